// Device helpers of the top-k selection shared by the standalone top-k kernels and the fused
// indexer + top-k kernel (not installed).
//
// Scores are ranked through order-preserving uint32 keys: a larger float gives a larger key,
// and -0 and +0 give the same key.  A chunk keeps a superset of its own top R keys (every key
// whose digit is at least the digit of its R-th largest), where a digit is a window of key bits
// placed from the chunk's key range: (k >> s) - (min >> s) takes at most 2^11 + 1 values, so
// scores concentrated in a narrow range still spread over the LDS histogram.
#pragma once

#include "lsa_internal.h"

namespace lsa {
namespace sel {

constexpr int kBins = 4096;  // histogram bins (digits are at most 2^11)

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) return 0x80000000u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Positions of one query row as the selection sees them.
struct RowGeom {
  int n, p;    // visible keys, query position
  bool dense;  // n <= topk: keep everything
  int lo, hi;  // middle positions [lo, hi] that compete for the free slots (empty if dense)
};

__device__ __forceinline__ RowGeom row_geom(const int32_t* seqlens, int row, int Lq, int S_max,
                                            int topk, int I, int W) {
  RowGeom g;
  const int b = row / Lq;
  g.n = min(seqlens[b] - Lq + (row - b * Lq) + 1, S_max);
  g.p = g.n - 1;
  g.dense = g.n <= topk;
  g.lo = I;
  g.hi = g.dense ? I - 1 : g.p - W;
  return g;
}

// LDS word of histogram bin d when each of THREADS threads owns PER = kBins / THREADS
// consecutive bins: bin PER*t + i sits at word i*THREADS + t, so when every owner reads its
// i-th bin the workgroup reads consecutive words (no bank conflicts).
template <int THREADS>
__device__ __forceinline__ uint32_t bin_slot(uint32_t d) {
  constexpr uint32_t PER = kBins / THREADS;
  static_assert(PER * THREADS == kBins && (PER & (PER - 1)) == 0, "power-of-two split");
  return (d % PER) * THREADS + d / PER;
}

// Which bin holds the target-th largest item: thread t owns bins [PER*t, PER*t + PER) with
// counts c; afterwards out[0] = that bin, out[1] = the number of items in higher bins and
// out[2] = the items in that bin.  Requires 1 <= target <= the sum of all counts.  Two barriers.
template <int PER, int WAVES>
__device__ void select_bin(const uint32_t (&c)[PER], uint32_t target, uint32_t* sh_scan,
                           uint32_t* out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) mine += c[i];
  // inclusive suffix sum over the lanes of this wave: the wave total minus the exclusive prefix
  const uint32_t pre = wave_prefix_sum(mine);
  const uint32_t x = wave_last(pre) - pre + mine;
  if (lane == 0) sh_scan[wave] = x;
  __syncthreads();
  uint32_t acc = x - mine;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) acc += w > wave ? sh_scan[w] : 0u;
#pragma unroll
  for (int i = PER - 1; i >= 0; --i) {
    if (acc < target && acc + c[i] >= target) {
      out[0] = static_cast<uint32_t>(PER * tid + i);
      out[1] = acc;
      out[2] = c[i];
    }
    acc += c[i];
  }
  __syncthreads();
}

// Exclusive prefix of a per-thread count over the workgroup, and the total.  One barrier.
template <int WAVES>
__device__ __forceinline__ uint32_t block_prefix(uint32_t mine, uint32_t* sh_scan, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_prefix_sum(mine);
  if (lane == 63) sh_scan[wave] = x;
  __syncthreads();
  uint32_t at = x - mine, t = 0;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    at += w < wave ? sh_scan[w] : 0u;
    t += sh_scan[w];
  }
  *total = t;
  return at;
}

// Minimum and maximum of per-thread values over the workgroup.  One barrier; sh holds 2*WAVES.
template <int WAVES>
__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, uint32_t* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (lane == 0) {
    sh[wave] = mn;
    sh[WAVES + wave] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    mn = min(mn, sh[w]);
    mx = max(mx, sh[WAVES + w]);
  }
}

// Shift s for keys in [mn, mx] such that (k >> s) - (mn >> s) <= 2^11 for all of them.
__device__ __forceinline__ int digit_shift(uint32_t mn, uint32_t mx) {
  const uint32_t d = mx - mn;
  const int bits = d ? 32 - __clz(static_cast<int>(d)) : 0;
  return max(0, bits - 11);
}

// LDS words chunk_candidates needs besides its histogram.
template <int THREADS>
constexpr int chunk_scratch_words() { return 3 * (THREADS / kWave) + 4; }

// Candidates of one chunk: item j of this thread (bit j of `valid`) holds the key at position
// base + j*THREADS + threadIdx.x; m = number of valid items in the workgroup.  Writes to `out`
// every valid key when m <= R, else those whose digit is at least that of the chunk's R-th
// largest (always a superset of the chunk's contribution to the row's top R), as (key,
// position) pairs, their number to *count, and bounds lo <= every written key <= hi to
// range[0], range[1].  hist: 2*kBins words of LDS, zeroed here; sh:
// chunk_scratch_words<THREADS>() words.  Call from every thread, with m >= 1.
// PREPARED: the caller has already zeroed hist (and ordered that before this call by a
// barrier) and passes in (mn, mx) bounds whose workgroup-wide min and max are those of the
// valid keys -- a scan that produced the keys can track them on the way.
template <int THREADS, int ITEMS, bool PREPARED = false>
__device__ void chunk_candidates(const uint32_t (&key)[ITEMS], uint32_t valid, int m, int R,
                                 int base, uint32_t* hist, uint32_t* sh, uint2* out,
                                 uint32_t* count, uint32_t* range, uint32_t mn = 0xffffffffu,
                                 uint32_t mx = 0u) {
  constexpr int WAVES = THREADS / kWave;
  uint32_t* sh_scan = sh;
  uint32_t* sh_mm = sh + WAVES;
  uint32_t* sh_out = sh + 3 * WAVES;
  const int tid = threadIdx.x, wave = tid >> 6;
  uint32_t keep = valid;
  if constexpr (!PREPARED) {
    if (m > R)  // hist is 16-byte aligned
      for (int i = tid; i < 2 * kBins / 4; i += THREADS) reinterpret_cast<u32x4*>(hist)[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      if (valid & (1u << j)) {
        mn = min(mn, key[j]);
        mx = max(mx, key[j]);
      }
    }
  }
  block_minmax<WAVES>(mn, mx, sh_mm);  // its barrier also orders the zeroing
  uint32_t lo = mn;
  if (m > R) {
    const int sh_bits = digit_shift(mn, mx);
    const uint32_t dbase = mn >> sh_bits;
    uint32_t* hw = hist + (wave & 1) * kBins;  // one copy per half of the waves
#pragma unroll
    for (int j = 0; j < ITEMS; ++j)
      if (valid & (1u << j)) atomicAdd(&hw[bin_slot<THREADS>((key[j] >> sh_bits) - dbase)], 1u);
    __syncthreads();
    constexpr int kPer = kBins / THREADS;
    uint32_t c[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) c[i] = hist[i * THREADS + tid] + hist[kBins + i * THREADS + tid];
    select_bin<kPer, WAVES>(c, static_cast<uint32_t>(R), sh_scan, sh_out);
    const uint32_t dmin = sh_out[0];
    lo = (dbase + dmin) << sh_bits;  // no kept key is below the first kept digit
    keep = 0;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j)
      keep |= ((valid & (1u << j)) && (key[j] >> sh_bits) - dbase >= dmin ? 1u : 0u) << j;
  }
  // Stores: the kept items of one wavefront and one item index j go to one contiguous run
  // (ordered by wavefront, then j, then lane; the list is a set).
  uint32_t mine = 0;  // this wavefront's kept items
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) mine += static_cast<uint32_t>(__popcll(wave_ballot((keep >> j) & 1u)));
  if ((tid & (kWave - 1)) == 0) sh_scan[wave] = mine;
  __syncthreads();
  uint32_t at = 0, total = 0;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    at += w < wave ? sh_scan[w] : 0u;
    total += sh_scan[w];
  }
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const uint64_t bj = wave_ballot((keep >> j) & 1u);
    if ((keep >> j) & 1u)
      out[at + lanes_below(bj)] = make_uint2(key[j], static_cast<uint32_t>(base + j * THREADS + tid));
    at += static_cast<uint32_t>(__popcll(bj));
  }
  if (tid == 0) {
    *count = total;
    range[0] = lo;
    range[1] = mx;
  }
}

}  // namespace sel
}  // namespace lsa
