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

// Most pairs a chunk list keeps for R free slots: the superset rule's list grows past R only by
// the keys that share the R-th largest's digit; beyond R + R/4 the list is cut to the exact top R.
// (The merge holds R + R/4 <= 1280 candidates per list in registers at R = 1008.)
__host__ __device__ constexpr int list_cap(int R) { return R + (R >> 2); }

// Pairs a candidate list of a chunk of `chunk` positions can hold: at most list_cap(R), and never
// more than the chunk has positions.  The lists are laid out with this stride.
__host__ __device__ constexpr int list_capacity(int R, int chunk) {
  return list_cap(R) < chunk ? list_cap(R) : chunk;
}

// LDS words chunk_candidates needs besides its histogram (ITEMS: items per thread).
template <int THREADS, int ITEMS = 32>
constexpr int chunk_scratch_words() { return 3 * (THREADS / kWave) + 8 + ITEMS; }

// Candidates of one chunk: item j of this thread holds the key at position
// base + j*THREADS + threadIdx.x, or 0 if that position does not compete; m = number of
// competing items in the workgroup.  No per-item validity mask is kept: scores are finite, so a
// competing key is at least order_key(-inf) = 0x007fffff and the digit window, which starts at
// the smallest competing key >> s (s <= 21), starts at 1 or above; the absent key 0 therefore
// never enters a histogram, a boundary bin or the list.  Writes to `out`
// every valid key when m <= R, else a superset of the chunk's contribution to the row's top R:
// every key whose digit is at least that of the chunk's R-th largest.  When that superset would
// exceed `cap` pairs (cap >= R; many keys share the R-th largest's digit), narrower digits are
// taken inside the boundary bin until it fits, and if a single key value remains, the lowest
// positions among its copies fill the list up to exactly R -- the chunk's exact top R by (key
// descending, position ascending), which still holds every row winner from this chunk.  The
// pairs (key, position) go to `out`, their number to *count, and bounds lo <= every written
// key <= hi to range[0], range[1].  hist: 2*kBins words of LDS (8-byte aligned; it also
// stages the list before the stores), zeroed here; sh:
// chunk_scratch_words<THREADS, ITEMS>() words.  Call from every thread, with m >= 1.
// PREPARED: the caller has already zeroed hist (and ordered that before this call by a
// barrier) and passes in (mn, mx) bounds whose workgroup-wide min and max are those of the
// valid keys -- a scan that produced the keys can track them on the way.
template <int THREADS, int ITEMS, bool PREPARED = false>
__device__ void chunk_candidates(const uint32_t (&key)[ITEMS], int m, int R,
                                 int cap, int base, uint32_t* hist, uint32_t* sh, uint2* out,
                                 uint32_t* count, uint32_t* range, uint32_t mn = 0xffffffffu,
                                 uint32_t mx = 0u) {
  constexpr int WAVES = THREADS / kWave;
  constexpr int kPer = kBins / THREADS;
  static_assert(ITEMS <= 32, "keep masks are 32 bits");
  uint32_t* sh_scan = sh;
  uint32_t* sh_mm = sh + WAVES;
  uint32_t* sh_out = sh + 3 * WAVES;
  uint32_t* sh_tie = sh + 3 * WAVES + 8;  // [ITEMS] tied items per item index
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & (kWave - 1);
  uint32_t keep = 0;
  if constexpr (!PREPARED) {
    if (m > R)  // hist is 16-byte aligned
      for (int i = tid; i < 2 * kBins / 4; i += THREADS) reinterpret_cast<u32x4*>(hist)[i] = u32x4{0u, 0u, 0u, 0u};
    // key - 1 wraps the absent key 0 to the largest value, so it never lowers the minimum; it
    // never raises the maximum
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      mn = min(mn, key[j] - 1u);
      mx = max(mx, key[j]);
    }
    mn += 1u;  // a thread with no competing item keeps 0xffffffff (wrapped back to 0 here)
    mn = mn ? mn : 0xffffffffu;
  }
  block_minmax<WAVES>(mn, mx, sh_mm);  // its barrier also orders the zeroing
  uint32_t lo = mn;
  if (m > R) {
    int s_in = digit_shift(mn, mx);
    const uint32_t dbase = mn >> s_in;
    uint32_t* hw = hist + (wave & 1) * kBins;  // one copy per half of the waves
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const uint32_t d = (key[j] >> s_in) - dbase;  // wraps past kBins for the absent key 0
      if (d < static_cast<uint32_t>(kBins)) atomicAdd(&hw[bin_slot<THREADS>(d)], 1u);
    }
    __syncthreads();
    uint32_t c[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) c[i] = hist[i * THREADS + tid] + hist[kBins + i * THREADS + tid];
    select_bin<kPer, WAVES>(c, static_cast<uint32_t>(R), sh_scan, sh_out);
    // boundary bin: keys with (k >> s_in) == pref; `above` keys lie above it
    uint32_t pref = dbase + sh_out[0], above = sh_out[1], inbin = sh_out[2];
    bool tie_break = false;  // the boundary holds one key value; only some of its copies are kept
    uint32_t need = static_cast<uint32_t>(R) - above;
    while (above + inbin > static_cast<uint32_t>(cap)) {
      if (s_in == 0) {
        tie_break = true;
        break;
      }
      const int s2 = max(0, s_in - 12);
      const uint32_t base2 = pref << (s_in - s2);  // digits below 2^12 = kBins
      for (int i = tid; i < kBins; i += THREADS) hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < ITEMS; ++j)
        if ((key[j] >> s_in) == pref)
          atomicAdd(&hist[bin_slot<THREADS>((key[j] >> s2) - base2)], 1u);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kPer; ++i) c[i] = hist[i * THREADS + tid];
      select_bin<kPer, WAVES>(c, need, sh_scan, sh_out);
      pref = base2 + sh_out[0];
      above += sh_out[1];
      need -= sh_out[1];
      inbin = sh_out[2];
      s_in = s2;
    }
    lo = pref << s_in;  // no kept key is below the boundary bin
#pragma unroll
    for (int j = 0; j < ITEMS; ++j)
      keep |= ((key[j] >> s_in) >= pref ? 1u : 0u) << j;
    if (tie_break) {
      // `inbin` copies of the key `pref` and `need` of them kept: the lowest positions, i.e. by
      // item index j, then thread -- count the copies per j, find the item index j* where the
      // count reaches `need`, and rank the copies at j* by thread
      if (tid < ITEMS) sh_tie[tid] = 0u;
      __syncthreads();
      uint32_t tied = 0;
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        const bool t = key[j] == pref;
        tied |= (t ? 1u : 0u) << j;
        const uint32_t n = static_cast<uint32_t>(__popcll(wave_ballot(t)));
        if (lane == 0 && n) atomicAdd(&sh_tie[j], n);
      }
      __syncthreads();
      uint32_t before = 0;
      int jstar = ITEMS;
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        const uint32_t n = sh_tie[j];
        if (jstar == ITEMS && before + n >= need) jstar = j;
        else if (jstar == ITEMS) before += n;
      }
      uint32_t total;
      const uint32_t rank = block_prefix<WAVES>(jstar < ITEMS ? (tied >> jstar) & 1u : 0u, sh_scan, &total);
      // copies at j < j* are kept, at j* the first need - before by thread, after j* none
      const uint32_t lower = (jstar >= 32) ? 0xffffffffu : ((1u << jstar) - 1u);
      uint32_t drop = tied & ~lower;
      if (jstar < ITEMS && rank < need - before) drop &= ~(1u << jstar);
      keep &= ~drop;
      __syncthreads();  // every thread has read sh_scan before the stores below reuse it
    }
  } else {
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) keep |= (key[j] != 0u ? 1u : 0u) << j;
  }
  // Stores: each thread's kept items form one contiguous run at the exclusive prefix of the
  // kept counts (ordered by thread, then j; the list is a set).  A list of at most kBins pairs is
  // staged in LDS first -- the histogram is free once the prefix's barrier has passed -- so that
  // it leaves as consecutive 8-byte pairs across the lanes; a longer one is written directly.
  uint32_t total;
  uint32_t at = block_prefix<WAVES>(static_cast<uint32_t>(__popc(keep)), sh_scan, &total);
  if (total <= static_cast<uint32_t>(kBins)) {
    uint2* staged = reinterpret_cast<uint2*>(hist);  // 2 * kBins words
#pragma unroll
    for (int j = 0; j < ITEMS; ++j)
      if ((keep >> j) & 1u)
        staged[at++] = make_uint2(key[j], static_cast<uint32_t>(base + j * THREADS + tid));
    __syncthreads();
    for (uint32_t i = tid; i < total; i += THREADS) out[i] = staged[i];
  } else {
#pragma unroll
    for (int j = 0; j < ITEMS; ++j)
      if ((keep >> j) & 1u)
        out[at++] = make_uint2(key[j], static_cast<uint32_t>(base + j * THREADS + tid));
  }
  if (tid == 0) {
    *count = total;
    range[0] = lo;
    range[1] = mx;
  }
}

}  // namespace sel
}  // namespace lsa
