// Top-k selection with forced sink/window columns (stage 2 of the LSA hot path).
//
// Semantics (page "MLX-VLM 的 LongCat-Flash-Lite-Sparse ...", section "LSA"): keep the
// index_topk best-scoring keys of each query row, where the index_init_tokens first positions
// (sink) and the index_local_tokens most recent positions (sliding window) are forced in; a row
// with no more keys than index_topk keeps all of them.  Equal scores go to the lowest position
// and the output is ascending, so the selected set is unique.
//
// Design.  Scores become order-preserving uint32 keys (larger float <=> larger key, -0 == +0).
// In a row with n > topk the forced positions are the I lowest and the W highest, so they fill
// the first I and the last W output slots directly; only the middle positions [I, p - W]
// compete, for the R = topk - I - W slots in between.
//  1. chunk (many workgroups per row, one per 16384 positions): each keeps a superset of its
//     local top R -- every middle key whose digit is at least that of its local R-th largest,
//     found with an LDS histogram -- and writes them as (key, position) pairs with a count.
//     No global atomics and nothing that must be cleared beforehand.
//  2. merge (one workgroup per row): an exact radix select over the union of the chunk lists
//     (candidates held in registers) narrows the threshold to a bin of at most 1024 keys, which
//     are then ranked by (key descending, position ascending) in LDS.  Winners are set in an
//     LDS bitmap over the middle range, which a popcount prefix compacts into ascending
//     indices.
// Digits adapt to the data: a digit is a window of key bits placed from the min/max of the keys
// still in play ((k >> s) - base, at most 2^11 + 1 values), so scores concentrated in a narrow
// range still spread over the histogram instead of piling into a few bins.
// Every step counts exactly, so the result does not depend on scheduling.
#include <algorithm>

#include "lsa_internal.h"

namespace lsa {
namespace {

constexpr int kBins = 4096;          // 12-bit digit histograms
constexpr int kLowBins = 256;        // last 8-bit digit
constexpr int kChunk = 16384;        // positions per chunk workgroup
constexpr int kChunkThreads = 512;
constexpr int kChunkWaves = kChunkThreads / kWave;
constexpr int kChunkItems = kChunk / kChunkThreads;  // 32 per thread
constexpr int kMergeThreads = 1024;
constexpr int kMergeWaves = kMergeThreads / kWave;
constexpr int kRegItems = 16;        // candidates held in registers per merge thread
constexpr int kMaxPositions = 1 << 20;
constexpr int kMaxChunks = kMaxPositions / kChunk;  // 64
constexpr int kTieList = kMergeThreads;             // ties ranked in LDS up to this many
constexpr size_t kWorkspaceBudget = size_t(256) << 20;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) return 0x80000000u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct RowGeom {
  int n, p;    // visible keys, query position
  bool dense;  // n <= topk: keep everything
  int lo, hi;  // middle positions [lo, hi] (empty if dense)
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

struct TopkParams {
  const float* scores;
  const int32_t* seqlens;
  int Lq, S_max, topk, init, local, R;
  int row0;          // first row of this group
  int chunks;        // chunks per row
  uint32_t* count;   // [group rows][chunks]
  uint2* cand;       // [group rows][chunks][kChunk] (key, position)
  int32_t* indices;  // [rows][topk]
  int32_t* n_sel;    // [rows]
};

// Which bin holds the target-th largest item: thread t owns bins [PER*t, PER*t + PER) with
// counts c; afterwards out[0] = that bin, out[1] = the number of items in higher bins and
// out[2] = the items in that bin.
// Requires 1 <= target <= the sum of all counts.  Two barriers.
template <int PER, int WAVES>
__device__ void select_bin(const uint32_t (&c)[PER], uint32_t target, uint32_t* sh_scan,
                           uint32_t* out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) mine += c[i];
  uint32_t x = mine;  // inclusive suffix sum over the lanes of this wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_down(x, off);
    if (lane + off < 64) x += y;
  }
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
  uint32_t x = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
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
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mn = min(mn, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mn), off)));
    mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), off)));
  }
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

// ------------------------------------------------------------------ 1. per-chunk candidates
__global__ __launch_bounds__(kChunkThreads) void topk_chunk_kernel(TopkParams P) {
  __shared__ uint32_t h[2][kBins];  // one copy per half of the waves
  __shared__ uint32_t sh_scan[kChunkWaves];
  __shared__ uint32_t sh_mm[2 * kChunkWaves];
  __shared__ uint32_t sh_out[4];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int grow = blockIdx.x / P.chunks;  // row within the group
  const int chunk = blockIdx.x - grow * P.chunks;
  const int row = P.row0 + grow;
  const RowGeom g = row_geom(P.seqlens, row, P.Lq, P.S_max, P.topk, P.init, P.local);
  const int base = chunk * kChunk;
  const int a = max(g.lo, base), z = min(g.hi, base + kChunk - 1);
  const int m = (g.dense || P.R == 0) ? 0 : max(0, z - a + 1);  // competing positions here
  if (m == 0) {
    if (tid == 0) P.count[blockIdx.x] = 0u;
    return;
  }
  const float* srow = P.scores + static_cast<size_t>(row) * P.S_max;
  // all loads issued at once: out-of-range items read a clamped in-range address and are masked
  uint32_t key[kChunkItems];
  uint32_t valid = 0;
#pragma unroll
  for (int j = 0; j < kChunkItems; ++j) {
    const int s = base + j * kChunkThreads + tid;
    key[j] = order_key(srow[min(max(s, a), z)]);
    valid |= ((s >= a && s <= z) ? 1u : 0u) << j;
  }
  // keep every key when the chunk has no more than R of them, else the digits from the one
  // holding the local R-th largest upwards
  uint32_t keep = valid;
  if (m > P.R) {
    for (int i = tid; i < 2 * kBins; i += kChunkThreads) (&h[0][0])[i] = 0u;
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int j = 0; j < kChunkItems; ++j) {
      if (valid & (1u << j)) {
        mn = min(mn, key[j]);
        mx = max(mx, key[j]);
      }
    }
    block_minmax<kChunkWaves>(mn, mx, sh_mm);  // its barrier also orders the zeroing
    const int sh = digit_shift(mn, mx);
    const uint32_t dbase = mn >> sh;
    uint32_t* hw = h[wave & 1];
#pragma unroll
    for (int j = 0; j < kChunkItems; ++j)
      if (valid & (1u << j)) atomicAdd(&hw[(key[j] >> sh) - dbase], 1u);
    __syncthreads();
    constexpr int kPer = kBins / kChunkThreads;
    uint32_t c[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) c[i] = h[0][kPer * tid + i] + h[1][kPer * tid + i];
    select_bin<kPer, kChunkWaves>(c, static_cast<uint32_t>(P.R), sh_scan, sh_out);
    const uint32_t dmin = sh_out[0];
    keep = 0;
#pragma unroll
    for (int j = 0; j < kChunkItems; ++j)
      keep |= ((valid & (1u << j)) && (key[j] >> sh) - dbase >= dmin ? 1u : 0u) << j;
  }
  uint32_t total;
  uint32_t at = block_prefix<kChunkWaves>(__popc(keep), sh_scan, &total);
  uint2* out = P.cand + static_cast<size_t>(blockIdx.x) * kChunk;
#pragma unroll
  for (int j = 0; j < kChunkItems; ++j) {
    if (keep & (1u << j)) {
      out[at] = make_uint2(key[j], static_cast<uint32_t>(base + j * kChunkThreads + tid));
      ++at;
    }
  }
  if (tid == 0) P.count[blockIdx.x] = total;
}

// ------------------------------------------------------------------ 2. merge per row
// Dynamic LDS layout of the merge kernel (32-bit words).
constexpr int kMsScan = 0;                          // [kMergeWaves]
constexpr int kMsRes = kMsScan + kMergeWaves;       // [16] results of select_bin / counters
constexpr int kMsCnt = kMsRes + 16;                 // [2][kMergeWaves] block_count / min-max
constexpr int kMsOff = kMsCnt + 2 * kMergeWaves;    // [kMaxChunks + 1] candidate offsets
constexpr int kMsHist = kMsOff + kMaxChunks + 16;   // [kBins] radix rounds, then the rank list
constexpr int kMsBits = kMsHist + kBins;            // bitmap over the middle range
static_assert(2 * kTieList <= kBins, "the rank list reuses the histogram");

// Block-wide sum of a per-thread count (one barrier; alternating slots).
__device__ __forceinline__ uint32_t block_count(uint32_t v, uint32_t* cnt, int& parity) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if (lane == 0) cnt[parity * kMergeWaves + wave] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) t += cnt[parity * kMergeWaves + w];
  parity ^= 1;
  return t;
}

__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(TopkParams P) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  uint32_t* sh_scan = lds + kMsScan;
  uint32_t* sh_res = lds + kMsRes;
  uint32_t* sh_cnt = lds + kMsCnt;
  uint32_t* sh_off = lds + kMsOff;
  uint32_t* sh_h = lds + kMsHist;
  uint32_t* sh_lk = lds + kMsHist;                                     // rank list keys
  int32_t* sh_lp = reinterpret_cast<int32_t*>(lds + kMsHist + kTieList);  // rank list positions
  uint32_t* sh_bits = lds + kMsBits;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grow = blockIdx.x;
  const int row = P.row0 + grow;
  const RowGeom g = row_geom(P.seqlens, row, P.Lq, P.S_max, P.topk, P.init, P.local);
  const int K = P.topk, I = P.init, W = P.local, R = P.R;
  int32_t* out = P.indices + static_cast<size_t>(row) * K;
  if (g.dense) {  // every visible position, then padding
    for (int j = tid; j < K; j += kMergeThreads) out[j] = j < g.n ? j : -1;
    if (tid == 0) P.n_sel[row] = max(g.n, 0);
    return;
  }
  // forced positions: the I lowest and the W highest fill the ends of the output
  for (int j = tid; j < I; j += kMergeThreads) out[j] = j;
  for (int j = tid; j < W; j += kMergeThreads) out[K - W + j] = g.p - W + 1 + j;
  if (tid == 0) P.n_sel[row] = K;
  if (R == 0) return;

  const int mid_words = (g.hi - g.lo + 32) >> 5;
  for (int i = tid; i < mid_words; i += kMergeThreads) sh_bits[i] = 0u;
  for (int i = tid; i < kBins; i += kMergeThreads) sh_h[i] = 0u;
  if (tid == 0) sh_res[8] = 0u;  // rank-list length
  // candidate offsets of the row's chunks (one wave: at most 64 chunks)
  const uint32_t* cnt = P.count + static_cast<size_t>(grow) * P.chunks;
  if (wave == 0) {
    const uint32_t c = lane < P.chunks ? cnt[lane] : 0u;
    uint32_t x = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    sh_off[lane] = x - c;
    if (lane == 63) sh_off[64] = x;
  }
  __syncthreads();
  const uint32_t nc = sh_off[64];
  const uint2* crow = P.cand + static_cast<size_t>(grow) * P.chunks * kChunk;
  // candidate q of the concatenated lists -> its pair
  auto locate = [&](uint32_t q) -> const uint2* {
    int lo = 0, hi = P.chunks - 1;  // last chunk c with sh_off[c] <= q
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sh_off[mid] <= q) lo = mid; else hi = mid - 1;
    }
    return crow + static_cast<size_t>(lo) * kChunk + (q - sh_off[lo]);
  };
  const bool in_regs = nc <= static_cast<uint32_t>(kRegItems * kMergeThreads);
  uint32_t rk[kRegItems];
  int32_t rp[kRegItems];
  if (in_regs) {
    const uint2* src[kRegItems];
#pragma unroll
    for (int i = 0; i < kRegItems; ++i) {
      const uint32_t q = static_cast<uint32_t>(i * kMergeThreads + tid);
      src[i] = q < nc ? locate(q) : crow;  // crow[0] is always readable
    }
#pragma unroll
    for (int i = 0; i < kRegItems; ++i) {  // all loads issued at once
      const uint2 v = *src[i];
      rk[i] = v.x;
      rp[i] = static_cast<int32_t>(v.y);
    }
  }
  auto each = [&](auto f) {
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < kRegItems; ++i)
        if (static_cast<uint32_t>(i * kMergeThreads + tid) < nc) f(rk[i], rp[i]);
    } else {
      for (uint32_t q = tid; q < nc; q += kMergeThreads) {
        const uint2 v = *locate(q);
        f(v.x, static_cast<int32_t>(v.y));
      }
    }
  };
  // radix rounds over adaptive digits.  Keys still in play are those with (k >> s_in) == pref
  // (all of them while s_in == 32); a round histograms the digit (k >> s) - dbase of those keys,
  // finds the digit of the need-th largest and narrows to it.
  uint32_t mn = 0xffffffffu, mx = 0u;
  each([&](uint32_t k, int32_t) {
    mn = min(mn, k);
    mx = max(mx, k);
  });
  block_minmax<kMergeWaves>(mn, mx, sh_cnt);
  int s_in = 32, s = digit_shift(mn, mx);
  uint32_t pref = 0, dbase = mn >> s;
  uint32_t need = static_cast<uint32_t>(R), pop;
  auto in_play = [&](uint32_t k) { return s_in >= 32 || (k >> s_in) == pref; };
  for (;;) {
    each([&](uint32_t k, int32_t) {
      if (in_play(k)) atomicAdd(&sh_h[(k >> s) - dbase], 1u);
    });
    __syncthreads();
    constexpr int kPer = kBins / kMergeThreads;
    uint32_t c[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) c[i] = sh_h[kPer * tid + i];
    select_bin<kPer, kMergeWaves>(c, need, sh_scan, sh_res);
    need -= sh_res[1];
    pop = sh_res[2];
    pref = dbase + sh_res[0];
    s_in = s;
    if (pop <= static_cast<uint32_t>(kTieList) || s == 0) break;
    const int s_next = max(0, s - 12);
    dbase = pref << (s - s_next);
    s = s_next;
    for (int i = tid; i < kBins; i += kMergeThreads) sh_h[i] = 0u;
    __syncthreads();
  }
  // keys above the final bin win; `need` of the `pop` keys in it win too
  const int lo = g.lo;
  auto set_bit = [&](int32_t p) { atomicOr(&sh_bits[(p - lo) >> 5], 1u << ((p - lo) & 31)); };
  each([&](uint32_t k, int32_t p) {
    if ((k >> s_in) > pref || (need == pop && (k >> s_in) == pref)) set_bit(p);
  });
  if (need < pop) {
    if (pop <= static_cast<uint32_t>(kTieList)) {
      // rank the bin's keys by (key descending, position ascending)
      each([&](uint32_t k, int32_t p) {
        if ((k >> s_in) == pref) {
          const uint32_t slot = atomicAdd(&sh_res[8], 1u);
          sh_lk[slot] = k;
          sh_lp[slot] = p;
        }
      });
      __syncthreads();
      if (static_cast<uint32_t>(tid) < pop) {
        const uint32_t kt = sh_lk[tid];
        const int32_t pt = sh_lp[tid];
        uint32_t rank = 0;
        for (uint32_t u = 0; u < pop; ++u) {
          const uint32_t ku = sh_lk[u];
          rank += (ku > kt || (ku == kt && sh_lp[u] < pt)) ? 1u : 0u;
        }
        if (rank < need) set_bit(pt);
      }
    } else {  // more than kTieList equal keys (s_in == 0): bisect for the cut-off position
      int parity = 0, cut = -1;
      for (int bit = 20; bit >= 0; --bit) {
        const int mid = cut + (1 << bit);
        if (mid >= P.S_max) continue;
        uint32_t v = 0;
        each([&](uint32_t k, int32_t p) { v += (k == pref && p <= mid) ? 1u : 0u; });
        if (block_count(v, sh_cnt, parity) < need) cut = mid;
      }
      each([&](uint32_t k, int32_t p) {
        if (k == pref && p <= cut + 1) set_bit(p);
      });
    }
  }
  __syncthreads();
  // compact the middle bitmap into out[I .. I + R)
  const int wpt = (mid_words + kMergeThreads - 1) / kMergeThreads;
  const int w0 = tid * wpt, w1 = min(mid_words, w0 + wpt);
  uint32_t mine = 0;
  for (int w = w0; w < w1; ++w) mine += __popc(sh_bits[w]);
  uint32_t total;
  uint32_t at = block_prefix<kMergeWaves>(mine, sh_scan, &total);
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = sh_bits[w];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      if (at < static_cast<uint32_t>(R)) out[I + at] = lo + 32 * w + b;
      ++at;
    }
  }
}

struct Plan {
  long rows = 0;
  int R = 0, chunks = 1;
  long group = 1;  // rows per launch pair
  size_t count_bytes = 0, cand_bytes = 0;
  size_t total() const { return count_bytes + cand_bytes; }
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

Plan make_plan(int B, int Lq, int S_max, int topk, int init_tokens, int local_tokens) {
  Plan pl;
  pl.rows = static_cast<long>(B) * Lq;
  pl.R = topk - init_tokens - local_tokens;
  pl.chunks = (S_max + kChunk - 1) / kChunk;
  const size_t per_row = static_cast<size_t>(pl.chunks) * kChunk * sizeof(uint2);
  pl.group = std::max<long>(1, std::min<long>(pl.rows, static_cast<long>(kWorkspaceBudget / per_row)));
  pl.count_bytes = align256(static_cast<size_t>(pl.group) * pl.chunks * 4);
  pl.cand_bytes = static_cast<size_t>(pl.group) * per_row;
  return pl;
}

size_t merge_lds_bytes(int S_max) {
  return sizeof(uint32_t) * (static_cast<size_t>(kMsBits) + (S_max + 31) / 32 + 1);
}

}  // namespace

int topk_max_positions() { return kMaxPositions; }

size_t topk_workspace_bytes(int B, int Lq, int S_max, int topk, int init_tokens, int local_tokens) {
  return make_plan(B, Lq, S_max, topk, init_tokens, local_tokens).total();
}

hipError_t launch_topk(const float* scores, const int32_t* seqlens, int B, int Lq, int S_max,
                       int topk, int init_tokens, int local_tokens, int32_t* indices,
                       int32_t* n_sel, void* workspace, hipStream_t stream) {
  const Plan pl = make_plan(B, Lq, S_max, topk, init_tokens, local_tokens);
  if (pl.group * pl.chunks > 0x7fffffffL || pl.rows > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const size_t lds = merge_lds_bytes(S_max);
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(topk_merge_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (err != hipSuccess) return err;
  TopkParams P{};
  P.scores = scores;
  P.seqlens = seqlens;
  P.Lq = Lq;
  P.S_max = S_max;
  P.topk = topk;
  P.init = init_tokens;
  P.local = local_tokens;
  P.R = pl.R;
  P.chunks = pl.chunks;
  char* ws = static_cast<char*>(workspace);
  P.count = reinterpret_cast<uint32_t*>(ws);
  P.cand = reinterpret_cast<uint2*>(ws + pl.count_bytes);
  P.indices = indices;
  P.n_sel = n_sel;
  for (long r0 = 0; r0 < pl.rows; r0 += pl.group) {
    const long g = std::min(pl.group, pl.rows - r0);
    P.row0 = static_cast<int>(r0);
    hipLaunchKernelGGL(topk_chunk_kernel, dim3(static_cast<unsigned>(g * pl.chunks)), dim3(kChunkThreads), 0,
                       stream, P);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(static_cast<unsigned>(g)), dim3(kMergeThreads), lds, stream, P);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace lsa
