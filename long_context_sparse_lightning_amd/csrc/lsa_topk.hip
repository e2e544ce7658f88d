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
#include <atomic>

#include "lsa_select.h"

namespace lsa {
namespace {

using sel::bin_slot;
using sel::block_minmax;
using sel::block_prefix;
using sel::digit_shift;
using sel::kBins;
using sel::order_key;
using sel::row_geom;
using sel::RowGeom;
using sel::select_bin;

constexpr int kChunk = 16384;        // positions per chunk workgroup
constexpr int kChunkThreads = 512;
constexpr int kChunkItems = kChunk / kChunkThreads;  // 32 per thread
constexpr int kMergeThreads = 1024;
constexpr int kMergeWaves = kMergeThreads / kWave;
constexpr int kRegItems = 20;        // candidates held in registers per merge thread
constexpr int kMaxPositions = 1 << 20;
constexpr int kMaxChunks = 128;      // chunk lists per row the merge accepts
constexpr int kTieList = kMergeThreads;             // ties ranked in LDS up to this many
constexpr size_t kWorkspaceBudget = size_t(1024) << 20;

struct TopkParams {
  const float* scores;
  const int32_t* seqlens;
  int Lq, S_max, topk, init, local, R;
  int row0;          // first row of this group
  int chunks;        // chunk lists per row
  int chunk_keys;    // positions per chunk (= capacity of its list)
  uint32_t* count;   // [group rows][chunks]
  uint32_t* range;   // [group rows][chunks][2] bounds of each list's keys
  uint2* cand;       // [group rows][chunks][chunk_keys] (key, position)
  int32_t* indices;  // [rows][topk]
  int32_t* n_sel;    // [rows]
};

// ------------------------------------------------------------------ 1. per-chunk candidates
// at most 128 VGPRs, so two 512-thread workgroups share a CU and overlap their load waits
__global__ __launch_bounds__(kChunkThreads, 4) void topk_chunk_kernel(TopkParams P) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[2 * kBins];
  __shared__ uint32_t sh[sel::chunk_scratch_words<kChunkThreads>()];
  const int tid = threadIdx.x;
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
  sel::chunk_candidates<kChunkThreads, kChunkItems>(key, valid, m, P.R, base, hist, sh,
                                                    P.cand + static_cast<size_t>(blockIdx.x) * kChunk,
                                                    P.count + blockIdx.x, P.range + 2 * blockIdx.x);
}

// ------------------------------------------------------------------ 2. merge per row
// Dynamic LDS layout of the merge kernel (32-bit words).
constexpr int kMsScan = 0;                          // [kMergeWaves]
constexpr int kMsRes = kMsScan + kMergeWaves;       // [16] results of select_bin / counters
constexpr int kMsCnt = kMsRes + 16;                 // [2][kMergeWaves] spare
constexpr int kMsOff = kMsCnt + 2 * kMergeWaves;    // [kMaxChunks + 1] candidate offsets
constexpr int kMsHist = kMsOff + kMaxChunks + 16;   // [kBins] radix rounds, then the rank list
static_assert(kMaxChunks <= kMergeThreads, "one thread per chunk list");
constexpr int kMsBits = kMsHist + kBins;            // bitmap over the middle range
static_assert(2 * kTieList <= kBins, "the rank list reuses the histogram");

__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(TopkParams P) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  uint32_t* sh_scan = lds + kMsScan;
  uint32_t* sh_res = lds + kMsRes;
  uint32_t* sh_off = lds + kMsOff;
  uint32_t* sh_h = lds + kMsHist;
  uint32_t* sh_lk = lds + kMsHist;                                     // rank list keys
  int32_t* sh_lp = reinterpret_cast<int32_t*>(lds + kMsHist + kTieList);  // rank list positions
  uint32_t* sh_bits = lds + kMsBits;
  const int tid = threadIdx.x;
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
  // list lengths and key bounds (thread c: list c), requested first: loads complete in order
  const size_t lc = static_cast<size_t>(grow) * P.chunks + tid;
  const uint32_t c_len = tid < P.chunks ? P.count[lc] : 0u;
  const uint32_t c_lo = tid < P.chunks ? P.range[2 * lc] : 0xffffffffu;
  const uint32_t c_hi = tid < P.chunks ? P.range[2 * lc + 1] : 0u;
  const size_t ck = static_cast<size_t>(P.chunk_keys);
  const uint2* crow = P.cand + static_cast<size_t>(grow) * P.chunks * ck;
  // candidate offsets of the row's lists (thread c: list c), the longest list, the key bounds
  if (tid == 0) {
    sh_res[9] = 0u;
    sh_res[10] = 0xffffffffu;
    sh_res[11] = 0u;
  }
  {
    uint32_t total;
    const uint32_t at = block_prefix<kMergeWaves>(c_len, sh_scan, &total);
    if (tid < P.chunks) {
      sh_off[tid] = at;
      atomicMax(&sh_res[9], c_len);
      if (c_len > 0) {
        atomicMin(&sh_res[10], c_lo);
        atomicMax(&sh_res[11], c_hi);
      }
    }
    if (tid == 0) sh_off[kMaxChunks] = total;
  }
  __syncthreads();
  const uint32_t nc = sh_off[kMaxChunks];
  // candidate q of the concatenated lists -> its pair
  auto locate = [&](uint32_t q) -> const uint2* {
    int lo = 0, hi = P.chunks - 1;  // last chunk c with sh_off[c] <= q
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sh_off[mid] <= q) lo = mid; else hi = mid - 1;
    }
    return crow + static_cast<size_t>(lo) * ck + (q - sh_off[lo]);
  };
  // in registers: list c is held by the TPL threads [c * TPL, (c + 1) * TPL), entry j of it by
  // thread c * TPL + j % TPL in slot j / TPL -- when every list fits
  const int tpl = kMergeThreads / P.chunks;
  const int my_list = tid / tpl, my_j = tid - my_list * tpl;
  const bool in_regs = sh_res[9] <= static_cast<uint32_t>(kRegItems * tpl);
  uint32_t rk[kRegItems];
  int32_t rp[kRegItems];
  uint32_t held = 0;  // bit i: slot i holds a candidate
  if (in_regs) {
    const uint32_t my_cnt =
        my_list < P.chunks ? (my_list + 1 < P.chunks ? sh_off[my_list + 1] : nc) - sh_off[my_list] : 0u;
    const uint2* lst = crow + static_cast<size_t>(my_list < P.chunks ? my_list : 0) * ck;
#pragma unroll
    for (int i = 0; i < kRegItems; ++i) {  // all loads issued at once, from in-range addresses
      const uint32_t j = static_cast<uint32_t>(my_j + i * tpl);
      const bool ok = j < my_cnt;
      const uint2 v = lst[ok ? j : 0u];
      rk[i] = v.x;
      rp[i] = static_cast<int32_t>(v.y);
      held |= (ok ? 1u : 0u) << i;
    }
  }
  auto each = [&](auto f) {
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < kRegItems; ++i)
        if (held & (1u << i)) f(rk[i], rp[i]);
    } else {
      for (uint32_t q = tid; q < nc; q += kMergeThreads) {
        const uint2 v = *locate(q);
        f(v.x, static_cast<int32_t>(v.y));
      }
    }
  };
  // radix rounds over adaptive digits.  Keys still in play are those with (k >> s_in) == pref
  // (all of them while s_in == 32); a round histograms the digit (k >> s) - dbase of those keys,
  // finds the digit of the need-th largest and narrows to it.  The first window comes from the
  // key bounds the chunk lists carry.
  const uint32_t mn = sh_res[10], mx = sh_res[11];
  int s_in = 32, s = digit_shift(mn, mx);
  uint32_t pref = 0, dbase = mn >> s;
  uint32_t need = static_cast<uint32_t>(R), pop;
  auto in_play = [&](uint32_t k) { return s_in >= 32 || (k >> s_in) == pref; };
  for (;;) {
    each([&](uint32_t k, int32_t) {
      if (in_play(k)) atomicAdd(&sh_h[bin_slot<kMergeThreads>((k >> s) - dbase)], 1u);
    });
    __syncthreads();
    constexpr int kPer = kBins / kMergeThreads;
    uint32_t c[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) c[i] = sh_h[i * kMergeThreads + tid];
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
    } else {
      // more than kTieList equal keys (s_in == 0): the `need` lowest positions among them, by a
      // radix select on the position (below 2^20): its top 12 bits, then its low 8.  Digits are
      // mirrored so that select_bin's target-th largest is the target-th lowest position.
      constexpr int kPer = kBins / kMergeThreads;
      uint32_t want = need, hi_digit = 0, cut = 0;
      for (int round = 0; round < 2; ++round) {
        for (int i = tid; i < kBins; i += kMergeThreads) sh_h[i] = 0u;
        __syncthreads();
        each([&](uint32_t k, int32_t p) {
          const uint32_t u = static_cast<uint32_t>(p);
          if (k != pref) return;
          if (round == 0) atomicAdd(&sh_h[bin_slot<kMergeThreads>(kBins - 1 - (u >> 8))], 1u);
          else if ((u >> 8) == hi_digit) atomicAdd(&sh_h[bin_slot<kMergeThreads>(kBins - 1 - (u & 255u))], 1u);
        });
        __syncthreads();
        uint32_t c[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) c[i] = sh_h[i * kMergeThreads + tid];
        select_bin<kPer, kMergeWaves>(c, want, sh_scan, sh_res);
        want -= sh_res[1];
        const uint32_t d = kBins - 1 - sh_res[0];
        if (round == 0) hi_digit = d;
        else cut = (hi_digit << 8) | d;
      }
      each([&](uint32_t k, int32_t p) {
        if (k == pref && static_cast<uint32_t>(p) <= cut) set_bit(p);
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
  size_t count_bytes = 0, range_bytes = 0, cand_bytes = 0;
  size_t total() const { return count_bytes + range_bytes + cand_bytes + kWorkspaceAlign; }
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
  pl.range_bytes = align256(static_cast<size_t>(pl.group) * pl.chunks * 8);
  pl.cand_bytes = static_cast<size_t>(pl.group) * per_row;
  return pl;
}

size_t merge_lds_bytes(int S_max) {
  return sizeof(uint32_t) * (static_cast<size_t>(kMsBits) + (S_max + 31) / 32 + 1);
}

// The attribute is a maximum: it is raised only when a launch needs more than the device's
// current setting, so calls of different sizes do not reset it back and forth.
hipError_t set_merge_lds(size_t lds) {
  constexpr int kDevices = 64;
  static std::atomic<size_t> set_to[kDevices];
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev >= 0 && dev < kDevices && set_to[dev].load(std::memory_order_relaxed) >= lds) return hipSuccess;
  err = hipFuncSetAttribute(reinterpret_cast<const void*>(topk_merge_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (err == hipSuccess && dev >= 0 && dev < kDevices) {
    size_t cur = set_to[dev].load(std::memory_order_relaxed);
    while (cur < lds && !set_to[dev].compare_exchange_weak(cur, lds)) {
    }
  }
  return err;
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
  hipError_t err = set_merge_lds(lds);
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
  P.chunk_keys = kChunk;
  char* ws = align_workspace(workspace);
  P.count = reinterpret_cast<uint32_t*>(ws);
  P.range = reinterpret_cast<uint32_t*>(ws + pl.count_bytes);
  P.cand = reinterpret_cast<uint2*>(ws + pl.count_bytes + pl.range_bytes);
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

int topk_merge_max_chunks() { return kMaxChunks; }

hipError_t launch_topk_merge(const int32_t* seqlens, int Lq, int S_max, int topk, int init_tokens,
                             int local_tokens, int row0, int rows, int chunks, int chunk_keys,
                             uint32_t* count, uint32_t* range, uint2* cand, int32_t* indices,
                             int32_t* n_sel, hipStream_t stream) {
  if (chunks > kMaxChunks || rows <= 0) return hipErrorInvalidConfiguration;
  const size_t lds = merge_lds_bytes(S_max);
  hipError_t err = set_merge_lds(lds);
  if (err != hipSuccess) return err;
  TopkParams P{};
  P.seqlens = seqlens;
  P.Lq = Lq;
  P.S_max = S_max;
  P.topk = topk;
  P.init = init_tokens;
  P.local = local_tokens;
  P.R = topk - init_tokens - local_tokens;
  P.row0 = row0;
  P.chunks = chunks;
  P.chunk_keys = chunk_keys;
  P.count = count;
  P.range = range;
  P.cand = cand;
  P.indices = indices;
  P.n_sel = n_sel;
  hipLaunchKernelGGL(topk_merge_kernel, dim3(static_cast<unsigned>(rows)), dim3(kMergeThreads), lds, stream, P);
  return hipGetLastError();
}

}  // namespace lsa
