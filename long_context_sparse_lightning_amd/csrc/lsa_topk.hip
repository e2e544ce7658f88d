// Top-k selection with forced sink/window columns (stage 2 of the LSA hot path).
//
// Semantics (page "MLX-VLM 的 LongCat-Flash-Lite-Sparse ...", section "LSA"): keep the
// index_topk best-scoring keys of each query row, where the index_init_tokens first positions
// (sink) and the index_local_tokens most recent positions (sliding window) are forced in; a row
// with no more keys than index_topk keeps all of them.  Equal scores go to the lowest position
// and the output is ascending, so the selected set is unique.
//
// Design.  The forced columns are written directly, so only the middle positions
// [init, p - local] compete for R = topk - init - local slots.  Scores become order-preserving
// uint32 keys (larger float <=> larger key, -0 == +0), and the selection runs as a tree:
//  * level 0: each 1024-thread workgroup takes a 16384-position chunk of one row (16 items per
//    thread, coalesced) and keeps that chunk's best R positions under the order
//    (key desc, position asc);
//  * merge levels: one workgroup takes the candidate lists of up to floor(16384 / R) chunks
//    and keeps the best R again, until one list per row remains.
// Every element of the row's best R is in its own chunk's best R, so the tree is exact.
// Inside a workgroup: a 3-pass radix select (11, 11 and 10 bits) with a replicated LDS
// histogram finds the exact threshold key T and how many items equal to T are still needed;
// then wavefront ballots with lane prefix counts (mbcnt) rank the tied items by position and
// compact the selected ones in position order.  Nothing depends on atomics' ordering, so the
// output is deterministic.
#include "lsa_internal.h"

namespace lsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kItems = 16;                     // items per thread
constexpr int kSegItems = kThreads * kItems;   // 16384 items per workgroup
constexpr int kBins = 2048;
constexpr int kRep = 4;                        // histogram replicas (fewer same-address atomics)

struct TopkParams {
  const float* scores;
  const int32_t* seqlens;
  int Lq, S_max, topk, init, local, R;
  // candidate lists read by merge levels: [rows][nseg_in][R] keys / positions, [rows][nseg_in] counts
  const uint32_t* in_key;
  const int32_t* in_pos;
  const int32_t* in_cnt;
  int nseg_in, group;
  // candidate lists written by non-final levels
  uint32_t* out_key;
  int32_t* out_pos;
  int32_t* out_cnt;
  int nseg_out;
  // final output
  int32_t* indices;
  int32_t* n_sel;
};

struct TopkShared {
  uint32_t hist[kRep][kBins];
  uint32_t wave_a[kWaves];
  uint32_t wave_b[kWaves];
  uint32_t digit, above;
};

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) return 0x80000000u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Sum of v over all threads with a larger thread index (exclusive suffix sum).
__device__ __forceinline__ uint32_t block_suffix_exclusive(uint32_t v, uint32_t* wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t y = __shfl_down(x, off);
    if (lane + off < 64) x += y;
  }
  if (lane == 0) wave_tot[wave] = x;
  __syncthreads();
  uint32_t above = 0;
  for (int w = wave + 1; w < kWaves; ++w) above += wave_tot[w];
  __syncthreads();
  return x - v + above;
}

// Sum over the block of a wave-uniform value supplied by every wave.
__device__ __forceinline__ uint32_t block_sum_waves(uint32_t wave_val, uint32_t* wave_tot,
                                                    uint32_t* below) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) wave_tot[wave] = wave_val;
  __syncthreads();
  uint32_t tot = 0, bel = 0;
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t t = wave_tot[w];
    tot += t;
    bel += w < wave ? t : 0u;
  }
  __syncthreads();
  *below = bel;
  return tot;
}

// Exact R-th largest key among the valid items (requires #valid > R >= 1).  Returns the
// threshold T; *need_eq receives how many items equal to T belong to the selection.
__device__ uint32_t radix_select(const uint32_t (&key)[kItems], uint32_t valid, int R,
                                 TopkShared& sh, int* need_eq) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t prefix = 0, pmask = 0;
  uint32_t remaining = static_cast<uint32_t>(R);
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
    uint32_t* hflat = &sh.hist[0][0];
    for (int k = tid; k < kRep * kBins; k += kThreads) hflat[k] = 0u;
    __syncthreads();
    uint32_t* myh = sh.hist[lane & (kRep - 1)];
#pragma unroll
    for (int j = 0; j < kItems; ++j)
      if (((valid >> j) & 1u) && (key[j] & pmask) == prefix)
        atomicAdd(&myh[(key[j] >> shift) & dmask], 1u);
    __syncthreads();
    const int b0 = 2 * tid, b1 = 2 * tid + 1;
    uint32_t c0 = 0, c1 = 0;
#pragma unroll
    for (int r = 0; r < kRep; ++r) {
      c0 += sh.hist[r][b0];
      c1 += sh.hist[r][b1];
    }
    const uint32_t above = block_suffix_exclusive(c0 + c1, sh.wave_a);
    if (above < remaining && above + c1 >= remaining) {
      sh.digit = static_cast<uint32_t>(b1);
      sh.above = above;
    } else if (above + c1 < remaining && above + c1 + c0 >= remaining) {
      sh.digit = static_cast<uint32_t>(b0);
      sh.above = above + c1;
    }
    __syncthreads();
    prefix |= sh.digit << shift;
    pmask |= dmask << shift;
    remaining -= sh.above;
    __syncthreads();
  }
  *need_eq = static_cast<int>(remaining);
  return prefix;
}

template <bool FROM_SCORES, bool FINAL>
__global__ __launch_bounds__(kThreads) void topk_level_kernel(TopkParams P) {
  __shared__ TopkShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x / P.nseg_out;
  const int seg = blockIdx.x - row * P.nseg_out;
  const int b = row / P.Lq;
  const int n = min(P.seqlens[b] - P.Lq + (row - b * P.Lq) + 1, P.S_max);
  const int p = n - 1;
  const int K = P.topk, I = P.init, W = P.local, R = P.R;
  const bool dense = n <= K;

  if (FINAL) {
    int32_t* out = P.indices + static_cast<size_t>(row) * K;
    if (dense) {
      for (int j = tid; j < K; j += kThreads) out[j] = j < n ? j : -1;
      if (tid == 0) P.n_sel[row] = n > 0 ? n : 0;
      return;
    }
    for (int j = tid; j < I; j += kThreads) out[j] = j;
    for (int j = tid; j < W; j += kThreads) out[I + R + j] = p - W + 1 + j;
    if (tid == 0) P.n_sel[row] = K;
    if (R == 0) return;
  } else if (dense || R == 0) {
    if (tid == 0) P.out_cnt[row * P.nseg_out + seg] = 0;
    return;
  }

  // ---- gather this workgroup's items; layout order (wave, j, lane) == position order
  uint32_t key[kItems];
  int32_t pos[kItems];
  uint32_t valid = 0;
  if (FROM_SCORES) {
    const int lo = I, hi = p - W;  // middle positions, inclusive
    const int base = seg * kSegItems + wave * (kItems * kWave) + lane;
    const float* srow = P.scores + static_cast<size_t>(row) * P.S_max;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const int s = base + j * kWave;
      const bool v = s >= lo && s <= hi;
      key[j] = v ? order_key(srow[s]) : 0u;
      pos[j] = s;
      valid |= (v ? 1u : 0u) << j;
    }
  } else {
    const int seg0 = seg * P.group;
    const int nsegs = min(P.group, P.nseg_in - seg0);
    const size_t cbase = static_cast<size_t>(row) * P.nseg_in + seg0;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const int q = wave * (kItems * kWave) + j * kWave + lane;
      const int sg = q / R;
      const int k = q - sg * R;
      bool v = false;
      key[j] = 0u;
      pos[j] = 0;
      if (sg < nsegs && k < P.in_cnt[cbase + sg]) {
        const size_t off = (cbase + sg) * R + k;
        key[j] = P.in_key[off];
        pos[j] = P.in_pos[off];
        v = true;
      }
      valid |= (v ? 1u : 0u) << j;
    }
  }

  // ---- how many valid items?
  uint32_t wcount = 0;
#pragma unroll
  for (int j = 0; j < kItems; ++j) wcount += __popcll(wave_ballot((valid >> j) & 1u));
  uint32_t below_unused;
  const uint32_t nvalid = block_sum_waves(wcount, sh.wave_a, &below_unused);

  // ---- threshold
  uint32_t T = 0;
  int need_eq = 0;
  const bool take_all = nvalid <= static_cast<uint32_t>(R);
  if (!take_all) T = radix_select(key, valid, R, sh, &need_eq);

  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const bool v = (valid >> j) & 1u;
    const bool g = v && (take_all || key[j] > T);
    const bool e = v && !take_all && key[j] == T;
    gt |= (g ? 1u : 0u) << j;
    eq |= (e ? 1u : 0u) << j;
  }
  // rank tied items by position: count ties in earlier waves first
  uint32_t weq = 0;
#pragma unroll
  for (int j = 0; j < kItems; ++j) weq += __popcll(wave_ballot((eq >> j) & 1u));
  uint32_t eq_base;
  block_sum_waves(weq, sh.wave_a, &eq_base);
  uint32_t sel = 0, run = eq_base, wsel = 0;
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const bool e = (eq >> j) & 1u;
    const uint64_t m = wave_ballot(e);
    const uint32_t rank = run + lanes_below(m);
    run += __popcll(m);
    const bool s = ((gt >> j) & 1u) || (e && rank < static_cast<uint32_t>(need_eq));
    sel |= (s ? 1u : 0u) << j;
    wsel += __popcll(wave_ballot(s));
  }
  uint32_t sel_base;
  const uint32_t total = block_sum_waves(wsel, sh.wave_b, &sel_base);

  // ---- compact in position order
  uint32_t at = sel_base;
  if (FINAL) {
    int32_t* out = P.indices + static_cast<size_t>(row) * K + I;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const bool s = (sel >> j) & 1u;
      const uint64_t m = wave_ballot(s);
      const uint32_t dst = at + lanes_below(m);
      if (s && dst < static_cast<uint32_t>(R)) out[dst] = pos[j];
      at += __popcll(m);
    }
  } else {
    const size_t obase = (static_cast<size_t>(row) * P.nseg_out + seg) * R;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const bool s = (sel >> j) & 1u;
      const uint64_t m = wave_ballot(s);
      const uint32_t dst = at + lanes_below(m);
      if (s && dst < static_cast<uint32_t>(R)) {
        P.out_key[obase + dst] = key[j];
        P.out_pos[obase + dst] = pos[j];
      }
      at += __popcll(m);
    }
    if (tid == 0) P.out_cnt[row * P.nseg_out + seg] = static_cast<int32_t>(min(total, static_cast<uint32_t>(R)));
  }
}

struct Plan {
  int R = 0, nseg0 = 1, group = 1, nseg1 = 1;
  size_t bytes_a = 0, bytes_b = 0;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

size_t list_bytes(long rows, int nseg, int R) {
  const size_t slots = static_cast<size_t>(rows) * nseg;
  return align256(slots * R * 4) * 2 + align256(slots * 4);
}

Plan make_plan(int B, int Lq, int S_max, int topk, int init_tokens, int local_tokens) {
  Plan pl;
  const long rows = static_cast<long>(B) * Lq;
  pl.R = topk - init_tokens - local_tokens;
  pl.nseg0 = (S_max + kSegItems - 1) / kSegItems;
  if (pl.nseg0 <= 1 || pl.R == 0) return pl;
  pl.group = kSegItems / pl.R;  // >= 2 because R <= topk <= 8192
  pl.nseg1 = (pl.nseg0 + pl.group - 1) / pl.group;
  pl.bytes_a = list_bytes(rows, pl.nseg0, pl.R);
  pl.bytes_b = pl.nseg1 > 1 ? list_bytes(rows, pl.nseg1, pl.R) : 0;
  return pl;
}

struct Lists {
  uint32_t* key;
  int32_t* pos;
  int32_t* cnt;
};

Lists carve(char* base, long rows, int nseg, int R) {
  const size_t slots = static_cast<size_t>(rows) * nseg;
  Lists l;
  l.key = reinterpret_cast<uint32_t*>(base);
  l.pos = reinterpret_cast<int32_t*>(base + align256(slots * R * 4));
  l.cnt = reinterpret_cast<int32_t*>(base + 2 * align256(slots * R * 4));
  return l;
}

}  // namespace

size_t topk_workspace_bytes(int B, int Lq, int S_max, int topk, int init_tokens, int local_tokens) {
  const Plan pl = make_plan(B, Lq, S_max, topk, init_tokens, local_tokens);
  return pl.bytes_a + pl.bytes_b;
}

hipError_t launch_topk(const float* scores, const int32_t* seqlens, int B, int Lq, int S_max,
                       int topk, int init_tokens, int local_tokens, int32_t* indices,
                       int32_t* n_sel, void* workspace, hipStream_t stream) {
  const Plan pl = make_plan(B, Lq, S_max, topk, init_tokens, local_tokens);
  const long rows = static_cast<long>(B) * Lq;
  TopkParams P{};
  P.scores = scores;
  P.seqlens = seqlens;
  P.Lq = Lq;
  P.S_max = S_max;
  P.topk = topk;
  P.init = init_tokens;
  P.local = local_tokens;
  P.R = pl.R;
  P.indices = indices;
  P.n_sel = n_sel;

  if (pl.nseg0 <= 1 || pl.R == 0) {
    P.nseg_out = 1;
    if (rows > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((topk_level_kernel<true, true>), dim3(static_cast<unsigned>(rows)),
                       dim3(kThreads), 0, stream, P);
    return hipGetLastError();
  }

  char* ws = static_cast<char*>(workspace);
  Lists cur = carve(ws, rows, pl.nseg0, pl.R);
  Lists other = carve(ws + pl.bytes_a, rows, pl.nseg1, pl.R);

  // level 0: chunks of the score rows -> candidate lists
  P.out_key = cur.key;
  P.out_pos = cur.pos;
  P.out_cnt = cur.cnt;
  P.nseg_out = pl.nseg0;
  long grid = rows * pl.nseg0;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((topk_level_kernel<true, false>), dim3(static_cast<unsigned>(grid)),
                     dim3(kThreads), 0, stream, P);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  int nseg = pl.nseg0;
  for (;;) {
    const int next = (nseg + pl.group - 1) / pl.group;
    P.in_key = cur.key;
    P.in_pos = cur.pos;
    P.in_cnt = cur.cnt;
    P.nseg_in = nseg;
    P.group = pl.group;
    P.nseg_out = next;
    grid = rows * next;
    if (next == 1) {
      hipLaunchKernelGGL((topk_level_kernel<false, true>), dim3(static_cast<unsigned>(grid)),
                         dim3(kThreads), 0, stream, P);
      return hipGetLastError();
    }
    // buffer capacities: `cur` alternates between the level-0 buffer (nseg0 slots per row) and
    // the level-1 buffer (nseg1 slots per row); every later level needs no more than either.
    Lists dst = {other.key, other.pos, other.cnt};
    P.out_key = dst.key;
    P.out_pos = dst.pos;
    P.out_cnt = dst.cnt;
    hipLaunchKernelGGL((topk_level_kernel<false, false>), dim3(static_cast<unsigned>(grid)),
                       dim3(kThreads), 0, stream, P);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    other = cur;
    cur = dst;
    nseg = next;
  }
}

}  // namespace lsa
