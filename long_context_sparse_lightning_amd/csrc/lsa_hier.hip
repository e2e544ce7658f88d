// Hierarchical indexing (page "LongCat Sparse Attention技术深度解析", section on LSA's three
// strategies, "分层索引": a coarse block-level score first, then the token selection inside the
// chosen blocks, so the indexer scores far fewer candidates).  The page fixes neither the block
// size nor the block score; this implementation takes:
//   block j = tokens [j*Bk, (j+1)*Bk) (Bk a power of two); block key = bf16(mean of the block's
//   index keys); a block is scored like a token, sum_h w[h] * max(0, q[h] . key); the blocks
//   scored are the nb = w0 / Bk complete ones before the sliding window (w0 = max(p - local + 1,
//   0)); the M best are kept; tokens outside the sink, the window, the partial block before it
//   and the kept blocks are excluded (they would score -inf); then the usual selection, which
//   never reaches an excluded token when M*Bk >= topk - local (required).
//
// Design for gfx950.  Block keys are a summary of the key cache, built once per completed block
// (lsa_block_keys), so a decode pass reads nb block keys (1/Bk of the cache) plus the kept
// blocks' tokens instead of every key.
//  * One wavefront scores 32 key rows against the row's (up to) 32 index heads with the
//    32x32x16 bf16 MFMA, heads as the A rows and keys as the B columns, so a lane ends with 16
//    head dot products of one key: the ReLU-weighted head sum is 16 FMAs and one lane swap.
//  * hier_block_scores_kernel: the block scores and each row's block count; it also empties the
//    row's candidate lists for stage 2.
//  * hier_block_select_kernel: one 1024-thread workgroup per row keeps the M best blocks: three
//    radix rounds over the 32-bit order key in an LDS histogram, the lowest blocks among equal
//    keys, and an ascending compaction of a block bitmap.
//  * hier_candidates_kernel: one wavefront per 32-token tile of a kept block (or of the partial
//    block before the window) scores its middle tokens and appends them, with one atomic per
//    wavefront, to the (key, position) list of their chunk of positions, in the format of the
//    exact merge of lsa_topk.hip, which makes the final selection.  Only kept tokens are
//    scored or written, so the merge sees about M*Bk candidates per row; the order inside a list
//    varies, the merge's result does not.  This needs at least R = topk - init - local middle
//    candidates per row: M*Bk >= topk - local.
#include <algorithm>

#include "lsa_internal.h"
#include "lsa_select.h"

namespace lsa {
namespace {

constexpr int kHierThreads = 256;  // 4 wavefronts, 32 key rows each
constexpr int kRowsPerGroup = 128;
constexpr int kMaxHeads = 32;

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// grid (ceil(S_max / Bk / 4), B): 4 blocks per workgroup, one wavefront per block, a lane per
// pair of dims (Di <= 128, even).  Blocks [first, seqlens[b] / Bk) are written.
__global__ __launch_bounds__(kHierThreads) void block_keys_kernel(const uint16_t* k_idx,
                                                                  const int32_t* seqlens, int S_max,
                                                                  int Di, int Bk, int first,
                                                                  uint16_t* out) {
  const int b = blockIdx.y;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int d = 2 * (threadIdx.x & 63);
  const int nb = min(seqlens[b], S_max) / Bk;
  if (j < first || j >= nb || d >= Di) return;
  const uint16_t* src = k_idx + (static_cast<size_t>(b) * S_max + static_cast<size_t>(j) * Bk) * Di + d;
  float u = 0.0f, v = 0.0f;
#pragma unroll 8
  for (int t = 0; t < Bk; ++t) {
    const uint32_t x = *reinterpret_cast<const uint32_t*>(src + static_cast<size_t>(t) * Di);
    u += bf16_lo(x);
    v += bf16_hi(x);
  }
  const float inv = 1.0f / static_cast<float>(Bk);  // exact: Bk is a power of two
  const uint32_t packed = static_cast<uint32_t>(bf16_bits_rne(u * inv)) |
                          (static_cast<uint32_t>(bf16_bits_rne(v * inv)) << 16);
  *reinterpret_cast<uint32_t*>(out + (static_cast<size_t>(b) * (S_max / Bk) + j) * Di + d) = packed;
}

struct HierParams {
  const uint16_t* q;      // [B, Hi, Di]
  const float* w;         // [B, Hi]
  const uint16_t* keys;   // stage 1: block keys [B, nblk, Di]; stage 2: k_idx [B, S_max, Di]
  const int32_t* seqlens;
  int Hi, Di, S_max, Bk, init, local;
  int nblk;               // S_max / Bk
  float* scores;          // stage 1: [B, nblk] block scores
  int32_t* nb_out;        // stage 1: blocks scored per row
  int32_t* kept;          // [B, M] kept blocks (ascending), kept_n[B] of them
  int32_t* kept_n;
  int M, topk;
  int chunk_keys, chunks;  // stage 2: candidate lists, one per chunk of positions
  uint32_t* count;         // [B, chunks]
  uint32_t* range;         // [B, chunks, 2] smallest and largest key of each list
  uint2* cand;             // [B, chunks, chunk_keys] (order key, position)
  int32_t* indices;        // [B, topk] the selection
  int32_t* n_sel;          // [B]
};

// Scores of key rows r0 .. r0 + 31 (row = lane & 31) against the row's heads; valid in every
// lane (both halves hold the same sum).  Rows past `last` re-read row `last`.
__device__ __forceinline__ float score32(const HierParams& P, int b, const uint16_t* keys,
                                         size_t keys_per_b, int r0, int last) {
  const int lane = threadIdx.x & 63, col = lane & 31, g = lane >> 5;
  const int head = col;
  const int row = min(r0 + col, last);
  const uint16_t* qrow = P.q + (static_cast<size_t>(b) * P.Hi + min(head, P.Hi - 1)) * P.Di + 8 * g;
  const uint16_t* krow = keys + static_cast<size_t>(b) * keys_per_b + static_cast<size_t>(row) * P.Di + 8 * g;
  f32x16 acc = f32x16{};
  const int steps = P.Di / 16;
  for (int k = 0; k < steps; ++k) {
    const bf16x8 a = head < P.Hi ? load_bf16x8(qrow + 16 * k) : zero_bf16x8();
    acc = mfma32(a, load_bf16x8(krow + 16 * k), acc);
  }
  // lane (col, g) register r: head acc_row(r, g) of key col
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int h = acc_row(r, g);
    const float wh = h < P.Hi ? P.w[static_cast<size_t>(b) * P.Hi + h] : 0.0f;
    s += wh * fmaxf(acc[r], 0.0f);
  }
  return sum_xor32(s);
}

// grid (ceil(nblk / 128), B): scores of blocks [0, nb) and the row's nb.
__global__ __launch_bounds__(kHierThreads) void hier_block_scores_kernel(HierParams P) {
  const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = min(P.seqlens[b], P.S_max), p = n - 1;
  const int nb = max(p - P.local + 1, 0) / P.Bk;
  const int r0 = blockIdx.x * kRowsPerGroup + wave * 32;
  if (blockIdx.x == 0) {  // the row's block count and empty candidate lists for stage 2
    if (tid == 0) P.nb_out[b] = nb;
    for (int c = tid; c < P.chunks; c += kHierThreads) {
      const size_t lc = static_cast<size_t>(b) * P.chunks + c;
      P.count[lc] = 0u;
      P.range[2 * lc] = 0xffffffffu;
      P.range[2 * lc + 1] = 0u;
    }
  }
  if (r0 >= nb) return;
  const float s = score32(P, b, P.keys, static_cast<size_t>(P.nblk) * P.Di, r0, nb - 1);
  const int j = r0 + lane;
  if (lane < 32 && j < nb) P.scores[static_cast<size_t>(b) * P.nblk + j] = s;
}

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelPer = sel::kBins / kSelThreads;
constexpr int kMaxSelBlocks = 1 << 17;  // S_max / Bk with S_max <= 2^20 and Bk >= 8

// grid (B): the M best of the row's nb block scores (larger score, then the lower block) in
// ascending order, or every block when nb <= M.
__global__ __launch_bounds__(kSelThreads) void hier_block_select_kernel(HierParams P) {
  __shared__ uint32_t hist[sel::kBins];
  __shared__ uint32_t win[kMaxSelBlocks / 32], tie[kMaxSelBlocks / 32];
  __shared__ uint32_t sh_scan[kSelWaves], sh_res[4];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int nb = P.nb_out[b];
  const float* sc = P.scores + static_cast<size_t>(b) * P.nblk;
  int32_t* out = P.kept + static_cast<size_t>(b) * P.M;
  if (nb <= P.M) {
    for (int j = tid; j < P.M; j += kSelThreads) out[j] = j < nb ? j : -1;
    if (tid == 0) P.kept_n[b] = max(nb, 0);
    return;
  }
  // the M-th largest key: its top 12 bits, the next 12, the last 8
  uint32_t want = static_cast<uint32_t>(P.M), pref = 0;
  for (int round = 0; round < 3; ++round) {
    const int shift = round == 0 ? 20 : round == 1 ? 8 : 0;
    const int prev = round == 1 ? 20 : 8;  // in play: (k >> prev) == pref (rounds 1, 2)
    const uint32_t mask = round < 2 ? 0xfffu : 0xffu;
    for (int i = tid; i < sel::kBins; i += kSelThreads) hist[i] = 0u;
    __syncthreads();
    for (int j = tid; j < nb; j += kSelThreads) {
      const uint32_t k = sel::order_key(sc[j]);
      if (round == 0 || (k >> prev) == pref)
        atomicAdd(&hist[sel::bin_slot<kSelThreads>((k >> shift) & mask)], 1u);
    }
    __syncthreads();
    uint32_t c[kSelPer];
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) c[i] = hist[i * kSelThreads + tid];
    sel::select_bin<kSelPer, kSelWaves>(c, want, sh_scan, sh_res);
    want -= sh_res[1];
    pref = (pref << (round < 2 ? 12 : 8)) | sh_res[0];
  }
  // winners: keys above pref, and the `want` lowest blocks whose key equals it
  const int words = (nb + 31) / 32;
  for (int i = tid; i < words; i += kSelThreads) win[i] = tie[i] = 0u;
  __syncthreads();
  for (int j = tid; j < nb; j += kSelThreads) {
    const uint32_t k = sel::order_key(sc[j]);
    if (k > pref) atomicOr(&win[j >> 5], 1u << (j & 31));
    else if (k == pref) atomicOr(&tie[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  const int wpt = (words + kSelThreads - 1) / kSelThreads;  // contiguous words per thread
  const int w0 = tid * wpt, w1 = min(words, w0 + wpt);
  uint32_t mine = 0, total;
  for (int w = w0; w < w1; ++w) mine += __popc(tie[w]);
  uint32_t rank = sel::block_prefix<kSelWaves>(mine, sh_scan, &total);
  for (int w = w0; w < w1 && rank < want; ++w) {
    uint32_t bits = tie[w];
    while (bits && rank < want) {
      const uint32_t low = bits & (~bits + 1u);
      win[w] |= low;
      bits ^= low;
      ++rank;
    }
  }
  __syncthreads();
  mine = 0;
  for (int w = w0; w < w1; ++w) mine += __popc(win[w]);
  uint32_t at = sel::block_prefix<kSelWaves>(mine, sh_scan, &total);
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = win[w];
    while (bits) {
      const int i = __ffs(bits) - 1;
      bits &= bits - 1;
      if (at < static_cast<uint32_t>(P.M)) out[at] = 32 * w + i;
      ++at;
    }
  }
  if (tid == 0) P.kept_n[b] = P.M;
}

// grid (ceil(tiles / 4), B), tiles = (M + 1) * ceil(Bk / 32): tile t < M * tpb covers the
// tokens of kept block t / tpb (32 of them from 32 * (t % tpb)); the last tpb tiles cover the
// partial block before the window.  A tile's tokens lie in one block, hence in one chunk list.
__global__ __launch_bounds__(kHierThreads) void hier_candidates_kernel(HierParams P) {
  const int b = blockIdx.y, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n = min(P.seqlens[b], P.S_max), p = n - 1;
  if (n <= P.topk) return;  // dense: the merge fills the row
  const int hi = p - P.local;  // middle positions [init, hi]
  const int nb = max(p - P.local + 1, 0) / P.Bk;
  const int tpb = (P.Bk + 31) / 32;
  int first, last;  // the tile's positions [first, last]
  if (t < P.M * tpb) {
    const int i = t / tpb;
    if (i >= P.kept_n[b]) return;
    const int blk0 = P.kept[static_cast<size_t>(b) * P.M + i] * P.Bk;
    first = blk0 + 32 * (t % tpb);
    last = min(first + 31, blk0 + P.Bk - 1);
  } else if (t < (P.M + 1) * tpb) {
    first = nb * P.Bk + 32 * (t - P.M * tpb);
    last = min(first + 31, nb * P.Bk + P.Bk - 1);
  } else {
    return;
  }
  const int s = first + (lane & 31);
  const bool cand = lane < 32 && s <= last && s >= P.init && s <= hi;
  const uint64_t mask = __ballot(cand);
  if (mask == 0) return;  // wavefront-uniform
  const float v = score32(P, b, P.keys, static_cast<size_t>(P.S_max) * P.Di, first, p);
  const uint32_t key = sel::order_key(v);
  // one list slot range per wavefront, and the list's key bounds
  const size_t lc = static_cast<size_t>(b) * P.chunks + first / P.chunk_keys;
  uint32_t at = 0;
  if (lane == 0) at = atomicAdd(&P.count[lc], static_cast<uint32_t>(__popcll(mask)));
  at = __shfl(at, 0) + lanes_below(mask);
  const uint32_t kmin = wave_min(cand ? key : 0xffffffffu), kmax = wave_max(cand ? key : 0u);
  if (lane == 0) {
    atomicMin(&P.range[2 * lc], kmin);
    atomicMax(&P.range[2 * lc + 1], kmax);
  }
  if (cand) P.cand[lc * static_cast<size_t>(P.chunk_keys) + at] = make_uint2(key, static_cast<uint32_t>(s));
}

constexpr int kMergeItems = 4;                                  // candidates per thread
constexpr int kMaxMergeCand = kSelThreads * kMergeItems;        // 4096
constexpr int kMaxLists = 128;

// grid (B): the selection of row b from its candidate lists when they hold at most
// kMaxMergeCand = (M + 1) * Bk candidates: sink and window at the ends, the R = topk - init -
// local best candidates (larger key, then lower position) in between, ascending.  A candidate's
// slot is (its block's rank among the kept blocks, or kept_n for the partial block) * Bk + its
// offset in the block, so slot order is position order.
__global__ __launch_bounds__(kSelThreads) void hier_merge_kernel(HierParams P) {
  __shared__ uint32_t hist[sel::kBins];
  __shared__ uint32_t win[kMaxMergeCand / 32], tie[kMaxMergeCand / 32];
  __shared__ uint32_t sh_scan[kSelWaves], sh_res[4], sh_off[kMaxLists + 1];
  __shared__ int32_t sh_kept[kMaxMergeCand / 8];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int K = P.topk, I = P.init, W = P.local, R = K - I - W;
  const int n = min(P.seqlens[b], P.S_max), p = n - 1;
  int32_t* out = P.indices + static_cast<size_t>(b) * K;
  if (n <= K) {  // dense: every visible position, then padding
    for (int j = tid; j < K; j += kSelThreads) out[j] = j < n ? j : -1;
    if (tid == 0) P.n_sel[b] = max(n, 0);
    return;
  }
  for (int j = tid; j < I; j += kSelThreads) out[j] = j;
  for (int j = tid; j < W; j += kSelThreads) out[K - W + j] = p - W + 1 + j;
  if (tid == 0) P.n_sel[b] = K;
  if (R == 0) return;
  const int nb = max(p - P.local + 1, 0) / P.Bk;
  const int kn = P.kept_n[b];
  for (int i = tid; i < kn; i += kSelThreads) sh_kept[i] = P.kept[static_cast<size_t>(b) * P.M + i];
  // list offsets
  const uint32_t c_len = tid < P.chunks ? P.count[static_cast<size_t>(b) * P.chunks + tid] : 0u;
  uint32_t nc;
  const uint32_t at0 = sel::block_prefix<kSelWaves>(c_len, sh_scan, &nc);
  if (tid < P.chunks) sh_off[tid] = at0;
  __syncthreads();
  // candidates into registers: entry q of the concatenated lists
  uint32_t key[kMergeItems];
  int32_t slot[kMergeItems];
  uint32_t held = 0;
#pragma unroll
  for (int i = 0; i < kMergeItems; ++i) {
    const uint32_t q = static_cast<uint32_t>(tid + kSelThreads * i);
    key[i] = 0u;
    slot[i] = 0;
    if (q < nc) {
      int lo = 0, hi = P.chunks - 1;  // last list c with sh_off[c] <= q
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sh_off[mid] <= q) lo = mid; else hi = mid - 1;
      }
      const uint2 v = P.cand[(static_cast<size_t>(b) * P.chunks + lo) * P.chunk_keys + (q - sh_off[lo])];
      const int pos = static_cast<int>(v.y), blk = pos / P.Bk;
      int r = kn;  // the partial block before the window
      if (blk < nb) {
        int a = 0, z = kn - 1;  // kept blocks ascending
        while (a < z) {
          const int mid = (a + z) >> 1;
          if (sh_kept[mid] < blk) a = mid + 1; else z = mid;
        }
        r = a;
      }
      key[i] = v.x;
      slot[i] = r * P.Bk + (pos - blk * P.Bk);
      held |= 1u << i;
    }
  }
  // the R-th largest key
  uint32_t want = static_cast<uint32_t>(R), pref = 0;
  for (int round = 0; round < 3; ++round) {
    const int shift = round == 0 ? 20 : round == 1 ? 8 : 0;
    const int prev = round == 1 ? 20 : 8;
    const uint32_t mask = round < 2 ? 0xfffu : 0xffu;
    for (int i = tid; i < sel::kBins; i += kSelThreads) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kMergeItems; ++i)
      if ((held >> i & 1u) && (round == 0 || (key[i] >> prev) == pref))
        atomicAdd(&hist[sel::bin_slot<kSelThreads>((key[i] >> shift) & mask)], 1u);
    __syncthreads();
    uint32_t c[kSelPer];
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) c[i] = hist[i * kSelThreads + tid];
    sel::select_bin<kSelPer, kSelWaves>(c, want, sh_scan, sh_res);
    want -= sh_res[1];
    pref = (pref << (round < 2 ? 12 : 8)) | sh_res[0];
  }
  // winners: keys above pref, and the `want` lowest slots whose key equals it
  const int words = ((kn + 1) * P.Bk + 31) / 32;
  for (int i = tid; i < words; i += kSelThreads) win[i] = tie[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kMergeItems; ++i) {
    if (!(held >> i & 1u)) continue;
    if (key[i] > pref) atomicOr(&win[slot[i] >> 5], 1u << (slot[i] & 31));
    else if (key[i] == pref) atomicOr(&tie[slot[i] >> 5], 1u << (slot[i] & 31));
  }
  __syncthreads();
  const int wpt = (words + kSelThreads - 1) / kSelThreads;
  const int w0 = tid * wpt, w1 = min(words, w0 + wpt);
  uint32_t mine = 0, total;
  for (int w = w0; w < w1; ++w) mine += __popc(tie[w]);
  uint32_t rank = sel::block_prefix<kSelWaves>(mine, sh_scan, &total);
  for (int w = w0; w < w1 && rank < want; ++w) {
    uint32_t bits = tie[w];
    while (bits && rank < want) {
      const uint32_t low = bits & (~bits + 1u);
      win[w] |= low;
      bits ^= low;
      ++rank;
    }
  }
  __syncthreads();
  mine = 0;
  for (int w = w0; w < w1; ++w) mine += __popc(win[w]);
  uint32_t at = sel::block_prefix<kSelWaves>(mine, sh_scan, &total);
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = win[w];
    while (bits) {
      const int sl = 32 * w + __ffs(bits) - 1;
      bits &= bits - 1;
      const int r = sl / P.Bk, o = sl - r * P.Bk;
      if (at < static_cast<uint32_t>(R)) out[I + at] = (r < kn ? sh_kept[r] : nb) * P.Bk + o;
      ++at;
    }
  }
}

size_t align_up(size_t x) { return (x + kWorkspaceAlign - 1) & ~(kWorkspaceAlign - 1); }

struct HierLayout {
  size_t blk_scores, nb, kept, kept_n, count, range, cand, total;
  int chunk_keys, chunks;
};

HierLayout hier_layout(int B, int S_max, int Bk, int M) {
  HierLayout L{};
  const size_t nblk = static_cast<size_t>(S_max / Bk);
  size_t off = 0;
  L.blk_scores = off;
  off += align_up(static_cast<size_t>(B) * nblk * sizeof(float));
  L.nb = off;
  off += align_up(static_cast<size_t>(B) * sizeof(int32_t));
  L.kept = off;
  off += align_up(static_cast<size_t>(B) * M * sizeof(int32_t));
  L.kept_n = off;
  off += align_up(static_cast<size_t>(B) * sizeof(int32_t));
  // candidate lists: a power-of-two chunk length (a multiple of every block size), at most
  // topk_merge_max_chunks() lists per row.  16384 positions (8 lists at 128K) measured best for
  // the merge: fewer lists cost less to walk, and each still fits its threads' registers when
  // M*Bk stays near 2048 (2 or 64 lists were slower).
  L.chunk_keys = 16384;
  while (static_cast<long>(L.chunk_keys) * topk_merge_max_chunks() < S_max) L.chunk_keys *= 2;
  L.chunks = (S_max + L.chunk_keys - 1) / L.chunk_keys;
  const size_t lists = static_cast<size_t>(B) * L.chunks;
  L.count = off;
  off += align_up(lists * sizeof(uint32_t));
  L.range = off;
  off += align_up(lists * 2 * sizeof(uint32_t));
  L.cand = off;
  off += align_up(lists * L.chunk_keys * sizeof(uint2));
  L.total = off + kWorkspaceAlign;
  return L;
}

}  // namespace

int hier_max_heads() { return kMaxHeads; }

size_t hier_workspace_bytes(int B, int S_max, int Bk, int topk, int init, int local, int M) {
  (void)topk, (void)init, (void)local;  // the final selection runs on the candidate lists
  return hier_layout(B, S_max, Bk, M).total;
}

hipError_t launch_block_keys(const uint16_t* k_idx, const int32_t* seqlens, int B, int S_max, int Di,
                             int Bk, int first_block, uint16_t* block_keys, hipStream_t stream) {
  const int nblk = S_max / Bk;
  if (nblk <= first_block) return hipSuccess;
  hipLaunchKernelGGL(block_keys_kernel, dim3(static_cast<unsigned>((nblk + 3) / 4), static_cast<unsigned>(B)),
                     dim3(kHierThreads), 0, stream, k_idx, seqlens, S_max, Di, Bk, first_block,
                     block_keys);
  return hipGetLastError();
}

hipError_t launch_hier_index_topk(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                                  const uint16_t* block_keys, const int32_t* seqlens, int B, int Hi,
                                  int Di, int S_max, int topk, int init, int local, int Bk, int M,
                                  int32_t* indices, int32_t* n_sel, void* workspace,
                                  hipStream_t stream) {
  const HierLayout L = hier_layout(B, S_max, Bk, M);
  char* ws = align_workspace(workspace);
  const int nblk = S_max / Bk;
  HierParams P{};
  P.q = q_idx;
  P.w = w;
  P.seqlens = seqlens;
  P.Hi = Hi;
  P.Di = Di;
  P.S_max = S_max;
  P.Bk = Bk;
  P.init = init;
  P.local = local;
  P.nblk = nblk;
  P.M = M;
  float* blk_scores = reinterpret_cast<float*>(ws + L.blk_scores);
  int32_t* nb = reinterpret_cast<int32_t*>(ws + L.nb);
  int32_t* kept = reinterpret_cast<int32_t*>(ws + L.kept);
  int32_t* kept_n = reinterpret_cast<int32_t*>(ws + L.kept_n);
  P.topk = topk;
  P.chunk_keys = L.chunk_keys;
  P.chunks = L.chunks;
  P.count = reinterpret_cast<uint32_t*>(ws + L.count);
  P.range = reinterpret_cast<uint32_t*>(ws + L.range);
  P.cand = reinterpret_cast<uint2*>(ws + L.cand);
  // stage 1: block scores, the row's block count, empty candidate lists
  P.keys = block_keys;
  P.scores = blk_scores;
  P.nb_out = nb;
  const unsigned gb = static_cast<unsigned>(std::max(1, (nblk + kRowsPerGroup - 1) / kRowsPerGroup));
  hipLaunchKernelGGL(hier_block_scores_kernel, dim3(gb, static_cast<unsigned>(B)), dim3(kHierThreads),
                     0, stream, P);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // the M best blocks of each row (every block when nb <= M)
  if (nblk > kMaxSelBlocks) return hipErrorInvalidConfiguration;
  P.kept = kept;
  P.kept_n = kept_n;
  hipLaunchKernelGGL(hier_block_select_kernel, dim3(static_cast<unsigned>(B)), dim3(kSelThreads), 0,
                     stream, P);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // stage 2: candidate lists of the kept blocks' tokens, then the exact merge
  P.keys = k_idx;
  const int tiles = (M + 1) * ((Bk + 31) / 32);
  hipLaunchKernelGGL(hier_candidates_kernel, dim3(static_cast<unsigned>((tiles + 3) / 4), static_cast<unsigned>(B)),
                     dim3(kHierThreads), 0, stream, P);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // the dedicated merge keeps the kept blocks' ids in LDS (sh_kept: kMaxMergeCand / 8 entries)
  if (static_cast<long>(M + 1) * Bk <= kMaxMergeCand && M <= kMaxMergeCand / 8 &&
      L.chunks <= kMaxLists) {
    P.indices = indices;
    P.n_sel = n_sel;
    hipLaunchKernelGGL(hier_merge_kernel, dim3(static_cast<unsigned>(B)), dim3(kSelThreads), 0, stream, P);
    return hipGetLastError();
  }
  return launch_topk_merge(seqlens, 1, S_max, topk, init, local, 0, B, L.chunks, L.chunk_keys, P.count,
                           P.range, P.cand, nullptr, indices, n_sel, stream);
}

}  // namespace lsa
