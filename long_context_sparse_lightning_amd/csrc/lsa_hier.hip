// Hierarchical indexing (page "LongCat Sparse Attention技术深度解析", section on LSA's three
// strategies, "分层索引": a coarse block-level score first, then the token selection inside the
// chosen blocks, so the indexer scores far fewer candidates).  The page fixes neither the block
// size nor the block score; this implementation takes:
//   block j = tokens [j*Bk, (j+1)*Bk) (Bk a power of two); block key = bf16(mean of the block's
//   index keys); a block is scored like a token, sum_h w[h] * max(0, q[h] . key); the blocks
//   scored are the nb = w0 / Bk complete ones before the sliding window (w0 = max(p - local + 1,
//   0)); the M best are kept; tokens outside the sink, the window, the partial block before it
//   and the kept blocks get the score -inf; then the usual selection.
//
// Design for gfx950.  Block keys are a summary of the key cache, built once per completed block
// (lsa_block_keys), so a decode pass reads nb block keys (1/Bk of the cache) plus the kept
// blocks' tokens instead of every key.
//  * hier_score_kernel<TOKENS>: one wavefront scores 32 key rows against the row's (up to) 32
//    index heads with the 32x32x16 bf16 MFMA, heads as the A rows and keys as the B columns, so
//    a lane ends with 16 head dot products of one key: the ReLU-weighted head sum is 16 FMAs and
//    one lane swap (xor 32).  Stage 1 (blocks) writes the block scores and each row's block
//    count; stage 2 (tokens) writes a dense score row: the score for candidates, -inf for
//    tokens outside the kept blocks (a wavefront whose 32 tokens are all excluded loads no key).
//  * The two selections (M blocks, then topk tokens) are the top-k kernels of lsa_topk.hip.
#include <algorithm>

#include "lsa_internal.h"

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
  float* scores;          // stage 1: [B, nblk]; stage 2: [B, S_max]
  int32_t* nb_out;        // stage 1: blocks scored per row
  const int32_t* kept;    // stage 2: [B, M] kept blocks (ascending), kept_n[B] of them
  const int32_t* kept_n;
  int M;
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
  return s + xor32(s);
}

// grid (ceil(rows / 128), B).  TOKENS = false: block scores of blocks [0, nb); true: the dense
// token score row [0, p] of stage 2.
template <bool TOKENS>
__global__ __launch_bounds__(kHierThreads) void hier_score_kernel(HierParams P) {
  __shared__ int keep[kRowsPerGroup / 8 + 2];  // kept flags of the blocks this group touches
  const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = min(P.seqlens[b], P.S_max), p = n - 1;
  const int w0 = max(p - P.local + 1, 0);
  const int nb = w0 / P.Bk;
  const int r0 = blockIdx.x * kRowsPerGroup + wave * 32;
  if constexpr (!TOKENS) {
    if (blockIdx.x == 0 && tid == 0) P.nb_out[b] = nb;
    if (r0 >= nb) return;
    const float s = score32(P, b, P.keys, static_cast<size_t>(P.nblk) * P.Di, r0, nb - 1);
    const int j = r0 + lane;
    if (lane < 32 && j < nb) P.scores[static_cast<size_t>(b) * P.nblk + j] = s;
  } else {
    // kept flags of blocks [first_blk, first_blk + span)
    const int g0 = blockIdx.x * kRowsPerGroup;
    const int first_blk = g0 / P.Bk;
    const int span = (kRowsPerGroup - 1) / P.Bk + 2;
    for (int i = tid; i < span; i += kHierThreads) keep[i] = 0;
    __syncthreads();
    const int cnt = P.kept_n[b];
    for (int i = tid; i < cnt; i += kHierThreads) {
      const int j = P.kept[static_cast<size_t>(b) * P.M + i] - first_blk;
      if (j >= 0 && j < span) keep[j] = 1;
    }
    __syncthreads();
    if (r0 > p) return;
    const int s = r0 + (lane & 31);
    const bool forced = s < P.init || s > p - P.local;
    const bool cand = s < P.init || s >= nb * P.Bk || keep[s / P.Bk - first_blk] != 0;
    float v = -INFINITY;
    if (__ballot(cand && !forced) != 0)  // wavefront-uniform
      v = score32(P, b, P.keys, static_cast<size_t>(P.S_max) * P.Di, r0, p);
    if (forced) v = 0.0f;  // the selection forces these; the value is not used
    else if (!cand) v = -INFINITY;
    if (lane < 32 && s <= p) P.scores[static_cast<size_t>(b) * P.S_max + s] = v;
  }
}

size_t align_up(size_t x) { return (x + kWorkspaceAlign - 1) & ~(kWorkspaceAlign - 1); }

struct HierLayout {
  size_t blk_scores, nb, kept, kept_n, tok_scores, topk_ws, total;
};

HierLayout hier_layout(int B, int S_max, int Bk, int topk, int init, int local, int M) {
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
  L.tok_scores = off;
  off += align_up(static_cast<size_t>(B) * S_max * sizeof(float));
  L.topk_ws = off;
  off += align_up(std::max(topk_workspace_bytes(B, 1, static_cast<int>(nblk), M, 0, 0),
                           topk_workspace_bytes(B, 1, S_max, topk, init, local)));
  L.total = off + kWorkspaceAlign;
  return L;
}

}  // namespace

int hier_max_heads() { return kMaxHeads; }

size_t hier_workspace_bytes(int B, int S_max, int Bk, int topk, int init, int local, int M) {
  return hier_layout(B, S_max, Bk, topk, init, local, M).total;
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
  const HierLayout L = hier_layout(B, S_max, Bk, topk, init, local, M);
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
  float* tok = reinterpret_cast<float*>(ws + L.tok_scores);
  void* tws = ws + L.topk_ws;
  // stage 1: block scores and the row's block count
  P.keys = block_keys;
  P.scores = blk_scores;
  P.nb_out = nb;
  const unsigned gb = static_cast<unsigned>(std::max(1, (nblk + kRowsPerGroup - 1) / kRowsPerGroup));
  hipLaunchKernelGGL((hier_score_kernel<false>), dim3(gb, static_cast<unsigned>(B)), dim3(kHierThreads),
                     0, stream, P);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // the M best blocks of each row (every block when nb <= M)
  if ((err = launch_topk(blk_scores, nb, B, 1, nblk, M, 0, 0, kept, kept_n, tws, stream)) != hipSuccess)
    return err;
  // stage 2: the dense token score row, then the selection
  P.keys = k_idx;
  P.scores = tok;
  P.kept = kept;
  P.kept_n = kept_n;
  const unsigned gt = static_cast<unsigned>((S_max + kRowsPerGroup - 1) / kRowsPerGroup);
  hipLaunchKernelGGL((hier_score_kernel<true>), dim3(gt, static_cast<unsigned>(B)), dim3(kHierThreads),
                     0, stream, P);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return launch_topk(tok, seqlens, B, 1, S_max, topk, init, local, indices, n_sel, tws, stream);
}

}  // namespace lsa
