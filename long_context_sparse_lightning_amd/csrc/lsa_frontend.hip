// Indexer front end: the inputs of the lightning indexer for the current tokens (page "MLX-VLM
// 的 LongCat-Flash-Lite-Sparse ...", section "LSA": wq_b projects the q-LoRA representation to
// index_n_heads x index_head_dim; wk projects the hidden state to the index key, which is
// RMS-normalised; weights_proj gives one weight per index head; index queries and keys take
// the attention's rotary settings, qk_rope_head_dim and rope_theta of section "架构总览").
// Per token at position p:
//   q_idx[h]   = rot_p(cq . wq_b[h*Di .. h*Di + Di)^T)            (bf16)
//   w[h]       = hid . w_proj[h]^T                                 (fp32)
//   k_cache[p] = rot_p(g * x / sqrt(mean(x^2) + eps)), x = hid . wk^T (bf16)
// rot_p turns pair (2m, 2m+1) of the last R dims by p * theta^(-2m/R).
//
// Design for gfx950.  Two small GEMMs (decode: 32 tokens against 12.6 MB of wq_b, an
// HBM-bound stream of weight rows; prefill: 4096 tokens, a matrix-core contraction).
//  * frontend_proj_kernel: a workgroup computes 32 tokens x 128 outputs over one range of the
//    reduction dimension with the 32x32x16 bf16 MFMA (four wavefronts, 32 outputs each).  The
//    weights are stored [outputs, inputs] (as a linear layer's), so a lane's 16-byte operand
//    pieces of both A (a token row) and B (a weight row) are contiguous.  The reduction is split
//    over enough workgroups to fill the CUs when there are few tokens; fp32 partial sums go to
//    the workspace.  frontend_proj_lds_kernel stages 128 x 128 tiles through LDS for many tokens.
//  * frontend_finalize_kernel: per token, adds the partials in a fixed order and applies the
//    rotation (angles in fp64), the key's RMS normalisation (one wavefront) and the roundings;
//    the key is written to its cache row.
//  * With many tokens the index query needs no reduction split: its projection then runs last,
//    rotating and rounding in its epilogue from an angle table the finalize kernel writes, so
//    the query never makes an fp32 round trip through HBM.
#include <algorithm>
#include <cmath>

#include "lsa_internal.h"

namespace lsa {
namespace {

constexpr int kProjThreads = 256;  // 4 wavefronts
constexpr int kTargetGroups = 512; // two workgroups per CU
constexpr int kMinChunk = 256;     // reduction entries per split (16 matrix-core steps)
constexpr int kFinThreads = 256;
constexpr int kMaxRot = 128;       // rotated dims the finalize kernel holds angles for
constexpr int kFinBatch = 8;       // partial sums a finalize thread has in flight

struct ProjParams {
  const uint16_t* A;   // [T, K]
  const uint16_t* W0;  // rows [0, n_split) of the weights, [n_split, K]
  const uint16_t* W1;  // rows [n_split, N), [N - n_split, K]
  int n_split, T, N, K, kchunk, splits;
  float* out;          // [splits, T, N] fp32 partial sums (unrotated kernels)
  // rotated bf16 output (frontend_proj_lds_kernel<true>): the index query of one split
  const float2* table; // [T, R/2] (cos, sin) of each token's rotation angles
  int Di, R;
  uint16_t* q_out;     // [T, N]
};

// One launch for two projections of the same tiling (the index query, and the key with the head
// weights): x blocks [0, nx0) belong to p[0], the rest to p[1]; z is the reduction split.
struct ProjGroup {
  ProjParams p[2];
  int nx0;
};

// This workgroup's problem and x block; false when the problem has fewer splits than the grid.
__device__ __forceinline__ bool pick(const ProjGroup& G, ProjParams& P, int& bx) {
  const bool second = static_cast<int>(blockIdx.x) >= G.nx0;
  P = second ? G.p[1] : G.p[0];
  bx = second ? static_cast<int>(blockIdx.x) - G.nx0 : static_cast<int>(blockIdx.x);
  return static_cast<int>(blockIdx.z) < P.splits;
}

__device__ __forceinline__ uint16_t bf16_of(float x) {  // round to nearest even
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// A wavefront computes TM x TN blocks of 32 tokens x 32 outputs (each loaded fragment feeds TN
// or TM matrix-core steps); the four wavefronts of a workgroup sit side by side along the
// outputs, so they share the token rows through the cache.  Workgroup tile: 32*TM tokens x
// 128*TN outputs.
template <int TM, int TN>
__global__ __launch_bounds__(kProjThreads) void frontend_proj_kernel(ProjGroup G) {
  ProjParams P;
  int bx;
  if (!pick(G, P, bx)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, g = lane >> 5;
  const int t0 = blockIdx.y * 32 * TM;
  const int n0 = (bx * 4 + wave) * 32 * TN;
  const int s = blockIdx.z;
  const int k0 = s * P.kchunk, k1 = min(P.K, k0 + P.kchunk);
  // rows past the end re-read the last row (their results are not stored)
  const uint16_t* arow[TM];
  const uint16_t* wrow[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
    arow[i] = P.A + static_cast<size_t>(min(t0 + 32 * i + col, P.T - 1)) * P.K + 8 * g;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int nc = min(n0 + 32 * j + col, P.N - 1);
    wrow[j] = (nc < P.n_split ? P.W0 + static_cast<size_t>(nc) * P.K
                              : P.W1 + static_cast<size_t>(nc - P.n_split) * P.K) + 8 * g;
  }
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};
  constexpr int U = 4 / (TM * TN > 2 ? 2 : 1);  // 16-wide steps whose loads are issued together
  int k = k0;
  for (; k + 16 * U <= k1; k += 16 * U) {
    bf16x8 a[U][TM], b[U][TN];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int i = 0; i < TM; ++i) a[u][i] = load_bf16x8(arow[i] + k + 16 * u);
#pragma unroll
      for (int j = 0; j < TN; ++j) b[u][j] = load_bf16x8(wrow[j] + k + 16 * u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(a[u][i], b[u][j], acc[i][j]);
  }
  for (; k < k1; k += 16) {  // K is a multiple of 16
    bf16x8 a[TM], b[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = load_bf16x8(arow[i] + k);
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = load_bf16x8(wrow[j] + k);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
  }
  // lane (col, g) of block (i, j) holds output n0 + 32j + col for tokens t0 + 32i + acc_row(r, g)
  float* o = P.out + static_cast<size_t>(s) * P.T * P.N;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = n0 + 32 * j + col;
    if (n >= P.N) continue;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + 32 * i + acc_row(r, g);
        if (t < P.T) o[static_cast<size_t>(t) * P.N + n] = acc[i][j][r];
      }
  }
}

// Epilogue of the unsplit index query: a wavefront's 2 x 2 blocks of 32 tokens x 32 outputs
// (tokens from t0, outputs from n0) are rotated and written as bf16.  Output n = n0 + 32j + col
// has the parity of col (n0 is a multiple of 32), so lanes col and col ^ 1 hold the two halves
// of a pair; the even lane stores both.
__device__ __forceinline__ void rotate_store(const ProjParams& P, const f32x16 (&acc)[2][2], int t0,
                                             int n0, int col, int g) {
  const int half = P.R / 2, rot0 = P.Di - P.R;
  const bool even = (col & 1) == 0;
  auto partner = [](float x) {  // value of lane ^ 1 (quad_perm [1,0,3,2])
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));
  };
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + 32 * j + col;
    const int d = min(n, P.N - 1) % P.Di;
    const bool rot = d >= rot0;
    const bool any_rot = __ballot(rot) != 0;  // wavefront-uniform (false when R = 0)
    const float2* tab = P.table + (rot ? (d - rot0) >> 1 : 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      // the 16 tokens' angles of this block, requested together
      float2 cs[16];
      if (any_rot) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          cs[r] = tab[static_cast<size_t>(min(t0 + 32 * i + acc_row(r, g), P.T - 1)) * half];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + 32 * i + acc_row(r, g);
        const float own = acc[i][j][r], other = partner(own);
        float out = own;
        if (any_rot && rot)  // pair (x, y) -> (x c - y s, x s + y c)
          out = even ? own * cs[r].x - other * cs[r].y : other * cs[r].y + own * cs[r].x;
        const float hi = partner(out);
        if (even && n < P.N && t < P.T)
          *reinterpret_cast<uint32_t*>(P.q_out + static_cast<size_t>(t) * P.N + n) =
              static_cast<uint32_t>(bf16_of(out)) | (static_cast<uint32_t>(bf16_of(hi)) << 16);
      }
    }
  }
}

// Many tokens (prefill): a workgroup computes 128 tokens x 128 outputs, staging 32-wide steps of
// both operands in LDS (double-buffered) so each fragment read feeds two matrix-core steps; the
// next step's global loads are in flight during the current step's matrix-core work.  Wavefront
// w computes rows 64*(w/2) .. +63 and outputs 64*(w%2) .. +63 as 2 x 2 blocks of 32 x 32.  LDS
// rows are padded to 80 bytes, so the 16 lanes of each fragment-read phase hit distinct banks.
// Requires K (and so every chunk) to be a multiple of 64.  With ROT (the index query without a
// reduction split) the epilogue applies the rotation and writes bf16 directly: the two outputs
// of a pair sit in adjacent lanes, exchanged with one DPP swap.
constexpr int kLdsTile = 128;  // tokens and outputs per workgroup
constexpr int kLdsRow = 40;    // bf16 per LDS row: 32 plus 8 of padding

template <bool ROT>
__global__ __launch_bounds__(kProjThreads, 2) void frontend_proj_lds_kernel(ProjGroup G) {
  ProjParams P;
  int bx;
  if (!pick(G, P, bx)) return;
  __shared__ __attribute__((aligned(16))) uint16_t as[2][kLdsTile * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][kLdsTile * kLdsRow];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, g = lane >> 5;
  const int t0 = blockIdx.y * kLdsTile, n0 = bx * kLdsTile;
  const int s = blockIdx.z;
  const int k0 = s * P.kchunk, k1 = min(P.K, k0 + P.kchunk);
  // global -> LDS: 16-byte piece u = tid + 256 j (j < 2) of a 128 x 32 tile is row u / 4, part u % 4
  const uint16_t* asrc[2];
  const uint16_t* wsrc[2];
  int loff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int u = tid + kProjThreads * j, row = u >> 2, part = u & 3;
    asrc[j] = P.A + static_cast<size_t>(min(t0 + row, P.T - 1)) * P.K + 8 * part;
    const int nc = min(n0 + row, P.N - 1);
    wsrc[j] = (nc < P.n_split ? P.W0 + static_cast<size_t>(nc) * P.K
                              : P.W1 + static_cast<size_t>(nc - P.n_split) * P.K) + 8 * part;
    loff[j] = row * kLdsRow + 8 * part;
  }
  // two register sets of global loads: the step two ahead is requested while this one computes
  struct Set {
    u32x4 a[2], w[2];
  };
  auto gload = [&](Set& x, int k) {  // k past the chunk re-reads its last step (no branch)
    k = min(k, k1 - 32);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      x.a[j] = *reinterpret_cast<const u32x4*>(asrc[j] + k);
      x.w[j] = *reinterpret_cast<const u32x4*>(wsrc[j] + k);
    }
  };
  auto lstore = [&](int buf, const Set& x) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      *reinterpret_cast<u32x4*>(&as[buf][loff[j]]) = x.a[j];
      *reinterpret_cast<u32x4*>(&ws[buf][loff[j]]) = x.w[j];
    }
  };
  const int wr = 64 * (wave >> 1), wc = 64 * (wave & 1);
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  auto compute = [&](int buf) {
    bf16x8 fa[2][2], fw[2][2];  // [block][k half]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        fa[i][h] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                  &as[buf][(wr + 32 * i + col) * kLdsRow + 16 * h + 8 * g]));
        fw[i][h] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                  &ws[buf][(wc + 32 * i + col) * kLdsRow + 16 * h + 8 * g]));
      }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(fa[i][h], fw[j][h], acc[i][j]);
  };
  Set x0, x1;
  gload(x0, k0);
  gload(x1, k0 + 32);
  lstore(0, x0);  // waits for x0 only: x1 was requested after it
  __syncthreads();
  // steps k (LDS buffer 0) and k + 32 (buffer 1) per iteration, so every register set and buffer
  // has a fixed role and the loop has no exit in the middle (every chunk is a multiple of 64);
  // each buffer was last read before the barrier that precedes its store, and the last
  // iteration's stores (clamped re-reads) are never computed
  for (int k = k0; k < k1; k += 64) {
    gload(x0, k + 64);
    __builtin_amdgcn_sched_barrier(0);  // keep the request ahead of this step's work
    compute(0);
    lstore(1, x1);
    __syncthreads();
    gload(x1, k + 96);
    __builtin_amdgcn_sched_barrier(0);
    compute(1);
    lstore(0, x0);
    __syncthreads();
  }
  if constexpr (ROT) {
    rotate_store(P, acc, t0 + wr, n0 + wc, col, g);
    return;
  }
  float* o = P.out + static_cast<size_t>(s) * P.T * P.N;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wc + 32 * j + col;
    if (n >= P.N) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + wr + 32 * i + acc_row(r, g);
        if (t < P.T) o[static_cast<size_t>(t) * P.N + n] = acc[i][j][r];
      }
  }
}

struct FinParams {
  const float* qp;  // [sq, T, Hi*Di] partials of the index query (null: written by the projection)
  const float* kp;  // [skw, T, Di + Hi] partials of the raw key and the head weights
  int sq, skw;
  const float* gain;
  const int32_t* seqlens;
  int Lq, Hi, Di, R, S_max;
  float eps;
  uint16_t* q_idx;  // [T, Hi, Di]
  float* w;         // [T, Hi]
  uint16_t* k_cache;  // [B, S_max, Di]
  float2* table;    // [T, R/2] (cos, sin) for the rotated projection epilogue, or null
  double inv_freq[kMaxRot / 2];  // theta^(-2m/R)
};

// Two adjacent bf16 values (round to nearest even) at dst: one 4-byte store when dst allows it.
__device__ __forceinline__ void store_pair(uint16_t* dst, float u, float v) {
  const uint16_t a = bf16_of(u), b = bf16_of(v);
  if ((reinterpret_cast<uintptr_t>(dst) & 3u) == 0u) {
    *reinterpret_cast<uint32_t*>(dst) = static_cast<uint32_t>(a) | (static_cast<uint32_t>(b) << 16);
  } else {
    dst[0] = a;
    dst[1] = b;
  }
}

// Sum of the pairs src[0], src[stride], ... (n of them) in split order, kFinBatch loads in flight
// (indexes past n re-read the last pair and are not added).
__device__ __forceinline__ float2 sum_splits(const float* src, size_t stride, int n) {
  float u = 0.0f, v = 0.0f;
  for (int s0 = 0; s0 < n; s0 += kFinBatch) {
    float2 x[kFinBatch];
#pragma unroll
    for (int j = 0; j < kFinBatch; ++j)
      x[j] = *reinterpret_cast<const float2*>(src + static_cast<size_t>(min(s0 + j, n - 1)) * stride);
#pragma unroll
    for (int j = 0; j < kFinBatch; ++j)
      if (s0 + j < n) {
        u += x[j].x;
        v += x[j].y;
      }
  }
  return float2{u, v};
}

// The same for single values.
__device__ __forceinline__ float sum_splits1(const float* src, size_t stride, int n) {
  float u = 0.0f;
  for (int s0 = 0; s0 < n; s0 += kFinBatch) {
    float x[kFinBatch];
#pragma unroll
    for (int j = 0; j < kFinBatch; ++j) x[j] = src[static_cast<size_t>(min(s0 + j, n - 1)) * stride];
#pragma unroll
    for (int j = 0; j < kFinBatch; ++j)
      if (s0 + j < n) u += x[j];
  }
  return u;
}

// Grid (T, 1 + q blocks).  Block (t, 0): the key (one wavefront), the head weights and, for the
// rotated projection epilogue, token t's row of the angle table.  Block (t, y > 0): q pairs
// 256 (y - 1) .. + 255 of token t, one per thread.  Each block forms the angles it uses once
// (fp64: p up to 2^20 times a frequency up to 1 would lose most of an fp32 angle's bits).
__global__ __launch_bounds__(kFinThreads) void frontend_finalize_kernel(FinParams P) {
  __shared__ float cs[kMaxRot / 2], sn[kMaxRot / 2];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int T = gridDim.x;
  const int b = t / P.Lq;
  const int p = P.seqlens[b] - P.Lq + (t - b * P.Lq);
  const int half = P.R / 2, Di = P.Di, rot0 = Di - P.R;
  const int Nq = P.Hi * Di, Nkw = Di + P.Hi;
  const bool key_block = blockIdx.y == 0;
  // this thread's pair: q elements (e, e + 1) or key dims (e, e + 1); its partials are requested
  // before the angles are formed
  const int e = key_block ? 2 * tid : 2 * ((blockIdx.y - 1) * kFinThreads + tid);
  const bool mine = key_block ? (tid < kWave && e < Di) : e < Nq;
  float2 x = float2{0.0f, 0.0f};
  if (mine)
    x = key_block ? sum_splits(P.kp + static_cast<size_t>(t) * Nkw + e, static_cast<size_t>(T) * Nkw, P.skw)
                  : sum_splits(P.qp + static_cast<size_t>(t) * Nq + e, static_cast<size_t>(T) * Nq, P.sq);
  if (tid < half) {
    const double a = static_cast<double>(p) * P.inv_freq[tid];
    const float c = static_cast<float>(cos(a)), sv = static_cast<float>(sin(a));
    cs[tid] = c;
    sn[tid] = sv;
    if (key_block && P.table) P.table[static_cast<size_t>(t) * half + tid] = float2{c, sv};
  }
  __syncthreads();
  auto rotate = [&](int d, float& u, float& v) {  // pair (d, d + 1), d even
    if (d >= rot0) {
      const int m = (d - rot0) >> 1;
      const float c = cs[m], s = sn[m];
      const float x0 = u, y0 = v;
      u = x0 * c - y0 * s;
      v = x0 * s + y0 * c;
    }
  };
  float u = x.x, v = x.y;
  if (!key_block) {
    if (mine) {
      rotate(e % Di, u, v);
      store_pair(P.q_idx + static_cast<size_t>(t) * Nq + e, u, v);
    }
    return;
  }
  // head weights
  for (int h = tid; h < P.Hi; h += kFinThreads)
    P.w[static_cast<size_t>(t) * P.Hi + h] =
        sum_splits1(P.kp + static_cast<size_t>(t) * Nkw + Di + h, static_cast<size_t>(T) * Nkw, P.skw);
  // key: one wavefront, lane l holds dims 2l and 2l + 1 (Di <= 128)
  if (tid < kWave) {
    const float ss = wave_sum_f(u * u + v * v);
    const float inv = 1.0f / sqrtf(ss / static_cast<float>(Di) + P.eps);
    if (mine) {
      u = P.gain[e] * (u * inv);
      v = P.gain[e + 1] * (v * inv);
      rotate(e, u, v);
      if (p >= 0 && p < P.S_max)  // the caller guarantees it; a bad position writes nothing
        store_pair(P.k_cache + (static_cast<size_t>(b) * P.S_max + p) * Di + e, u, v);
    }
  }
}

// Workgroup tile: 32 tokens x 128 outputs for few tokens (decode), 64 x 256 from 64 tokens on,
// 128 x 128 through LDS from 128 tokens on when K is a multiple of 64.
bool lds_tiles(long T, int K) { return T >= 128 && K % 64 == 0; }
bool big_tiles(long T) { return T >= 64; }
long tile_t(long T, int K) { return lds_tiles(T, K) ? kLdsTile : big_tiles(T) ? 64 : 32; }
long tile_n(long T, int K) { return lds_tiles(T, K) ? kLdsTile : big_tiles(T) ? 256 : 128; }

struct Split {
  int splits = 1, kchunk = 64;
};

// Reduction split: enough workgroups to fill the CUs, but at least kMinChunk entries each; the
// chunk is a multiple of 64 (so the kernel's unrolled steps cover every chunk but the last).
Split plan_split(long T, long N, int K) {
  Split sp;
  const long tiles = ((T + tile_t(T, K) - 1) / tile_t(T, K)) * ((N + tile_n(T, K) - 1) / tile_n(T, K));
  long s = tiles > 0 ? (kTargetGroups + tiles - 1) / tiles : 1;
  s = std::max<long>(1, std::min<long>(s, K / kMinChunk));
  long chunk = (K + s - 1) / s;
  chunk = (chunk + 63) / 64 * 64;
  sp.kchunk = static_cast<int>(std::min<long>(chunk, K));
  sp.splits = static_cast<int>((K + sp.kchunk - 1) / sp.kchunk);
  return sp;
}

size_t align_up(size_t x) { return (x + kWorkspaceAlign - 1) & ~(kWorkspaceAlign - 1); }

// Workspace plan.  When the index query needs no reduction split and takes the LDS tiles, its
// projection rotates and writes bf16 itself (after the finalize kernel has written the angle
// table); otherwise its fp32 partials go through the finalize kernel.
struct Plan {
  Split sq, skw;
  bool rot_q;
  size_t q_bytes, k_bytes, table_bytes;
};

Plan make_plan(long T, int q_lora, int hidden, int Hi, int Di) {
  Plan pl;
  pl.sq = plan_split(T, static_cast<long>(Hi) * Di, q_lora);
  pl.skw = plan_split(T, Di + Hi, hidden);
  pl.rot_q = lds_tiles(T, q_lora) && pl.sq.splits == 1;
  pl.q_bytes = pl.rot_q ? 0 : align_up(static_cast<size_t>(pl.sq.splits) * T * Hi * Di * sizeof(float));
  pl.k_bytes = align_up(static_cast<size_t>(pl.skw.splits) * T * (Di + Hi) * sizeof(float));
  pl.table_bytes = pl.rot_q ? align_up(static_cast<size_t>(T) * (Di / 2) * sizeof(float2)) : 0;  // R <= Di
  return pl;
}

}  // namespace

int frontend_max_rot() { return kMaxRot; }

size_t frontend_workspace_bytes(int B, int Lq, int q_lora, int hidden, int Hi, int Di) {
  const long T = static_cast<long>(B) * Lq;
  if (T <= 0) return 0;
  const Plan pl = make_plan(T, q_lora, hidden, Hi, Di);
  return pl.q_bytes + pl.k_bytes + pl.table_bytes + kWorkspaceAlign;
}

hipError_t launch_frontend(const uint16_t* cq, const uint16_t* hid, const uint16_t* wq_b,
                           const uint16_t* wk, const float* gain, const uint16_t* w_proj,
                           const int32_t* seqlens, int B, int Lq, int q_lora, int hidden, int Hi,
                           int Di, int rope_dim, double theta, float eps, int S_max,
                           uint16_t* q_idx, float* w, uint16_t* k_cache, void* workspace,
                           hipStream_t stream) {
  const long T = static_cast<long>(B) * Lq;
  const long Nq = static_cast<long>(Hi) * Di, Nkw = Di + Hi;
  const Plan pl = make_plan(T, q_lora, hidden, Hi, Di);
  char* ws = align_workspace(workspace);
  float* qp = reinterpret_cast<float*>(ws);
  float* kp = reinterpret_cast<float*>(ws + pl.q_bytes);
  float2* table = reinterpret_cast<float2*>(ws + pl.q_bytes + pl.k_bytes);
  if ((T + 31) / 32 > 65535 || T > 0x7fffffffL) return hipErrorInvalidConfiguration;
  // tiles along the outputs of a problem with N outputs and reduction length K
  auto nx = [&](long N, int K) { return static_cast<int>((N + tile_n(T, K) - 1) / tile_n(T, K)); };
  auto same_tiling = [&](int K0, int K1) {
    return lds_tiles(T, K0) == lds_tiles(T, K1);  // tile sizes depend on T and on this alone
  };
  // launches one or two projections of the same tiling
  auto proj = [&](const ProjParams& a, long Na, const ProjParams* b, long Nb, bool rot) {
    ProjGroup G{{a, b ? *b : a}, nx(Na, a.K)};
    const int K = a.K;
    const dim3 grid(static_cast<unsigned>(G.nx0 + (b ? nx(Nb, b->K) : 0)),
                    static_cast<unsigned>((T + tile_t(T, K) - 1) / tile_t(T, K)),
                    static_cast<unsigned>(std::max(a.splits, b ? b->splits : 0)));
    if (rot)
      hipLaunchKernelGGL(frontend_proj_lds_kernel<true>, grid, dim3(kProjThreads), 0, stream, G);
    else if (lds_tiles(T, K))
      hipLaunchKernelGGL(frontend_proj_lds_kernel<false>, grid, dim3(kProjThreads), 0, stream, G);
    else if (big_tiles(T))
      hipLaunchKernelGGL((frontend_proj_kernel<2, 2>), grid, dim3(kProjThreads), 0, stream, G);
    else
      hipLaunchKernelGGL((frontend_proj_kernel<1, 1>), grid, dim3(kProjThreads), 0, stream, G);
    return hipGetLastError();
  };
  ProjParams pq{cq, wq_b, wq_b, static_cast<int>(Nq), static_cast<int>(T), static_cast<int>(Nq),
                q_lora, pl.sq.kchunk, pl.sq.splits, qp, table, Di, rope_dim, q_idx};
  ProjParams pk{hid, wk, w_proj, Di, static_cast<int>(T), static_cast<int>(Nkw), hidden, pl.skw.kchunk,
                pl.skw.splits, kp, nullptr, Di, rope_dim, nullptr};
  FinParams pf{pl.rot_q ? nullptr : qp, kp, pl.sq.splits, pl.skw.splits, gain, seqlens, Lq, Hi, Di,
               rope_dim, S_max, eps, q_idx, w, k_cache, pl.rot_q ? table : nullptr, {}};
  for (int m = 0; m < rope_dim / 2; ++m) pf.inv_freq[m] = std::pow(theta, -2.0 * m / rope_dim);
  const unsigned q_blocks = pl.rot_q ? 0u : static_cast<unsigned>((Nq / 2 + kFinThreads - 1) / kFinThreads);
  hipError_t err;
  if (pl.rot_q) {
    err = proj(pk, Nkw, nullptr, 0, false);
  } else if (same_tiling(q_lora, hidden)) {
    err = proj(pq, Nq, &pk, Nkw, false);
  } else if ((err = proj(pq, Nq, nullptr, 0, false)) == hipSuccess) {
    err = proj(pk, Nkw, nullptr, 0, false);
  }
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(frontend_finalize_kernel, dim3(static_cast<unsigned>(T), 1 + q_blocks),
                     dim3(kFinThreads), 0, stream, pf);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (pl.rot_q) return proj(pq, Nq, nullptr, 0, true);  // reads the angle table the finalize kernel wrote
  return hipSuccess;
}

}  // namespace lsa
