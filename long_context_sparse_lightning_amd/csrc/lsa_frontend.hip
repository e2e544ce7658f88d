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
//    the workspace.
//  * frontend_finalize_kernel: one workgroup per token adds the partials in a fixed order and
//    applies the rotation (angles in fp64, once per token), the key's RMS normalisation (one
//    wavefront) and the roundings; the key is written to its cache row.
#include <algorithm>

#include "lsa_internal.h"

namespace lsa {
namespace {

constexpr int kProjThreads = 256;  // 4 wavefronts
constexpr int kTargetGroups = 512; // two workgroups per CU
constexpr int kMinChunk = 256;     // reduction entries per split (16 matrix-core steps)
constexpr int kFinThreads = 256;
constexpr int kMaxRot = 128;       // rotated dims the finalize kernel holds angles for

struct ProjParams {
  const uint16_t* A;   // [T, K]
  const uint16_t* W0;  // rows [0, n_split) of the weights, [n_split, K]
  const uint16_t* W1;  // rows [n_split, N), [N - n_split, K]
  int n_split, T, N, K, kchunk;
  float* out;          // [splits, T, N]
};

// A wavefront computes TM x TN blocks of 32 tokens x 32 outputs (each loaded fragment feeds TN
// or TM matrix-core steps); the four wavefronts of a workgroup sit side by side along the
// outputs, so they share the token rows through the cache.  Workgroup tile: 32*TM tokens x
// 128*TN outputs.
template <int TM, int TN>
__global__ __launch_bounds__(kProjThreads) void frontend_proj_kernel(ProjParams P) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, g = lane >> 5;
  const int t0 = blockIdx.y * 32 * TM;
  const int n0 = (blockIdx.x * 4 + wave) * 32 * TN;
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

// Many tokens (prefill): a workgroup computes 128 tokens x 128 outputs, staging 32-wide steps of
// both operands in LDS (double-buffered) so each fragment read feeds two matrix-core steps; the
// next step's global loads are in flight during the current step's matrix-core work.  Wavefront
// w computes rows 64*(w/2) .. +63 and outputs 64*(w%2) .. +63 as 2 x 2 blocks of 32 x 32.  LDS
// rows are padded to 80 bytes, so the 16 lanes of each fragment-read phase hit distinct banks.
// Requires K (and so every chunk) to be a multiple of 64.
constexpr int kLdsTile = 128;  // tokens and outputs per workgroup
constexpr int kLdsRow = 40;    // bf16 per LDS row: 32 plus 8 of padding

__global__ __launch_bounds__(kProjThreads, 2) void frontend_proj_lds_kernel(ProjParams P) {
  __shared__ __attribute__((aligned(16))) uint16_t as[2][kLdsTile * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][kLdsTile * kLdsRow];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, g = lane >> 5;
  const int t0 = blockIdx.y * kLdsTile, n0 = blockIdx.x * kLdsTile;
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
  const float* qp;  // [sq, T, Hi*Di] partials of the index query
  const float* kp;  // [skw, T, Di + Hi] partials of the raw key and the head weights
  int sq, skw;
  const float* gain;
  const int32_t* seqlens;
  int Lq, Hi, Di, R, S_max;
  double theta;
  float eps;
  uint16_t* q_idx;  // [T, Hi, Di]
  float* w;         // [T, Hi]
  uint16_t* k_cache;  // [B, S_max, Di]
};

__device__ __forceinline__ uint16_t bf16_of(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

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

__global__ __launch_bounds__(kFinThreads) void frontend_finalize_kernel(FinParams P) {
  __shared__ float cs[kMaxRot / 2], sn[kMaxRot / 2];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int T = gridDim.x;
  const int b = t / P.Lq;
  const int p = P.seqlens[b] - P.Lq + (t - b * P.Lq);
  const int half = P.R / 2;
  // rotation of pair m at position p; the angle is formed and reduced in fp64 (p up to 2^20 times
  // a frequency up to 1 would lose most of an fp32 angle's bits)
  for (int m = tid; m < half; m += kFinThreads) {
    const double a = static_cast<double>(p) * pow(P.theta, -2.0 * m / P.R);
    cs[m] = static_cast<float>(cos(a));
    sn[m] = static_cast<float>(sin(a));
  }
  __syncthreads();
  const int Di = P.Di, rot0 = Di - P.R;
  auto rotate = [&](int d, float& u, float& v) {  // pair (d, d + 1), d even
    if (d >= rot0) {
      const int m = (d - rot0) >> 1;
      const float c = cs[m], s = sn[m];
      const float x = u, y = v;
      u = x * c - y * s;
      v = x * s + y * c;
    }
  };
  // index query: pairs of outputs, partials added in split order
  const int Nq = P.Hi * Di;
  for (int e = 2 * tid; e < Nq; e += 2 * kFinThreads) {
    float u = 0.0f, v = 0.0f;
#pragma unroll 4
    for (int s = 0; s < P.sq; ++s) {
      const float2 x = *reinterpret_cast<const float2*>(P.qp + (static_cast<size_t>(s) * T + t) * Nq + e);
      u += x.x;
      v += x.y;
    }
    rotate(e % Di, u, v);
    store_pair(P.q_idx + static_cast<size_t>(t) * Nq + e, u, v);
  }
  const int Nkw = Di + P.Hi;
  // head weights
  for (int h = tid; h < P.Hi; h += kFinThreads) {
    float x = 0.0f;
    for (int s = 0; s < P.skw; ++s) x += P.kp[(static_cast<size_t>(s) * T + t) * Nkw + Di + h];
    P.w[static_cast<size_t>(t) * P.Hi + h] = x;
  }
  // key: one wavefront, lane l holds dims 2l and 2l + 1 (Di <= 128)
  if (tid < kWave) {
    const int d = 2 * tid;
    const bool mine = d < Di;
    float u = 0.0f, v = 0.0f;
    if (mine) {
#pragma unroll 4
      for (int s = 0; s < P.skw; ++s) {
        const float* src = P.kp + (static_cast<size_t>(s) * T + t) * Nkw + d;
        u += src[0];
        v += src[1];
      }
    }
    const float ss = wave_sum_f(u * u + v * v);
    const float inv = 1.0f / sqrtf(ss / static_cast<float>(Di) + P.eps);
    if (mine) {
      u = P.gain[d] * (u * inv);
      v = P.gain[d + 1] * (v * inv);
      rotate(d, u, v);
      if (p >= 0 && p < P.S_max)  // the caller guarantees it; a bad position writes nothing
        store_pair(P.k_cache + (static_cast<size_t>(b) * P.S_max + p) * Di + d, u, v);
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

}  // namespace

int frontend_max_rot() { return kMaxRot; }

size_t frontend_workspace_bytes(int B, int Lq, int q_lora, int hidden, int Hi, int Di) {
  const long T = static_cast<long>(B) * Lq;
  if (T <= 0) return 0;
  const Split sq = plan_split(T, static_cast<long>(Hi) * Di, q_lora);
  const Split skw = plan_split(T, Di + Hi, hidden);
  return align_up(static_cast<size_t>(sq.splits) * T * Hi * Di * sizeof(float)) +
         align_up(static_cast<size_t>(skw.splits) * T * (Di + Hi) * sizeof(float)) + kWorkspaceAlign;
}

hipError_t launch_frontend(const uint16_t* cq, const uint16_t* hid, const uint16_t* wq_b,
                           const uint16_t* wk, const float* gain, const uint16_t* w_proj,
                           const int32_t* seqlens, int B, int Lq, int q_lora, int hidden, int Hi,
                           int Di, int rope_dim, double theta, float eps, int S_max,
                           uint16_t* q_idx, float* w, uint16_t* k_cache, void* workspace,
                           hipStream_t stream) {
  const long T = static_cast<long>(B) * Lq;
  const long Nq = static_cast<long>(Hi) * Di, Nkw = Di + Hi;
  const Split sq = plan_split(T, Nq, q_lora);
  const Split skw = plan_split(T, Nkw, hidden);
  char* ws = align_workspace(workspace);
  float* qp = reinterpret_cast<float*>(ws);
  float* kp = reinterpret_cast<float*>(ws + align_up(static_cast<size_t>(sq.splits) * T * Nq * sizeof(float)));
  if ((T + 31) / 32 > 65535 || T > 0x7fffffffL) return hipErrorInvalidConfiguration;
  auto proj = [&](const ProjParams& pp, long N, int splits) {
    const int K = pp.K;
    const dim3 grid(static_cast<unsigned>((N + tile_n(T, K) - 1) / tile_n(T, K)),
                    static_cast<unsigned>((T + tile_t(T, K) - 1) / tile_t(T, K)),
                    static_cast<unsigned>(splits));
    if (lds_tiles(T, K))
      hipLaunchKernelGGL(frontend_proj_lds_kernel, grid, dim3(kProjThreads), 0, stream, pp);
    else if (big_tiles(T))
      hipLaunchKernelGGL((frontend_proj_kernel<2, 2>), grid, dim3(kProjThreads), 0, stream, pp);
    else
      hipLaunchKernelGGL((frontend_proj_kernel<1, 1>), grid, dim3(kProjThreads), 0, stream, pp);
    return hipGetLastError();
  };
  ProjParams pq{cq, wq_b, wq_b, static_cast<int>(Nq), static_cast<int>(T), static_cast<int>(Nq),
                q_lora, sq.kchunk, qp};
  hipError_t err = proj(pq, Nq, sq.splits);
  if (err != hipSuccess) return err;
  ProjParams pk{hid, wk, w_proj, Di, static_cast<int>(T), static_cast<int>(Nkw), hidden, skw.kchunk, kp};
  if ((err = proj(pk, Nkw, skw.splits)) != hipSuccess) return err;
  FinParams pf{qp, kp, sq.splits, skw.splits, gain, seqlens, Lq, Hi, Di, rope_dim, S_max, theta, eps,
               q_idx, w, k_cache};
  hipLaunchKernelGGL(frontend_finalize_kernel, dim3(static_cast<unsigned>(T)), dim3(kFinThreads), 0,
                     stream, pf);
  return hipGetLastError();
}

}  // namespace lsa
