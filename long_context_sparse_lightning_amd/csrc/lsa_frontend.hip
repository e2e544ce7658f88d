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

constexpr int kProjThreads = 256;  // 4 wavefronts x 32 outputs
constexpr int kTileT = 32;         // tokens per workgroup
constexpr int kTileN = 128;        // outputs per workgroup
constexpr int kTargetGroups = 512; // two workgroups per CU
constexpr int kFinThreads = 256;
constexpr int kMaxRot = 128;       // rotated dims the finalize kernel holds angles for

struct ProjParams {
  const uint16_t* A;   // [T, K]
  const uint16_t* W0;  // rows [0, n_split) of the weights, [n_split, K]
  const uint16_t* W1;  // rows [n_split, N), [N - n_split, K]
  int n_split, T, N, K, kchunk;
  float* out;          // [splits, T, N]
};

__global__ __launch_bounds__(kProjThreads) void frontend_proj_kernel(ProjParams P) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, g = lane >> 5;
  const int t0 = blockIdx.y * kTileT;
  const int n = blockIdx.x * kTileN + wave * 32 + col;  // this lane's weight row (B column)
  const int s = blockIdx.z;
  const int k0 = s * P.kchunk, k1 = min(P.K, k0 + P.kchunk);
  // rows past the end re-read the last row (their results are not stored)
  const uint16_t* arow = P.A + static_cast<size_t>(min(t0 + col, P.T - 1)) * P.K + 8 * g;
  const int nc = min(n, P.N - 1);
  const uint16_t* wrow = (nc < P.n_split ? P.W0 + static_cast<size_t>(nc) * P.K
                                         : P.W1 + static_cast<size_t>(nc - P.n_split) * P.K) + 8 * g;
  f32x16 acc = {};
  constexpr int U = 4;  // 16-wide steps whose loads are issued together
  int k = k0;
  for (; k + 16 * U <= k1; k += 16 * U) {
    bf16x8 a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a[u] = load_bf16x8(arow + k + 16 * u);
      b[u] = load_bf16x8(wrow + k + 16 * u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc = mfma32(a[u], b[u], acc);
  }
  for (; k < k1; k += 16) acc = mfma32(load_bf16x8(arow + k), load_bf16x8(wrow + k), acc);
  // lane (col, g) holds outputs n for tokens t0 + acc_row(r, g)
  if (n < P.N) {
    float* o = P.out + static_cast<size_t>(s) * P.T * P.N + n;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = t0 + acc_row(r, g);
      if (t < P.T) o[static_cast<size_t>(t) * P.N] = acc[r];
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
    for (int s = 0; s < P.sq; ++s) {
      const float* src = P.qp + (static_cast<size_t>(s) * T + t) * Nq + e;
      u += src[0];
      v += src[1];
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
    if (mine)
      for (int s = 0; s < P.skw; ++s) {
        const float* src = P.kp + (static_cast<size_t>(s) * T + t) * Nkw + d;
        u += src[0];
        v += src[1];
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

struct Split {
  int splits = 1, kchunk = 16;
};

Split plan_split(long T, long N, int K) {
  Split sp;
  const long tiles = ((T + kTileT - 1) / kTileT) * ((N + kTileN - 1) / kTileN);
  long s = tiles > 0 ? (kTargetGroups + tiles - 1) / tiles : 1;
  s = std::max<long>(1, std::min<long>(s, K / 16));
  long chunk = (K + s - 1) / s;
  chunk = (chunk + 15) / 16 * 16;
  sp.kchunk = static_cast<int>(chunk);
  sp.splits = static_cast<int>((K + chunk - 1) / chunk);
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
  const long ty = (T + kTileT - 1) / kTileT;
  if (ty > 65535 || T > 0x7fffffffL) return hipErrorInvalidConfiguration;

  ProjParams pq{cq, wq_b, wq_b, static_cast<int>(Nq), static_cast<int>(T), static_cast<int>(Nq),
                q_lora, sq.kchunk, qp};
  hipLaunchKernelGGL(frontend_proj_kernel,
                     dim3(static_cast<unsigned>((Nq + kTileN - 1) / kTileN), static_cast<unsigned>(ty),
                          static_cast<unsigned>(sq.splits)),
                     dim3(kProjThreads), 0, stream, pq);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  ProjParams pk{hid, wk, w_proj, Di, static_cast<int>(T), static_cast<int>(Nkw), hidden, skw.kchunk, kp};
  hipLaunchKernelGGL(frontend_proj_kernel,
                     dim3(static_cast<unsigned>((Nkw + kTileN - 1) / kTileN), static_cast<unsigned>(ty),
                          static_cast<unsigned>(skw.splits)),
                     dim3(kProjThreads), 0, stream, pk);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  FinParams pf{qp, kp, sq.splits, skw.splits, gain, seqlens, Lq, Hi, Di, rope_dim, S_max, theta, eps,
               q_idx, w, k_cache};
  hipLaunchKernelGGL(frontend_finalize_kernel, dim3(static_cast<unsigned>(T)), dim3(kFinThreads), 0,
                     stream, pf);
  return hipGetLastError();
}

}  // namespace lsa
