// Absorbed-MLA attention over the selected latent rows (stage 3 of the LSA hot path).
//
// For each query row and head: logits l_s = scale * q . kv[s, :Dqk] over the selected rows s,
// softmax, and out = sum_s p_s kv[s, :Dv]  (page "MLX-VLM 的 LongCat-Flash-Lite-Sparse ...",
// section "LSA": decode gathers the latent rows named by the top-k indices, prefill applies
// the same selection as a sparse mask; section "架构总览": kv_lora_rank 512 and rope 64, so a
// row is 576 values and the value vector is its first 512).  Decode and prefill share this
// kernel: a prefill chunk is B*Lq independent query rows, each with its own selection.
//
// Design for gfx950.  A workgroup (4 wavefronts) owns one (query row, group of 32 heads,
// slice of the selected rows).  Rows arrive 32 at a time: each thread gathers 16-byte pieces
// of whole 1152-byte latent rows (consecutive threads read consecutive pieces of a row, so
// every row is read as full cache lines) into registers, and they are stored to LDS at a
// padded pitch (an odd number of 16-byte units, so the per-row fragment reads below hit
// distinct banks).  The next tile's gather is in flight while the current tile is computed.
//  * logits: S^T = KV_tile (32 rows x Dqk) . Q^T on the 32x32x16 bf16 matrix core; the Dqk/16
//    steps are split over the 4 wavefronts and their partial sums added in LDS in a fixed
//    order.  With rows as the M dimension each lane holds 16 rows of one head, so the
//    softmax max/sum needs one cross-lane exchange.
//  * online softmax in fp32 (base-2 exponentials with log2(e) folded into the scale); the
//    probabilities are rounded to bf16 and the running sum adds the rounded values, so the
//    normalisation matches what the value product sees.
//  * values: O (32 heads x Dv) += P (32 x 32 rows) . V; each wavefront owns Dv/4 output
//    columns.  P is already in the A-operand layout (the row order inside a k-step only has
//    to agree between A and B), and the B operand is read from the LDS tile per lane.
//  * several workgroups per query row when rows are few (decode): each writes fp32 partial
//    O with its max and sum, and a small combine kernel merges them with log-sum-exp weights.
#include <algorithm>

#include "lsa_internal.h"

namespace lsa {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;       // latent rows per tile
constexpr int kHeadGroup = 32;  // heads per workgroup (matrix-core M)
constexpr int kMaxSplits = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int DQK, int DV>
struct Cfg {
  static constexpr int NC = DQK / 16;           // matrix-core steps over Dqk
  static constexpr int NCW = (NC + 3) / 4;      // steps per wavefront (max)
  static constexpr int NB = DV / 32;            // 32-column output blocks
  static constexpr int NBW = (NB + 3) / 4;      // output blocks per wavefront (max)
  static constexpr int PITCH = DQK + 8;         // LDS row pitch in bf16 elements
  static constexpr int CPR = DQK / 8;           // 16-byte pieces per latent row
  static constexpr int TILE_PIECES = kTile * CPR;
  static constexpr int PPT = (TILE_PIECES + kThreads - 1) / kThreads;  // pieces per thread
  static_assert(DQK % 16 == 0 && DV % 32 == 0 && DV <= DQK, "unsupported head dims");
  static_assert(((PITCH * 2 / 16) & 1) == 1, "pitch must be an odd number of 16-byte units");
};

struct MlaParams {
  const uint16_t* q;
  const uint16_t* kv;
  const int32_t* indices;
  const int32_t* n_sel;
  const int32_t* seqlens;
  int Lq, H, S_max, topk;
  int hgroups, splits, kps;  // head groups, workgroups per (row, head group), rows per split
  float scale_log2;
  uint16_t* out;
  float* lse;
  float* ws_o;   // [rows][hgroups][splits][32][DV] partial outputs
  float* ws_ml;  // [rows][hgroups][splits][32][2]  running max (base 2) and sum
};

template <int DQK, int DV>
__global__ __launch_bounds__(kThreads, 2) void sparse_mla_kernel(MlaParams P) {
  using C = Cfg<DQK, DV>;
  __shared__ __attribute__((aligned(16))) uint16_t kvt[kTile * C::PITCH];
  __shared__ __attribute__((aligned(16))) float spart[4][4][kWave][4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, g = lane >> 5;
  int bid = blockIdx.x;
  const int split = bid % P.splits;
  bid /= P.splits;
  const int hg = bid % P.hgroups;
  const int row = bid / P.hgroups;
  const int b = row / P.Lq;
  const int n = min(P.seqlens[b] - P.Lq + (row - b * P.Lq) + 1, P.S_max);
  const int32_t* ilist = P.indices ? P.indices + static_cast<size_t>(row) * P.topk : nullptr;
  const int cnt = ilist ? min(P.n_sel[row], P.topk) : max(n, 0);
  const int j0 = split * P.kps;
  const int j1 = min(cnt, j0 + P.kps);
  const uint16_t* kv_b = P.kv + static_cast<size_t>(b) * P.S_max * DQK;

  // query fragments of this wavefront's Dqk steps (B operand: column = head, k = 8g..8g+7)
  const int head = hg * kHeadGroup + col;
  bf16x8 qf[C::NCW];
#pragma unroll
  for (int cc = 0; cc < C::NCW; ++cc) {
    const int c = wave + 4 * cc;
    qf[cc] = (head < P.H && c < C::NC)
                 ? load_bf16x8(P.q + (static_cast<size_t>(row) * P.H + head) * DQK + 16 * c + 8 * g)
                 : zero_bf16x8();
  }

  float m_run = -INFINITY, l_run = 0.0f;  // for head `col` (same in both lane halves)
  f32x16 o[C::NBW];
#pragma unroll
  for (int i = 0; i < C::NBW; ++i) o[i] = f32x16{};

  u32x4 stg[C::PPT];
  auto gather = [&](int tile) {
#pragma unroll
    for (int k = 0; k < C::PPT; ++k) {
      const int piece = tid + kThreads * k;
      stg[k] = u32x4{0, 0, 0, 0};
      if (piece < C::TILE_PIECES) {
        const int r = piece / C::CPR;
        const int pc = piece - r * C::CPR;
        const int j = tile + r;
        if (j < j1) {
          int s = ilist ? ilist[j] : j;
          s = min(max(s, 0), P.S_max - 1);
          stg[k] = *reinterpret_cast<const u32x4*>(kv_b + static_cast<size_t>(s) * DQK + 8 * pc);
        }
      }
    }
  };

  if (j0 < j1) gather(j0);
  for (int tile = j0; tile < j1; tile += kTile) {
    __syncthreads();  // the previous tile's LDS reads are done
#pragma unroll
    for (int k = 0; k < C::PPT; ++k) {
      const int piece = tid + kThreads * k;
      if (piece < C::TILE_PIECES) {
        const int r = piece / C::CPR;
        const int pc = piece - r * C::CPR;
        *reinterpret_cast<u32x4*>(&kvt[r * C::PITCH + 8 * pc]) = stg[k];
      }
    }
    __syncthreads();
    if (tile + kTile < j1) gather(tile + kTile);

    // ---- logits (partial over this wavefront's Dqk steps)
    f32x16 acc = {};
#pragma unroll
    for (int cc = 0; cc < C::NCW; ++cc) {
      const int c = wave + 4 * cc;
      if (c < C::NC) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(&kvt[col * C::PITCH + 16 * c + 8 * g]));
        acc = mfma32(a, qf[cc], acc);
      }
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *reinterpret_cast<f32x4*>(&spart[wave][q4][lane][0]) =
          f32x4{acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]};
    __syncthreads();
    float s[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      f32x4 t = *reinterpret_cast<const f32x4*>(&spart[0][q4][lane][0]);
#pragma unroll
      for (int w = 1; w < 4; ++w) t += *reinterpret_cast<const f32x4*>(&spart[w][q4][lane][0]);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[4 * q4 + e] = t[e];
    }

    // ---- online softmax for head `col` over this tile's rows acc_row(r, g)
    float mloc = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool ok = tile + acc_row(r, g) < j1;
      s[r] = ok ? s[r] * P.scale_log2 : -INFINITY;
      mloc = fmaxf(mloc, s[r]);
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);  // finite: every tile has a valid row
    const float alpha = exp2f(m_run - m_new);  // 0 on the first tile
    bf16x8 pa[2];
    float psum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint16_t pb = bf16_bits_rne(exp2f(s[r] - m_new));
      psum += bf16_bits_to_float(pb);
      pa[r >> 3][r & 7] = __builtin_bit_cast(__bf16, pb);
    }
    psum += __shfl_xor(psum, 32);
    l_run = alpha * l_run + psum;
    m_run = m_new;

    // ---- rescale and accumulate the value product
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float a = __shfl(alpha, acc_row(r, g));
#pragma unroll
      for (int nbw = 0; nbw < C::NBW; ++nbw) o[nbw][r] *= a;
    }
#pragma unroll
    for (int nbw = 0; nbw < C::NBW; ++nbw) {
      const int nb = wave + 4 * nbw;
      if (nb < C::NB) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8 vb;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            // the row that A's k index 8g + t refers to in step ks (rows acc_row(8ks + t, g))
            const int vr = 16 * ks + 8 * (t >> 2) + 4 * g + (t & 3);
            vb[t] = __builtin_bit_cast(__bf16, kvt[vr * C::PITCH + 32 * nb + col]);
          }
          o[nbw] = mfma32(pa[ks], vb, o[nbw]);
        }
      }
    }
  }

  // ---- epilogue
  if (P.splits == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float lr = __shfl(l_run, acc_row(r, g));
      const int hh = hg * kHeadGroup + acc_row(r, g);
      const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
#pragma unroll
      for (int nbw = 0; nbw < C::NBW; ++nbw) {
        const int nb = wave + 4 * nbw;
        if (nb < C::NB && hh < P.H)
          P.out[(static_cast<size_t>(row) * P.H + hh) * DV + 32 * nb + col] =
              bf16_bits_rne(o[nbw][r] * inv);
      }
    }
    if (wave == 0 && g == 0 && head < P.H && P.lse)
      P.lse[static_cast<size_t>(row) * P.H + head] =
          l_run > 0.0f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
  } else {
    const size_t slot = (static_cast<size_t>(row) * P.hgroups + hg) * P.splits + split;
    float* wo = P.ws_o + slot * kHeadGroup * DV;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
      for (int nbw = 0; nbw < C::NBW; ++nbw) {
        const int nb = wave + 4 * nbw;
        if (nb < C::NB) wo[acc_row(r, g) * DV + 32 * nb + col] = o[nbw][r];
      }
    }
    if (wave == 0 && g == 0) {
      P.ws_ml[slot * kHeadGroup * 2 + 2 * col] = m_run;
      P.ws_ml[slot * kHeadGroup * 2 + 2 * col + 1] = l_run;
    }
  }
}

// Merge the split partials of one (row, head): log-sum-exp weights in a fixed order.
template <int DV>
__global__ __launch_bounds__(128) void mla_combine_kernel(MlaParams P) {
  const int row = blockIdx.x / P.H;
  const int head = blockIdx.x - row * P.H;
  const int hg = head / kHeadGroup, hl = head - hg * kHeadGroup;
  const size_t slot0 = (static_cast<size_t>(row) * P.hgroups + hg) * P.splits;
  float mmax = -INFINITY;
  for (int s = 0; s < P.splits; ++s) mmax = fmaxf(mmax, P.ws_ml[(slot0 + s) * kHeadGroup * 2 + 2 * hl]);
  float L = 0.0f;
  for (int s = 0; s < P.splits; ++s) {
    const float ms = P.ws_ml[(slot0 + s) * kHeadGroup * 2 + 2 * hl];
    const float ls = P.ws_ml[(slot0 + s) * kHeadGroup * 2 + 2 * hl + 1];
    L += ms == -INFINITY ? 0.0f : exp2f(ms - mmax) * ls;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  for (int c = threadIdx.x; c < DV; c += blockDim.x) {
    float acc = 0.0f;
    for (int s = 0; s < P.splits; ++s) {
      const float ms = P.ws_ml[(slot0 + s) * kHeadGroup * 2 + 2 * hl];
      if (ms != -INFINITY)
        acc += exp2f(ms - mmax) * P.ws_o[((slot0 + s) * kHeadGroup + hl) * DV + c];
    }
    P.out[(static_cast<size_t>(row) * P.H + head) * DV + c] = bf16_bits_rne(acc * inv);
  }
  if (threadIdx.x == 0 && P.lse)
    P.lse[static_cast<size_t>(row) * P.H + head] = L > 0.0f ? (mmax + __log2f(L)) * kLn2 : -INFINITY;
}

struct MlaPlan {
  int hgroups = 1, splits = 1, kps = 0;
  size_t ws_o_bytes = 0, ws_ml_bytes = 0;
};

MlaPlan make_plan(long rows, int H, int Dv, int S_max, int topk, int dense) {
  MlaPlan pl;
  pl.hgroups = (H + kHeadGroup - 1) / kHeadGroup;
  const long keys = dense ? S_max : topk;
  const long units = rows * pl.hgroups;
  long splits = units > 0 ? (640 + units - 1) / units : 1;
  splits = std::min<long>(splits, (keys + kTile - 1) / kTile);
  splits = std::min<long>(splits, kMaxSplits);
  splits = std::max<long>(splits, 1);
  long kps = (keys + splits - 1) / splits;
  kps = ((kps + kTile - 1) / kTile) * kTile;
  if (kps < kTile) kps = kTile;
  splits = (keys + kps - 1) / kps;
  if (splits < 1) splits = 1;
  pl.splits = static_cast<int>(splits);
  pl.kps = static_cast<int>(std::min<long>(kps, 0x7fffffffL));
  if (pl.splits > 1) {
    const size_t slots = static_cast<size_t>(units) * pl.splits;
    pl.ws_o_bytes = (slots * kHeadGroup * Dv * 4 + 255) & ~static_cast<size_t>(255);
    pl.ws_ml_bytes = (slots * kHeadGroup * 2 * 4 + 255) & ~static_cast<size_t>(255);
  }
  return pl;
}

template <int DQK, int DV>
hipError_t launch_dims(const MlaParams& P, long rows, hipStream_t stream) {
  const long grid = rows * P.hgroups * P.splits;
  if (grid > 0x7fffffffL || rows * P.H > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((sparse_mla_kernel<DQK, DV>), dim3(static_cast<unsigned>(grid)),
                     dim3(kThreads), 0, stream, P);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || P.splits == 1) return err;
  hipLaunchKernelGGL((mla_combine_kernel<DV>), dim3(static_cast<unsigned>(rows * P.H)), dim3(128), 0,
                     stream, P);
  return hipGetLastError();
}

}  // namespace

size_t mla_workspace_bytes(int B, int Lq, int H, int Dv, int S_max, int topk, int dense) {
  const MlaPlan pl = make_plan(static_cast<long>(B) * Lq, H, Dv, S_max, topk, dense);
  return pl.ws_o_bytes + pl.ws_ml_bytes;
}

hipError_t launch_mla(const uint16_t* q, const uint16_t* kv, const int32_t* indices,
                      const int32_t* n_sel, const int32_t* seqlens, int B, int Lq, int H, int Dqk,
                      int Dv, int S_max, int topk, float softmax_scale, uint16_t* out, float* lse,
                      void* workspace, hipStream_t stream) {
  const long rows = static_cast<long>(B) * Lq;
  const MlaPlan pl = make_plan(rows, H, Dv, S_max, topk, indices == nullptr);
  MlaParams P{};
  P.q = q;
  P.kv = kv;
  P.indices = indices;
  P.n_sel = n_sel;
  P.seqlens = seqlens;
  P.Lq = Lq;
  P.H = H;
  P.S_max = S_max;
  P.topk = topk;
  P.hgroups = pl.hgroups;
  P.splits = pl.splits;
  P.kps = pl.kps;
  P.scale_log2 = softmax_scale * kLog2e;
  P.out = out;
  P.lse = lse;
  P.ws_o = static_cast<float*>(workspace);
  P.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.ws_o_bytes);
  if (Dqk == 576 && Dv == 512) return launch_dims<576, 512>(P, rows, stream);
  if (Dqk == 80 && Dv == 64) return launch_dims<80, 64>(P, rows, stream);
  return hipErrorInvalidValue;
}

}  // namespace lsa
