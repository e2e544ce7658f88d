// Lightning-indexer scores (stage 1 of the LSA hot path).
//
//   scores[b,i,s] = sum_h w[b,i,h] * max(0, q_idx[b,i,h,:] . k_idx[b,s,:])     for s <= p
//
// (page "MLX-VLM 的 LongCat-Flash-Lite-Sparse ...", section "LSA" for the score, section
// "预填充优化" for the ReLU-weighted head sum done in one fused epilogue without a
// [heads x keys] intermediate.)
//
// Design for gfx950.  One wavefront scores 32 keys at a time with the 32x32x16 bf16 matrix
// core: A = the query's index heads (32 rows, zero-padded past Hi), B = 32 keys; Di/16
// instructions cover the head dimension.  The query fragment stays in registers for the
// whole scan, so the only HBM stream is the key cache, read exactly once.  Each lane loads
// one 16-byte piece of a key per instruction; the two lanes holding a key cover its two
// halves, so the dims are assigned to the k index as: lane half g, step c -> dims
// [g*Di/2 + 8c, +8), identically for A and B (any consistent assignment gives the same dot
// product).  The epilogue multiplies each accumulator row (head) by its weight after the
// ReLU, sums the 16 heads a lane holds, and adds the partner lane's 16 heads: scores leave
// the kernel as one fp32 per key and the [heads x keys] tile never touches memory.
// Loads for the next tile are issued before the matrix-core work of the current one.
#include "lsa_internal.h"

namespace lsa {
namespace {

constexpr int kThreads = 256;             // 4 wavefronts
constexpr int kTileKeys = 32;             // keys per wavefront step
constexpr int kWgStride = kTileKeys * 4;  // keys per workgroup step

template <int DI>
__global__ __launch_bounds__(kThreads) void index_scores_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint16_t* __restrict__ k_idx, const int32_t* __restrict__ seqlens, int Lq, int Hi,
    int S_max, int keys_per_wg, int chunks_per_row, float* __restrict__ scores) {
  constexpr int NC = DI / 16;  // matrix-core steps over the head dimension
  const int row = blockIdx.x / chunks_per_row;
  const int chunk = blockIdx.x - row * chunks_per_row;
  const int b = row / Lq;
  // keys visible to this query (clamped so a bad seqlens value cannot write past the row)
  const int n = min(seqlens[b] - Lq + (row - b * Lq) + 1, S_max);
  const int start = chunk * keys_per_wg;
  if (start >= n) return;
  const int end = min(n, start + keys_per_wg);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 31;
  const int g = lane >> 5;

  bf16x8 qa[NC];
  {
    const uint16_t* qp = q_idx + (static_cast<size_t>(row) * Hi + col) * DI + g * (DI / 2);
#pragma unroll
    for (int c = 0; c < NC; ++c) qa[c] = col < Hi ? load_bf16x8(qp + 8 * c) : zero_bf16x8();
  }
  float wr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int h = acc_row(r, g);
    wr[r] = h < Hi ? w[static_cast<size_t>(row) * Hi + h] : 0.0f;
  }

  const uint16_t* kb_base = k_idx + static_cast<size_t>(b) * S_max * DI + g * (DI / 2);
  float* srow = scores + static_cast<size_t>(row) * S_max;

  int t = start + wave * kTileKeys;
  bf16x8 kb[NC];
  if (t < end) {
    const uint16_t* kp = kb_base + static_cast<size_t>(min(t + col, S_max - 1)) * DI;
#pragma unroll
    for (int c = 0; c < NC; ++c) kb[c] = load_bf16x8(kp + 8 * c);
  }
  for (; t < end; t += kWgStride) {
    // prefetch the next tile of this wavefront
    const int tn = t + kWgStride;
    bf16x8 kn[NC];
    if (tn < end) {
      const uint16_t* kp = kb_base + static_cast<size_t>(min(tn + col, S_max - 1)) * DI;
#pragma unroll
      for (int c = 0; c < NC; ++c) kn[c] = load_bf16x8(kp + 8 * c);
    }
    f32x16 acc = {};
#pragma unroll
    for (int c = 0; c < NC; ++c) acc = mfma32(qa[c], kb[c], acc);
    float part = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) part += wr[r] * fmaxf(acc[r], 0.0f);
    const float other = __shfl_xor(part, 32);
    const int key = t + col;
    if (g == 0 && key < end) srow[key] = part + other;
#pragma unroll
    for (int c = 0; c < NC; ++c) kb[c] = kn[c];
  }
}

template <int DI>
hipError_t launch_di(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                     const int32_t* seqlens, int B, int Lq, int Hi, int S_max, float* scores,
                     hipStream_t stream) {
  const long rows = static_cast<long>(B) * Lq;
  // Aim for >= ~2048 workgroups in total (8 per CU) with whole workgroup steps per chunk.
  long per = (rows * S_max + 2047) / 2048;
  per = ((per + kWgStride - 1) / kWgStride) * kWgStride;
  if (per < kWgStride) per = kWgStride;
  if (per > 16384) per = 16384;
  const int keys_per_wg = static_cast<int>(per);
  const int chunks = (S_max + keys_per_wg - 1) / keys_per_wg;
  const long grid = rows * chunks;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(index_scores_kernel<DI>, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                     stream, q_idx, w, k_idx, seqlens, Lq, Hi, S_max, keys_per_wg, chunks, scores);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_index_scores(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                               const int32_t* seqlens, int B, int Lq, int Hi, int Di, int S_max,
                               float* scores, hipStream_t stream) {
  switch (Di) {
    case 32: return launch_di<32>(q_idx, w, k_idx, seqlens, B, Lq, Hi, S_max, scores, stream);
    case 64: return launch_di<64>(q_idx, w, k_idx, seqlens, B, Lq, Hi, S_max, scores, stream);
    case 128: return launch_di<128>(q_idx, w, k_idx, seqlens, B, Lq, Hi, S_max, scores, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lsa
