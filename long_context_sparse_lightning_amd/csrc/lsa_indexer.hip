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
// Loads for the next tile are issued before the matrix-core work of the current one, into the
// other of two register buffers (the loop is unrolled by two, so no register copy has to wait
// for a load in flight), and without a condition (past the end they re-read a clamped in-range
// row): a conditional prefetch makes the compiler wait for it together with the current tile.
// Scores are staged in LDS and written with coalesced stores after the scan: a global store in
// the loop would make the next overwrite of its data register wait for the store -- and, since
// loads and stores share one counter, for every prefetch issued before it.
#include "lsa_internal.h"

namespace lsa {
namespace {

constexpr int kThreads = 256;             // 4 wavefronts
constexpr int kTileKeys = 32;             // keys per wavefront step
constexpr int kWgStride = kTileKeys * 4;  // keys per workgroup step
constexpr int kMaxKeysPerWg = 8192;       // LDS score staging: 32 KB

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
  // wave index made provably uniform, so the tile loop below is scalar control flow (a
  // divergent loop exit would add a path on which the compiler waits for every load in flight)
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
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
  wait_vmcnt<0>();  // the query and weights are in: only key tiles are in flight below

  const uint16_t* kb_base = k_idx + static_cast<size_t>(b) * S_max * DI + g * (DI / 2);
  extern __shared__ float stage[];  // [keys_per_wg] scores of this workgroup's chunk

  auto load_tile = [&](bf16x8 (&dst)[NC], int t0) {
    const uint16_t* kp = kb_base + static_cast<size_t>(min(t0 + col, S_max - 1)) * DI;
#pragma unroll
    for (int c = 0; c < NC; ++c) dst[c] = load_bf16x8(kp + 8 * c);
  };
  auto score_tile = [&](const bf16x8 (&src)[NC], int t0) {
    f32x16 acc = {};
#pragma unroll
    for (int c = 0; c < NC; ++c) acc = mfma32(qa[c], src[c], acc);
    float part = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) part += wr[r] * fmaxf(acc[r], 0.0f);
    const float other = __shfl_xor(part, 32);
    if (g == 0) stage[t0 - start + col] = part + other;  // t0 - start + col < keys_per_wg
  };

  // tiles of this wavefront: t0 + i * kWgStride for i < ntiles; two per iteration, so both
  // register buffers have fixed roles and the loop has no exit in the middle
  int t = start + wave * kTileKeys;
  const int ntiles = t < end ? (end - t + kWgStride - 1) / kWgStride : 0;
  bf16x8 ka[NC], kc[NC];
  load_tile(ka, t);
  int i = 0;
  for (; i + 2 <= ntiles; i += 2) {
    load_tile(kc, t + kWgStride);
    __builtin_amdgcn_sched_barrier(0);  // keep the whole prefetch ahead of the matrix-core work
    score_tile(ka, t);
    load_tile(ka, t + 2 * kWgStride);  // past the end this re-reads a clamped row
    __builtin_amdgcn_sched_barrier(0);
    score_tile(kc, t + kWgStride);
    t += 2 * kWgStride;
  }
  if (i < ntiles) score_tile(ka, t);
  __syncthreads();
  float* srow = scores + static_cast<size_t>(row) * S_max + start;
  for (int i = threadIdx.x; i < end - start; i += kThreads) srow[i] = stage[i];
}

template <int DI>
hipError_t launch_di(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                     const int32_t* seqlens, int B, int Lq, int Hi, int S_max, float* scores,
                     hipStream_t stream) {
  const long rows = static_cast<long>(B) * Lq;
  // About 512 workgroups (two per CU, all resident at once) with whole workgroup steps per
  // chunk; long chunks amortise the query/weight loads and the ramp of each workgroup.
  long per = (rows * S_max + 511) / 512;
  per = ((per + kWgStride - 1) / kWgStride) * kWgStride;
  if (per < kWgStride) per = kWgStride;
  if (per > kMaxKeysPerWg) per = kMaxKeysPerWg;
  const int keys_per_wg = static_cast<int>(per);
  const int chunks = (S_max + keys_per_wg - 1) / keys_per_wg;
  const long grid = rows * chunks;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const size_t lds = static_cast<size_t>(keys_per_wg) * sizeof(float);
  hipLaunchKernelGGL(index_scores_kernel<DI>, dim3(static_cast<unsigned>(grid)), dim3(kThreads), lds,
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
