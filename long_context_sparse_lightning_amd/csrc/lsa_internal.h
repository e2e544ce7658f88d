// Internal declarations shared by the LSA kernels and the C-ABI layer (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lsa {

// ------------------------------------------------------------------ vector types (gfx950)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBufferFlags = 0x00020000;  // buffer resource word 3 for gfx9-family raw buffers

// 16-byte global load of 8 bf16 values.
__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() { return __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0}); }

// D = A * B + C on the 32x32x16 bf16 matrix core.  Per lane l (c = l % 32, g = l / 32):
//   A: row c, k = 8g .. 8g+7;  B: column c, k = 8g .. 8g+7;
//   C/D register r: column c, row 8*(r/4) + 4*g + (r%4).
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 accumulator held in register r by lanes of half g.
__device__ __forceinline__ constexpr int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Lane prefix count of a 64-bit wave mask: number of set bits in lanes below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

__device__ __forceinline__ uint64_t wave_ballot(bool pred) { return __ballot(pred); }

// x combined with x of lane ^ 32 by the gfx950 permlane swap (VALU, no LDS round trip).  Swapping
// a value with itself leaves the lower half's value in every lane of r[0] and the upper half's
// in every lane of r[1], so the sum or maximum of the pair needs no per-lane select and is the
// same in both halves.
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Inclusive scan of op over the 64 lanes of a wavefront on the vector ALU (gfx9 DPP): shifts by
// 1, 2, 4 and 8 lanes within each row of 16, then the last lane of row 0 / row 2 into rows 1 / 3
// (row_bcast:15) and lane 31 into rows 2 and 3 (row_bcast:31).  Lanes with no source take
// `identity`.  No LDS round trip, unlike the __shfl family.
template <typename Op>
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t x, uint32_t identity, Op op) {
  const int id = static_cast<int>(identity);
  x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(id, static_cast<int>(x), 0x111, 0xf, 0xf, false)));
  x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(id, static_cast<int>(x), 0x112, 0xf, 0xf, false)));
  x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(id, static_cast<int>(x), 0x114, 0xf, 0xf, false)));
  x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(id, static_cast<int>(x), 0x118, 0xf, 0xf, false)));
  x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(id, static_cast<int>(x), 0x142, 0xa, 0xf, false)));
  x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(id, static_cast<int>(x), 0x143, 0xc, 0xf, false)));
  return x;
}

// Inclusive prefix sum over the lanes of a wavefront.
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t x) {
  return wave_scan_incl(x, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

// Value of lane 63 (the wavefront total of an inclusive scan), wave-uniform.
__device__ __forceinline__ uint32_t wave_last(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}

__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
  return wave_last(wave_scan_incl(x, 0xffffffffu, [](uint32_t a, uint32_t b) { return a < b ? a : b; }));
}

__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  return wave_last(wave_scan_incl(x, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; }));
}

// Float reductions over the wavefront (the scan on the bit patterns, combined as floats).
__device__ __forceinline__ float wave_max_f(float x) {
  const uint32_t r = wave_last(wave_scan_incl(__float_as_uint(x), __float_as_uint(-INFINITY),
                                              [](uint32_t a, uint32_t b) {
                                                return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
                                              }));
  return __uint_as_float(r);
}

__device__ __forceinline__ float wave_sum_f(float x) {
  const uint32_t r = wave_last(wave_scan_incl(__float_as_uint(x), 0u, [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
  return __uint_as_float(r);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).  The compiler
// folds it into its own wait tracking, so later waits count from here.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// ------------------------------------------------------------------ workspaces
// A caller's workspace may start at any address.  Every workspace size includes this much slack
// and the launchers use the buffer from its first kWorkspaceAlign-byte boundary, so the regions
// inside it can be read and written with 16-byte (and wider) accesses.
constexpr size_t kWorkspaceAlign = 256;
inline char* align_workspace(void* p) {
  return reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(p) + kWorkspaceAlign - 1) &
                                 ~static_cast<uintptr_t>(kWorkspaceAlign - 1));
}

// ------------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error; arguments were validated by the C-ABI layer.
hipError_t launch_index_scores(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                               const int32_t* seqlens, int B, int Lq, int Hi, int Di, int S_max,
                               float* scores, hipStream_t stream);

int topk_max_positions();  // largest S_max the top-k kernels accept
size_t topk_workspace_bytes(int B, int Lq, int S_max, int topk, int init_tokens, int local_tokens);
hipError_t launch_topk(const float* scores, const int32_t* seqlens, int B, int Lq, int S_max,
                       int topk, int init_tokens, int local_tokens, int32_t* indices,
                       int32_t* n_sel, void* workspace, hipStream_t stream);

// Exact merge of per-chunk candidate lists into the selection of rows [row0, row0 + rows):
// count[r][c] pairs (key, position) at cand[r][c][0 .. count), r relative to row0, each list the
// candidates of positions [c * chunk_keys, (c + 1) * chunk_keys) (a superset of that chunk's
// contribution to the row's top R, or all of its middle positions), with range[r][c][0..1]
// bounding its keys.  Rows with more than 16 lists are merged in two levels when `level1` (a
// device region of topk_merge_level1_bytes(rows, chunks, ...) bytes) is given, else in one.
int topk_merge_max_chunks();
size_t topk_merge_level1_bytes(long rows, int chunks, int topk, int init_tokens, int local_tokens);
hipError_t launch_topk_merge(const int32_t* seqlens, int Lq, int S_max, int topk, int init_tokens,
                             int local_tokens, int row0, int rows, int chunks, int chunk_keys,
                             uint32_t* count, uint32_t* range, uint2* cand, void* level1,
                             int32_t* indices, int32_t* n_sel, hipStream_t stream);

// Indexer and top-k in one pass: the scores never leave the chip.
size_t index_topk_workspace_bytes(int B, int Lq, int S_max, int topk, int init_tokens, int local_tokens);
hipError_t launch_index_topk(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                             const int32_t* seqlens, int B, int Lq, int Hi, int Di, int S_max,
                             int topk, int init_tokens, int local_tokens, int32_t* indices,
                             int32_t* n_sel, void* workspace, hipStream_t stream);

// With index_seqlens, each row also attends to the positions appended after the index pass
// ([index_seqlens[b], p], at most max_app); `app` sizes the plan for them.
size_t mla_workspace_bytes(int B, int Lq, int H, int Dv, int S_max, int topk, int dense, int app = 0);
hipError_t launch_mla(const uint16_t* q, const uint16_t* kv, const int32_t* indices,
                      const int32_t* n_sel, const int32_t* seqlens, int B, int Lq, int H, int Dqk,
                      int Dv, int S_max, int topk, float softmax_scale, uint16_t* out, float* lse,
                      void* workspace, hipStream_t stream, const int32_t* index_seqlens = nullptr,
                      int max_app = 0);

// Hierarchical indexing: block-mean keys, block scores, the kept blocks' token selection.
int hier_max_heads();
size_t hier_workspace_bytes(int B, int S_max, int Bk, int topk, int init, int local, int M);
hipError_t launch_block_keys(const uint16_t* k_idx, const int32_t* seqlens, int B, int S_max, int Di,
                             int Bk, int first_block, uint16_t* block_keys, hipStream_t stream);
hipError_t launch_hier_index_topk(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                                  const uint16_t* block_keys, const int32_t* seqlens, int B, int Hi,
                                  int Di, int S_max, int topk, int init, int local, int Bk, int M,
                                  int32_t* indices, int32_t* n_sel, void* workspace,
                                  hipStream_t stream);

// Indexer front end: index queries, head weights and the new keys of the current tokens.
int frontend_max_rot();
size_t frontend_workspace_bytes(int B, int Lq, int q_lora, int hidden, int Hi, int Di);
hipError_t launch_frontend(const uint16_t* cq, const uint16_t* hid, const uint16_t* wq_b,
                           const uint16_t* wk, const float* gain, const uint16_t* w_proj,
                           const int32_t* seqlens, int B, int Lq, int q_lora, int hidden, int Hi,
                           int Di, int rope_dim, double theta, float eps, int S_max,
                           uint16_t* q_idx, float* w, uint16_t* k_cache, void* workspace,
                           hipStream_t stream);

}  // namespace lsa
