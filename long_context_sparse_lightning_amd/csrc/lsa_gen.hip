// Seeded synthetic-input fills (host loop and GPU kernel) for the counter-based SplitMix64
// generator defined in inputs.py.  No LSA arithmetic lives here: these functions only turn
// (stream state, flat element index) into values, identically on host and device.
//
// Kinds: 0 = dyadic bf16 ((h mod 7) - 3)/4; 1 = fp32 weight (1 + h mod 4)/8;
//        2 = unit-variance bf16 (Irwin-Hall n=4 over the 16-bit fields of h, scaled by c).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z;
}

__host__ __device__ inline uint32_t f32_bits(float f) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __float_as_uint(f);
#else
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
#endif
}

__host__ __device__ inline uint16_t bf16_rne(float f) {
  uint32_t u = f32_bits(f);
  uint32_t lsb = (u >> 16) & 1u;
  return static_cast<uint16_t>((u + 0x7FFFu + lsb) >> 16);
}

// One element: writes 2 bytes (bf16 kinds) or 4 bytes (weight kind) at dst.
__host__ __device__ inline void gen_one(void* dst, uint64_t j, int kind, uint64_t base, uint64_t idx,
                                        double c) {
  uint64_t h = mix64(base + (idx + 1ull) * kGamma);
  if (kind == 1) {
    float v = static_cast<float>(static_cast<int>(h % 4ull) + 1) * 0.125f;
    static_cast<float*>(dst)[j] = v;
  } else if (kind == 0) {
    float v = static_cast<float>(static_cast<int>(h % 7ull) - 3) * 0.25f;
    static_cast<uint16_t*>(dst)[j] = bf16_rne(v);
  } else {
    uint64_t s = (h & 0xFFFFull) + ((h >> 16) & 0xFFFFull) + ((h >> 32) & 0xFFFFull) + (h >> 48);
    double z = static_cast<double>(static_cast<int64_t>(s) - 131070) * c;
    static_cast<uint16_t*>(dst)[j] = bf16_rne(static_cast<float>(z));
  }
}

__global__ void gen_fill_kernel(void* dst, int kind, uint64_t base, uint64_t start, uint64_t count,
                                double c) {
  uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  for (uint64_t j = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; j < count;
       j += stride)
    gen_one(dst, j, kind, base, start + j, c);
}

}  // namespace

extern "C" {

// Host fill: dst[j] = value(start + j) for j < count.  Returns 0, or 1 on a bad kind.
int lsa_gen_fill_host(void* dst, int kind, uint64_t base, uint64_t start, uint64_t count, double c) {
  if (kind < 0 || kind > 2) return 1;
  for (uint64_t j = 0; j < count; ++j) gen_one(dst, j, kind, base, start + j, c);
  return 0;
}

// Host fill of selected rows: dst[r*row_len + d] = value(row_ids[r]*row_len + d).
int lsa_gen_fill_host_rows(void* dst, int kind, uint64_t base, const uint64_t* row_ids,
                           uint64_t nrows, uint64_t row_len, double c) {
  if (kind < 0 || kind > 2) return 1;
  for (uint64_t r = 0; r < nrows; ++r)
    for (uint64_t d = 0; d < row_len; ++d)
      gen_one(dst, r * row_len + d, kind, base, row_ids[r] * row_len + d, c);
  return 0;
}

// Device fill (enqueued on `stream`, no host sync).  Returns 0, 1 on a bad kind, 2 on a
// launch error.
int lsa_gen_fill_device(void* dst, int kind, uint64_t base, uint64_t start, uint64_t count, double c,
                        void* stream) {
  if (kind < 0 || kind > 2) return 1;
  if (count == 0) return 0;
  uint64_t blocks = (count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(gen_fill_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), dst, kind, base, start, count, c);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
