// Peak calibration for the roofline figures: the bf16 MFMA rate and the HBM
// read / copy rates this MI355X reaches in practice, next to the published
// peaks.  Measurement only: nothing on the attention path calls this library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pdllm_calib.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 4;                 // independent accumulators per wave

// Operand bits from a hash of the lane and a salt: full-entropy bf16 values
// (the MFMA rate depends on the data, so zero operands would overstate it).
__device__ __forceinline__ bf16x8 noise(uint32_t x) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    w[i] = (x & 0xbfffbfffu) | 0x3c003c00u;   // finite, random sign, magnitudes below 2
  }
  return __builtin_bit_cast(bf16x8, w);
}

__global__ __launch_bounds__(256) void mfma_peak_kernel(int64_t iters, float* sink) {
  const uint32_t id = blockIdx.x * 256u + threadIdx.x;
  const bf16x8 a = noise(id * 2654435761u + 1u), b = noise(id * 2246822519u + 7u);
  f32x16 c[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) c[k] = f32x16{};
  for (int64_t it = 0; it < iters; ++it)
#pragma unroll
    for (int k = 0; k < kChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += c[k][j];
  sink[id] = s;
}

// Workgroup w streams the w-th contiguous block of the buffer: consecutive
// threads take consecutive 16-byte vectors, four loads in flight each.
__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4* __restrict__ buf, int64_t n_vec,
                                                        int64_t per_wg, uint32_t* sink) {
  const int64_t v0 = (int64_t)blockIdx.x * per_wg;
  const int64_t v1 = v0 + per_wg < n_vec ? v0 + per_wg : n_vec;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t i = v0 + threadIdx.x;
  for (; i + 3 * 256 < v1; i += 4 * 256) {
    const u32x4 x0 = buf[i], x1 = buf[i + 256], x2 = buf[i + 512], x3 = buf[i + 768];
    acc ^= x0 ^ x1 ^ x2 ^ x3;
  }
  for (; i < v1; i += 256) acc ^= buf[i];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

__global__ __launch_bounds__(256) void hbm_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        int64_t n_vec, int64_t per_wg) {
  const int64_t v0 = (int64_t)blockIdx.x * per_wg;
  const int64_t v1 = v0 + per_wg < n_vec ? v0 + per_wg : n_vec;
  int64_t i = v0 + threadIdx.x;
  for (; i + 3 * 256 < v1; i += 4 * 256) {
    const u32x4 x0 = src[i], x1 = src[i + 256], x2 = src[i + 512], x3 = src[i + 768];
    dst[i] = x0;
    dst[i + 256] = x1;
    dst[i + 512] = x2;
    dst[i + 768] = x3;
  }
  for (; i < v1; i += 256) dst[i] = src[i];
}

}  // namespace

extern "C" {

int pdllm_calib_mfma_bf16(int64_t iters, int32_t n_wg, float* sink, void* stream) {
  if (iters < 1 || n_wg < 1 || sink == nullptr) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(n_wg), dim3(256), 0, (hipStream_t)stream, iters, sink);
  return (int)hipGetLastError();
}

int64_t pdllm_calib_mfma_bf16_flops(int64_t iters, int32_t n_wg) {
  return (int64_t)n_wg * 4 * iters * kChains * 32 * 32 * 16 * 2;
}

int pdllm_calib_hbm_read(const void* buf, int64_t bytes, int32_t n_wg, uint32_t* sink, void* stream) {
  if (buf == nullptr || sink == nullptr || bytes < 16 || bytes % 16 || n_wg < 1 ||
      reinterpret_cast<uintptr_t>(buf) % 16)
    return (int)hipErrorInvalidValue;
  const int64_t n_vec = bytes / 16;
  hipLaunchKernelGGL(hbm_read_kernel, dim3(n_wg), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(buf), n_vec, (n_vec + n_wg - 1) / n_wg, sink);
  return (int)hipGetLastError();
}

int pdllm_calib_hbm_copy(const void* src, void* dst, int64_t bytes, int32_t n_wg, void* stream) {
  if (src == nullptr || dst == nullptr || bytes < 16 || bytes % 16 || n_wg < 1 ||
      reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16)
    return (int)hipErrorInvalidValue;
  const int64_t n_vec = bytes / 16;
  hipLaunchKernelGGL(hbm_copy_kernel, dim3(n_wg), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n_vec, (n_vec + n_wg - 1) / n_wg);
  return (int)hipGetLastError();
}

}  // extern "C"
