// Calibration kernels for measurement (built into libdhsa_calib.so, not into the DHSA library):
// what this device sustains for the two bounds the DHSA kernels are measured against.
//
//  * dense bf16 MFMA: back-to-back independent v_mfma_f32_32x32x16_bf16 (four accumulator chains
//    per wave, two waves per SIMD), no memory traffic in the loop;
//  * HBM read: each workgroup streams one contiguous range of a device buffer, 16 bytes per lane
//    per load and eight loads in flight, folded into one value per thread so the loads cannot be
//    dropped (the fastest of the read shapes measured on this device).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dhsa_calib.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256, 2) void mfma_loop_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1e-3f * (float)(lane + e));
    b[e] = (__bf16)(1e-3f * (float)(lane - e));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ src, size_t n16,
                                                   float* __restrict__ out) {
  // workgroup b reads the contiguous range [b * per, (b + 1) * per), 8 loads in flight per lane
  constexpr int U = 8;
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  size_t x = lo + threadIdx.x;
  for (; x + (U - 1) * 256 < hi; x += U * 256) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[x + u * 256];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x + v[u].w;
  }
  for (; x < hi; x += 256) acc ^= src[x].x;
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = (float)(acc & 0xFFFF);
}

}  // namespace

extern "C" {

int dhsa_calib_mfma_bf16(int blocks, int iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || out == nullptr) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
  return (int)hipGetLastError();
}

int dhsa_calib_read(const void* src, size_t bytes, int blocks, float* out, void* stream) {
  if (src == nullptr || out == nullptr || blocks <= 0 || bytes % 16 != 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint4*)src, bytes / 16, out);
  return (int)hipGetLastError();
}

}  // extern "C"
