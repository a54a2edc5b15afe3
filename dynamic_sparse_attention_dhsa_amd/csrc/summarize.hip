// Stage 1: length-normalised chunk summaries on gfx950.
//
// "Long-Context Modeling with Dynamic Hierarchical Sparse Attention for
// On-Device LLMs" (Abstract, Innovation): a chunk is represented by the
// mean of its token vectors times sqrt(n) for a chunk of n tokens, i.e.
//   sum[c, h, :] = (sum over tokens t of chunk c of x[t, h, :]) / sqrt(n_c).
//
// In the packed THD layout the tokens of chunk c form one contiguous block of
// n_c rows of W = H * d elements, so the stage is a segmented column sum of a
// row-major matrix: a pure HBM stream.  A workgroup owns one (chunk, block of
// 512 columns); its eight waves take every eighth row, each lane accumulates 8
// adjacent columns in fp32 from 16-byte loads (bf16) with eight rows in
// flight, and the eight partial sums are combined through LDS in a fixed order,
// so results are reproducible run to run.  Q and K chunks go in one launch,
// column blocks fastest: the workgroups resident at any time read whole rows of
// neighbouring chunks, not one column slice of every chunk.
#include "dhsa_internal.hpp"

namespace dhsa {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kColsPerLane = 8;
constexpr int kColsPerBlock = 64 * kColsPerLane;  // 512
constexpr int kUnroll = 8;

struct Vec8 { float v[8]; };

__device__ inline void load8(const uint16_t* p, Vec8& o) {
  uint4 raw = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o.v[2 * i] = __uint_as_float(w[i] << 16);
    o.v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ inline void load8(const float* p, Vec8& o) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  o.v[0] = a.x; o.v[1] = a.y; o.v[2] = a.z; o.v[3] = a.w;
  o.v[4] = b.x; o.v[5] = b.y; o.v[6] = b.z; o.v[7] = b.w;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void summarize_kernel(
    const T* __restrict__ q, const T* __restrict__ k, float* __restrict__ q_sum,
    float* __restrict__ k_sum, const int32_t* __restrict__ cu_chunks, int Wq, int Wk, int nbq) {
  __shared__ float part[kWaves][kColsPerBlock];
  const int c = blockIdx.y;
  const bool is_q = (int)blockIdx.x < nbq;
  const int cb = is_q ? blockIdx.x : blockIdx.x - nbq;
  const int W = is_q ? Wq : Wk;
  const T* __restrict__ src = is_q ? q : k;
  float* __restrict__ dst = is_q ? q_sum : k_sum;

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int col = cb * kColsPerBlock + lane * kColsPerLane;
  const bool col_ok = col < W;
  const int s = cu_chunks[c];
  const int e = cu_chunks[c + 1];

  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;

  if (col_ok) {
    const T* base = src + (size_t)col;
    int r = s + wave;
    for (; r + (kUnroll - 1) * kWaves < e; r += kUnroll * kWaves) {
      Vec8 x[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) load8(base + (size_t)(r + u * kWaves) * W, x[u]);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += x[u].v[i];
    }
    for (; r < e; r += kWaves) {
      Vec8 x;
      load8(base + (size_t)r * W, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += x.v[i];
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[wave][lane * kColsPerLane + i] = acc[i];
  __syncthreads();

  const float inv_norm = 1.0f / sqrtf((float)(e - s));
  for (int x = threadIdx.x; x < kColsPerBlock; x += kThreads) {
    const int cc = cb * kColsPerBlock + x;
    if (cc < W) {
      float t = part[0][x];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) t += part[w][x];
      dst[(size_t)c * W + cc] = t * inv_norm;
    }
  }
}

}  // namespace

hipError_t launch_summarize(const Plan& p, const void* q, const void* k, float* q_sum, float* k_sum,
                            hipStream_t stream) {
  if (p.C == 0) return hipSuccess;
  const int Wq = p.Hq * p.d, Wk = p.Hkv * p.d;
  const int nbq = (Wq + kColsPerBlock - 1) / kColsPerBlock;
  const int nbk = (Wk + kColsPerBlock - 1) / kColsPerBlock;
  dim3 grid(nbq + nbk, p.C);
  if (p.dtype == 1) {
    hipLaunchKernelGGL(summarize_kernel<uint16_t>, grid, dim3(kThreads), 0, stream,
                       (const uint16_t*)q, (const uint16_t*)k, q_sum, k_sum, p.cu_chunks, Wq, Wk, nbq);
  } else {
    hipLaunchKernelGGL(summarize_kernel<float>, grid, dim3(kThreads), 0, stream, (const float*)q,
                       (const float*)k, q_sum, k_sum, p.cu_chunks, Wq, Wk, nbq);
  }
  return hipGetLastError();
}

}  // namespace dhsa
