// Stage 3 in full fp32 (vector ALU; no reduced-precision matrix path).
//
// Same operation as the bf16 kernel (ICML 2026 spotlight page, Abstract: exact
// attention over the kept interactions): query token t of chunk i, head h
// attends to the keys u <= t of the kept chunks of row (h, i).  One wave owns
// 64 query rows of one chunk and one head, one query row per lane.  Keys are
// staged 16 at a time in LDS and read as broadcasts; each lane scores the 16
// keys, updates its running max and sum once per batch (natural exponent on
// the scaled logits) and accumulates the value rows in fp32.
#include "dhsa_internal.hpp"

namespace dhsa {
namespace {

constexpr int kRows = 64;
constexpr int kKB = 16;

template <int D>
__global__ __launch_bounds__(kRows) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ block_idx,
    const int32_t* __restrict__ cu_chunks, float* __restrict__ out, float* __restrict__ lse,
    int C, int T, int Hq, int Hkv, long long nnz, float scale, int row_tiles) {
  __shared__ __attribute__((aligned(16))) float Ks[kKB][D];
  __shared__ __attribute__((aligned(16))) float Vs[kKB][D];
  int bid = blockIdx.x;
  const int rt = bid % row_tiles; bid /= row_tiles;
  const int i = bid % C;          bid /= C;
  const int h = bid;
  const int s_i = cu_chunks[i], e_i = cu_chunks[i + 1];
  const int q0 = s_i + rt * kRows;
  if (q0 >= e_i) return;
  const int g = h / (Hq / Hkv);
  const int tid = threadIdx.x;
  const int t = q0 + tid;
  const bool row_ok = t < e_i;
  const int last_row = min(q0 + kRows, e_i) - 1;

  float qv[D], o[D];
#pragma unroll
  for (int x = 0; x < D; ++x) {
    qv[x] = row_ok ? q[((size_t)t * Hq + h) * D + x] : 0.f;
    o[x] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;

  const int rp0 = row_ptr[i], rlen = row_ptr[i + 1] - rp0;
  for (int e = 0; e < rlen; ++e) {
    const int j = block_idx[(size_t)h * nnz + rp0 + e];
    if (j < 0 || j > i) continue;            // only causal chunks of this row are read
    const bool diag = j == i;
    const int ks = cu_chunks[j];
    const int ke = diag ? last_row + 1 : cu_chunks[j + 1];
    for (int kt = ks; kt < ke; kt += kKB) {
      __syncthreads();
      for (int x = tid; x < kKB * D / 4; x += kRows) {
        const int key = x / (D / 4), c4 = x % (D / 4);
        const int u = kt + key;
        float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
        if (u < ke) {
          kk = reinterpret_cast<const float4*>(k + ((size_t)u * Hkv + g) * D)[c4];
          vv = reinterpret_cast<const float4*>(v + ((size_t)u * Hkv + g) * D)[c4];
        }
        reinterpret_cast<float4*>(&Ks[key][0])[c4] = kk;
        reinterpret_cast<float4*>(&Vs[key][0])[c4] = vv;
      }
      __syncthreads();
      float z[kKB];
      float mx = -INFINITY;
#pragma unroll
      for (int x = 0; x < kKB; ++x) {
        float s = 0.f;
#pragma unroll
        for (int y = 0; y < D; ++y) s = fmaf(qv[y], Ks[x][y], s);
        const int u = kt + x;
        const bool ok = u < ke && !(diag && u > t);
        z[x] = ok ? s * scale : -INFINITY;
        mx = fmaxf(mx, z[x]);
      }
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = expf(m_run - m_use);
      float ls = 0.f;
#pragma unroll
      for (int x = 0; x < kKB; ++x) { z[x] = expf(z[x] - m_use); ls += z[x]; }
      l_run = l_run * alpha + ls;
      m_run = m_new;
#pragma unroll
      for (int y = 0; y < D; ++y) {
        float acc = o[y] * alpha;
#pragma unroll
        for (int x = 0; x < kKB; ++x) acc = fmaf(z[x], Vs[x][y], acc);
        o[y] = acc;
      }
    }
  }
  if (!row_ok) return;
  const float inv_l = 1.0f / l_run;
#pragma unroll
  for (int y = 0; y < D; ++y) out[((size_t)t * Hq + h) * D + y] = o[y] * inv_l;
  if (lse != nullptr) lse[(size_t)h * T + t] = m_run + logf(l_run);
}

template <int D>
hipError_t launch_d(const Plan& p, const void* q, const void* k, const void* v, const int32_t* row_ptr,
                    int64_t nnz, const int32_t* block_idx, float scale, void* out, float* lse,
                    hipStream_t stream) {
  const int row_tiles = (p.max_chunk_len + kRows - 1) / kRows;
  const long long blocks = (long long)p.Hq * p.C * row_tiles;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(prefill_f32_kernel<D>, dim3((unsigned)blocks), dim3(kRows), 0, stream, (const float*)q,
                     (const float*)k, (const float*)v, row_ptr, block_idx, p.cu_chunks, (float*)out, lse,
                     p.C, p.T, p.Hq, p.Hkv, (long long)nnz, scale, row_tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const Plan& p, const void* q, const void* k, const void* v,
                              const int32_t* row_ptr, int64_t nnz, const int32_t* block_idx,
                              float softmax_scale, void* out, float* lse, hipStream_t stream) {
  if (p.C == 0) return hipSuccess;
  switch (p.d) {
    case 32: return launch_d<32>(p, q, k, v, row_ptr, nnz, block_idx, softmax_scale, out, lse, stream);
    case 64: return launch_d<64>(p, q, k, v, row_ptr, nnz, block_idx, softmax_scale, out, lse, stream);
    case 128: return launch_d<128>(p, q, k, v, row_ptr, nnz, block_idx, softmax_scale, out, lse, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dhsa
