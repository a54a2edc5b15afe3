// Stage 3 in full fp32 (vector ALU; no reduced-precision matrix path).
//
// Same operation as the bf16 kernel (ICML 2026 spotlight page, Abstract: exact
// attention over the kept interactions): query token t of chunk i, head h
// attends to the keys u <= t of the kept chunks of row (h, i).  A workgroup
// owns 64 query rows of one chunk and one head, one query row per lane of each
// of its SPLIT waves; the row's key batches (16 keys, in kept-chunk order) are
// dealt round robin to the waves, each staging its batches in its own LDS
// slice and keeping its own running max, sum and output per row (natural
// exponent on the scaled logits, value rows accumulated in fp32).  At the end
// the waves' states are merged through LDS by the first wave.
#include "dhsa_internal.hpp"

namespace dhsa {
namespace {

constexpr int kRows = 64;
constexpr int kKB = 16;
template <int D> struct F32Geo {
  static constexpr int SPLIT = D >= 128 ? 2 : 4;   // waves per workgroup (LDS and registers at d = 128)
};

__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
__global__ __launch_bounds__(kRows * F32Geo<D>::SPLIT) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ block_idx,
    const int32_t* __restrict__ cu_chunks, const int32_t* __restrict__ seq_chunk_start, float* __restrict__ out,
    float* __restrict__ lse, int B, int C, int T, int Hq, int Hkv, long long nnz, float scale, int row_tiles) {
  constexpr int SPLIT = F32Geo<D>::SPLIT;
  __shared__ __attribute__((aligned(16))) float Ks[SPLIT][kKB][D];
  __shared__ __attribute__((aligned(16))) float Vs[SPLIT][kKB][D];
  __shared__ float part[SPLIT - 1][D + 2][kRows];    // waves 1.. : (m, l, o[D]) per row
  int bid = blockIdx.x;
  const int rt = bid % row_tiles; bid /= row_tiles;
  const int i = bid % C;          bid /= C;
  const int h = bid;
  const int s_i = cu_chunks[i], e_i = cu_chunks[i + 1];
  const int q0 = s_i + rt * kRows;
  if (q0 >= e_i) return;                       // workgroup-uniform
  const int g = h / (Hq / Hkv);
  const int lane = threadIdx.x & (kRows - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kRows);
  const int t = q0 + lane;
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
  const int first = seq_chunk_start[seq_of_chunk(seq_chunk_start, B, i)];   // first chunk of i's sequence
  int batch = 0;                               // key batches of the row so far, in kept-chunk order
  for (int e = 0; e < rlen; ++e) {
    const int j = block_idx[(size_t)h * nnz + rp0 + e];
    if (j < first || j > i) continue;        // only chunks of i's sequence up to i are read (-1 padding too)
    const bool diag = j == i;
    const int ks = cu_chunks[j];
    const int ke = diag ? last_row + 1 : cu_chunks[j + 1];
    const int nbt = (ke - ks + kKB - 1) / kKB;
    // this wave's batches of the chunk: the ones whose row-wide number is w modulo SPLIT
    for (int bt = (w - batch % SPLIT + SPLIT) % SPLIT; bt < nbt; bt += SPLIT) {
      const int kt = ks + bt * kKB;
      wave_sync();                             // the previous batch's LDS reads are done
      for (int x = lane; x < kKB * D / 4; x += kRows) {
        const int key = x / (D / 4), c4 = x % (D / 4);
        const int u = kt + key;
        float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
        if (u < ke) {
          kk = reinterpret_cast<const float4*>(k + ((size_t)u * Hkv + g) * D)[c4];
          vv = reinterpret_cast<const float4*>(v + ((size_t)u * Hkv + g) * D)[c4];
        }
        reinterpret_cast<float4*>(&Ks[w][key][0])[c4] = kk;
        reinterpret_cast<float4*>(&Vs[w][key][0])[c4] = vv;
      }
      wave_sync();
      float z[kKB];
      float mx = -INFINITY;
#pragma unroll
      for (int x = 0; x < kKB; ++x) {
        float sc = 0.f;
#pragma unroll
        for (int y = 0; y < D; ++y) sc = fmaf(qv[y], Ks[w][x][y], sc);
        const int u = kt + x;
        const bool ok = u < ke && !(diag && u > t);
        z[x] = ok ? sc * scale : -INFINITY;
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
        for (int x = 0; x < kKB; ++x) acc = fmaf(z[x], Vs[w][x][y], acc);
        o[y] = acc;
      }
    }
    batch += nbt;
  }
  // merge: waves 1.. hand their states to the first wave, which rescales each to the common max
  if (w > 0) {
    part[w - 1][0][lane] = m_run;
    part[w - 1][1][lane] = l_run;
#pragma unroll
    for (int y = 0; y < D; ++y) part[w - 1][2 + y][lane] = o[y];
  }
  __syncthreads();
  if (w > 0 || !row_ok) return;
  float M = m_run;
#pragma unroll
  for (int x = 0; x < SPLIT - 1; ++x) M = fmaxf(M, part[x][0][lane]);
  const float M_use = (M == -INFINITY) ? 0.f : M;
  const float a0 = expf(m_run - M_use);
  float l_tot = l_run * a0;
#pragma unroll
  for (int y = 0; y < D; ++y) o[y] *= a0;
#pragma unroll
  for (int x = 0; x < SPLIT - 1; ++x) {
    const float ax = expf(part[x][0][lane] - M_use);
    l_tot = fmaf(part[x][1][lane], ax, l_tot);
#pragma unroll
    for (int y = 0; y < D; ++y) o[y] = fmaf(part[x][2 + y][lane], ax, o[y]);
  }
  const float inv_l = 1.0f / l_tot;
#pragma unroll
  for (int y = 0; y < D; ++y) out[((size_t)t * Hq + h) * D + y] = o[y] * inv_l;
  if (lse != nullptr) lse[(size_t)h * T + t] = M + logf(l_tot);
}

template <int D>
hipError_t launch_d(const Plan& p, const void* q, const void* k, const void* v, const int32_t* row_ptr,
                    int64_t nnz, const int32_t* block_idx, float scale, void* out, float* lse,
                    hipStream_t stream) {
  const int row_tiles = (p.max_chunk_len + kRows - 1) / kRows;
  const long long blocks = (long long)p.Hq * p.C * row_tiles;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(prefill_f32_kernel<D>, dim3((unsigned)blocks), dim3(kRows * F32Geo<D>::SPLIT), 0, stream,
                     (const float*)q,
                     (const float*)k, (const float*)v, row_ptr, block_idx, p.cu_chunks, p.seq_chunk_start,
                     (float*)out, lse, p.B, p.C, p.T, p.Hq, p.Hkv, (long long)nnz, scale, row_tiles);
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
