// Stage 2: causal chunk routing on gfx950.
//
// "Long-Context Modeling with Dynamic Hierarchical Sparse Attention for
// On-Device LLMs" (Abstract): chunk-level similarity scores, upsampled to token
// level, decide which token interactions are kept; the ICML 2026 page
// (Abstract) makes the routing causal.  With a budget counted in chunks the
// broadcast of chunk scores to token pairs keeps whole chunks, so a row
// (q head h, query chunk i) keeps
//   the top-k earlier chunks j of its sequence by s_j = q_sum[i,h] . k_sum[j,h/G],
//   ranked by (s_j descending, j ascending), plus the diagonal chunk i,
// written ascending into its slice of the CSR block list.
//
// Routing once per KV head (a reading of the open GQA granularity) scores with
// the sum of the group's query summaries instead of one head's and gives every
// head of the group the same row.
//
// Ranking uses a 64-bit key (order-preserving bits of the fp32 score, then
// the complemented chunk id), so a larger key is a better candidate and every
// key is distinct: ties resolve to the lower chunk id exactly.
//
// Main kernel: a wave owns one q head and one query chunk (a workgroup: four q
// heads of one chunk; chunks with the most candidates are launched first).  It
// walks the candidates in batches of 64 (one per lane), computes the row's fp32
// dot products (when the four heads share a KV head, each batch of K summaries
// is staged once in LDS for all of them), and keeps the row's best 64 keys as a sorted
// wave-wide list: a batch is bitonic-sorted across lanes, merged with the list
// by an element-wise max against the reversed order, and re-sorted with a
// bitonic half-cleaner cascade.  Batches that cannot beat the row's current
// k-th key are skipped.  Rows keeping more than 64 chunks out of a longer
// candidate list go to a general kernel that bitonic-sorts all of the row's
// keys in LDS.
#include "dhsa_internal.hpp"

namespace dhsa {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxTop = 64;
constexpr int kWideThreads = 256;
constexpr int kMaxCand = 8192;

__device__ inline uint32_t ordered_bits(float s) {
  uint32_t u = (s == 0.0f) ? 0u : __float_as_uint(s);   // -0 and +0 rank equal
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline uint64_t rank_key(float s, int j) {
  return ((uint64_t)ordered_bits(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}

__device__ inline int key_chunk(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

__device__ inline uint64_t shfl_xor_u64(uint64_t x, int m) {
  uint32_t lo = __shfl_xor((unsigned)x, m);
  uint32_t hi = __shfl_xor((unsigned)(x >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

__device__ inline uint64_t shfl_u64(uint64_t x, int src) {
  uint32_t lo = __shfl((unsigned)x, src);
  uint32_t hi = __shfl((unsigned)(x >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

// Bitonic sort of one key per lane across the wave; ascending (lane 0 smallest)
// when `ascending`, else descending.
__device__ inline uint64_t wave_sort(uint64_t key, int lane, bool ascending) {
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      uint64_t other = shfl_xor_u64(key, stride);
      bool lower = (lane & stride) == 0;
      bool block_up = ((lane & size) == 0) == ascending;   // direction of this block
      bool keep_small = (lower == block_up);
      key = keep_small ? (key < other ? key : other) : (key > other ? key : other);
    }
  }
  return key;
}

__device__ inline uint32_t wave_sort_u32_asc(uint32_t v, int lane) {
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      uint32_t other = __shfl_xor(v, stride);
      bool lower = (lane & stride) == 0;
      bool block_up = (lane & size) == 0;
      bool keep_small = (lower == block_up);
      v = keep_small ? min(v, other) : max(v, other);
    }
  }
  return v;
}

// `top` is sorted descending across lanes; returns the best 64 of top U batch, sorted descending.
__device__ inline uint64_t merge_batch(uint64_t top, uint64_t batch, int lane) {
  uint64_t b = wave_sort(batch, lane, /*ascending=*/true);
  uint64_t m = top > b ? top : b;                 // bitonic: falls, then rises
#pragma unroll
  for (int stride = 32; stride > 0; stride >>= 1) {
    uint64_t other = shfl_xor_u64(m, stride);
    bool lower = (lane & stride) == 0;
    m = lower ? (m > other ? m : other) : (m < other ? m : other);
  }
  return m;
}

template <int D, bool GROUPED>
__global__ __launch_bounds__(kWaves * 64) void route_kernel(
    const float* __restrict__ q_sum, const float* __restrict__ k_sum,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ seq_chunk_start,
    int32_t* __restrict__ block_idx, int B, int C, int Hq, int Hkv, long long nnz) {
  __shared__ float qs[kWaves][D];
  __shared__ __attribute__((aligned(16))) float ks[64][D + 4];   // a batch of K summaries (padded rows)
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.y * kWaves + wave;
  const int i = C - 1 - blockIdx.x;            // latest chunks (most candidates) first
  const int G = Hq / Hkv;
  // When the workgroup's four q heads share one KV head, each batch of K summaries is loaded once
  // into LDS for all of them (block-uniform; then Hq % 4 == 0 and no wave leaves early).
  const bool shared_kv = G % kWaves == 0;
  if (h >= Hq) return;                         // only when Hq % 4 != 0: no block barrier is used then
  const int g = h / G;

  const int first = seq_chunk_start[seq_of_chunk(seq_chunk_start, B, i)];
  const int nc = i - first;
  const int kk = row_ptr[i + 1] - row_ptr[i] - 1;
  const bool select = kk > 0 && kk < nc && kk <= kMaxTop;   // same for every head of the chunk
  // the query side of the score: this head's summary, or (routing per KV head) the sum of the
  // group's summaries in ascending head order
  for (int x = lane; x < D; x += 64) {
    float acc = q_sum[((size_t)i * Hq + (GROUPED ? g * G : h)) * D + x];
    if constexpr (GROUPED)
      for (int hh = 1; hh < G; ++hh) acc += q_sum[((size_t)i * Hq + g * G + hh) * D + x];
    qs[wave][x] = acc;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // shared batches: each thread holds its share of the next batch in registers while the current
  // one is scored and merged
  constexpr int PER = 64 * (D / 4) / (kWaves * 64);
  float4 pre[PER];
  auto fetch = [&](int jb) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int x = threadIdx.x + p * kWaves * 64;
      const int row = x / (D / 4), c4 = x % (D / 4);
      const int jj = jb + row;
      pre[p] = jj < i ? reinterpret_cast<const float4*>(k_sum + ((size_t)jj * Hkv + g) * D)[c4]
                      : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  uint64_t top = 0;
  if (select) {
    if (shared_kv) fetch(first);
    for (int jb = first; jb < i; jb += 64) {
      const int j = jb + lane;
      float acc = 0.f;
      if (shared_kv) {
        __syncthreads();                       // the previous batch has been read
#pragma unroll
        for (int p = 0; p < PER; ++p) {
          const int x = threadIdx.x + p * kWaves * 64;
          *reinterpret_cast<float4*>(&ks[x / (D / 4)][4 * (x % (D / 4))]) = pre[p];
        }
        __syncthreads();
        if (jb + 64 < i) fetch(jb + 64);
#pragma unroll 8
        for (int x = 0; x < D / 4; ++x) {
          const float4 kv = *reinterpret_cast<const float4*>(&ks[lane][4 * x]);
          const float4 qv = *reinterpret_cast<const float4*>(&qs[wave][4 * x]);
          acc = fmaf(qv.x, kv.x, acc);
          acc = fmaf(qv.y, kv.y, acc);
          acc = fmaf(qv.z, kv.z, acc);
          acc = fmaf(qv.w, kv.w, acc);
        }
      } else if (j < i) {
        const float4* kr = reinterpret_cast<const float4*>(k_sum + ((size_t)j * Hkv + g) * D);
#pragma unroll 4
        for (int x = 0; x < D / 4; ++x) {
          const float4 kv = kr[x];
          const float4 qv = *reinterpret_cast<const float4*>(&qs[wave][4 * x]);
          acc = fmaf(qv.x, kv.x, acc);
          acc = fmaf(qv.y, kv.y, acc);
          acc = fmaf(qv.z, kv.z, acc);
          acc = fmaf(qv.w, kv.w, acc);
        }
      }
      const uint64_t key = j < i ? rank_key(acc, j) : 0ull;
      const uint64_t kth = shfl_u64(top, kk - 1);
      if (__ballot(key > kth) == 0ull) continue;
      top = merge_batch(top, key, lane);
    }
  }

  int32_t* out = block_idx + (size_t)h * nnz + row_ptr[i];
  if (select) {
    const uint32_t jj = lane < kk ? (uint32_t)key_chunk(top) : 0xFFFFFFFFu;
    const uint32_t srt = wave_sort_u32_asc(jj, lane);
    if (lane < kk) out[lane] = (int32_t)srt;
    if (lane == 0) out[kk] = i;
  } else if (kk >= nc) {                       // every earlier chunk is kept
    for (int x = lane; x < nc; x += 64) out[x] = first + x;
    if (lane == 0) out[nc] = i;
  } else if (kk == 0) {
    if (lane == 0) out[0] = i;
  }
  // otherwise 64 < kk < nc: the general kernel writes this row
}

// General rows: more than 64 kept chunks out of a longer candidate list.
template <int D, bool GROUPED>
__global__ __launch_bounds__(kWideThreads) void route_wide_kernel(
    const float* __restrict__ q_sum, const float* __restrict__ k_sum,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ seq_chunk_start,
    int32_t* __restrict__ block_idx, int B, int C, int Hq, int Hkv, long long nnz) {
  __shared__ uint64_t keys[kMaxCand];
  __shared__ uint32_t flags[kMaxCand / 32];
  __shared__ float qrow[D];
  __shared__ int warp_total[kWideThreads / 64];
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int first = seq_chunk_start[seq_of_chunk(seq_chunk_start, B, i)];
  const int n = i - first;
  const int kk = row_ptr[i + 1] - row_ptr[i] - 1;
  if (!(kk > kMaxTop && kk < n)) return;     // block-uniform
  const int g = h / (Hq / Hkv);
  int npad = 1;
  while (npad < n) npad <<= 1;

  for (int x = tid; x < D; x += kWideThreads) {
    const int G = Hq / Hkv, g0 = (h / G) * G;
    float acc = q_sum[((size_t)i * Hq + (GROUPED ? g0 : h)) * D + x];
    if constexpr (GROUPED)
      for (int hh = 1; hh < G; ++hh) acc += q_sum[((size_t)i * Hq + g0 + hh) * D + x];
    qrow[x] = acc;
  }
  for (int x = tid; x < kMaxCand / 32; x += kWideThreads) flags[x] = 0u;
  __syncthreads();
  for (int x = tid; x < npad; x += kWideThreads) {
    uint64_t key = 0ull;
    if (x < n) {
      const int j = first + x;
      const float* kr = k_sum + ((size_t)j * Hkv + g) * D;
      float acc = 0.f;
      for (int y = 0; y < D; ++y) acc = fmaf(qrow[y], kr[y], acc);
      key = rank_key(acc, j);
    }
    keys[x] = key;
  }
  __syncthreads();
  for (int size = 2; size <= npad; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int p = tid; p < npad / 2; p += kWideThreads) {
        const int a = 2 * stride * (p / stride) + (p % stride);
        const int b = a + stride;
        const bool desc = (a & size) == 0;
        const uint64_t ka = keys[a], kb = keys[b];
        if ((ka < kb) == desc) { keys[a] = kb; keys[b] = ka; }
      }
      __syncthreads();
    }
  }
  for (int x = tid; x < kk; x += kWideThreads) {
    const int loc = key_chunk(keys[x]) - first;
    atomicOr(&flags[loc >> 5], 1u << (loc & 31));
  }
  __syncthreads();
  // Ascending compaction of the flagged chunks: each wave counts a quarter, then writes.
  int32_t* out = block_idx + (size_t)h * nnz + row_ptr[i];
  const int wave = tid >> 6, lane = tid & 63;
  const int per = (n + 4 * 64 - 1) / (4 * 64) * 64;
  const int lo = wave * per, hi = min(n, lo + per);
  int cnt = 0;
  for (int base = lo; base < hi; base += 64) {
    const int x = base + lane;
    const bool f = x < hi && ((flags[x >> 5] >> (x & 31)) & 1u);
    cnt += __popcll(__ballot(f));
  }
  if (lane == 0) warp_total[wave] = cnt;
  __syncthreads();
  int pos = 0;
  for (int w = 0; w < wave; ++w) pos += warp_total[w];
  for (int base = lo; base < hi; base += 64) {
    const int x = base + lane;
    const bool f = x < hi && ((flags[x >> 5] >> (x & 31)) & 1u);
    const uint64_t bal = __ballot(f);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (f) out[pos + before] = first + x;
    pos += __popcll(bal);
  }
  if (tid == 0) out[kk] = i;
}

template <int D, bool GROUPED>
hipError_t launch_route_d(const Plan& p, const float* q_sum, const float* k_sum, const int32_t* row_ptr,
                          int64_t nnz, int32_t* block_idx, bool wide_rows, hipStream_t stream) {
  dim3 grid(p.C, (p.Hq + kWaves - 1) / kWaves);
  hipLaunchKernelGGL((route_kernel<D, GROUPED>), grid, dim3(kWaves * 64), 0, stream, q_sum, k_sum, row_ptr,
                     p.seq_chunk_start, block_idx, p.B, p.C, p.Hq, p.Hkv, (long long)nnz);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !wide_rows) return err;
  hipLaunchKernelGGL((route_wide_kernel<D, GROUPED>), dim3(p.C, p.Hq), dim3(kWideThreads), 0, stream, q_sum,
                     k_sum, row_ptr, p.seq_chunk_start, block_idx, p.B, p.C, p.Hq, p.Hkv, (long long)nnz);
  return hipGetLastError();
}

template <int D>
hipError_t launch_route_g(const Plan& p, const float* q_sum, const float* k_sum, const int32_t* row_ptr,
                          int64_t nnz, int32_t* block_idx, bool wide_rows, bool grouped, hipStream_t stream) {
  return grouped ? launch_route_d<D, true>(p, q_sum, k_sum, row_ptr, nnz, block_idx, wide_rows, stream)
                 : launch_route_d<D, false>(p, q_sum, k_sum, row_ptr, nnz, block_idx, wide_rows, stream);
}

}  // namespace

hipError_t launch_route(const Plan& p, const float* q_sum, const float* k_sum, const int32_t* row_ptr,
                        int64_t nnz, int32_t* block_idx, bool wide_rows, bool grouped, hipStream_t stream) {
  if (p.C == 0) return hipSuccess;
  switch (p.d) {
    case 32: return launch_route_g<32>(p, q_sum, k_sum, row_ptr, nnz, block_idx, wide_rows, grouped, stream);
    case 64: return launch_route_g<64>(p, q_sum, k_sum, row_ptr, nnz, block_idx, wide_rows, grouped, stream);
    case 128: return launch_route_g<128>(p, q_sum, k_sum, row_ptr, nnz, block_idx, wide_rows, grouped, stream);
    case 256: return launch_route_g<256>(p, q_sum, k_sum, row_ptr, nnz, block_idx, wide_rows, grouped, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dhsa
