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
// Scores are ranked by their order-preserving bits (the fp32 order, with -0
// equal to +0); the general kernel appends the complemented chunk id, so a
// larger 64-bit key is a better candidate and ties resolve to the lower chunk
// id exactly.
//
// Main kernel: a workgroup owns one query chunk and four q heads (chunks with
// the most candidates are launched first).  Scoring: when the four heads share
// a KV head, each wave takes blocks of 16 candidates, four lanes per candidate
// (each a quarter of the row), and computes all four heads' dot products (one,
// when routing per KV head) from one read of the K summary, reduced across the
// four lanes; otherwise each wave scores its own head, one candidate per lane.
// The scores go to LDS.
// Selection, one wave per head: the row's scores are loaded into registers (64
// candidates per register), the k-th best score is found by a most-significant-
// bit-first binary search over the order-preserving score bits (each step
// counts the candidates at or above a trial value with wave ballots), and one
// pass in chunk order writes those above it plus the first ones equal to it,
// which is the (score desc, chunk asc) top-k already in ascending chunk order.
// Rows with more candidates than the registers hold go to a general kernel
// that bitonic-sorts all of the row's keys in LDS (under a chunk count or a
// token budget).
#include "dhsa_internal.hpp"
#include "select.hpp"

namespace dhsa {
namespace {

constexpr int kWaves = 4;
constexpr int kRegCand = kRouteRegCand;          // candidates held in registers
constexpr int kRegBatches = sel::kSelBatches;    // 64 per batch, one per lane
static_assert(kRegCand == sel::kSelCand, "selection capacity");
using sel::ordered_bits;
constexpr int kWideThreads = 256;
constexpr int kMaxCand = 8192;

__device__ inline uint64_t rank_key(float s, int j) {
  return ((uint64_t)ordered_bits(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}

__device__ inline int key_chunk(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

// TOKENS: the budget is token_budget[i] tokens instead of the row length (longest fitting prefix of
// the ranking; the row's unused entries get -1).
template <int D, bool GROUPED, bool TOKENS>
__global__ __launch_bounds__(kWaves * 64) void route_kernel(
    const float* __restrict__ q_sum, const float* __restrict__ k_sum,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ seq_chunk_start,
    int32_t* __restrict__ block_idx, int B, int C, int Hq, int Hkv, long long nnz,
    const int32_t* __restrict__ cu_chunks, const int32_t* __restrict__ token_budget) {
  __shared__ __attribute__((aligned(16))) float qs[kWaves][D];
  __shared__ float sc[kWaves][kRegCand];       // the four rows' scores
  const int nhb = (Hq + kWaves - 1) / kWaves;  // head blocks per chunk
  const int i = C - 1 - (int)blockIdx.x / nhb; // latest chunks (most candidates) first, all heads
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h0 = ((int)blockIdx.x % nhb) * kWaves;
  const int h = h0 + wave;
  const int G = Hq / Hkv;
  // When the workgroup's four q heads share one KV head, candidates are scored for all four at
  // once (block-uniform; then Hq % 4 == 0 and no wave leaves early).
  const bool shared_kv = G % kWaves == 0;
  if (h >= Hq) return;                         // only when Hq % 4 != 0: no block barrier is used then
  const int g = h / G;

  const int first = seq_chunk_start[seq_of_chunk(seq_chunk_start, B, i)];
  const int nc = i - first;
  const int kk = row_ptr[i + 1] - row_ptr[i] - 1;
  int32_t* out = block_idx + (size_t)h * nnz + row_ptr[i];
  // the same for every head of the chunk, so block-uniform
  if constexpr (TOKENS) {
    // every earlier chunk fits (the row then holds them all, ascending), or there is none
    if (token_budget[i] >= cu_chunks[i] - cu_chunks[first]) {
      for (int x = lane; x < nc; x += 64) out[x] = first + x;
      if (lane == 0) out[nc] = i;
      return;
    }
    if (nc > kRegCand) return;                 // more candidates than registers: the general kernel
  } else if (!(kk > 0 && kk < nc && nc <= kRegCand)) {
    if (kk >= nc) {                            // every earlier chunk is kept
      for (int x = lane; x < nc; x += 64) out[x] = first + x;
      if (lane == 0) out[nc] = i;
    } else if (kk == 0) {
      if (lane == 0) out[0] = i;
    }
    return;                                    // otherwise the general kernel writes this row
  }
  // the query side of the score: this head's summary, or (routing per KV head) the sum of the
  // group's summaries in ascending head order (one wave forms it when the four heads share a group)
  if (!(GROUPED && shared_kv) || wave == 0) {
    for (int x = lane; x < D; x += 64) {
      float acc = q_sum[((size_t)i * Hq + (GROUPED ? g * G : h)) * D + x];
      if constexpr (GROUPED)
        for (int hh = 1; hh < G; ++hh) acc += q_sum[((size_t)i * Hq + g * G + hh) * D + x];
      qs[wave][x] = acc;
    }
  }

  if (shared_kv) {
    __syncthreads();                           // every head's query vector is in LDS
    // lane = (candidate c of a block of 16, quarter qd); quarter qd holds float4 columns qd,
    // qd + 4, ... of the candidate's K summary
    constexpr int NV = D / 16;                 // float4 per lane per candidate
    // routing per KV head: the four heads share one group, so one query vector serves all
    constexpr int R = GROUPED ? 1 : kWaves;
    const int c = lane >> 2, qd = lane & 3;
    const int nblk = (nc + 15) >> 4;
    for (int blk = wave; blk < nblk; blk += kWaves) {
      float4 cur[NV];
      const int j = min(first + 16 * blk + c, i - 1);   // rows past the end re-read the last one
      const float4* kr = reinterpret_cast<const float4*>(k_sum + ((size_t)j * Hkv + g) * D);
#pragma unroll
      for (int x = 0; x < NV; ++x) cur[x] = kr[qd + 4 * x];
      asm volatile("" ::: "memory");           // re-read the query vectors from LDS each block
      float acc[kWaves] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int x = 0; x < NV; ++x) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float4 qv = *reinterpret_cast<const float4*>(&qs[r][4 * (qd + 4 * x)]);
          acc[r] = fmaf(qv.x, cur[x].x, acc[r]);
          acc[r] = fmaf(qv.y, cur[x].y, acc[r]);
          acc[r] = fmaf(qv.z, cur[x].z, acc[r]);
          acc[r] = fmaf(qv.w, cur[x].w, acc[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        acc[r] += __shfl_xor(acc[r], 1);
        acc[r] += __shfl_xor(acc[r], 2);
      }
      const float mine = qd == 0 ? acc[0] : qd == 1 ? acc[1] : qd == 2 ? acc[2] : acc[3];
      if (16 * blk + c < nc && qd < R) sc[qd][16 * blk + c] = mine;
    }
    __syncthreads();
  } else {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int jb = 0; jb < nc; jb += 64) {
      const int x0 = jb + lane;
      if (x0 >= nc) continue;
      const float4* kr = reinterpret_cast<const float4*>(k_sum + ((size_t)(first + x0) * Hkv + g) * D);
      float acc = 0.f;
#pragma unroll 4
      for (int x = 0; x < D / 4; ++x) {
        const float4 kv = kr[x];
        const float4 qv = *reinterpret_cast<const float4*>(&qs[wave][4 * x]);
        acc = fmaf(qv.x, kv.x, acc);
        acc = fmaf(qv.y, kv.y, acc);
        acc = fmaf(qv.z, kv.z, acc);
        acc = fmaf(qv.w, kv.w, acc);
      }
      sc[wave][x0] = acc;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  const int nb = (nc + 63) >> 6;
  const float* row = sc[GROUPED && shared_kv ? 0 : wave];
  uint32_t ob[kRegBatches];
#pragma unroll
  for (int b = 0; b < kRegBatches; ++b)
    ob[b] = (b < nb && 64 * b + lane < nc) ? ordered_bits(row[64 * b + lane]) : 0u;
  if constexpr (TOKENS) {
    int len[kRegBatches];
#pragma unroll
    for (int b = 0; b < kRegBatches; ++b) {
      const int j = first + 64 * b + lane;
      len[b] = (b < nb && j < i) ? cu_chunks[j + 1] - cu_chunks[j] : 0;
    }
    const int m = sel::select_tokens_dispatch<1>(nb, ob, len, token_budget[i], first, lane, out);
    for (int x = m + 1 + lane; x <= kk; x += 64) out[x] = -1;   // the row's unused capacity
    if (lane == 0) out[m] = i;
  } else {
    sel::select_dispatch<1>(nb, ob, kk, first, lane, out);
    if (lane == 0) out[kk] = i;
  }
}

// General rows: more candidates than the main kernel holds in registers.  The row's keys are sorted
// in LDS (a bitonic network, best first); with a chunk count the first kk are kept, with a token budget
// (TOKENS) the longest prefix of the sorted order whose chunk lengths fit (a block scan of the lengths
// in sorted order: the inclusive sums rise strictly, so the kept count is how many stay within the
// budget).  The kept chunks are written ascending, then the diagonal, then (TOKENS) -1 to the row's end.
template <int D, bool GROUPED, bool TOKENS>
__global__ __launch_bounds__(kWideThreads) void route_wide_kernel(
    const float* __restrict__ q_sum, const float* __restrict__ k_sum,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ seq_chunk_start,
    int32_t* __restrict__ block_idx, int B, int C, int Hq, int Hkv, long long nnz,
    const int32_t* __restrict__ cu_chunks, const int32_t* __restrict__ token_budget) {
  __shared__ uint64_t keys[kMaxCand];
  __shared__ uint32_t flags[kMaxCand / 32];
  __shared__ float qrow[D];
  __shared__ int warp_total[kWideThreads / 64];
  __shared__ int kept_total;
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int first = seq_chunk_start[seq_of_chunk(seq_chunk_start, B, i)];
  const int n = i - first;
  const int kk = row_ptr[i + 1] - row_ptr[i] - 1;
  if constexpr (TOKENS) {
    // rows the main kernel writes: few enough candidates, or a budget every earlier chunk fits in
    if (n <= kRegCand || token_budget[i] >= cu_chunks[i] - cu_chunks[first]) return;   // block-uniform
  } else {
    if (!(kk > 0 && kk < n && n > kRegCand)) return;   // block-uniform
  }
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
  const int wave = tid >> 6, lane = tid & 63;
  int m = kk;                                          // chunks kept before the diagonal
  if constexpr (TOKENS) {
    // thread tid takes the consecutive sorted positions [lo, hi): its lengths' sum, a block-wide
    // exclusive scan of those sums, then its positions whose inclusive sum stays within the budget
    const int budget = token_budget[i];
    const int per = (n + kWideThreads - 1) / kWideThreads;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int seg = 0;
    for (int x = lo; x < hi; ++x) {
      const int j = key_chunk(keys[x]);
      seg += cu_chunks[j + 1] - cu_chunks[j];
    }
    int incl = seg;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (lane == 63) warp_total[wave] = incl;
    if (tid == 0) kept_total = 0;
    __syncthreads();
    int acc = incl - seg;
    for (int w = 0; w < wave; ++w) acc += warp_total[w];
    int cnt = 0;
    for (int x = lo; x < hi; ++x) {
      const int j = key_chunk(keys[x]);
      acc += cu_chunks[j + 1] - cu_chunks[j];
      if (acc > budget) break;
      ++cnt;
    }
    atomicAdd(&kept_total, cnt);
    __syncthreads();
    m = kept_total;
    __syncthreads();                                   // warp_total is reused below
  }
  for (int x = tid; x < m; x += kWideThreads) {
    const int loc = key_chunk(keys[x]) - first;
    atomicOr(&flags[loc >> 5], 1u << (loc & 31));
  }
  __syncthreads();
  // Ascending compaction of the flagged chunks: each wave counts a quarter, then writes.
  int32_t* out = block_idx + (size_t)h * nnz + row_ptr[i];
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
  if (tid == 0) out[m] = i;
  if constexpr (TOKENS)
    for (int x = m + 1 + tid; x <= kk; x += kWideThreads) out[x] = -1;   // the row's unused capacity
}

template <int D, bool GROUPED>
hipError_t launch_route_d(const Plan& p, const float* q_sum, const float* k_sum, const int32_t* row_ptr,
                          int64_t nnz, int32_t* block_idx, bool wide_rows, hipStream_t stream) {
  dim3 grid(p.C * ((p.Hq + kWaves - 1) / kWaves));
  hipLaunchKernelGGL((route_kernel<D, GROUPED, false>), grid, dim3(kWaves * 64), 0, stream, q_sum, k_sum, row_ptr,
                     p.seq_chunk_start, block_idx, p.B, p.C, p.Hq, p.Hkv, (long long)nnz, p.cu_chunks, nullptr);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !wide_rows) return err;
  hipLaunchKernelGGL((route_wide_kernel<D, GROUPED, false>), dim3(p.C, p.Hq), dim3(kWideThreads), 0, stream, q_sum,
                     k_sum, row_ptr, p.seq_chunk_start, block_idx, p.B, p.C, p.Hq, p.Hkv, (long long)nnz,
                     p.cu_chunks, nullptr);
  return hipGetLastError();
}

template <int D>
hipError_t launch_route_g(const Plan& p, const float* q_sum, const float* k_sum, const int32_t* row_ptr,
                          int64_t nnz, int32_t* block_idx, bool wide_rows, bool grouped, hipStream_t stream) {
  return grouped ? launch_route_d<D, true>(p, q_sum, k_sum, row_ptr, nnz, block_idx, wide_rows, stream)
                 : launch_route_d<D, false>(p, q_sum, k_sum, row_ptr, nnz, block_idx, wide_rows, stream);
}

template <int D, bool GROUPED>
hipError_t launch_route_tokens_g(const Plan& p, const float* q_sum, const float* k_sum, const int32_t* token_budget,
                                 const int32_t* row_ptr, int64_t nnz, int32_t* block_idx, bool wide_rows,
                                 hipStream_t stream) {
  dim3 grid(p.C * ((p.Hq + kWaves - 1) / kWaves));
  hipLaunchKernelGGL((route_kernel<D, GROUPED, true>), grid, dim3(kWaves * 64), 0, stream, q_sum, k_sum, row_ptr,
                     p.seq_chunk_start, block_idx, p.B, p.C, p.Hq, p.Hkv, (long long)nnz, p.cu_chunks, token_budget);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !wide_rows) return err;
  hipLaunchKernelGGL((route_wide_kernel<D, GROUPED, true>), dim3(p.C, p.Hq), dim3(kWideThreads), 0, stream, q_sum,
                     k_sum, row_ptr, p.seq_chunk_start, block_idx, p.B, p.C, p.Hq, p.Hkv, (long long)nnz,
                     p.cu_chunks, token_budget);
  return hipGetLastError();
}

template <int D>
hipError_t launch_route_tokens_d(const Plan& p, const float* q_sum, const float* k_sum, const int32_t* token_budget,
                                 const int32_t* row_ptr, int64_t nnz, int32_t* block_idx, bool wide_rows,
                                 bool grouped, hipStream_t stream) {
  return grouped ? launch_route_tokens_g<D, true>(p, q_sum, k_sum, token_budget, row_ptr, nnz, block_idx, wide_rows,
                                                  stream)
                 : launch_route_tokens_g<D, false>(p, q_sum, k_sum, token_budget, row_ptr, nnz, block_idx, wide_rows,
                                                   stream);
}

}  // namespace

hipError_t launch_route_tokens(const Plan& p, const float* q_sum, const float* k_sum, const int32_t* token_budget,
                               const int32_t* row_ptr, int64_t nnz, int32_t* block_idx, bool wide_rows, bool grouped,
                               hipStream_t stream) {
  if (p.C == 0) return hipSuccess;
  switch (p.d) {
    case 32:
      return launch_route_tokens_d<32>(p, q_sum, k_sum, token_budget, row_ptr, nnz, block_idx, wide_rows, grouped,
                                       stream);
    case 64:
      return launch_route_tokens_d<64>(p, q_sum, k_sum, token_budget, row_ptr, nnz, block_idx, wide_rows, grouped,
                                       stream);
    case 128:
      return launch_route_tokens_d<128>(p, q_sum, k_sum, token_budget, row_ptr, nnz, block_idx, wide_rows, grouped,
                                        stream);
    case 256:
      return launch_route_tokens_d<256>(p, q_sum, k_sum, token_budget, row_ptr, nnz, block_idx, wide_rows, grouped,
                                        stream);
    default: return hipErrorInvalidValue;
  }
}

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
