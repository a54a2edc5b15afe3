// Online chunking on gfx950: this library's own chunk-boundary rule.
//
// The pages claim online variable-length chunking as the step before the
// chunk summaries ("Long-Context Modeling with Dynamic Hierarchical Sparse
// Attention for On-Device LLMs", Abstract and Innovation; ICML 2026 page,
// Abstract) but state no rule.  The rule here is a plain one of our own:
//   sim[t] = cos(K[t-1], K[t]) over all KV heads of the two key rows (1 at a
//            sequence's first token and where either row is all zeros);
//   a chunk starting at c0 in a sequence ending at e ends at the first t in
//   [c0 + lo, min(c0 + hi, e)) with sim[t] < tau, else at min(c0 + hi, e).
//
// Kernel 1 (HBM-bound): a wave covers 64 consecutive tokens, with its lanes
// spread across the key row (16-byte loads, so each load instruction reads one
// contiguous span of the row); the previous row stays in registers, so every
// row is read once.  Per token the dot product and the two squared norms are
// reduced across the wave in fp32; the lane of the token writes sim and the
// cut decisions go into the word's bits by a ballot.
// Kernel 2 (latency-bound, one wave): walks the sequences in order.  The cut
// bitmap is staged in LDS 64 KB at a time, and a window of 64 words (4096
// tokens, one word per lane) sits in registers, so a step that stays inside
// the window is a mask, a ballot and a lane read, with no memory access.
#include "dhsa_internal.hpp"

namespace dhsa {
namespace {

constexpr int kSimWaves = 4;
constexpr int kSegWords = 8192;                   // bitmap words staged in LDS at a time (64 KB)
constexpr int kSimTok = 16;                       // tokens per wave of the similarity kernel

__device__ inline int seq_of_token(const int32_t* __restrict__ cu_seqlens, int B, int t) {
  int lo = 0, hi = B - 1;                         // last b with cu_seqlens[b] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_seqlens[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ inline void widen(const uint4& raw, float (&x)[8], uint16_t) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ inline void widen(const uint4& raw, float (&x)[4], float) {
  x[0] = __uint_as_float(raw.x); x[1] = __uint_as_float(raw.y);
  x[2] = __uint_as_float(raw.z); x[3] = __uint_as_float(raw.w);
}

template <int CTRL, int ROW_MASK>
__device__ inline float dpp_get(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK,
                                                               0xF, false));
}

// Sum over the wave on the VALU's cross-lane paths (DPP): pairs and quads by quad permutes, 8 and 16
// lanes by the half-row and row mirrors, then the row broadcasts of lanes 15 and 31 carry the rows'
// sums up to the last row; lane 63 ends with the total, which every lane reads.
__device__ inline float wave_sum(float x) {
  x += dpp_get<0xB1, 0xF>(x);                     // quad_perm [1,0,3,2]
  x += dpp_get<0x4E, 0xF>(x);                     // quad_perm [2,3,0,1]
  x += dpp_get<0x141, 0xF>(x);                    // row_half_mirror
  x += dpp_get<0x140, 0xF>(x);                    // row_mirror
  x += dpp_get<0x142, 0xA>(x);                    // row_bcast:15 into rows 1 and 3
  x += dpp_get<0x143, 0xC>(x);                    // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// NJ 16-byte pieces per lane cover the row (pieces j * 64 + lane; lanes past the row's end idle).
// A wave takes kSimTok consecutive tokens with R rows in flight: a ring of R row buffers, each refilled
// with the row R tokens ahead as soon as it has been consumed (refills past the wave's last token
// re-read that token, a cache hit).  Its kSimTok cut bits are one 16-bit quarter of a bitmap word.
template <typename T, int NJ, int R>
__global__ __launch_bounds__(kSimWaves * 64) void adjacent_sim_kernel(
    const T* __restrict__ k, const int32_t* __restrict__ cu_seqlens, int B, int ntok, int W, float tau,
    float* __restrict__ sim, uint16_t* __restrict__ cut_quarters) {
  constexpr int VEC = 16 / sizeof(T);             // elements per 16-byte load
  const int lane = threadIdx.x & 63;
  const int part = blockIdx.x * kSimWaves + (threadIdx.x >> 6);
  const int t0 = part * kSimTok;
  if (t0 >= ntok) {                               // wave-uniform: a quarter past T in the last word
    if (lane == 0 && part < (ntok + 63) / 64 * (64 / kSimTok)) cut_quarters[part] = 0;
    return;
  }
  const int npieces = W / VEC;
  const int t_end = min(t0 + kSimTok, ntok);
  // the sequence holding t0 and where the next one starts (wave-uniform)
  int b = seq_of_token(cu_seqlens, B, t0);
  int cur_start = cu_seqlens[b];
  int next_start = cu_seqlens[b + 1];
  // rows are kept as loaded (16-byte words) and widened to fp32 when used
  auto load_row = [&](int t, uint4 (&x)[NJ]) {
    const uint4* row = reinterpret_cast<const uint4*>(k + (size_t)t * W);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int p = j * 64 + lane;
      x[j] = p < npieces ? row[p] : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  uint4 ring[R][NJ];
  float prv[NJ][VEC];
  {
    uint4 raw[NJ];
    load_row(t0 > 0 ? t0 - 1 : 0, raw);
#pragma unroll
    for (int j = 0; j < NJ; ++j) widen(raw[j], prv[j], T{});
  }
#pragma unroll
  for (int r = 0; r < R; ++r) load_row(min(t0 + r, t_end - 1), ring[r]);
  float s_mine = 1.0f;
  uint32_t bits = 0u;
  for (int t = t0; t < t_end; t += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int tt = t + r;
      if (tt < t_end) {                           // wave-uniform
        while (tt >= next_start) {                // crossed into a later sequence (skips empty ones)
          ++b;
          cur_start = next_start;
          next_start = cu_seqlens[b + 1];
        }
        float cur[NJ][VEC];
#pragma unroll
        for (int j = 0; j < NJ; ++j) widen(ring[r][j], cur[j], T{});
        float dot = 0.f, na = 0.f, nc = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            dot = fmaf(prv[j][e], cur[j][e], dot);
            na = fmaf(prv[j][e], prv[j][e], na);
            nc = fmaf(cur[j][e], cur[j][e], nc);
          }
        dot = wave_sum(dot);
        na = wave_sum(na);
        nc = wave_sum(nc);
        float s = 1.0f;
        if (tt != cur_start && na > 0.f && nc > 0.f) s = dot / (sqrtf(na) * sqrtf(nc));
        if (s < tau) bits |= 1u << (tt - t0);
        if (lane == tt - t0) s_mine = s;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int e = 0; e < VEC; ++e) prv[j][e] = cur[j][e];
        load_row(min(tt + R, t_end - 1), ring[r]);
      }
    }
  }
  if (lane < t_end - t0) sim[t0 + lane] = s_mine;
  if (lane == 0) cut_quarters[part] = (uint16_t)bits;
}

__global__ __launch_bounds__(64) void chunk_walk_kernel(
    const unsigned long long* __restrict__ cut_bits, const int32_t* __restrict__ cu_seqlens, int B, int ntok,
    int lo, int hi, int32_t* __restrict__ cu_chunks, int32_t* __restrict__ seq_chunk_start,
    int32_t* __restrict__ num_chunks) {
  __shared__ unsigned long long seg[kSegWords];
  const int lane = threadIdx.x;
  const int nwords = (ntok + 63) >> 6;
  int seg0 = -1;                                  // first word staged in seg (-1: nothing yet)
  int win0 = -1;                                  // first word of the register window
  unsigned long long win = 0ull;                  // word win0 + lane
  unsigned long long nz = 0ull;                   // bit i: word win0 + i has a cut bit
  auto load_window = [&](int w0) {                // wave-uniform
    if (seg0 < 0 || w0 < seg0 || w0 + 64 > seg0 + kSegWords) {
      // stage the words the batch still has (at most kSegWords), 16 loads in flight per lane
      const int n = min(kSegWords, max(nwords - w0, 64));
      __builtin_amdgcn_wave_barrier();
      for (int x0 = 0; x0 < n; x0 += 16 * 64) {
        unsigned long long tmp[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int w = w0 + x0 + j * 64 + lane;
          tmp[j] = (w < nwords) ? cut_bits[w] : 0ull;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) seg[x0 + j * 64 + lane] = tmp[j];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      seg0 = w0;
    }
    // words of the segment past n are past the bitmap: zero them here rather than trust stale LDS
    win = (w0 + lane < nwords) ? seg[w0 - seg0 + lane] : 0ull;
    nz = __ballot(win != 0ull);
    win0 = w0;
  };
  auto word_at = [&](int i) {                     // word win0 + i, i wave-uniform
    const unsigned lo32 = __builtin_amdgcn_readlane((unsigned)win, i);
    const unsigned hi32 = __builtin_amdgcn_readlane((unsigned)(win >> 32), i);
    return ((unsigned long long)hi32 << 32) | lo32;
  };
  int pos = 0;                                    // chunks written so far
  int32_t outv = 0;                               // cu_chunks[(pos & ~63) + lane], stored 64 at a time
  auto emit = [&](int value) {                    // cu_chunks[pos] = value
    if (lane == (pos & 63)) outv = value;
    if ((pos & 63) == 63) cu_chunks[(pos & ~63) + lane] = outv;
    ++pos;
  };
  emit(0);
  if (lane == 0) seq_chunk_start[0] = 0;
  for (int b = 0; b < B; ++b) {
    const int e = cu_seqlens[b + 1];
    int c0 = cu_seqlens[b];
    while (c0 < e) {
      const int a = c0 + lo;
      const int end = min(c0 + hi, e);            // the host clamps lo, hi to T: no int overflow
      int cut = end;
      if (a < end) {
        const int wa = a >> 6, wb = (end - 1) >> 6;
        int w = wa;
        while (w <= wb) {                         // scan the words [w, wb] for the first cut bit
          if (win0 < 0 || w < win0 || w >= win0 + 64) load_window(w);
          const int i0 = w - win0, i1 = min(wb - win0, 63);
          unsigned long long cand = nz & (~0ull << i0) & (i1 == 63 ? ~0ull : ((2ull << i1) - 1ull));
          bool found = false;
          while (cand) {
            const int i = __builtin_ctzll(cand);
            const int wi = win0 + i;
            unsigned long long v = word_at(i);
            if (wi == wa) v &= ~0ull << (a & 63);
            if (wi == wb && (end & 63)) v &= (1ull << (end & 63)) - 1ull;
            if (v) {
              cut = (wi << 6) + __builtin_ctzll(v);
              found = true;
              break;
            }
            cand &= cand - 1ull;
          }
          if (found) break;
          w = win0 + 64;                          // continue past this window
        }
      }
      emit(cut);
      c0 = cut;
    }
    if (lane == 0) seq_chunk_start[b + 1] = pos - 1;
  }
  if ((pos & 63) != 0 && lane < (pos & 63)) cu_chunks[(pos & ~63) + lane] = outv;
  if (lane == 0) *num_chunks = pos - 1;
}

}  // namespace

hipError_t launch_adjacent_similarity(int B, int ntok, int W, int dtype, const int32_t* cu_seqlens, const void* k,
                                      float tau, float* sim, uint64_t* cut_bits, hipStream_t stream) {
  if (ntok == 0) return hipSuccess;
  const int parts = (ntok + 63) / 64 * (64 / kSimTok);   // every quarter of every bitmap word
  const dim3 grid((parts + kSimWaves - 1) / kSimWaves);
  const int npieces = W / (dtype == 1 ? 8 : 4);
  const int nj = (npieces + 63) / 64;             // the host allows npieces <= kSimMaxPieces
#define DHSA_SIM_LAUNCH(TY, NJ, R)                                                                           \
  hipLaunchKernelGGL((adjacent_sim_kernel<TY, NJ, R>), grid, dim3(kSimWaves * 64), 0, stream, (const TY*)k, \
                     cu_seqlens, B, ntok, W, tau, sim, (uint16_t*)cut_bits)
  if (dtype == 1) {
    if (nj <= 1) DHSA_SIM_LAUNCH(uint16_t, 1, 4);
    else if (nj <= 2) DHSA_SIM_LAUNCH(uint16_t, 2, 4);
    else if (nj <= 4) DHSA_SIM_LAUNCH(uint16_t, 4, 2);
    else DHSA_SIM_LAUNCH(uint16_t, 8, 1);
  } else {
    if (nj <= 1) DHSA_SIM_LAUNCH(float, 1, 4);
    else if (nj <= 2) DHSA_SIM_LAUNCH(float, 2, 4);
    else if (nj <= 4) DHSA_SIM_LAUNCH(float, 4, 2);
    else DHSA_SIM_LAUNCH(float, 8, 1);
  }
#undef DHSA_SIM_LAUNCH
  return hipGetLastError();
}

hipError_t launch_chunk_walk(int B, int ntok, const int32_t* cu_seqlens, const uint64_t* cut_bits, int lo, int hi,
                             int32_t* cu_chunks, int32_t* seq_chunk_start, int32_t* num_chunks, hipStream_t stream) {
  hipLaunchKernelGGL(chunk_walk_kernel, dim3(1), dim3(64), 0, stream, (const unsigned long long*)cut_bits,
                     cu_seqlens, B, ntok, lo, hi, cu_chunks, seq_chunk_start, num_chunks);
  return hipGetLastError();
}

}  // namespace dhsa
