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
// Kernel 1 (HBM-bound): a wave covers 8 consecutive tokens, all their rows in
// flight at once (at rows of up to 2 KB), with its lanes spread across the key
// row (16-byte loads, so each load instruction reads one contiguous span of the
// row); the previous row stays in registers, so a row is read once per wave.
// Per token the dot product with the previous row and the row's squared norm
// (packed bf16 dot products for bf16 rows) are reduced across the wave in fp32,
// the previous row's norm being the last token's; the lane of the token writes
// sim, and the wave's cut decisions are one byte of a bitmap word.
// Kernel 2 (latency-bound, one workgroup): the greedy walk, split into segments
// walked speculatively by 16 waves and stitched by one (walks from different
// starts merge at their first common cut); a window of 64 bitmap words (4096
// tokens, one word per lane) sits in registers, so a step that stays inside
// the window is a mask, a ballot and a lane read, with no memory access.
#include "dhsa_internal.hpp"

namespace dhsa {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kSimWaves = 4;
constexpr int kSimTok = 8;                        // tokens per wave of the similarity kernel: one byte of a bitmap word

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
// with the row R tokens ahead as soon as it has been consumed.  Its kSimTok cut bits are one byte of a
// bitmap word.
template <typename T, int NJ, int R>
__global__ __launch_bounds__(kSimWaves * 64) void adjacent_sim_kernel(
    const T* __restrict__ k, const int32_t* __restrict__ cu_seqlens, int B, int ntok, int W, float tau,
    float* __restrict__ sim, uint8_t* __restrict__ cut_bytes) {
  constexpr int VEC = 16 / sizeof(T);             // elements per 16-byte load
  const int lane = threadIdx.x & 63;
  const int part = blockIdx.x * kSimWaves + (threadIdx.x >> 6);
  const int t0 = part * kSimTok;
  if (t0 >= ntok) {                               // wave-uniform: a byte past T in the last word
    if (lane == 0 && part < (ntok + 63) / 64 * (64 / kSimTok)) cut_bytes[part] = 0;
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
  constexpr bool BF = sizeof(T) == 2;
  // bf16: packed dot products of the rows as loaded (exact products, fp32 sums); fp32: rows widened
  // (a no-op) and multiply-added.  A lane's partial sums over its pieces: dot(prev, cur) and |cur|^2.
  auto partials = [&](const uint4 (&pv)[NJ], const uint4 (&cu)[NJ], float& dot, float& nc)
      __attribute__((always_inline)) {
    dot = 0.f;
    nc = 0.f;
    if constexpr (BF) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const uint32_t a[4] = {pv[j].x, pv[j].y, pv[j].z, pv[j].w};
        const uint32_t c[4] = {cu[j].x, cu[j].y, cu[j].z, cu[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 av = __builtin_bit_cast(bf16x2, a[e]), cv = __builtin_bit_cast(bf16x2, c[e]);
          dot = __builtin_amdgcn_fdot2_f32_bf16(av, cv, dot, false);
          nc = __builtin_amdgcn_fdot2_f32_bf16(cv, cv, nc, false);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        float a[VEC], c[VEC];
        widen(pv[j], a, T{});
        widen(cu[j], c, T{});
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          dot = fmaf(a[e], c[e], dot);
          nc = fmaf(c[e], c[e], nc);
        }
      }
    }
  };
  uint4 ring[R][NJ];
  uint4 prv[NJ];
  load_row(t0 > 0 ? t0 - 1 : 0, prv);
#pragma unroll
  for (int r = 0; r < R; ++r) load_row(min(t0 + r, t_end - 1), ring[r]);
  // |row t0 - 1|^2; afterwards each token's |previous row|^2 is the last token's |row|^2
  float na;
  {
    float unused;
    partials(prv, prv, unused, na);
    na = wave_sum(na);
  }
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
        float dot, nc;
        partials(prv, ring[r], dot, nc);
        dot = wave_sum(dot);
        nc = wave_sum(nc);
        float s = 1.0f;
        if (tt != cur_start && na > 0.f && nc > 0.f) s = dot / (sqrtf(na) * sqrtf(nc));
        if (s < tau) bits |= 1u << (tt - t0);
        if (lane == tt - t0) s_mine = s;
        na = nc;
#pragma unroll
        for (int j = 0; j < NJ; ++j) prv[j] = ring[r][j];
        if (tt + R < t_end) load_row(tt + R, ring[r]);   // (wave-uniform)
      }
    }
  }
  if (lane < t_end - t0) sim[t0 + lane] = s_mine;
  if (lane == 0) cut_bytes[part] = (uint8_t)bits;
}

// One greedy step for one wave: the chunk starting at c0, in a sequence ending at e, ends at the
// returned position.  The wave keeps a window of 64 bitmap words in registers (word win0 + lane in
// `win`, bit i of `nz` set when word win0 + i has a cut bit) and reloads it from memory when a scan
// leaves it.  win0 and nz are wave-uniform.
__device__ inline int walk_step(const unsigned long long* __restrict__ cut_bits, int nwords, int lane, int c0, int e,
                                int lo, int hi, int& win0, unsigned long long& win, unsigned long long& nz) {
  const int a = c0 + lo;
  const int end = min(c0 + hi, e);                // the host clamps lo, hi to T: no int overflow
  if (a >= end) return end;
  const int wa = a >> 6, wb = (end - 1) >> 6;
  int w = wa;
  while (w <= wb) {                               // scan the words [w, wb] for the first cut bit
    if (win0 < 0 || w < win0 || w >= win0 + 64) {
      win = (w + lane < nwords) ? cut_bits[w + lane] : 0ull;
      nz = __ballot(win != 0ull);
      win0 = w;
    }
    const int i0 = w - win0, i1 = min(wb - win0, 63);
    unsigned long long cand = nz & (~0ull << i0) & (i1 == 63 ? ~0ull : ((2ull << i1) - 1ull));
    while (cand) {
      const int i = __builtin_ctzll(cand);
      const int wi = win0 + i;
      const unsigned lo32 = __builtin_amdgcn_readlane((unsigned)win, i);
      const unsigned hi32 = __builtin_amdgcn_readlane((unsigned)(win >> 32), i);
      unsigned long long v = ((unsigned long long)hi32 << 32) | lo32;
      if (wi == wa) v &= ~0ull << (a & 63);
      if (wi == wb && (end & 63)) v &= (1ull << (end & 63)) - 1ull;
      if (v) return (wi << 6) + __builtin_ctzll(v);
      cand &= cand - 1ull;
    }
    w = win0 + 64;                                // continue past this window
  }
  return end;
}

// The greedy cut is sequential, but walks from different starts merge once they reach a common cut.
// Walk: the token line (sequences back to back; a sequence's end is always a cut) is split into
// kWalkWaves segments, and each wave walks from its segment's first token as if a chunk started there,
// keeping its cuts in LDS up to the first one at or past the segment's end (a list that would exceed
// kWalkCap is dropped).  Stitch: wave 0 carries the true chain through the segments in order; where
// the chain's position is in a segment's list, the rest of that list is the chain and is copied out,
// otherwise it takes exact steps until it lands in the list or leaves the segment.  The result is the
// sequential walk's, whatever the lists hold.  Last, every sequence start is looked up in cu_chunks.
constexpr int kWalkWaves = 16;
constexpr int kWalkCap = 2040;                    // cuts kept per segment

__global__ __launch_bounds__(kWalkWaves * 64) void chunk_walk_kernel(
    const unsigned long long* __restrict__ cut_bits, const int32_t* __restrict__ cu_seqlens, int B, int ntok,
    int lo, int hi, int32_t* __restrict__ cu_chunks, int32_t* __restrict__ seq_chunk_start,
    int32_t* __restrict__ num_chunks) {
  __shared__ int32_t cuts[kWalkWaves][kWalkCap];
  __shared__ int32_t count[kWalkWaves];           // cuts kept, or -1 for a dropped list
  __shared__ int32_t total;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nwords = (ntok + 63) >> 6;
  // segments of S tokens, a whole number of bitmap words; kWalkWaves * S >= ntok
  const int S = max(64, ((ntok + kWalkWaves - 1) / kWalkWaves + 63) / 64 * 64);
  int win0 = -1;
  unsigned long long win = 0ull, nz = 0ull;

  // ---- walk (speculative), one segment per wave
  {
    const int s0 = wv * S, s1 = min(ntok, s0 + S);
    int n = 0;
    if (s0 < ntok) {
      int c = s0;
      int e = cu_seqlens[seq_of_token(cu_seqlens, B, c) + 1];
      if (lane == 0) cuts[wv][0] = c;
      n = 1;
      while (c < s1) {
        const int cut = walk_step(cut_bits, nwords, lane, c, e, lo, hi, win0, win, nz);
        if (n < kWalkCap && lane == 0) cuts[wv][n] = cut;
        ++n;
        c = cut;
        if (c == e && c < ntok) e = cu_seqlens[seq_of_token(cu_seqlens, B, c) + 1];
        if (n > kWalkCap) break;
      }
    }
    if (lane == 0) count[wv] = n > kWalkCap ? -1 : n;
  }
  __syncthreads();

  // ---- stitch, one wave
  if (wv == 0) {
    win0 = -1;
    if (lane == 0) cu_chunks[0] = 0;
    int c = 0, pos = 0;
    while (c < ntok) {
      const int k = c / S;
      const int n = count[k];
      int m = -1;
      if (n > 0) {                                // the list is strictly increasing: binary search for c
        int l = 0, r = n - 1;
        while (l < r) {
          const int mid = (l + r) >> 1;
          if (cuts[k][mid] < c) l = mid + 1; else r = mid;
        }
        if (cuts[k][l] == c) m = l;
      }
      if (m >= 0) {                               // the chain from c is this list's: copy the rest out
        const int cnt = n - 1 - m;
        for (int x = lane; x < cnt; x += 64) cu_chunks[pos + 1 + x] = cuts[k][m + 1 + x];
        pos += cnt;
        c = cuts[k][n - 1];                       // at or past the segment's end, or the last token
      } else {                                    // one exact step
        const int e = cu_seqlens[seq_of_token(cu_seqlens, B, c) + 1];
        const int cut = walk_step(cut_bits, nwords, lane, c, e, lo, hi, win0, win, nz);
        if (lane == 0) cu_chunks[pos + 1] = cut;
        ++pos;
        c = cut;
      }
    }
    if (lane == 0) { total = pos; *num_chunks = pos; }
  }
  __syncthreads();

  // ---- sequence starts: each is a cut (or 0), found in cu_chunks[0 .. total]
  const int nc = total;
  for (int b = tid; b <= B; b += kWalkWaves * 64) {
    const int v = cu_seqlens[b];
    int l = 0, r = nc;
    while (l < r) {
      const int mid = (l + r) >> 1;
      if (cu_chunks[mid] < v) l = mid + 1; else r = mid;
    }
    seq_chunk_start[b] = l;
  }
}

}  // namespace

hipError_t launch_adjacent_similarity(int B, int ntok, int W, int dtype, const int32_t* cu_seqlens, const void* k,
                                      float tau, float* sim, uint64_t* cut_bits, hipStream_t stream) {
  if (ntok == 0) return hipSuccess;
  const int parts = (ntok + 63) / 64 * (64 / kSimTok);   // every byte of every bitmap word
  const dim3 grid((parts + kSimWaves - 1) / kSimWaves);
  const int npieces = W / (dtype == 1 ? 8 : 4);
  const int nj = (npieces + 63) / 64;             // the host allows npieces <= kSimMaxPieces
#define DHSA_SIM_LAUNCH(TY, NJ, R)                                                                           \
  hipLaunchKernelGGL((adjacent_sim_kernel<TY, NJ, R>), grid, dim3(kSimWaves * 64), 0, stream, (const TY*)k, \
                     cu_seqlens, B, ntok, W, tau, sim, (uint8_t*)cut_bits)
  if (dtype == 1) {
    if (nj <= 1) DHSA_SIM_LAUNCH(uint16_t, 1, 8);
    else if (nj <= 2) DHSA_SIM_LAUNCH(uint16_t, 2, 8);
    else if (nj <= 4) DHSA_SIM_LAUNCH(uint16_t, 4, 4);
    else DHSA_SIM_LAUNCH(uint16_t, 8, 2);
  } else {
    if (nj <= 1) DHSA_SIM_LAUNCH(float, 1, 8);
    else if (nj <= 2) DHSA_SIM_LAUNCH(float, 2, 8);
    else if (nj <= 4) DHSA_SIM_LAUNCH(float, 4, 4);
    else DHSA_SIM_LAUNCH(float, 8, 2);
  }
#undef DHSA_SIM_LAUNCH
  return hipGetLastError();
}

hipError_t launch_chunk_walk(int B, int ntok, const int32_t* cu_seqlens, const uint64_t* cut_bits, int lo, int hi,
                             int32_t* cu_chunks, int32_t* seq_chunk_start, int32_t* num_chunks, hipStream_t stream) {
  hipLaunchKernelGGL(chunk_walk_kernel, dim3(1), dim3(kWalkWaves * 64), 0, stream, (const unsigned long long*)cut_bits,
                     cu_seqlens, B, ntok, lo, hi, cu_chunks, seq_chunk_start, num_chunks);
  return hipGetLastError();
}

}  // namespace dhsa
