// Stage 3: block-sparse causal prefill, bf16 in, fp32 accumulate, on gfx950 MFMA.
//
// ICML 2026 spotlight page (Abstract): DHSA runs attention through a
// memory-efficient tiled backend over the interactions its router keeps;
// "... for On-Device LLMs" (Abstract): the kept token interactions follow from
// chunk scores upsampled to token level.  Query token t of chunk i, head h
// attends to every key u <= t inside a kept chunk of row (h, i):
//   out[t,h] = sum_u softmax_u(scale * q_t . k_u) v_u,   lse[h,t] = log sum_u exp(scale * q_t . k_u).
//
// Work decomposition.  A workgroup (4 waves) owns one query chunk i, one KV
// head g and a tile of query rows.  Its waves are HP query heads of g (HP =
// gcd(G, 4)) times RB = 4 / HP blocks of 32 query rows, so one K/V tile staged
// in LDS feeds every q head of the group that keeps it.  The workgroup walks
// the union of its heads' kept chunks in ascending order (a per-head bitmap in
// LDS); a wave whose head does not keep a chunk skips its MFMAs but still
// helps stage the tiles.  Keys go in tiles of 64 that never cross a chunk
// boundary; a tile's tail beyond its chunk is zero-filled and masked, and the
// diagonal chunk is masked causally.
//
// Per tile and wave (32 queries x 64 keys) with v_mfma_f32_32x32x16_bf16:
//   S^T = K Q^T     A = K rows from LDS, B = Q^T held in registers for the whole walk
//   online softmax  base-2 exponent with scale*log2(e) folded in one FMA
//   O^T += V^T P^T  A = V^T from LDS (stored transposed), B = P^T straight from
//                   the S^T accumulators after rounding to bf16
// The transposed products keep every softmax quantity of a query in one lane
// pair (lanes l and l^32), and P never leaves registers.  The next tile's
// global loads are issued before the current tile is computed.
#include "dhsa_internal.hpp"

namespace dhsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBK = 64;          // keys per tile
constexpr int kQW = 32;          // query rows per wave
constexpr int kMaxWords = DHSA_MAX_WORDS;  // bitmap words per head (32 chunks each)
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Tile {
  static constexpr int KSTR = D + 8;        // K row stride in LDS (bf16), breaks bank aliasing
  static constexpr int VSTR = kBK + 4;      // V^T row stride in LDS (bf16)
  static constexpr int GR = D / 8;          // 16-byte granules per row
  static constexpr int KLOADS = kBK * GR / kThreads;        // K granules per thread
  static constexpr int VUNITS = (kBK / 4) * GR;             // (4 keys x 8 dims) units per tile
  static constexpr int VLOADS = (VUNITS + kThreads - 1) / kThreads;
  static constexpr int DSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
};

__device__ inline uint32_t lds_union_word(const uint32_t (*bm)[kMaxWords], int hp, int w) {
  uint32_t u = 0;
  for (int x = 0; x < hp; ++x) u |= bm[x][w];
  return u;
}

// Lowest kept local chunk index >= x in the union of the heads' bitmaps, or -1.
__device__ inline int next_union(const uint32_t (*bm)[kMaxWords], int hp, int x, int nbits) {
  if (x >= nbits) return -1;
  int w = x >> 5;
  uint32_t u = lds_union_word(bm, hp, w) & (0xFFFFFFFFu << (x & 31));
  const int nw = (nbits + 31) >> 5;
  while (true) {
    if (u) return (w << 5) + __builtin_ctz(u);
    if (++w >= nw) return -1;
    u = lds_union_word(bm, hp, w);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, (D >= 256 ? 1 : 2)) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ block_idx,
    const int32_t* __restrict__ cu_chunks, const int32_t* __restrict__ seq_chunk_start,
    uint16_t* __restrict__ out, float* __restrict__ lse, int B, int C, int T, int Hq, int Hkv,
    long long nnz, float scale, int hp, int head_slots, int row_tiles) {
  using TL = Tile<D>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBK * TL::KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * TL::VSTR];
  __shared__ uint32_t bm[kWaves][kMaxWords];

  const int G = Hq / Hkv;
  const int rb_count = kWaves / hp;
  // block -> (kv head, head slot, chunk (heaviest first), row tile)
  int bid = blockIdx.x;
  const int rt = bid % row_tiles;  bid /= row_tiles;
  const int ci = bid % C;          bid /= C;
  const int hs = bid % head_slots; bid /= head_slots;
  const int gk = bid;
  const int i = C - 1 - ci;
  const int s_i = cu_chunks[i], e_i = cu_chunks[i + 1];
  const int q0 = s_i + rt * rb_count * kQW;
  if (q0 >= e_i) return;                                  // block-uniform

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hw = wave % hp;                               // head within the workgroup
  const int h = gk * G + hs * hp + hw;
  const int qr0 = q0 + (wave / hp) * kQW;                 // this wave's first query row
  const bool wave_rows = qr0 < e_i;
  const int wave_last = min(qr0 + kQW, e_i) - 1;
  const int first = seq_chunk_start[seq_of_chunk(seq_chunk_start, B, i)];
  const int nbits = i - first + 1;
  const int rp0 = row_ptr[i], rlen = row_ptr[i + 1] - rp0;
  const int diag_end = min(e_i, q0 + rb_count * kQW);

  // ---- kept-chunk bitmaps of the workgroup's heads
  for (int x = tid; x < kWaves * kMaxWords; x += kThreads) bm[x / kMaxWords][x % kMaxWords] = 0u;
  __syncthreads();
  for (int x = tid; x < hp * rlen; x += kThreads) {
    const int hh = x / rlen, e = x - hh * rlen;
    const int j = block_idx[(size_t)(gk * G + hs * hp + hh) * nnz + rp0 + e];
    const int loc = j - first;
    if (loc >= 0 && loc < nbits) atomicOr(&bm[hh][loc >> 5], 1u << (loc & 31));
  }
  __syncthreads();

  // ---- Q^T fragments (B operand) for the whole walk
  const int col = lane & 31, half = lane >> 5;
  const int tq = qr0 + col;
  bf16x8 qf[TL::DSTEPS];
  {
    const bool ok = tq < e_i;
    const uint16_t* qp = q + ((size_t)tq * Hq + h) * D + half * 8;
#pragma unroll
    for (int s = 0; s < TL::DSTEPS; ++s) {
      uint4 raw = ok ? *reinterpret_cast<const uint4*>(qp + s * 16) : make_uint4(0, 0, 0, 0);
      qf[s] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  f32x16 o[TL::DBLK];
#pragma unroll
  for (int db = 0; db < TL::DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = scale * kLog2e;

  // ---- tile walk state (identical in every thread)
  int jl = next_union(bm, hp, 0, nbits);                  // local chunk index
  int kt = 0, kend = 0;
  auto span = [&](int loc, int& a, int& b) {
    const int j = first + loc;
    a = cu_chunks[j];
    b = (j == i) ? diag_end : cu_chunks[j + 1];
  };
  if (jl >= 0) span(jl, kt, kend);

  uint4 kreg[TL::KLOADS];
  uint4 vreg[TL::VLOADS][4];
  auto load_tile = [&](int kt_, int kend_) {
#pragma unroll
    for (int m = 0; m < TL::KLOADS; ++m) {
      const int idx = tid + m * kThreads;
      const int key = idx / TL::GR, gg = idx % TL::GR;
      const int u = kt_ + key;
      kreg[m] = (u < kend_) ? *reinterpret_cast<const uint4*>(k + ((size_t)u * Hkv + gk) * D + gg * 8)
                            : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < TL::VLOADS; ++m) {
      const int idx = tid + m * kThreads;
      const int gg = idx % TL::GR, kq = idx / TL::GR;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int u = kt_ + kq * 4 + x;
        vreg[m][x] = (idx < TL::VUNITS && u < kend_)
                         ? *reinterpret_cast<const uint4*>(v + ((size_t)u * Hkv + gk) * D + gg * 8)
                         : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int m = 0; m < TL::KLOADS; ++m) {
      const int idx = tid + m * kThreads;
      const int key = idx / TL::GR, gg = idx % TL::GR;
      *reinterpret_cast<uint4*>(&Ks[key * TL::KSTR + gg * 8]) = kreg[m];
    }
#pragma unroll
    for (int m = 0; m < TL::VLOADS; ++m) {
      const int idx = tid + m * kThreads;
      if (idx >= TL::VUNITS) continue;
      const int gg = idx % TL::GR, kq = idx / TL::GR;
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vreg[m][0]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vreg[m][1]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vreg[m][2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vreg[m][3]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // dimension gg*8+e of keys 4kq..4kq+3 -> one 8-byte row segment of V^T
        const int sh = (e & 1) * 16;
        const uint32_t a0 = (w0[e >> 1] >> sh) & 0xFFFFu, a1 = (w1[e >> 1] >> sh) & 0xFFFFu;
        const uint32_t a2 = (w2[e >> 1] >> sh) & 0xFFFFu, a3 = (w3[e >> 1] >> sh) & 0xFFFFu;
        uint2 pk = make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
        *reinterpret_cast<uint2*>(&Vt[(gg * 8 + e) * TL::VSTR + kq * 4]) = pk;
      }
    }
  };

  if (jl >= 0) load_tile(kt, kend);
  while (jl >= 0) {
    __syncthreads();                 // previous tile fully consumed
    store_tile();
    __syncthreads();                 // tile visible
    // advance the walk and prefetch the next tile
    const int cur_jl = jl, cur_kt = kt, cur_kend = kend;
    kt += kBK;
    if (kt >= kend) {
      jl = next_union(bm, hp, jl + 1, nbits);
      if (jl >= 0) span(jl, kt, kend);
    }
    if (jl >= 0) load_tile(kt, kend);

    // ---- compute on the staged tile
    const bool keeps = (bm[hw][cur_jl >> 5] >> (cur_jl & 31)) & 1u;
    const bool diag = (first + cur_jl) == i;
    if (!wave_rows || !keeps || (diag && cur_kt > wave_last)) continue;   // wave-uniform
    const int nvalid = cur_kend - cur_kt;                 // 1..64
    const bool two = nvalid > 32;

    f32x16 s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
#pragma unroll
    for (int s = 0; s < TL::DSTEPS; ++s) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&Ks[col * TL::KSTR + s * 16 + half * 8]);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[s], s0, 0, 0, 0);
    }
    if (two) {
#pragma unroll
      for (int s = 0; s < TL::DSTEPS; ++s) {
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&Ks[(32 + col) * TL::KSTR + s * 16 + half * 8]);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[s], s1, 0, 0, 0);
      }
    }

    // S^T[r] holds key (8*(r/4) + 4*half + r%4) of its 32-key block for query `col`.
    if (!two) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s1[r] = -INFINITY;
    }
    if (nvalid < kBK || diag) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * half + (r & 3);
        if (key >= nvalid || (diag && cur_kt + key > tq)) s0[r] = -INFINITY;
        if (32 + key >= nvalid || (diag && cur_kt + 32 + key > tq)) s1[r] = -INFINITY;
      }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
    const float mb = m_use * c2;
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = __builtin_amdgcn_exp2f(fmaf(s0[r], c2, -mb));
      s1[r] = __builtin_amdgcn_exp2f(fmaf(s1[r], c2, -mb));
      ls += s0[r] + s1[r];
    }
    ls += __shfl_xor(ls, 32);
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < TL::DBLK; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;

    // P^T fragments: k-step ks covers keys 16ks..16ks+15 of the tile = S^T block ks/2, regs (ks%2)*8..+7
    bf16x8 pf[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pf[0][e] = (__bf16)s0[e];
      pf[1][e] = (__bf16)s0[8 + e];
      pf[2][e] = (__bf16)s1[e];
      pf[3][e] = (__bf16)s1[8 + e];
    }
    const int nks = two ? 4 : 2;
#pragma unroll
    for (int db = 0; db < TL::DBLK; ++db) {
      const uint16_t* vrow = &Vt[(db * 32 + col) * TL::VSTR + 4 * half];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (ks >= nks) break;
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow + ks * 16);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + ks * 16 + 8);
        bf16x8 a;
        a[0] = lo[0]; a[1] = lo[1]; a[2] = lo[2]; a[3] = lo[3];
        a[4] = hi[0]; a[5] = hi[1]; a[6] = hi[2]; a[7] = hi[3];
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], o[db], 0, 0, 0);
      }
    }
  }

  // ---- epilogue
  if (!wave_rows || tq >= e_i) return;
  const float inv_l = 1.0f / l_run;
  uint16_t* op = out + ((size_t)tq * Hq + h) * D;
#pragma unroll
  for (int db = 0; db < TL::DBLK; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x4 w;
#pragma unroll
      for (int x = 0; x < 4; ++x) w[x] = (__bf16)(o[db][g4 * 4 + x] * inv_l);
      *reinterpret_cast<bf16x4*>(op + db * 32 + 8 * g4 + 4 * half) = w;
    }
  }
  if (lse != nullptr && half == 0) lse[(size_t)h * T + tq] = m_run * scale + logf(l_run);
}

template <int D>
hipError_t launch_d(const Plan& p, const void* q, const void* k, const void* v, const int32_t* row_ptr,
                    int64_t nnz, const int32_t* block_idx, float scale, void* out, float* lse,
                    hipStream_t stream) {
  const int G = p.Hq / p.Hkv;
  int hp = 1;
  while (hp < kWaves && G % (hp * 2) == 0) hp *= 2;       // gcd(G, 4) for the supported group sizes
  if (G % hp) hp = 1;
  const int rows_per_block = (kWaves / hp) * kQW;
  const int row_tiles = (p.max_chunk_len + rows_per_block - 1) / rows_per_block;
  const int head_slots = G / hp;
  const long long blocks = (long long)p.Hkv * head_slots * p.C * row_tiles;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(prefill_bf16_kernel<D>, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, row_ptr, block_idx,
                     p.cu_chunks, p.seq_chunk_start, (uint16_t*)out, lse, p.B, p.C, p.T, p.Hq, p.Hkv,
                     (long long)nnz, scale, hp, head_slots, row_tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const Plan& p, const void* q, const void* k, const void* v,
                               const int32_t* row_ptr, int64_t nnz, const int32_t* block_idx,
                               float softmax_scale, void* out, float* lse, hipStream_t stream) {
  if (p.C == 0) return hipSuccess;
  switch (p.d) {
    case 64: return launch_d<64>(p, q, k, v, row_ptr, nnz, block_idx, softmax_scale, out, lse, stream);
    case 128: return launch_d<128>(p, q, k, v, row_ptr, nnz, block_idx, softmax_scale, out, lse, stream);
    case 256: return launch_d<256>(p, q, k, v, row_ptr, nnz, block_idx, softmax_scale, out, lse, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dhsa
