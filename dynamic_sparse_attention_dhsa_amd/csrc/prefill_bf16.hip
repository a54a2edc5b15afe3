// Stage 3: block-sparse causal prefill, bf16 in, fp32 accumulate, on gfx950 MFMA.
//
// ICML 2026 spotlight page (Abstract): DHSA runs attention through a
// memory-efficient tiled backend over the interactions its router keeps;
// "... for On-Device LLMs" (Abstract): the kept token interactions follow from
// chunk scores upsampled to token level.  Query token t of chunk i, head h
// attends to every key u <= t inside a kept chunk of row (h, i):
//   out[t,h] = sum_u softmax_u(scale * q_t . k_u) v_u,   lse[h,t] = log sum_u exp(scale * q_t . k_u).
//
// Work decomposition.  A workgroup of NW waves owns one query chunk i, one KV
// head g and a tile of query rows.  Its waves are HP query heads of g times
// NW / HP blocks of 32 query rows, so one K/V tile staged in LDS feeds every q
// head of the group that keeps it.  The workgroup walks the union of its
// heads' kept chunks in ascending order (per-head bitmaps in LDS); a wave
// whose head does not keep a chunk skips the math but still stages tiles.
// Key tiles never cross a chunk boundary; a tile holds 64 keys, or 32 at a
// chunk's tail when no more are left, and keys past the chunk (or past the
// diagonal) are masked.
//
// Blocks are numbered so that all row tiles of one (KV head, query chunk)
// land on the same XCD (blocks are dealt to the 8 XCDs round robin), where
// they stream the same kept K/V through one L2; KV heads go one after
// another across the chip, heaviest chunks first.
//
// Per tile and wave (32 queries x 64 keys), with v_mfma_f32_32x32x16_bf16:
//   S^T = K Q^T      A = K rows from LDS, B = Q^T held in registers for the whole walk
//   online softmax   base 2, scale*log2(e) folded into one FMA; the running max
//                    is only moved (and O rescaled) when a tile exceeds it by 2^8
//   O^T += V^T P^T   A = V^T read with the LDS transpose load from V stored as
//                    is, B = P^T straight from the S^T accumulators (bf16)
// The QK^T of the next tile is interleaved with the softmax of the current
// one, and the PV of the current tile with staging the tile after next, so
// the matrix cores and the vector ALUs of a wave overlap.  K/V come in through
// buffer loads whose range ends at the last token, so nothing past the
// tensors is read, and go through a three-stage LDS ring with one barrier per
// tile.
#include <type_traits>

#include "dhsa_internal.hpp"

namespace dhsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef s16x4 __attribute__((address_space(3))) lds_s16x4;

#ifndef DHSA_VPAD
#define DHSA_VPAD 32
#endif

constexpr int kMaxWords = DHSA_MAX_WORDS;      // bitmap words per head (32 chunks each)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleLog2 = 8.0f;           // move the running max only past 2^8
constexpr int kBufWord3 = 0x00020000;          // gfx9 buffer resource: raw 32-bit data

// scheduling-group masks for __builtin_amdgcn_sched_group_barrier
constexpr int kSgVALU = 0x002, kSgMFMA = 0x008, kSgVMEM = 0x020, kSgDSR = 0x100, kSgDSW = 0x200;

template <int D>
struct Geo {
  static constexpr int NW = 4;                           // waves per workgroup (two workgroups per CU)
  static constexpr int NT = NW * 64;
  static constexpr int BK = 64;                          // keys per tile (two 32-key blocks)
  static constexpr int GR = D / 8;                       // 16-byte granules per row
  static constexpr int KS = D + 8;                       // K row stride in LDS (bf16)
  static constexpr int VS = D + DHSA_VPAD;               // V row stride in LDS (bf16)
  static constexpr int KTILE = BK * KS;
  static constexpr int VTILE = BK * VS;
  static constexpr int LOADS = BK * GR / NT;             // granules per thread per tensor per tile
  static constexpr int DSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
  static constexpr int MINW = (D >= 256) ? 1 : 2;        // waves per SIMD
  static_assert(BK * GR % NT == 0, "tile must split evenly over the workgroup");
};

__device__ inline uint32_t union_word(const uint32_t (*bm)[kMaxWords], int hp, int w) {
  uint32_t u = 0;
  for (int x = 0; x < hp; ++x) u |= bm[x][w];
  return u;
}

// Lowest kept local chunk index >= x in the union of the heads' bitmaps, or -1.
__device__ inline int next_union(const uint32_t (*bm)[kMaxWords], int hp, int x, int nbits) {
  if (x >= nbits) return -1;
  int w = x >> 5;
  uint32_t u = union_word(bm, hp, w) & (0xFFFFFFFFu << (x & 31));
  const int nw = (nbits + 31) >> 5;
  while (true) {
    if (u) return (w << 5) + __builtin_ctz(u);
    if (++w >= nw) return -1;
    u = union_word(bm, hp, w);
  }
}

// Reductions over lanes l and l ^ 32 through the VALU lane swap (no LDS round trip): after the swap
// of x with itself, one result holds the lane's own value and the other its partner's.
__device__ inline float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline uint32_t pack_bf16(float a, float b) {
  f32x2 x = {a, b};
  bf16x2 r = __builtin_convertvector(x, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

template <int N> using ic = std::integral_constant<int, N>;

template <int D, bool WITH_LSE>
__global__ __launch_bounds__(Geo<D>::NT, Geo<D>::MINW) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ block_idx,
    const int32_t* __restrict__ cu_chunks, const int32_t* __restrict__ seq_chunk_start,
    uint16_t* __restrict__ out, float* __restrict__ lse, int B, int C, int T, int Hq, int Hkv,
    long long nnz, float scale, int hp, int head_slots, int row_tiles) {
  using GE = Geo<D>;
  constexpr int NW = GE::NW, NT = GE::NT, BK = GE::BK;
  // two-stage rings: K of the tile after next and V of the next tile are written while the
  // current tile is computed, so one barrier per tile suffices
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2 * GE::KTILE];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2 * GE::VTILE];
  __shared__ uint32_t bm[GE::NW][kMaxWords];

  // ---- block -> (KV head, chunk, head slot, row tile); one XCD per (KV head, chunk)
  const int G = Hq / Hkv;
  const int rb_count = NW / hp;
  const int per_group = head_slots * row_tiles;
  const int xcd = blockIdx.x & 7;
  const int kth = blockIdx.x >> 3;
  const int gid = (kth / per_group) * 8 + xcd;
  if (gid >= Hkv * C) return;                              // block-uniform
  const int sub = kth % per_group;
  const int rt = sub % row_tiles;
  const int hs = sub / row_tiles;
  const int gk = gid / C;
  const int i = C - 1 - (gid % C);                         // heaviest (latest) chunks first
  const int s_i = cu_chunks[i], e_i = cu_chunks[i + 1];
  const int q0 = s_i + rt * rb_count * 32;
  if (q0 >= e_i) return;                                   // block-uniform

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hw = wave % hp;
  const int h = gk * G + hs * hp + hw;
  const int qr0 = q0 + (wave / hp) * 32;
  const bool wave_rows = qr0 < e_i;
  const int wave_last = min(qr0 + 32, e_i) - 1;
  const int first = seq_chunk_start[seq_of_chunk(seq_chunk_start, B, i)];
  const int nbits = i - first + 1;
  const int rp0 = row_ptr[i], rlen = row_ptr[i + 1] - rp0;
  const int diag_end = min(e_i, q0 + rb_count * 32);

  // ---- kept-chunk bitmaps of the workgroup's heads
  const int nwords = (nbits + 31) >> 5;
  for (int x = tid; x < hp * nwords; x += NT) bm[x / nwords][x % nwords] = 0u;
  __syncthreads();
  for (int x = tid; x < hp * rlen; x += NT) {
    const int hh = x / rlen, e = x - hh * rlen;
    const int j = block_idx[(size_t)(gk * G + hs * hp + hh) * nnz + rp0 + e];
    const int loc = j - first;
    if (loc >= 0 && loc < nbits) atomicOr(&bm[hh][loc >> 5], 1u << (loc & 31));
  }
  __syncthreads();

  // ---- Q^T fragments (B operand), whole walk
  const int col = lane & 31, half = lane >> 5;
  const int tq = qr0 + col;
  bf16x8 qf[GE::DSTEPS];
  {
    const bool ok = tq < e_i;
    const uint16_t* qp = q + ((size_t)tq * Hq + h) * D + half * 8;
#pragma unroll
    for (int s = 0; s < GE::DSTEPS; ++s) {
      uint4 raw = ok ? *reinterpret_cast<const uint4*>(qp + s * 16) : make_uint4(0, 0, 0, 0);
      qf[s] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // ---- tile walk, kept in scalar registers (identical in every thread)
  struct TileRef {
    int jl, kt, kend;      // local chunk index (-1: walk over), key range [kt, kend) of the chunk part
  };
  auto chunk_span = [&](TileRef& t) {
    const int j = first + t.jl;
    t.kt = cu_chunks[j];
    t.kend = (j == i) ? diag_end : cu_chunks[j + 1];
  };
  auto next_tile = [&](TileRef t) {
    if (t.jl < 0) return t;
    t.kt += BK;
    if (t.kt >= t.kend) {
      t.jl = __builtin_amdgcn_readfirstlane(next_union(bm, hp, t.jl + 1, nbits));
      if (t.jl >= 0) chunk_span(t);
    }
    return t;
  };
  // a wave computes every tile of the walk when it has rows; tiles of chunks its head does not keep,
  // keys past the chunk end and keys past the diagonal are masked to -inf
  auto keeps = [&](const TileRef& t) { return ((bm[hw][t.jl >> 5] >> (t.jl & 31)) & 1u) != 0; };

  // ---- staging: buffer loads -> registers -> LDS (K and V both stored as rows, padded)
  auto voff = [&](int m) { const int idx = tid + m * NT; return ((idx / GE::GR) * Hkv * D + (idx % GE::GR) * 8) * 2; };
  auto lds_k = [&](int m) { const int idx = tid + m * NT; return (idx / GE::GR) * GE::KS + (idx % GE::GR) * 8; };
  auto lds_v = [&](int m) { const int idx = tid + m * NT; return (idx / GE::GR) * GE::VS + (idx % GE::GR) * 8; };
  // buffer range: this KV head's rows from the tile start to the last token (nothing past T is read)
  auto tile_rsrc = [&](const uint16_t* base_ptr, const TileRef& t) {
    const long long rows_left = (long long)(T - t.kt) * Hkv - gk;
    const long long cap = (long long)BK * Hkv * D * 2;
    const int nbytes = (int)min(rows_left * D * 2, cap);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base_ptr + ((size_t)t.kt * Hkv + gk) * D), (short)0, nbytes,
                                             kBufWord3);
  };
  uint4 kreg[GE::LOADS], vreg[GE::LOADS];
  auto load_k = [&](const TileRef& t) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(k, t);
#pragma unroll
    for (int m = 0; m < GE::LOADS; ++m)
      kreg[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff(m), 0, 0));
  };
  auto load_v = [&](const TileRef& t) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(v, t);
#pragma unroll
    for (int m = 0; m < GE::LOADS; ++m)
      vreg[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff(m), 0, 0));
  };
  auto store_k = [&](int stage) {
#pragma unroll
    for (int m = 0; m < GE::LOADS; ++m) *reinterpret_cast<uint4*>(k_lds + stage * GE::KTILE + lds_k(m)) = kreg[m];
  };
  auto store_v = [&](int stage) {
#pragma unroll
    for (int m = 0; m < GE::LOADS; ++m) *reinterpret_cast<uint4*>(v_lds + stage * GE::VTILE + lds_v(m)) = vreg[m];
  };

  // ---- per-lane LDS read bases
  const int k_lane = col * GE::KS + half * 8;               // K row 32b + col, dims 16s + 8*half
  const int grp = (lane >> 4) & 3, ii = lane & 15;          // transpose load: 4-key x 16-dim block per 16 lanes
  const int v_lane = (4 * (grp >> 1) + (ii >> 2)) * GE::VS + 16 * (grp & 1) + 4 * (ii & 3);

  f32x16 o[GE::DBLK];
#pragma unroll
  for (int db = 0; db < GE::DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  // lb_run: sum of the bf16 weights actually multiplied into V, which normalises O (a dominant
  // weight cancels exactly); l_run: sum of the fp32 weights, kept only when the LSE is wanted
  float m_ref = -INFINITY, l_run = 0.f, lb_run = 0.f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const float c2 = scale * kLog2e;
  const float grow_raw = kRescaleLog2 / c2;
  const f32x16 zero16 = {};

  // S^T[b][r] holds tile key 32b + 8(r/4) + 4*half + r%4 of query `col`
  auto needs_mask = [&](const TileRef& t) { return t.kend - t.kt < BK || first + t.jl == i || !keeps(t); };
  auto apply_mask = [&](f32x16 (&s)[2], const TileRef& t) {
    int lim = t.kend - t.kt - 1;
    if (first + t.jl == i) lim = min(lim, tq - t.kt);
    if (!keeps(t)) lim = -1;
    lim -= 4 * half;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * b + 8 * (r >> 2) + (r & 3) > lim) s[b][r] = -INFINITY;
  };

  // QK^T of the next tile (QN blocks) interleaved with the softmax of the current tile (CB blocks).
  // Leaves P^T of the current tile packed in pw and the running max / sum updated; returns alpha.
  uint32_t pw[16];
  auto region_a = [&](auto qn_c, auto cb_c, int stage_n, f32x16 (&sn)[2], f32x16 (&sc)[2], float& alpha) {
    constexpr int QN = decltype(qn_c)::value, CB = decltype(cb_c)::value;
    const uint16_t* kb0 = k_lds + stage_n * GE::KTILE + k_lane;
#pragma unroll
    for (int st = 0; st < GE::DSTEPS; ++st) {
      if constexpr (QN >= 1) {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(kb0 + st * 16);
        sn[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[st], st == 0 ? zero16 : sn[0], 0, 0, 0);
      }
      if constexpr (QN >= 2) {
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(kb0 + 32 * GE::KS + st * 16);
        sn[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[st], st == 0 ? zero16 : sn[1], 0, 0, 0);
      }
    }
    if constexpr (CB >= 1) {
      // reductions as shallow trees (four independent partial results) to keep dependency chains short
      float m4[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) m4[x] = fmaxf(fmaxf(sc[0][x], sc[0][x + 4]), fmaxf(sc[0][x + 8], sc[0][x + 12]));
#pragma unroll
      for (int b = 1; b < CB; ++b)
#pragma unroll
        for (int x = 0; x < 4; ++x)
          m4[x] = fmaxf(fmaxf(m4[x], sc[b][x]), fmaxf(fmaxf(sc[b][x + 4], sc[b][x + 8]), sc[b][x + 12]));
      const float mx = max_halves(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
      const bool grow = mx > m_ref + grow_raw;
      const float m_new = grow ? mx : m_ref;
      alpha = grow ? __builtin_amdgcn_exp2f((m_ref - m_new) * c2) : 1.f;   // 0 at the first tile
      const float mb = (m_new == -INFINITY ? 0.f : m_new) * c2;
      m_ref = m_new;
#pragma unroll
      for (int b = 0; b < CB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[b][r] = __builtin_amdgcn_exp2f(fmaf(sc[b][r], c2, -mb));
      float lb4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < CB; ++b)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          pw[b * 8 + r / 2] = pack_bf16(sc[b][r], sc[b][r + 1]);
          lb4[(r / 2) & 3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[b * 8 + r / 2]), ones,
                                                             lb4[(r / 2) & 3], false);
        }
      lb_run = lb_run * alpha + sum_halves((lb4[0] + lb4[1]) + (lb4[2] + lb4[3]));
      if constexpr (WITH_LSE) {
        float ls4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < CB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) ls4[r & 3] += sc[b][r];
        l_run = l_run * alpha + sum_halves((ls4[0] + ls4[1]) + (ls4[2] + ls4[3]));
      }
    }
    // interleave: each QK MFMA followed by its next K read and a slice of the softmax
    if constexpr (QN > 0 && CB > 0) {
      __builtin_amdgcn_sched_group_barrier(kSgDSR, 4, 0);
#pragma unroll
      for (int x = 0; x < GE::DSTEPS * QN; ++x) {
        __builtin_amdgcn_sched_group_barrier(kSgMFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDSR, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgVALU, (CB * 60) / (GE::DSTEPS * QN) + 1, 0);
      }
    }
  };

  // O^T += V^T P^T for the current tile (CB blocks), interleaved with staging the tile after next.
  auto region_b = [&](auto cb_c, int stage_c) {
    constexpr int CB = decltype(cb_c)::value;
    if constexpr (CB > 0) {
      const uint16_t* vb = v_lds + stage_c * GE::VTILE + v_lane;
#pragma unroll
      for (int ks = 0; ks < 2 * CB; ++ks) {
        const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(pw[ks * 4], pw[ks * 4 + 1], pw[ks * 4 + 2],
                                                                pw[ks * 4 + 3]));
#pragma unroll
        for (int db = 0; db < GE::DBLK; ++db) {
          const uint16_t* p0 = vb + (ks * 16) * GE::VS + db * 32;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 8 * GE::VS));
          const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
          const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(l2.x, l2.y, h2.x, h2.y));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf, o[db], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_group_barrier(kSgDSR, 6, 0);
#pragma unroll
      for (int x = 0; x < 2 * CB * GE::DBLK; ++x) {
        __builtin_amdgcn_sched_group_barrier(kSgMFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDSR, 2, 0);
      }
    }
  };

  auto run_a = [&](int qn, int cb, int stage_n, f32x16 (&sn)[2], f32x16 (&sc)[2], float& alpha) {
    if (qn && cb) region_a(ic<2>{}, ic<2>{}, stage_n, sn, sc, alpha);
    else if (qn) region_a(ic<2>{}, ic<0>{}, stage_n, sn, sc, alpha);
    else if (cb) region_a(ic<0>{}, ic<2>{}, stage_n, sn, sc, alpha);
  };
  auto run_b = [&](int cb, int stage_c) {
    if (cb) region_b(ic<2>{}, stage_c);
  };

  // ---- prologue: K ring holds tiles 0 and 1, V ring tile 0; registers hold K of tile 2 and V of tile 1
  TileRef t0;
  t0.jl = __builtin_amdgcn_readfirstlane(next_union(bm, hp, 0, nbits));
  t0.kt = 0; t0.kend = 0;
  if (t0.jl >= 0) chunk_span(t0);
  TileRef t1 = next_tile(t0);
  TileRef t2 = next_tile(t1);
  if (t0.jl >= 0) { load_k(t0); load_v(t0); store_k(0); store_v(0); }
  if (t1.jl >= 0) { load_k(t1); store_k(1); load_v(t1); }
  if (t2.jl >= 0) load_k(t2);
  __syncthreads();

  f32x16 sA[2], sB[2];
  const int busy = wave_rows ? 2 : 0;          // waves without rows only stage tiles
  int cb_cur = (t0.jl >= 0) ? busy : 0;
  {
    float dummy;
    run_a(cb_cur, 0, 0, sA, sB, dummy);        // S^T of tile 0
  }
  __syncthreads();                             // K stage 0 is rewritten by the first iteration
  int stage = 0;
  // one iteration: softmax + PV of t0 (S^T in sc), QK^T of t1 (into sn)
  auto step = [&](f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    const int st1 = stage ^ 1;
    // K(t2) -> K stage of t0 (read in the previous iteration), V(t1) -> V stage st1 (free since then)
    const TileRef t3 = next_tile(t2);
    if (t2.jl >= 0) store_k(stage);
    if (t1.jl >= 0) store_v(st1);
    if (t3.jl >= 0) load_k(t3);
    if (t2.jl >= 0) load_v(t2);
    const int cb_nxt = (t1.jl >= 0) ? busy : 0;
    if (cb_cur > 0 && needs_mask(t0)) apply_mask(sc, t0);
    float alpha = 1.f;
    run_a(cb_nxt, cb_cur, st1, sn, sc, alpha);
    if (cb_cur > 0 && __builtin_amdgcn_ballot_w64(alpha != 1.f)) {   // a running max moved
#pragma unroll
      for (int db = 0; db < GE::DBLK; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    run_b(cb_cur, stage);
    __syncthreads();
    t0 = t1; t1 = t2; t2 = t3;
    cb_cur = cb_nxt;
    stage = st1;
  };
  while (t0.jl >= 0) {
    step(sA, sB);
    if (t0.jl < 0) break;
    step(sB, sA);
  }

  // ---- epilogue
  if (!wave_rows || tq >= e_i) return;
  const float inv_l = 1.0f / lb_run;
  uint16_t* op = out + ((size_t)tq * Hq + h) * D;
#pragma unroll
  for (int db = 0; db < GE::DBLK; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      uint2 w;
      w.x = pack_bf16(o[db][g4 * 4 + 0] * inv_l, o[db][g4 * 4 + 1] * inv_l);
      w.y = pack_bf16(o[db][g4 * 4 + 2] * inv_l, o[db][g4 * 4 + 3] * inv_l);
      *reinterpret_cast<uint2*>(op + db * 32 + 8 * g4 + 4 * half) = w;
    }
  }
  if constexpr (WITH_LSE) {
    if (half == 0) lse[(size_t)h * T + tq] = m_ref * scale + logf(l_run);
  }
}

template <int D>
hipError_t launch_d(const Plan& p, const void* q, const void* k, const void* v, const int32_t* row_ptr,
                    int64_t nnz, const int32_t* block_idx, float scale, void* out, float* lse,
                    hipStream_t stream) {
  using GE = Geo<D>;
  const int G = p.Hq / p.Hkv;
  int hp = 1;
  while (hp < GE::NW && G % (hp * 2) == 0) hp *= 2;
  const int rows_per_block = (GE::NW / hp) * 32;
  const int row_tiles = (p.max_chunk_len + rows_per_block - 1) / rows_per_block;
  const int head_slots = G / hp;
  const long long groups = (long long)p.Hkv * p.C;
  const long long blocks = (groups + 7) / 8 * 8 * head_slots * row_tiles;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  auto kern = lse != nullptr ? prefill_bf16_kernel<D, true> : prefill_bf16_kernel<D, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(GE::NT), 0, stream, (const uint16_t*)q, (const uint16_t*)k,
                     (const uint16_t*)v, row_ptr, block_idx, p.cu_chunks, p.seq_chunk_start, (uint16_t*)out, lse,
                     p.B, p.C, p.T, p.Hq, p.Hkv, (long long)nnz, scale, hp, head_slots, row_tiles);
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
