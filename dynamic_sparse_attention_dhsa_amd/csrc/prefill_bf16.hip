// Stage 3: block-sparse causal prefill, bf16 in, fp32 accumulate, on gfx950 MFMA.
//
// ICML 2026 spotlight page (Abstract): DHSA runs attention through a
// memory-efficient tiled backend over the interactions its router keeps;
// "... for On-Device LLMs" (Abstract): the kept token interactions follow from
// chunk scores upsampled to token level.  Query token t of chunk i, head h
// attends to every key u <= t inside a kept chunk of row (h, i):
//   out[t,h] = sum_u softmax_u(scale * q_t . k_u) v_u,   lse[h,t] = log sum_u exp(scale * q_t . k_u).
//
// Work decomposition.  A workgroup of four waves owns one query chunk i, one
// KV head g and a tile of query rows; two workgroups share a CU.  Its waves
// are HP query heads of g (HP = the largest power of two dividing G, at most
// 4) times 4 / HP blocks of 32 query rows, so one K/V tile staged in LDS feeds
// every q head of the group that keeps it.  The workgroup walks the union of
// its heads' kept chunks in ascending order (per-head bitmaps in LDS); a
// head's scores on a chunk it does not keep are masked.  Key tiles hold 64
// keys and never cross a chunk boundary; keys past the chunk end or past the
// diagonal are masked.
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
// one, so the matrix cores and the vector ALUs of a wave overlap.  K and V
// reach LDS through buffer loads that write LDS directly (no registers),
// ranged so that nothing past the last token is read, into two-stage rings
// kept in separate LDS arrays.  Rows are unpadded; their 16-byte granules are
// XOR-swizzled by row so that the fragment reads hit 64 distinct banks.  An
// iteration issues the loads of the next V and of the K after next, computes,
// waits for its own loads and ends with one barrier.
#include <type_traits>

#include "dhsa_internal.hpp"

namespace dhsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef s16x4 __attribute__((address_space(3))) lds_s16x4;
typedef void __attribute__((address_space(3))) lds_void;

constexpr int kMaxWords = DHSA_MAX_WORDS;      // bitmap words per head (32 chunks each)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleLog2 = 8.0f;           // move the running max only past 2^8
constexpr int kBufWord3 = 0x00020000;          // gfx9 buffer resource: raw 32-bit data
constexpr int kWaitVmcnt0 = 0x0F70;            // s_waitcnt vmcnt(0), other counters unconstrained

// scheduling-group masks for __builtin_amdgcn_sched_group_barrier
constexpr int kSgVALU = 0x002, kSgMFMA = 0x008, kSgDSR = 0x100;

template <int D>
struct Geo {
  static constexpr int NW = 4;                           // waves per workgroup (two workgroups per CU)
  static constexpr int NT = NW * 64;
  static constexpr int BK = 64;                          // keys per tile (two 32-key blocks)
  static constexpr int ROWB = 2 * D;                     // bytes per K/V row in LDS (unpadded)
  static constexpr int SLOTS = ROWB / 16;                // 16-byte granules per row
  static constexpr int RPD = 64 / SLOTS;                 // rows per LDS-writing load (64 lanes x 16 B)
  static constexpr int TILEB = BK * ROWB;                // bytes per K (or V) tile
  static constexpr int DPW = TILEB / 1024 / NW;          // LDS-writing loads per wave per tile
  static constexpr int DSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
  static constexpr int MINW = (D >= 256) ? 1 : 2;        // waves per SIMD
  static_assert(DPW * NW * 1024 == TILEB, "tile must split evenly over the waves");
  // Granule swizzles (physical slot = logical granule ^ swizzle(row)) for 64 four-byte banks:
  //  K: the 16 lanes of a 16-byte fragment read take 16 consecutive rows at one logical granule;
  //  V: the 32 lanes of half a transpose read take 4 consecutive rows (4-aligned) x 4 granules.
  // Both are XOR-linear in the row bits they use, so the swizzle of row 32b + r, 16k + r, 8k + r or
  // RPD * m + r splits into a per-lane part and a constant.
  static constexpr __host__ __device__ int kswz(int r) { return D >= 128 ? (r & 15) : ((r >> 1) & 7); }
  static constexpr __host__ __device__ int vswz(int r) { return D >= 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

// Lowest set bit index >= x of the bitmap bu (nbits bits), or -1.
__device__ inline int next_set(const uint32_t* bu, int x, int nbits) {
  if (x >= nbits) return -1;
  int w = x >> 5;
  uint32_t u = bu[w] & (0xFFFFFFFFu << (x & 31));
  const int nw = (nbits + 31) >> 5;
  while (true) {
    if (u) return (w << 5) + __builtin_ctz(u);
    if (++w >= nw) return -1;
    u = bu[w];
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
  // Two-stage rings, one LDS array per stage: K of the tile after next and V of the next tile load
  // while the current tile is computed.  The stage of every access is known at compile time, so a
  // read of one array never waits for loads still landing in another.
  __shared__ __attribute__((aligned(1024))) uint8_t k_st0[GE::TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t k_st1[GE::TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t v_st0[GE::TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t v_st1[GE::TILEB];
  __shared__ uint32_t bm[GE::NW + 1][kMaxWords];            // per head slot, then their union

  // ---- block -> (KV head, chunk, head slot, row tile); one XCD per (KV head, chunk)
  const int G = Hq / Hkv;
  const int rb_count = NW / hp;
  const int per_group = head_slots * row_tiles;
  const int xcd = blockIdx.x & 7;
  const int kth = blockIdx.x >> 3;
  const int gid = (kth / per_group) * 8 + xcd;
  if (gid >= Hkv * C) return;                              // block-uniform
  const int sub = kth % per_group;
  const int rt = __builtin_amdgcn_readfirstlane(sub % row_tiles);
  const int hs = __builtin_amdgcn_readfirstlane(sub / row_tiles);
  const int gk = __builtin_amdgcn_readfirstlane(gid / C);  // (integer division runs on the VALU)
  const int i = __builtin_amdgcn_readfirstlane(C - 1 - (gid % C));   // heaviest (latest) chunks first
  const int s_i = cu_chunks[i], e_i = cu_chunks[i + 1];
  const int q0 = s_i + rt * rb_count * 32;
  if (q0 >= e_i) return;                                   // block-uniform

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hw = wave % hp;
  const int h = gk * G + hs * hp + hw;
  const int qr0 = q0 + (wave / hp) * 32;
  const bool wave_rows = qr0 < e_i;
  const int first = __builtin_amdgcn_readfirstlane(seq_chunk_start[seq_of_chunk(seq_chunk_start, B, i)]);
  const int nbits = i - first + 1;
  const int rp0 = row_ptr[i], rlen = row_ptr[i + 1] - rp0;
  const int diag_end = min(e_i, q0 + rb_count * 32);

  // ---- kept-chunk bitmaps of the workgroup's heads
  const int nwords = (nbits + 31) >> 5;
  for (int x = tid; x < (GE::NW + 1) * nwords; x += NT) bm[x / nwords][x % nwords] = 0u;
  __syncthreads();
  for (int x = tid; x < hp * rlen; x += NT) {
    const int hh = x / rlen, e = x - hh * rlen;
    const int j = block_idx[(size_t)(gk * G + hs * hp + hh) * nnz + rp0 + e];
    const int loc = j - first;
    if (loc >= 0 && loc < nbits) {
      atomicOr(&bm[hh][loc >> 5], 1u << (loc & 31));
      atomicOr(&bm[GE::NW][loc >> 5], 1u << (loc & 31));
    }
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

  // ---- tile walk, kept in scalar registers (identical in every thread of a wave)
  struct TileRef {
    int jl, kt, kend;      // local chunk index (-1: walk over), key range [kt, kend) of the chunk part
    int keep;              // whether this wave's head keeps the chunk
  };
  // (every field goes through readfirstlane: the walk is wave-uniform, and scalar registers keep the
  // buffer descriptors and branches built from it scalar)
  auto chunk_span = [&](TileRef& t) __attribute__((always_inline)) {
    const int j = first + t.jl;
    t.kt = __builtin_amdgcn_readfirstlane(cu_chunks[j]);
    t.kend = __builtin_amdgcn_readfirstlane((j == i) ? diag_end : cu_chunks[j + 1]);
    t.keep = __builtin_amdgcn_readfirstlane((bm[hw][t.jl >> 5] >> (t.jl & 31)) & 1u);
  };
  auto next_tile = [&](TileRef t) __attribute__((always_inline)) {
    if (t.jl < 0) return t;
    t.kt += BK;
    if (t.kt >= t.kend) {
      t.jl = __builtin_amdgcn_readfirstlane(next_set(bm[GE::NW], t.jl + 1, nbits));
      if (t.jl >= 0) chunk_span(t);
    }
    return t;
  };

  // ---- staging: LDS-writing buffer loads.  Load m of this wave writes the 1 KB at tile byte
  // (wave * DPW + m) * 1024, lane by lane in 16-byte steps: tile row RPD * (wave * DPW + m) + lane / SLOTS,
  // physical slot lane % SLOTS, which receives logical granule slot ^ swizzle(row).  The row block
  // goes into the scalar offset; the swizzle splits into the lane part below and a constant of m.
  // Every load of a tile writes all of its stage: rows past the last token are out of the buffer
  // range and arrive as zeros.
  const int row_in = lane / GE::SLOTS, slot = lane % GE::SLOTS;
  const int row_bytes = Hkv * D * 2;                       // global stride of one token's KV head row
  const int vk_lane = row_in * row_bytes + (slot ^ GE::kswz(row_in)) * 16;
  const int vv_lane = row_in * row_bytes + (slot ^ GE::vswz(row_in)) * 16;
  const int soff_wave = wave * GE::DPW * GE::RPD * row_bytes;
  // buffer range: this KV head's rows from the tile start to the last token (nothing past T is read)
  auto tile_rsrc = [&](const uint16_t* base_ptr, const TileRef& t) __attribute__((always_inline)) {
    const int kt = __builtin_amdgcn_readfirstlane(t.kt);
    const long long rows_left = (long long)(T - kt) * Hkv - gk;
    const long long cap = (long long)BK * Hkv * D * 2;
    const int nbytes = (int)min(rows_left * D * 2, cap);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base_ptr + ((size_t)kt * Hkv + gk) * D), (short)0, nbytes,
                                             kBufWord3);
  };
  auto load_k = [&](const TileRef& t, uint8_t* dst) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(k, t);
#pragma unroll
    for (int m = 0; m < GE::DPW; ++m) {
      // (the offsets are named first: clang drops the host stub of the kernel when a constexpr call
      // sits directly in this builtin's argument list)
      const int voff = vk_lane ^ (GE::kswz(GE::RPD * m) * 16);
      const int soff = soff_wave + m * GE::RPD * row_bytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + (wave * GE::DPW + m) * 1024), 16, voff, soff, 0, 0);
    }
  };
  auto load_v = [&](const TileRef& t, uint8_t* dst) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(v, t);
#pragma unroll
    for (int m = 0; m < GE::DPW; ++m) {
      // (the offsets are named first: clang drops the host stub of the kernel when a constexpr call
      // sits directly in this builtin's argument list)
      const int voff = vv_lane ^ (GE::vswz(GE::RPD * m) * 16);
      const int soff = soff_wave + m * GE::RPD * row_bytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + (wave * GE::DPW + m) * 1024), 16, voff, soff, 0, 0);
    }
  };

  // ---- per-lane LDS read offsets (bytes)
  // K fragment of S^T = K Q^T: row col (+32 for the second key block), logical granule 2s + half at
  // step s; physical byte (col * ROWB + 16 * (half ^ kswz(col))) ^ 32 s
  const int k_lane = col * GE::ROWB + 16 * (half ^ GE::kswz(col));
  // V^T fragment, transpose load: the 16-lane group grp reads key rows 4 (grp / 2) + ii / 4 (+8 for the
  // upper half, +16 per k-step), dims 16 (grp % 2) + 4 (ii % 4) of the 32-dim block db; physical byte
  // v_lane ^ 64 db
  const int grp = (lane >> 4) & 3, ii = lane & 15;
  const int vrow = 4 * (grp >> 1) + (ii >> 2);
  const int v_lane = vrow * GE::ROWB + 16 * ((2 * (grp & 1) + ((ii & 3) >> 1)) ^ GE::vswz(vrow)) + 8 * (ii & 1);

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
  // masking: tiles cut by the chunk end, tiles of chunks this head does not keep, and tiles of the
  // diagonal chunk with a key past the wave's first query row
  auto needs_mask = [&](const TileRef& t) __attribute__((always_inline)) {
    return t.kend - t.kt < BK || !t.keep || (first + t.jl == i && t.kt + BK - 1 > qr0);
  };
  auto apply_mask = [&](f32x16 (&s)[2], const TileRef& t) __attribute__((always_inline)) {
    int lim = t.kend - t.kt - 1;
    if (first + t.jl == i) lim = min(lim, tq - t.kt);
    if (!t.keep) lim = -1;
    lim -= 4 * half;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[b][r] = (32 * b + 8 * (r >> 2) + (r & 3) > lim) ? -INFINITY : s[b][r];
        __builtin_amdgcn_sched_barrier(0);     // compare and select in turn, through one condition register
      }
  };

  // QK^T of the next tile (if QN) interleaved with the softmax of the current tile (if SM).
  // Leaves P^T of the current tile packed in pw and the running max / sums updated; returns alpha.
  uint32_t pw[16];
  auto region_a = [&](auto qn_c, auto sm_c, const uint8_t* kst, f32x16 (&sn)[2], f32x16 (&sc)[2],
                      float& alpha) __attribute__((always_inline)) {
    constexpr bool QN = decltype(qn_c)::value, SM = decltype(sm_c)::value;
    if constexpr (QN) {
      const uint8_t* kb = kst + 0;
#pragma unroll
      for (int st = 0; st < GE::DSTEPS; ++st) {
        const int ko = k_lane ^ (32 * st);
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(kb + ko);
        sn[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[st], st == 0 ? zero16 : sn[0], 0, 0, 0);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(kb + 32 * GE::ROWB + ko);
        sn[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[st], st == 0 ? zero16 : sn[1], 0, 0, 0);
      }
    }
    if constexpr (SM) {
      // reductions as shallow trees (four independent partial results) to keep dependency chains short
      float m4[4];
#pragma unroll
      for (int x = 0; x < 4; ++x)
        m4[x] = fmaxf(fmaxf(fmaxf(sc[0][x], sc[0][x + 4]), fmaxf(sc[0][x + 8], sc[0][x + 12])),
                      fmaxf(fmaxf(sc[1][x], sc[1][x + 4]), fmaxf(sc[1][x + 8], sc[1][x + 12])));
      const float mx = max_halves(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
      const bool grow = mx > m_ref + grow_raw;
      const float m_new = grow ? mx : m_ref;
      alpha = grow ? __builtin_amdgcn_exp2f((m_ref - m_new) * c2) : 1.f;   // 0 at the first tile
      const float mb = (m_new == -INFINITY ? 0.f : m_new) * c2;
      m_ref = m_new;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[b][r] = __builtin_amdgcn_exp2f(fmaf(sc[b][r], c2, -mb));
      float lb4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < 2; ++b)
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
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) ls4[r & 3] += sc[b][r];
        l_run = l_run * alpha + sum_halves((ls4[0] + ls4[1]) + (ls4[2] + ls4[3]));
      }
    }
    // interleave: each QK MFMA followed by its next K read and a slice of the softmax
    if constexpr (QN && SM) {
      __builtin_amdgcn_sched_group_barrier(kSgDSR, 4, 0);
#pragma unroll
      for (int x = 0; x < 2 * GE::DSTEPS; ++x) {
        __builtin_amdgcn_sched_group_barrier(kSgMFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDSR, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgVALU, 120 / (2 * GE::DSTEPS) + 1, 0);
      }
    }
  };

  // O^T += V^T P^T for the current tile
  auto region_b = [&](const uint8_t* vst) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(pw[ks * 4], pw[ks * 4 + 1], pw[ks * 4 + 2],
                                                              pw[ks * 4 + 3]));
#pragma unroll
      for (int db = 0; db < GE::DBLK; ++db) {
        const uint8_t* p0 = vst + (v_lane ^ (64 * db)) + ks * 16 * GE::ROWB;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 8 * GE::ROWB));
        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
        const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(l2.x, l2.y, h2.x, h2.y));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf, o[db], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(kSgDSR, 6, 0);
#pragma unroll
    for (int x = 0; x < 4 * GE::DBLK; ++x) {
      __builtin_amdgcn_sched_group_barrier(kSgMFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSgDSR, 2, 0);
    }
  };

  // ---- prologue: K ring holds tiles 0 and 1, V ring tile 0
  TileRef t0;
  t0.jl = __builtin_amdgcn_readfirstlane(next_set(bm[GE::NW], 0, nbits));
  t0.kt = 0; t0.kend = 0; t0.keep = 0;
  if (t0.jl >= 0) chunk_span(t0);
  TileRef t1 = next_tile(t0);
  TileRef t2 = next_tile(t1);
  if (t0.jl >= 0) { load_k(t0, k_st0); load_v(t0, v_st0); }
  if (t1.jl >= 0) load_k(t1, k_st1);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();

  // Waves without query rows (possible when the workgroup holds several row blocks) only stage
  // tiles.  Every other wave runs the same straight-line tile body: after the last tile the QK^T of
  // the (absent) next tile reads a stale but finite K stage and is discarded.
  f32x16 sA[2], sB[2];
  if (wave_rows) {
    float dummy;
    region_a(std::true_type{}, std::false_type{}, k_st0, sA, sB, dummy);   // S^T of tile 0
  }
  __syncthreads();                             // K stage 0 is rewritten by the first iteration

  // One iteration with stage parity S: softmax and PV of t0 (S^T in sc, V in V stage S), QK^T of t1
  // (K in K stage 1 - S, into sn); meanwhile K of t2 lands in K stage S and V of t1 in V stage 1 - S.
  auto step = [&](auto s_c, f32x16 (&sc)[2], f32x16 (&sn)[2]) __attribute__((always_inline)) {
    constexpr int S = decltype(s_c)::value;
    uint8_t* const k_fill = S ? k_st1 : k_st0;
    uint8_t* const k_read = S ? k_st0 : k_st1;
    uint8_t* const v_fill = S ? v_st0 : v_st1;
    uint8_t* const v_read = S ? v_st1 : v_st0;
    const TileRef t3 = next_tile(t2);
    if (t2.jl >= 0) load_k(t2, k_fill);
    if (t1.jl >= 0) load_v(t1, v_fill);
    if (wave_rows) {
      if (needs_mask(t0)) apply_mask(sc, t0);
      float alpha = 1.f;
      // The half with the softmax issues first when both waves of the SIMD are ready: its VALU chain
      // is the latency-critical one, and the other wave's PV MFMAs fill the gaps.
      __builtin_amdgcn_s_setprio(2);
      region_a(std::true_type{}, std::true_type{}, k_read, sn, sc, alpha);
      __builtin_amdgcn_s_setprio(0);
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {   // a running max moved
#pragma unroll
        for (int db = 0; db < GE::DBLK; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
      region_b(v_read);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // this wave's loads have landed before others read them
    __syncthreads();
    t0 = t1; t1 = t2; t2 = t3;
  };
  while (t0.jl >= 0) {
    step(ic<0>{}, sA, sB);
    if (t0.jl < 0) break;
    step(ic<1>{}, sB, sA);
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
