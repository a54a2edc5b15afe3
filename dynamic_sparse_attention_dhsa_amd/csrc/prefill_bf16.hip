// Stage 3: block-sparse causal prefill, bf16 in, fp32 accumulate, on gfx950 MFMA.
//
// ICML 2026 spotlight page (Abstract): DHSA computes attention over the
// interactions its router keeps with a tiled kernel that keeps memory low;
// "... for On-Device LLMs" (Abstract): the kept token interactions follow from
// chunk scores upsampled to token level.  Query token t of chunk i, head h
// attends to every key u <= t inside a kept chunk of row (h, i):
//   out[t,h] = sum_u softmax_u(scale * q_t . k_u) v_u,   lse[h,t] = log sum_u exp(scale * q_t . k_u).
//
// Work decomposition.  A workgroup of four waves owns one query chunk i, one
// KV head g and a tile of query rows; two workgroups share a CU.  Its waves
// are HP query heads of g (HP = the largest power of two dividing G, at most
// 4) times 4 / HP blocks of R query rows, so one K/V tile staged in LDS feeds
// every q head of the group that keeps it.  The workgroup walks the union of
// its heads' kept chunks in ascending order (per-head bitmaps in LDS); a
// head's scores on a chunk it does not keep are masked, and a wave skips the
// iterations on runs of tiles its head keeps none of.  Key tiles hold 2R keys
// in groups of a few rows; a group never crosses a chunk boundary, a tile may
// (the kept chunks before the diagonal are packed back to back, the diagonal
// chunk takes tiles of its own); rows past a chunk's end or past the
// diagonal are masked.
//
// Blocks are numbered so that all row tiles of one (KV head, query chunk)
// land on the same XCD (blocks are dealt to the 8 XCDs round robin), where
// they stream the same kept K/V through one L2; KV heads go one after
// another across the chip, heaviest chunks first.  Each XCD's blocks are
// its groups' real row tiles back to back, with no block for rows past a
// chunk's end: the dispatcher hands blocks out in order, round robin over
// the XCDs, so an XCD whose slots are full holds back every other one, and
// padding blocks that make the XCDs' shares of real work differ from one
// dispatch position to the next leave slots idle.  (Past 2048 groups per
// XCD, where each block's scan over its XCD's groups would grow long, every
// group is padded to the longest chunk's row tiles instead.)
//
// Per tile and wave (R queries x 2R keys), with v_mfma_f32_32x32x16_bf16 (R = 32,
// head dims 64 and 128) or v_mfma_f32_16x16x32_bf16 (R = 16, head dim 256, where
// a 32-row wave's O, Q^T and scores would leave room for one wave per SIMD):
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
#include <algorithm>
#include <type_traits>

#include "dhsa_internal.hpp"

namespace dhsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef s16x4 __attribute__((address_space(3))) lds_s16x4;
typedef void __attribute__((address_space(3))) lds_void;

constexpr int kMaxWords = DHSA_MAX_WORDS;      // bitmap words per head (32 chunks each)
constexpr int kUnion = 4;                      // bitmap row of the union (head slots use rows 0..3)
constexpr int kCompactMaxGroups = 2048;        // (KV head, chunk) groups per XCD for compact block numbering
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleLog2 = 8.0f;           // move the running max only past 2^8
constexpr int kBufWord3 = 0x00020000;          // gfx9 buffer resource: raw 32-bit data
constexpr int kWaitVmcnt0 = 0x0F70;            // s_waitcnt vmcnt(0), other counters unconstrained

// scheduling-group masks for __builtin_amdgcn_sched_group_barrier
constexpr int kSgVALU = 0x002, kSgMFMA = 0x008, kSgDSR = 0x100;

template <int D>
struct Geo {
  // Query rows per wave: 32 with 32x32x16 MFMAs; at d = 256 a 32-row wave's O, Q^T and scores would
  // not fit two waves per SIMD, so there a wave takes 16 rows with 16x16x32 MFMAs and tiles hold 32 keys.
  static constexpr int ROWS = (D >= 256) ? 16 : 32;
  static constexpr int NW = 4;                           // waves per workgroup (two workgroups per CU)
  static constexpr int NT = NW * 64;
  static constexpr int BK = 2 * ROWS;                    // keys per tile (two key blocks of ROWS)
  static constexpr int ROWB = 2 * D;                     // bytes per K/V row in LDS (unpadded)
  static constexpr int SLOTS = ROWB / 16;                // 16-byte granules per row
  static constexpr int RPD = 64 / SLOTS;                 // rows per LDS-writing load (64 lanes x 16 B)
  static constexpr int TILEB = BK * ROWB;                // bytes per K (or V) tile
  static constexpr int DPW = TILEB / 1024 / NW;          // LDS-writing loads per wave per tile
  static constexpr int QK_K = (ROWS == 32) ? 16 : 32;    // head dims per S^T MFMA
  static constexpr int DSTEPS = D / QK_K;                // S^T MFMAs per key block
  static constexpr int OB = ROWS;                        // head dims per O^T block (the MFMA's M)
  static constexpr int DBLK = D / OB;                    // O^T blocks
  static constexpr int PVK = BK / QK_K;                  // PV MFMAs per O^T block and tile
  static constexpr int MINW = 2;                         // waves per SIMD
  static_assert(DPW * NW * 1024 == TILEB, "tile must split evenly over the waves");
  // Granule swizzles (physical slot = logical granule ^ swizzle(row)) for 64 four-byte banks:
  //  K: the 16 lanes of a 16-byte fragment read take 16 consecutive rows at one logical granule;
  //  V: the 32 lanes of half a transpose read take 4 consecutive rows (4-aligned) x 4 granules.
  // Both are XOR-linear in the row bits they use, so the swizzle of row 32b + r, 16k + r, 8k + r or
  // RPD * m + r splits into a per-lane part and a constant.
  static constexpr __host__ __device__ int kswz(int r) { return D >= 128 ? (r & 15) : ((r >> 1) & 7); }
  //  V with 16-row waves: the four 16-lane groups of a transpose read take rows 4g .. 4g + 3 of one
  //  column range; row bit 2 moves groups g and g + 1 (read in the same cycle) to other banks.
  static constexpr __host__ __device__ int vswz(int r) {
    return ROWS == 16 ? (4 * (r & 3)) ^ (2 * ((r >> 2) & 1)) : (D >= 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1));
  }
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
// the same over lanes l and l ^ 16 (16-lane rows swapped in pairs)
__device__ inline float max_rows16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_rows16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
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
    long long nnz, float scale, int hp, int head_slots, int row_tiles, int compact) {
  using GE = Geo<D>;
  constexpr int NW = GE::NW, NT = GE::NT, BK = GE::BK;
  // Two-stage rings, one LDS array per stage: K of the tile after next and V of the next tile load
  // while the current tile is computed.  The stage of every access is known at compile time, so a
  // read of one array never waits for loads still landing in another.
  __shared__ __attribute__((aligned(1024))) uint8_t k_st0[GE::TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t k_st1[GE::TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t v_st0[GE::TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t v_st1[GE::TILEB];
  __shared__ uint32_t bm[kUnion + 1][kMaxWords];            // per head slot, then their union

  // ---- block -> (KV head, chunk, head slot, row tile); group g = (KV head, chunk) on XCD g % 8
  const int G = Hq / Hkv;
  const int rb_count = NW / hp;
  constexpr int ROWS = GE::ROWS;
  const int rows_blk = rb_count * ROWS;
  const int xcd = blockIdx.x & 7;
  const int kth = blockIdx.x >> 3;                         // position among this XCD's blocks
  const int ngroups = Hkv * C;
  // group g holds KV head g / C and chunk C - 1 - g % C (heaviest, i.e. latest, chunks first)
  auto group_tiles = [&](int g) __attribute__((always_inline)) {
    const int ci = C - 1 - (g % C);
    return head_slots * ((cu_chunks[ci + 1] - cu_chunks[ci] + rows_blk - 1) / rows_blk);
  };
  int gid, sub;
  if (compact) {
    // this XCD's groups xcd + 8 m, m < ng_x, each with its real row tiles: an exclusive scan of the
    // per-thread tile counts (contiguous ranges of m) finds the group holding position kth
    __shared__ int s_wsum[NW];
    __shared__ int s_sel[2];
    const int t0 = threadIdx.x, l0 = t0 & 63, w0 = t0 >> 6;
    const int ng_x = ngroups > xcd ? (ngroups - xcd + 7) >> 3 : 0;
    const int per = (ng_x + NT - 1) / NT;
    const int m_lo = t0 * per, m_hi = min(ng_x, m_lo + per);
    int my = 0;
    for (int m = m_lo; m < m_hi; ++m) my += group_tiles(xcd + 8 * m);
    int incl = my;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (l0 >= off) incl += o;
    }
    if (l0 == 63) s_wsum[w0] = incl;
    if (t0 == 0) s_sel[0] = -1;
    __syncthreads();
    for (int x = 0; x < w0; ++x) incl += s_wsum[x];
    if (kth >= incl - my && kth < incl) {
      int acc = incl - my;
      for (int m = m_lo; m < m_hi; ++m) {
        const int t = group_tiles(xcd + 8 * m);
        if (kth < acc + t) { s_sel[0] = m; s_sel[1] = kth - acc; break; }
        acc += t;
      }
    }
    __syncthreads();
    const int msel = __builtin_amdgcn_readfirstlane(s_sel[0]);
    if (msel < 0) return;                                  // block-uniform: past this XCD's row tiles
    gid = xcd + 8 * msel;
    sub = __builtin_amdgcn_readfirstlane(s_sel[1]);
  } else {
    // every group padded to row_tiles x head_slots blocks (too many groups for the scan above)
    const int per_group = head_slots * row_tiles;
    gid = (kth / per_group) * 8 + xcd;
    if (gid >= ngroups) return;                            // block-uniform
    sub = kth % per_group;
  }
  const int gk = __builtin_amdgcn_readfirstlane(gid / C);  // (integer division runs on the VALU)
  const int i = __builtin_amdgcn_readfirstlane(C - 1 - (gid % C));
  const int s_i = cu_chunks[i], e_i = cu_chunks[i + 1];
  const int tiles_i = compact ? (e_i - s_i + rows_blk - 1) / rows_blk : row_tiles;
  const int rt = __builtin_amdgcn_readfirstlane(sub % tiles_i);
  const int hs = __builtin_amdgcn_readfirstlane(sub / tiles_i);
  const int q0 = s_i + rt * rows_blk;
  if (q0 >= e_i) return;                                   // block-uniform (padded blocks only)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hw = wave % hp;
  const int h = gk * G + hs * hp + hw;
  const int qr0 = q0 + (wave / hp) * ROWS;
  const bool wave_rows = qr0 < e_i;
  const int first = __builtin_amdgcn_readfirstlane(seq_chunk_start[seq_of_chunk(seq_chunk_start, B, i)]);
  const int nbits = i - first + 1;
  const int rp0 = row_ptr[i], rlen = row_ptr[i + 1] - rp0;
  const int diag_end = min(e_i, q0 + rb_count * ROWS);

  // ---- kept-chunk bitmaps of the workgroup's heads
  const int nwords = (nbits + 31) >> 5;
  for (int x = tid; x < (kUnion + 1) * nwords; x += NT) bm[x / nwords][x % nwords] = 0u;
  __syncthreads();
  for (int x = tid; x < hp * rlen; x += NT) {
    const int hh = x / rlen, e = x - hh * rlen;
    const int j = block_idx[(size_t)(gk * G + hs * hp + hh) * nnz + rp0 + e];
    const int loc = j - first;
    if (loc >= 0 && loc < nbits) {
      atomicOr(&bm[hh][loc >> 5], 1u << (loc & 31));
      atomicOr(&bm[kUnion][loc >> 5], 1u << (loc & 31));
    }
  }
  __syncthreads();

  // ---- Q^T fragments (B operand), whole walk
  // a lane's query column, and which slice of the MFMA's k (or of the accumulator's rows) it holds:
  // 0..1 with 32-row waves, 0..3 with 16-row waves
  const int col = lane & (ROWS - 1), half = lane / ROWS;
  const int tq = qr0 + col;
  bf16x8 qf[GE::DSTEPS];
  {
    const bool ok = tq < e_i;
    const uint16_t* qp = q + ((size_t)tq * Hq + h) * D + half * 8;
#pragma unroll
    for (int s = 0; s < GE::DSTEPS; ++s) {
      uint4 raw = ok ? *reinterpret_cast<const uint4*>(qp + s * GE::QK_K) : make_uint4(0, 0, 0, 0);
      qf[s] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // ---- tile walk, wave-uniform, in scalar registers (every value read from memory goes through
  // readfirstlane, so the descriptors and branches built from it stay scalar).  A tile is 64 key rows
  // in NGRP groups of GS rows, one group per LDS-writing load.  The kept chunks before the diagonal
  // are packed back to back: a group never crosses a chunk, but a tile does, so only the last group
  // of a chunk carries rows past its end.  The diagonal chunk follows in tiles of its own, which the
  // causal mask needs.  Per tile: how many rows of each group are real keys of a chunk this wave's
  // head keeps (NB bits per group), and the first key row of each of this wave's groups.
  constexpr int GS = GE::RPD;
  constexpr int NGRP = BK / GS;
  constexpr int NB = 64 / NGRP;
  constexpr uint64_t kFull = 0x0101010101010101ull * (uint64_t)(NB == 8 ? GS : (NB == 4 ? GS * 0x11 : GS * 0x55));
  struct TileRef {
    int valid;               // 0: the walk is over
    int kt;                  // tile of the diagonal chunk: its first key row; -1 for packed tiles
    uint64_t nval;           // real, kept rows per group (NB bits each)
    int src[GE::DPW];        // first key row of this wave's groups
  };
  auto groups_mask = [](int ng) __attribute__((always_inline)) {
    return ng * NB >= 64 ? ~0ull : ((1ull << (ng * NB)) - 1ull);
  };
  auto rf = [](int x) __attribute__((always_inline)) { return __builtin_amdgcn_readfirstlane(x); };
  // cursor: local chunk cj (-1: done), row offset coff in it, and the chunk's first row, length and
  // keep bit for this wave's head, fetched once per chunk
  int cj, coff = 0, cr0 = 0, clen = 0, ckeep = 0;
  auto enter = [&](int x) __attribute__((always_inline)) {
    cj = x;
    coff = 0;
    if (cj >= 0) {
      cr0 = rf(cu_chunks[first + cj]);
      clen = (first + cj == i) ? diag_end - cr0 : rf(cu_chunks[first + cj + 1]) - cr0;
      ckeep = rf((bm[hw][cj >> 5] >> (cj & 31)) & 1u);
    }
  };
  enter(rf(next_set(bm[kUnion], 0, nbits)));
  auto build = [&]() __attribute__((always_inline)) {
    TileRef t;
    t.valid = cj >= 0;
    t.kt = -1;
    t.nval = 0;
#pragma unroll
    for (int m = 0; m < GE::DPW; ++m) t.src[m] = 0;
    if (cj < 0) return t;
    if (first + cj == i) {                   // diagonal chunk: contiguous rows up to diag_end
      t.kt = cr0 + coff;
      const int nrows = min(BK, clen - coff);
      const int full = nrows / GS, rem = nrows % GS;
      t.nval = (kFull & groups_mask(full)) | (full < NGRP ? (uint64_t)rem << (full * NB) : 0ull);
#pragma unroll
      for (int m = 0; m < GE::DPW; ++m) t.src[m] = t.kt + GS * (wave * GE::DPW + m);
      coff += BK;
      if (coff >= clen) cj = -1;
      return t;
    }
    // the common case: the whole tile inside the current chunk (one key range, no partial group)
    if (clen - coff >= BK) {
      t.nval = ckeep ? kFull : 0ull;
#pragma unroll
      for (int m = 0; m < GE::DPW; ++m) t.src[m] = cr0 + coff + GS * (wave * GE::DPW + m);
      coff += BK;
      if (coff >= clen) enter(rf(next_set(bm[kUnion], cj + 1, nbits)));
      return t;
    }
    int slot = 0;
    while (slot < NGRP) {                    // pack groups from consecutive kept chunks
      const int left = clen - coff;
      if (left > 0) {
        const int ngr = min((left + GS - 1) / GS, NGRP - slot);
        const int last = min(GS, left - GS * (ngr - 1));
        if (ckeep) t.nval |= ((kFull & groups_mask(ngr - 1)) | ((uint64_t)last << ((ngr - 1) * NB))) << (slot * NB);
#pragma unroll
        for (int m = 0; m < GE::DPW; ++m) {
          const int g = wave * GE::DPW + m - slot;
          if (g >= 0 && g < ngr) t.src[m] = cr0 + coff + GS * g;
        }
        slot += ngr;
        coff += GS * ngr;
      }
      if (coff >= clen) {                    // chunk done: on to the next kept one
        enter(rf(next_set(bm[kUnion], cj + 1, nbits)));
        if (cj < 0 || first + cj == i) break;   // the diagonal chunk starts a tile of its own
      }
    }
    return t;
  };

  // ---- staging: LDS-writing buffer loads.  Load m of this wave writes the 1 KB at tile byte
  // (wave * DPW + m) * 1024, lane by lane in 16-byte steps: tile row GS * (wave * DPW + m) + lane / SLOTS,
  // physical slot lane % SLOTS, which receives logical granule slot ^ swizzle(row); the swizzle splits
  // into the lane part below and a constant of m.  The key row of the group is added to the lane's
  // offset (not the scalar one), so the buffer's range check covers it: rows past the last token are
  // out of range and arrive as zeros, and nothing past the tensors is read.
  const int row_in = lane / GE::SLOTS, slot = lane % GE::SLOTS;
  const int row_bytes = Hkv * D * 2;                       // global stride of one token's KV head row
  const int row0 = GE::RPD * GE::DPW * wave + row_in;      // tile row of this lane in the wave's first load
  const int vk_lane = row_in * row_bytes + (slot ^ GE::kswz(row0)) * 16;
  const int vv_lane = row_in * row_bytes + (slot ^ GE::vswz(row0)) * 16;
  const int kv_bytes = (int)(((long long)T * Hkv - gk) * D * 2);   // this KV head's rows, up to the last token
  const __amdgpu_buffer_rsrc_t rsrc_k =
      __builtin_amdgcn_make_buffer_rsrc((void*)(k + (size_t)gk * D), (short)0, kv_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t rsrc_v =
      __builtin_amdgcn_make_buffer_rsrc((void*)(v + (size_t)gk * D), (short)0, kv_bytes, kBufWord3);
  auto load_k = [&](const TileRef& t, uint8_t* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < GE::DPW; ++m) {
      // (the offset is named first: clang drops the host stub of the kernel when a constexpr call
      // sits directly in this builtin's argument list)
      const int voff = (vk_lane ^ (GE::kswz(GE::RPD * m) * 16)) + t.src[m] * row_bytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_k, (lds_void*)(dst + (wave * GE::DPW + m) * 1024), 16, voff, 0, 0, 0);
    }
  };
  auto load_v = [&](const TileRef& t, uint8_t* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < GE::DPW; ++m) {
      const int voff = (vv_lane ^ (GE::vswz(GE::RPD * m) * 16)) + t.src[m] * row_bytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_v, (lds_void*)(dst + (wave * GE::DPW + m) * 1024), 16, voff, 0, 0, 0);
    }
  };

  // ---- per-lane LDS read offsets (bytes)
  // K fragment of S^T = K Q^T: key row col of the block (col + ROWS for the second one), logical
  // granule (QK_K / 8) st + half at step st; physical byte (col * ROWB + 16 * (half ^ kswz(col))) ^ 2 QK_K st
  const int k_lane = col * GE::ROWB + 16 * (half ^ GE::kswz(col));
  // V^T fragment, transpose load (a 16-lane group reads 4 rows x 16 columns and each lane receives one
  // column of the 4 rows).  32-row waves: the group grp reads key rows 4 (grp / 2) + ii / 4 (+8 for the
  // upper half, +16 per k-step), dims 16 (grp % 2) + 4 (ii % 4) of the 32-dim block db; physical byte
  // v_lane ^ 64 db.  16-row waves: group grp reads key rows 4 grp + ii / 4 (+16 for the upper half),
  // dims 4 (ii % 4) of the 16-dim block db; physical byte v_lane ^ 32 db.
  const int grp = (lane >> 4) & 3, ii = lane & 15;
  int v_lane;
  if constexpr (ROWS == 32) {
    const int vrow = 4 * (grp >> 1) + (ii >> 2);
    v_lane = vrow * GE::ROWB + 16 * ((2 * (grp & 1) + ((ii & 3) >> 1)) ^ GE::vswz(vrow)) + 8 * (ii & 1);
  } else {
    const int vrow = 4 * grp + (ii >> 2);
    v_lane = vrow * GE::ROWB + 16 * (((ii & 3) >> 1) ^ GE::vswz(vrow)) + 8 * (ii & 1);
  }
  constexpr int VHI = (ROWS == 32) ? 8 : 16;               // rows between a transpose read's two halves
  constexpr int VDB = (ROWS == 32) ? 64 : 32;              // byte XOR per O^T block

  // accumulators: S^T of a tile as two ROWS x ROWS key blocks, O^T as DBLK blocks of OB dims
  using Acc = std::conditional_t<ROWS == 32, f32x16, f32x4>;
  constexpr int NA = (ROWS == 32) ? 16 : 4;                // accumulator registers per block
  constexpr int NPW = BK * ROWS / 128;                     // packed bf16 weight pairs per lane and tile
  Acc o[GE::DBLK];
#pragma unroll
  for (int db = 0; db < GE::DBLK; ++db)
#pragma unroll
    for (int r = 0; r < NA; ++r) o[db][r] = 0.f;
  // lb_run: sum of the bf16 weights actually multiplied into V, which normalises O (a dominant
  // weight cancels exactly); l_run: sum of the fp32 weights, kept only when the LSE is wanted
  float m_ref = -INFINITY, l_run = 0.f, lb_run = 0.f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const float c2 = scale * kLog2e;
  const float grow_raw = kRescaleLog2 / c2;
  const Acc zeroA = {};
  auto mfma = [](const bf16x8& a, const bf16x8& b, const Acc& c) __attribute__((always_inline)) {
    if constexpr (ROWS == 32) return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  };
  // reductions over the lanes holding one query column: l ^ 32 (32-row waves), l ^ 16 and l ^ 32 (16-row)
  auto col_max = [](float x) __attribute__((always_inline)) {
    if constexpr (ROWS == 16) x = max_rows16(x);
    return max_halves(x);
  };
  auto col_sum = [](float x) __attribute__((always_inline)) {
    if constexpr (ROWS == 16) x = sum_rows16(x);
    return sum_halves(x);
  };

  // 32-row waves: S^T[b][r] holds tile row 32b + 8(r/4) + 4*half + r%4 of query `col`.
  // 16-row waves: S^T[b][r] holds tile row 16b + 4*half + r of query `col`.
  // A tile needs masking when a group has fewer real, kept rows than GS, or when it is a tile of the
  // diagonal chunk with a key past the wave's first query row.
  auto needs_mask = [&](const TileRef& t) __attribute__((always_inline)) {
    return t.nval != kFull || (t.kt >= 0 && t.kt + BK - 1 > qr0);
  };
  auto apply_mask = [&](Acc (&s)[2], const TileRef& t) __attribute__((always_inline)) {
    const uint64_t nv = t.nval;
    if constexpr (ROWS == 32) {
      // rows past lim (in the lane's frame, which starts at row 4 * half) fail the causal test
      const int lim = (t.kt >= 0 ? tq - t.kt : BK) - 4 * half;
      const int hs4 = 4 * half;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int base = 32 * b + 8 * q4;  // lane-frame row of r = 4 q4 (plus 4 * half for the tile row)
          if constexpr (GS == 4) {           // group 8b + 2q4 + half, row in group r % 4
            const int n = (int)((nv >> (NB * (8 * b + 2 * q4) + NB * half)) & 0xF);
            const int nn = min(n, lim - base + 1);
#pragma unroll
            for (int e = 0; e < 4; ++e) s[b][4 * q4 + e] = (e < nn) ? s[b][4 * q4 + e] : -INFINITY;
          } else {                           // GS == 8: group 4b + q4, row in group 4 * half + r % 4
            const int n = (int)((nv >> (NB * (4 * b + q4))) & 0xFF) - hs4;
            const int nn = min(n, lim - base + 1);
#pragma unroll
            for (int e = 0; e < 4; ++e) s[b][4 * q4 + e] = (e < nn) ? s[b][4 * q4 + e] : -INFINITY;
          }
        }
    } else {
      // GS == 2: register r of block b is tile row 16b + 4 half + r, group 8b + 2 half + r / 2
      const int lim = (t.kt >= 0 ? tq - t.kt : BK) - 4 * half;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int p2 = 0; p2 < 2; ++p2) {
          const int n = (int)((nv >> (NB * (8 * b + p2) + 2 * NB * half)) & 0x3);
          const int nn = min(n, lim - 16 * b - 2 * p2 + 1);
#pragma unroll
          for (int e = 0; e < 2; ++e) s[b][2 * p2 + e] = (e < nn) ? s[b][2 * p2 + e] : -INFINITY;
        }
    }
  };

  // QK^T of the next tile (if QN) interleaved with the softmax of the current tile (if SM).
  // Leaves P^T of the current tile packed in pw and the running max / sums updated; returns alpha.
  uint32_t pw[NPW];
  auto region_a = [&](auto qn_c, auto sm_c, const uint8_t* kst, Acc (&sn)[2], Acc (&sc)[2],
                      float& alpha) __attribute__((always_inline)) {
    constexpr bool QN = decltype(qn_c)::value, SM = decltype(sm_c)::value;
    if constexpr (QN) {
      const uint8_t* kb = kst + 0;
#pragma unroll
      for (int st = 0; st < GE::DSTEPS; ++st) {
        const int ko = k_lane ^ (2 * GE::QK_K * st);
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(kb + ko);
        sn[0] = mfma(a0, qf[st], st == 0 ? zeroA : sn[0]);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(kb + ROWS * GE::ROWB + ko);
        sn[1] = mfma(a1, qf[st], st == 0 ? zeroA : sn[1]);
      }
    }
    if constexpr (SM) {
      // reductions as shallow trees (four independent partial results) to keep dependency chains short
      float mx;
      if constexpr (ROWS == 32) {
        // a tree of three-input maxima (v_max3_f32): 32 values in 16 instructions, three levels deep
        float t[12];
#pragma unroll
        for (int x = 0; x < 10; ++x) {
          const int a = 3 * x, b = a + 1, c = a + 2;
          t[x] = fmaxf(fmaxf(sc[a >> 4][a & 15], sc[b >> 4][b & 15]), sc[c >> 4][c & 15]);
        }
        t[10] = sc[1][14];
        t[11] = sc[1][15];
        float u[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) u[x] = fmaxf(fmaxf(t[3 * x], t[3 * x + 1]), t[3 * x + 2]);
        mx = col_max(fmaxf(fmaxf(fmaxf(u[0], u[1]), u[2]), u[3]));
      } else {
        mx = col_max(fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                           fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3]))));
      }
      const bool grow = mx > m_ref + grow_raw;
      const float m_new = grow ? mx : m_ref;
      alpha = grow ? __builtin_amdgcn_exp2f((m_ref - m_new) * c2) : 1.f;   // 0 at the first tile
      const float mb = (m_new == -INFINITY ? 0.f : m_new) * c2;
      m_ref = m_new;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < NA; ++r) sc[b][r] = __builtin_amdgcn_exp2f(fmaf(sc[b][r], c2, -mb));
      float lb4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < NA; r += 2) {
          const int x = b * (NA / 2) + r / 2;
          pw[x] = pack_bf16(sc[b][r], sc[b][r + 1]);
          lb4[x & 3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[x]), ones, lb4[x & 3], false);
        }
      lb_run = lb_run * alpha + col_sum((lb4[0] + lb4[1]) + (lb4[2] + lb4[3]));
      if constexpr (WITH_LSE) {
        float ls4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < NA; ++r) ls4[r & 3] += sc[b][r];
        l_run = l_run * alpha + col_sum((ls4[0] + ls4[1]) + (ls4[2] + ls4[3]));
      }
    }
    // interleave: each QK MFMA followed by its next K read and a slice of the softmax
    if constexpr (QN && SM) {
      constexpr int SMV = (ROWS == 32) ? 120 : 48;          // softmax VALU instructions, about
      __builtin_amdgcn_sched_group_barrier(kSgDSR, 4, 0);
#pragma unroll
      for (int x = 0; x < 2 * GE::DSTEPS; ++x) {
        __builtin_amdgcn_sched_group_barrier(kSgMFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDSR, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgVALU, SMV / (2 * GE::DSTEPS) + 1, 0);
      }
    }
  };

  // O^T += V^T P^T for the current tile
  auto region_b = [&](const uint8_t* vst) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < GE::PVK; ++ks) {
      const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(pw[ks * 4], pw[ks * 4 + 1], pw[ks * 4 + 2],
                                                              pw[ks * 4 + 3]));
#pragma unroll
      for (int db = 0; db < GE::DBLK; ++db) {
        const uint8_t* p0 = vst + (v_lane ^ (VDB * db)) + ks * 16 * GE::ROWB;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + VHI * GE::ROWB));
        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
        const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(l2.x, l2.y, h2.x, h2.y));
        o[db] = mfma(a, pf, o[db]);
      }
    }
    __builtin_amdgcn_sched_group_barrier(kSgDSR, 6, 0);
#pragma unroll
    for (int x = 0; x < GE::PVK * GE::DBLK; ++x) {
      __builtin_amdgcn_sched_group_barrier(kSgMFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSgDSR, 2, 0);
    }
  };

  // ---- prologue: K ring holds tiles 0 and 1, V ring tile 0
  TileRef t0 = build();
  TileRef t1 = build();
  TileRef t2 = build();
  if (t0.valid) { load_k(t0, k_st0); load_v(t0, v_st0); }
  if (t1.valid) load_k(t1, k_st1);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();

  // Waves without query rows (possible when the workgroup holds several row blocks) only stage
  // tiles.  Every other wave runs the same straight-line tile body: after the last tile the QK^T of
  // the (absent) next tile reads a stale but finite K stage and is discarded.
  Acc sA[2], sB[2] = {zeroA, zeroA};           // sB is first read after a skipped iteration
  if (wave_rows) {
    float dummy;
    region_a(std::true_type{}, std::false_type{}, k_st0, sA, sB, dummy);   // S^T of tile 0
  }
  __syncthreads();                             // K stage 0 is rewritten by the first iteration

  // One iteration with stage parity S: softmax and PV of t0 (S^T in sc, V in V stage S), QK^T of t1
  // (K in K stage 1 - S, into sn); meanwhile K of t2 lands in K stage S and V of t1 in V stage 1 - S.
  auto step = [&](auto s_c, Acc (&sc)[2], Acc (&sn)[2]) __attribute__((always_inline)) {
    constexpr int S = decltype(s_c)::value;
    uint8_t* const k_fill = S ? k_st1 : k_st0;
    uint8_t* const k_read = S ? k_st0 : k_st1;
    uint8_t* const v_fill = S ? v_st0 : v_st1;
    uint8_t* const v_read = S ? v_st1 : v_st0;
    const TileRef t3 = build();
    if (t2.valid) load_k(t2, k_fill);
    if (t1.valid) load_v(t1, v_fill);
    // A tile holding no row that this wave's head keeps (a chunk kept only by other heads of the
    // workgroup) has every score masked, and its softmax update changes nothing.  When the next tile
    // is such a tile too, the wave skips the iteration's QK^T, softmax and PV (a wave-uniform branch
    // on the scalar tile records); the stale scores it then leaves for the next tile are all
    // overwritten by that tile's mask, which selects -inf for every row.
    if (wave_rows && (t0.nval != 0 || t1.nval != 0)) {
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
          for (int r = 0; r < NA; ++r) o[db][r] *= alpha;
      }
      region_b(v_read);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // this wave's loads have landed before others read them
    __syncthreads();
    t0 = t1; t1 = t2; t2 = t3;
  };
  while (t0.valid) {
    step(ic<0>{}, sA, sB);
    if (!t0.valid) break;
    step(ic<1>{}, sB, sA);
  }

  // ---- epilogue
  if (!wave_rows || tq >= e_i) return;
  const float inv_l = 1.0f / lb_run;
  uint16_t* op = out + ((size_t)tq * Hq + h) * D;
  // O^T block db, accumulator register r: head dim OB db + (32-row waves) 8 (r / 4) + 4 half + r % 4,
  // (16-row waves) 4 half + r
#pragma unroll
  for (int db = 0; db < GE::DBLK; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < NA / 4; ++g4) {
      uint2 w;
      w.x = pack_bf16(o[db][g4 * 4 + 0] * inv_l, o[db][g4 * 4 + 1] * inv_l);
      w.y = pack_bf16(o[db][g4 * 4 + 2] * inv_l, o[db][g4 * 4 + 3] * inv_l);
      *reinterpret_cast<uint2*>(op + db * GE::OB + 8 * g4 + 4 * half) = w;
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
  const int rows_per_block = (GE::NW / hp) * GE::ROWS;
  const int row_tiles = (p.max_chunk_len + rows_per_block - 1) / rows_per_block;
  const int head_slots = G / hp;
  const long long groups = (long long)p.Hkv * p.C;
  // Compact numbering (each XCD's real row tiles only) while the kernel's per-block scan over an XCD's
  // groups stays short; the grid then covers the XCD with the most tiles.  Group g = gk C + (C-1-i)
  // sits on XCD g % 8, so the tiles of the chunks with (C-1-i) % 8 == r land on XCD (gk C + r) % 8.
  const bool compact = (groups + 7) / 8 <= kCompactMaxGroups;
  long long blocks;
  if (compact) {
    long long by_res[8] = {0, 0, 0, 0, 0, 0, 0, 0}, tiles_x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int ci = 0; ci < p.C; ++ci) {
      const int n = p.h_cu_chunks[ci + 1] - p.h_cu_chunks[ci];
      by_res[(p.C - 1 - ci) & 7] += (long long)head_slots * ((n + rows_per_block - 1) / rows_per_block);
    }
    for (int gk = 0; gk < p.Hkv; ++gk)
      for (int r = 0; r < 8; ++r) tiles_x[((long long)gk * p.C + r) & 7] += by_res[r];
    long long tmax = 0;
    for (int x = 0; x < 8; ++x) tmax = std::max(tmax, tiles_x[x]);
    blocks = 8 * tmax;
  } else {
    blocks = (groups + 7) / 8 * 8 * head_slots * row_tiles;
  }
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  auto kern = lse != nullptr ? prefill_bf16_kernel<D, true> : prefill_bf16_kernel<D, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(GE::NT), 0, stream, (const uint16_t*)q, (const uint16_t*)k,
                     (const uint16_t*)v, row_ptr, block_idx, p.cu_chunks, p.seq_chunk_start, (uint16_t*)out, lse,
                     p.B, p.C, p.T, p.Hq, p.Hkv, (long long)nnz, scale, hp, head_slots, row_tiles, compact ? 1 : 0);
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
