// Top-k selection over scores held in registers, shared by the routing kernels (prefill and
// decode).  A wave holds up to kSelCand candidate scores, 64 per register (candidate 64 b + lane in
// ob[b]), as order-preserving 32-bit keys (the fp32 order, -0 equal to +0; 0 marks an empty slot).
// The k-th best key is found by a most-significant-bit-first binary search (each step counts the
// candidates at or above a trial value with wave ballots), and one pass in candidate order writes
// those above it plus the first ones equal to it: the (score desc, index asc) top-k, ascending.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dhsa {
namespace sel {

constexpr int kSelCand = 1024;                    // candidates held in registers
constexpr int kSelBatches = kSelCand / 64;        // 64 per batch, one per lane

__device__ inline uint32_t ordered_bits(float s) {
  uint32_t u = (s == 0.0f) ? 0u : __float_as_uint(s);   // -0 and +0 rank equal
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}


// Sum of x over the wave on the DPP paths (the total lands in lane 63, read back for every lane).
__device__ inline int wave_sum_i32(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  x += __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);  // row_half_mirror
  x += __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false);  // row_mirror
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return __builtin_amdgcn_readlane(x, 63);
}

// Selection over the scores held in registers (ob[b]: ordered bits of candidate first + 64 b +
// lane, 0 where there is no candidate; a finite score never maps to 0 and every trial value is at
// least 1, so empty slots never count).  NB is the number of batches in use, fixed at compile time
// so the per-bit count is straight-line code.  Writes the row's kk kept chunks, ascending.
template <int NB>
__device__ inline void select_and_write(const uint32_t (&ob)[kSelBatches], int kk, int first, int lane,
                                        int32_t* __restrict__ out) {
  // thr: the largest value with at least kk candidates at or above it, i.e. the kk-th best score.
  // Few batches: one bit per step, counted with a ballot and popcount per batch.  From four batches on
  // the steps' dependency chain (count, wave sum, threshold) is what costs, so a step settles two bits:
  // the counts at thr | 01, thr | 10 and thr | 11 (per-lane vector counts, three wave sums in flight)
  // are monotone, and the largest trial value that keeps kk candidates is the one the bit-by-bit
  // search would reach.
  uint32_t thr = 0u;
  if constexpr (NB >= 4) {
    for (int bit = 30; bit >= 0; bit -= 2) {
      const uint32_t t1 = thr | (1u << bit), t2 = thr | (2u << bit), t3 = thr | (3u << bit);
      int c1 = 0, c2 = 0, c3 = 0;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        c1 += ob[b] >= t1 ? 1 : 0;
        c2 += ob[b] >= t2 ? 1 : 0;
        c3 += ob[b] >= t3 ? 1 : 0;
      }
      c1 = wave_sum_i32(c1);
      c2 = wave_sum_i32(c2);
      c3 = wave_sum_i32(c3);
      thr = c3 >= kk ? t3 : (c2 >= kk ? t2 : (c1 >= kk ? t1 : thr));
    }
  } else {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t t = thr | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int b = 0; b < NB; ++b) cnt += __popcll(__ballot(ob[b] >= t));
      if (cnt >= kk) thr = t;
    }
  }
  // Write in chunk order those above thr, then the first ones equal to it until kk are written.
  int above = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b) above += __popcll(__ballot(ob[b] > thr));
  const int need = kk - above;
  const uint64_t below = (1ull << lane) - 1ull;
  int pos = 0, eq_seen = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const bool eq = ob[b] == thr;              // thr >= 1, so only real candidates
    const uint64_t eqm = __ballot(eq);
    const bool keep = ob[b] > thr || (eq && eq_seen + __popcll(eqm & below) < need);
    eq_seen += __popcll(eqm);
    const uint64_t km = __ballot(keep);
    if (keep) out[pos + __popcll(km & below)] = first + 64 * b + lane;
    pos += __popcll(km);
  }
}

template <int NB>
__device__ inline void select_dispatch(int nb, const uint32_t (&ob)[kSelBatches], int kk, int first, int lane,
                                       int32_t* __restrict__ out) {
  if constexpr (NB > kSelBatches) {
    return;
  } else {
    if (nb == NB) select_and_write<NB>(ob, kk, first, lane, out);
    else select_dispatch<NB + 1>(nb, ob, kk, first, lane, out);
  }
}

// Token-budget selection: keep the longest prefix of the (score desc, index asc) ranking whose lengths
// (len[b] for candidate 64 b + lane, 0 for an empty slot) sum to at most `budget`.  With 64-bit keys
// K = (ordered score bits << 32) | ~index (distinct; larger = better ranked; 0 marks an empty slot),
// the kept set is {K >= X} for X the smallest value whose at-or-above length sum fits; X is found
// bit by bit from the top: bit b stays 0 when the largest value with that bit 0 (lower bits all 1)
// still fits.  Writes the kept indices ascending (first + 64 b + lane) and returns how many.
template <int NB>
__device__ inline int select_tokens_and_write(const uint32_t (&ob)[kSelBatches], const int (&len)[kSelBatches],
                                              int budget, int first, int lane, int32_t* __restrict__ out) {
  // Keys (score bits : complemented chunk id) order the candidates by the ranking; the kept set is
  // every key >= X for the smallest X whose kept lengths fit the budget.  The search runs over the
  // 32 score bits first, with one 64-bit compare per candidate: (score bits << 1) | [low word all
  // ones, i.e. chunk 0] against (threshold << 1) | 1 (empty slots are 0 and never pass); then, when
  // several candidates tie the chosen score bits, over the chunk bits among them.  A single tied
  // candidate is kept when it fits beside everything above it.
  uint32_t lo[NB];
  uint64_t k1[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    lo[b] = 0xFFFFFFFFu - (uint32_t)(first + 64 * b + lane);
    k1[b] = ob[b] != 0u ? (((uint64_t)ob[b] << 1) | (lo[b] == 0xFFFFFFFFu ? 1ull : 0ull)) : 0ull;
  }
  uint32_t Xh = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint64_t t1 = ((uint64_t)(Xh | ((1u << bit) - 1u)) << 1) | 1ull;
    int part = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b) part += k1[b] >= t1 ? len[b] : 0;
    if (wave_sum_i32(part) > budget) Xh |= 1u << bit;
  }
  // lengths above the chosen score bits, and the candidates that tie them
  int above = 0, tie_len = 0, ntied = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const bool tie = ob[b] != 0u && ob[b] == Xh;
    above += (ob[b] != 0u && ob[b] > Xh) ? len[b] : 0;
    tie_len += tie ? len[b] : 0;
    ntied += __popcll(__ballot(tie));
  }
  above = wave_sum_i32(above);
  uint32_t Xl = 0u;
  if (ntied == 1) {
    Xl = above + wave_sum_i32(tie_len) <= budget ? 0u : 0xFFFFFFFFu;   // keep it, or not (its low word < ~0)
  } else if (ntied > 1) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t xl = Xl | ((1u << bit) - 1u);
      int part = 0;
#pragma unroll
      for (int b = 0; b < NB; ++b) part += (ob[b] != 0u && ob[b] == Xh && lo[b] >= xl) ? len[b] : 0;
      if (above + wave_sum_i32(part) > budget) Xl |= 1u << bit;
    }
  }
  const uint64_t below = (1ull << lane) - 1ull;
  int pos = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const bool keep = ob[b] != 0u && (ob[b] > Xh || (ob[b] == Xh && lo[b] >= Xl));
    const uint64_t km = __ballot(keep);
    if (keep) out[pos + __popcll(km & below)] = first + 64 * b + lane;
    pos += __popcll(km);
  }
  return pos;
}

template <int NB>
__device__ inline int select_tokens_dispatch(int nb, const uint32_t (&ob)[kSelBatches], const int (&len)[kSelBatches],
                                             int budget, int first, int lane, int32_t* __restrict__ out) {
  if constexpr (NB > kSelBatches) {
    return 0;
  } else {
    if (nb == NB) return select_tokens_and_write<NB>(ob, len, budget, first, lane, out);
    return select_tokens_dispatch<NB + 1>(nb, ob, len, budget, first, lane, out);
  }
}

}  // namespace sel
}  // namespace dhsa
