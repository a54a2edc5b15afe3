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


// Selection over the scores held in registers (ob[b]: ordered bits of candidate first + 64 b +
// lane, 0 where there is no candidate; a finite score never maps to 0 and every trial value is at
// least 1, so empty slots never count).  NB is the number of batches in use, fixed at compile time
// so the per-bit count is straight-line code.  Writes the row's kk kept chunks, ascending.
template <int NB>
__device__ inline void select_and_write(const uint32_t (&ob)[kSelBatches], int kk, int first, int lane,
                                        int32_t* __restrict__ out) {
  // thr: the largest value with at least kk candidates at or above it, i.e. the kk-th best score
  uint32_t thr = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t t = thr | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b) cnt += __popcll(__ballot(ob[b] >= t));
    if (cnt >= kk) thr = t;
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

}  // namespace sel
}  // namespace dhsa
