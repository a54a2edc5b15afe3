// Decode on gfx950: one new token per sequence, appended and attended against the kept structure.
//
// The pages evaluate prefill ("Long-Context Modeling with Dynamic Hierarchical
// Sparse Attention for On-Device LLMs", Abstract; ICML 2026 page, Abstract) and
// describe the method as online; decode is the plain online reading of the same
// steps (this library's reading):
//   * the new token t joins the open (last) chunk of its sequence, which starts
//     at c0, unless the chunk-boundary rule cuts before it:
//     (t - c0 >= lo and cos(K[t-1], K[t]) < tau) or t - c0 >= hi; the open chunk
//     then closes and its key summary (sum of its key rows / sqrt(size)) is kept;
//   * routing: the open chunk's query summary so far, (sum of q over c0..t) /
//     sqrt(t - c0 + 1), scores every closed chunk of the sequence; the top-k by
//     (score desc, chunk asc) are kept, plus the open chunk (per query head, or
//     once per KV head with the group's summed query summaries);
//   * attention: exact softmax of the token's query over the tokens of the kept
//     closed chunks and of the open chunk up to t.
//
// Kernels, in stream order: route (one 1024-thread workgroup per (sequence,
// row), a row being a q head or, routed per KV head, a KV head: every workgroup
// takes the append decision from the pre-token state (similarity with the
// previous key row by a block reduction, the cut); the KV head's owner writes
// the cache row and the closing chunk's key summary; scores of the closed
// chunks in LDS, the radix top-k in registers up to 1024 candidates and an
// LDS selection beyond, then the kept spans' cache rows); attend (split-K: one
// wave per (sequence, q head, equal range of the kept tokens), or per
// (sequence, KV group, range) when routing per KV head, so the group's heads
// read each K/V row once; one round of waves fills the GPU; key rows read
// across lanes with the partial dot products summed on the DPP paths, online
// softmax in base 2 with one token per lane, PV with 16-byte value loads); combine (per (sequence, q head): the
// attention waves' partial softmax states, then the append's counters and
// running sums are committed).
#include <math.h>

#include <algorithm>
#include <mutex>

#include "dhsa_internal.hpp"
#include "select.hpp"

// Scratch of dhsa_decode_step_noalloc, for callers that cannot allocate device memory.  Every GPU
// the library runs on holds its own copy of this array from the library's first use there until the
// process ends.  In host code the name stands for a host-side shadow, not a device address: host code
// only ever passes the address that dhsa::decode_noalloc_scratch obtains for the current GPU.
static __device__ __align__(256) uint8_t scratch[dhsa::kNoAllocScratchBytes];

namespace dhsa {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float to_f(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ inline float to_f(float x) { return x; }
__device__ inline uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
__device__ inline void from_f(float f, uint16_t& o) { o = bf16_rne(f); }
__device__ inline void from_f(float f, float& o) { o = f; }

template <int CTRL, int ROW_MASK>
__device__ inline float dpp_get(float v, float fill) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill), __builtin_bit_cast(int, v),
                                                               CTRL, ROW_MASK, 0xF, false));
}
// Reductions over the wave on the DPP paths (quad permutes, half-row and row mirrors, then the row
// broadcasts of lanes 15 and 31 into the later rows); lane 63 ends with the result, which every lane
// reads.  Lanes a broadcast does not reach keep `fill`, the operation's identity.
__device__ inline float wave_add(float x) {
  x += dpp_get<0xB1, 0xF>(x, 0.f);
  x += dpp_get<0x4E, 0xF>(x, 0.f);
  x += dpp_get<0x141, 0xF>(x, 0.f);
  x += dpp_get<0x140, 0xF>(x, 0.f);
  x += dpp_get<0x142, 0xA>(x, 0.f);
  x += dpp_get<0x143, 0xC>(x, 0.f);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
__device__ inline float wave_max(float x) {
  x = fmaxf(x, dpp_get<0xB1, 0xF>(x, -INFINITY));
  x = fmaxf(x, dpp_get<0x4E, 0xF>(x, -INFINITY));
  x = fmaxf(x, dpp_get<0x141, 0xF>(x, -INFINITY));
  x = fmaxf(x, dpp_get<0x140, 0xF>(x, -INFINITY));
  x = fmaxf(x, dpp_get<0x142, 0xA>(x, -INFINITY));
  x = fmaxf(x, dpp_get<0x143, 0xC>(x, -INFINITY));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// ---------------------------------------------------------------------------------------------- route
// Sum over the LS consecutive lanes that read one summary row (LS in {16, 32, 64}) on the DPP paths;
// lane LS - 1 of each group holds the sum.
template <int LS>
__device__ inline float row_sum(float x) {
  x += dpp_get<0xB1, 0xF>(x, 0.f);
  x += dpp_get<0x4E, 0xF>(x, 0.f);
  x += dpp_get<0x141, 0xF>(x, 0.f);
  x += dpp_get<0x140, 0xF>(x, 0.f);
  if constexpr (LS >= 32) x += dpp_get<0x142, 0xA>(x, 0.f);
  if constexpr (LS >= 64) x += dpp_get<0x143, 0xC>(x, 0.f);
  return x;
}

// One workgroup (kRouteThreads) per (sequence, row); a row is a q head, or a KV head when routing per
// KV head.  The workgroup first takes the token's append decision itself (the cosine of the new key
// row with the previous one over every KV head, then the chunking rule), so every workgroup of a
// sequence reads the state as it was before the token and none waits for another: the owner of KV
// head g (the row itself when routing per KV head, else the group's first q head) writes the token's
// cache row and, at a cut, the closed chunk's key summary for head g; every workgroup keeps that
// summary in LDS and scores it from there; the sequence's counters and running sums are committed by
// the combine launch (from the pending record the row-0 workgroup leaves).  Then each wave scores a
// contiguous range of closed chunks into LDS, reading the key summaries across lanes; up to 1024
// closed chunks, wave 0 holds the scores in registers and selects the top-k, beyond that the whole
// workgroup selects (block_select); wave 0 lays out the row's kept spans (closed chunks ascending,
// then the open chunk) with their token offsets, from the chunk table; every wave writes the spans'
// cache rows into the row array, and wave 0 the row's total kept tokens.
constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;

// Top-kk of the n scores in LDS (n up to kDecodeMaxChunks, more than one wave holds in registers) by
// the whole workgroup, in the rule's order (score desc, chunk asc).  Thread tid owns candidates
// tid, tid + 1024, ... (their order-preserving bits are re-read from LDS where needed, which keeps
// the kernel's registers free).  The kk-th best value is found bit by bit from the top with a
// workgroup count per step (wave ballots, one LDS slot per wave, double-buffered by the step's parity
// so one barrier a step suffices); then one pass in chunk order keeps those above it and the first
// ones equal to it.  Writes kl[0 .. kk-1] ascending.  Every thread of the workgroup calls it.
__device__ inline uint32_t cand_bits(const float* scores, int n, int j) {
  return j < n ? sel::ordered_bits(scores[j]) : 0u;   // a finite score never maps to 0
}

__device__ inline int block_total(int (*cnt)[kRouteWaves], int slot, int c, int lane, int wv) {
  if (lane == 0) cnt[slot][wv] = c;
  __syncthreads();
  int tot = 0;
#pragma unroll 1
  for (int w = 0; w < kRouteWaves; ++w) tot += cnt[slot][w];
  return tot;
}

__device__ inline void block_select(const float* scores, int n, int kk, int32_t* kl, int (*cnt)[kRouteWaves],
                                    int tid) {
  const int lane = tid & 63, wv = tid >> 6;
  const int nb = (n + kRouteThreads - 1) / kRouteThreads;   // batches of 1024 candidates in use
  uint32_t thr = 0u;
#pragma unroll 1
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t t = thr | (1u << bit);
    int c = 0;
#pragma unroll 1
    for (int m = 0; m < nb; ++m) c += __popcll(__ballot(cand_bits(scores, n, m * kRouteThreads + tid) >= t));
    if (block_total(cnt, bit & 1, c, lane, wv) >= kk) thr = t;
  }
  int c_above = 0;
#pragma unroll 1
  for (int m = 0; m < nb; ++m) c_above += __popcll(__ballot(cand_bits(scores, n, m * kRouteThreads + tid) > thr));
  // slot 1: the last bit step (bit 0) used slot 0, which slower waves may still be reading
  const int need = kk - block_total(cnt, 1, c_above, lane, wv);     // equal ones to keep
  __syncthreads();                               // every wave has read slot 1 before batches reuse it
  const uint64_t below = (1ull << lane) - 1ull;
  int eq_base = 0, pos_base = 0;
#pragma unroll 1
  for (int m = 0; m < nb; ++m) {
    const int j = m * kRouteThreads + tid;
    const uint32_t x = cand_bits(scores, n, j);
    const bool eq = x == thr;                    // thr >= 1, so only real candidates
    const uint64_t eqm = __ballot(eq);
    if (lane == 0) cnt[0][wv] = __popcll(eqm);
    __syncthreads();
    int eq_before = eq_base + __popcll(eqm & below), eq_tot = 0;
#pragma unroll 1
    for (int w = 0; w < kRouteWaves; ++w) {
      const int cw = cnt[0][w];
      eq_before += w < wv ? cw : 0;
      eq_tot += cw;
    }
    const bool keep = x > thr || (eq && eq_before < need);
    const uint64_t km = __ballot(keep);
    if (lane == 0) cnt[1][wv] = __popcll(km);
    __syncthreads();
    int pos = pos_base + __popcll(km & below), k_tot = 0;
#pragma unroll 1
    for (int w = 0; w < kRouteWaves; ++w) {
      const int cw = cnt[1][w];
      pos += w < wv ? cw : 0;
      k_tot += cw;
    }
    if (keep) kl[pos] = j;
    eq_base += eq_tot;
    pos_base += k_tot;
    __syncthreads();                             // the counts are rewritten by the next batch
  }
}

template <typename T, int D, bool GROUPED>
__global__ __launch_bounds__(kRouteThreads) void decode_route_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ k_cache,
    T* __restrict__ v_cache, float* __restrict__ k_sum, const float* __restrict__ q_run,
    const float* __restrict__ k_run, const int32_t* __restrict__ seq_len, const int32_t* __restrict__ num_closed,
    const int32_t* __restrict__ chunk_start, const int32_t* __restrict__ status, int Hq, int Hkv, int Cmax, int L,
    int topk, int lo, int hi, float tau, int32_t* __restrict__ urow, int32_t* __restrict__ ntok,
    int32_t* __restrict__ kept_out, int4* __restrict__ pend) {
  __shared__ __attribute__((aligned(16))) float qv[D];
  __shared__ __attribute__((aligned(16))) float ksn[D];   // key summary of the chunk this token closes
  __shared__ float red[3][kRouteWaves];
  __shared__ float scores[kDecodeMaxChunks];
  __shared__ int32_t kl[kDecodeMaxTopk];          // the kept closed chunks, ascending
  __shared__ int3 span_lds[kDecodeMaxTopk + 1];
  __shared__ int sel_cnt[2][kRouteWaves];
  const int R = GROUPED ? Hkv : Hq;
  const int b = blockIdx.x / R, r = blockIdx.x % R, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int G = Hq / Hkv;
  const int g = GROUPED ? r : r / G;
  const bool owner = GROUPED || r % G == 0;       // writes KV head g's cache row and closed summary
  const int Wk = Hkv * D, Wq = Hq * D;
  const size_t row = (size_t)b * R + r;
  int32_t* ur = urow + row * (size_t)L;
  // ---- the append decision (block-uniform: every thread sums the same LDS values in the same order)
  const int t = seq_len[b];                       // tokens in the cache before this one
  const int nc0 = num_closed[b];
  const int32_t* cs = chunk_start + (size_t)b * (Cmax + 1);
  const int c00 = cs[nc0];
  int code = status[b] != 0 ? -1 : (t >= L ? 1 : 0);   // -1 stopped before, 1 cache full, 2 table full
  const T* kn = k + (size_t)b * Wk;
  T* kc = k_cache + (size_t)b * L * Wk;
  // this thread's first elements of the previous key row and of the new one, for the similarity
  // (unconditional loads, from the new row's first element where this thread has none, so nothing
  // consumes them before the loads below are issued)
  const bool app = code == 0 && t > 0;
  const bool pld = app && tid < Wk;
  const T pa = *(pld ? kc + (size_t)(t - 1) * Wk + tid : kn);
  const T pc = *(pld ? kn + tid : kn);
  // Loads that do not depend on the append decision go out next, so they are in flight while it is
  // taken: the first batch of this wave's closed-chunk key summaries (read across lanes: LS lanes x 16
  // bytes per summary row, RS rows per load, 16 loads per batch) and this thread's query-sum inputs.
  constexpr int LS = D / 4, RS = 64 / LS;
  const int sr = lane / LS, sp = lane % LS;
  const int per_wave = (nc0 + kRouteThreads / 64 - 1) / (kRouteThreads / 64);
  const int j_lo = wv * per_wave, j_hi = min(nc0, j_lo + per_wave);
  float4 kv[16];
  auto load_sums = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int j = j0 + x * RS + sr;
      kv[x] = j < j_hi ? *reinterpret_cast<const float4*>(k_sum + (((size_t)b * Cmax + j) * Hkv + g) * D + 4 * sp)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  load_sums(j_lo);
  constexpr int QH = GROUPED ? 8 : 1;             // query heads summed into the row's summary, at most
  float qrv[QH];
  T qnv[QH];                                      // (unconditional loads, converted where used)
  const float* qr = q_run + (size_t)b * Wq;
  const T* qn = q + (size_t)b * Wq;
#pragma unroll
  for (int hh = 0; hh < QH; ++hh) {
    const bool in = tid < D && (GROUPED ? hh < G : hh == 0);
    const int y = in ? ((GROUPED ? g * G : r) + hh) * D + tid : 0;
    qrv[hh] = qr[y];
    qnv[hh] = qn[y];
  }
  float dot = 0.f, na = 0.f, nb = 0.f;
  if (app) {
    const float fa = pld ? to_f(pa) : 0.f, fc = pld ? to_f(pc) : 0.f;
    dot = fmaf(fa, fc, dot);
    na = fmaf(fa, fa, na);
    nb = fmaf(fc, fc, nb);
    for (int x = tid + kRouteThreads; x < Wk; x += kRouteThreads) {
      const float a = to_f(kc[(size_t)(t - 1) * Wk + x]), c = to_f(kn[x]);
      dot = fmaf(a, c, dot);
      na = fmaf(a, a, na);
      nb = fmaf(c, c, nb);
    }
  }
  dot = wave_add(dot);
  na = wave_add(na);
  nb = wave_add(nb);
  if (lane == 0) { red[0][wv] = dot; red[1][wv] = na; red[2][wv] = nb; }
  __syncthreads();
  dot = na = nb = 0.f;
#pragma unroll
  for (int w = 0; w < kRouteThreads / 64; ++w) { dot += red[0][w]; na += red[1][w]; nb += red[2][w]; }
  const float sim = (t > 0 && na > 0.f && nb > 0.f) ? dot / (sqrtf(na) * sqrtf(nb)) : 1.0f;
  const int n_open = t - c00;
  const bool cut = code == 0 && t > 0 && ((n_open >= lo && sim < tau) || n_open >= hi);
  if (cut && nc0 + 1 > Cmax) code = 2;
  if (code != 0) {                                // stopped: nothing to attend, the state stays
    if (tid == 0) {
      ntok[row] = 0;
      if (r == 0) pend[b] = make_int4(code, 0, 0, 0);
    }
    return;
  }
  const int nc = nc0 + (cut ? 1 : 0);             // closed chunks with this token
  const int c0 = cut ? t : c00;                   // the open chunk's first token
  const int t_end = t + 1;                        // tokens in the cache, this one included
  if (cut) {
    const float inv_c = 1.0f / sqrtf((float)n_open);
    const float* kr = k_run + ((size_t)b * Hkv + g) * D;
    for (int x = tid; x < D; x += kRouteThreads) {
      const float a = kr[x] * inv_c;
      ksn[x] = a;
      if (owner) k_sum[(((size_t)b * Cmax + nc0) * Hkv + g) * D + x] = a;
    }
  }
  if (owner) {
    const T* vn = v + (size_t)b * Wk;
    T* vc = v_cache + (size_t)b * L * Wk;
    for (int x = tid; x < D; x += kRouteThreads) {
      kc[(size_t)t * Wk + g * D + x] = kn[g * D + x];
      vc[(size_t)t * Wk + g * D + x] = vn[g * D + x];
    }
  }
  if (r == 0 && tid == 0) pend[b] = make_int4(0, cut ? 1 : 0, t, nc0);
  // the open chunk's query summary with this token
  const float inv = 1.0f / sqrtf((float)(t_end - c0));
  if (tid < D) {
    float a = 0.f;
#pragma unroll
    for (int hh = 0; hh < QH; ++hh)
      if (GROUPED ? hh < G : hh == 0) a += (cut ? to_f(qnv[hh]) : qrv[hh] + to_f(qnv[hh])) * inv;
    if constexpr (GROUPED) {                      // groups of more than QH heads: the rest loaded here
      for (int hh = QH; hh < G; ++hh) {
        const int y = (g * G + hh) * D + tid;
        a += (cut ? to_f(qn[y]) : qr[y] + to_f(qn[y])) * inv;
      }
    }
    qv[tid] = a;
  }
  __syncthreads();
  const int kk = min(topk, nc);
  if (kk < nc && kk > 0) {
    // chunks closed before this token: summaries in memory, the first batch already loaded; each
    // lane's partial dot product summed over its row's lanes
    const float4 q4 = *reinterpret_cast<const float4*>(&qv[4 * sp]);
    for (int j0 = j_lo; j0 < j_hi; j0 += 16 * RS) {
      if (j0 != j_lo) load_sums(j0);
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        float a = q4.x * kv[x].x;
        a = fmaf(q4.y, kv[x].y, a);
        a = fmaf(q4.z, kv[x].z, a);
        a = fmaf(q4.w, kv[x].w, a);
        a = row_sum<LS>(a);
        const int j = j0 + x * RS + sr;
        if (sp == LS - 1 && j < j_hi) scores[j] = a;
      }
    }
    if (cut && wv == kRouteThreads / 64 - 1) {   // the chunk this token closes, from LDS, same arithmetic
      const float4 k4 = *reinterpret_cast<const float4*>(&ksn[4 * sp]);
      float a = q4.x * k4.x;
      a = fmaf(q4.y, k4.y, a);
      a = fmaf(q4.z, k4.z, a);
      a = fmaf(q4.w, k4.w, a);
      a = row_sum<LS>(a);
      if (sp == LS - 1 && sr == 0) scores[nc0] = a;
    }
  }
  __syncthreads();
  // more closed chunks than a wave holds in registers: the workgroup selects (kk, nc block-uniform)
  if (kk > 0 && kk < nc && nc > sel::kSelCand) block_select(scores, nc, kk, kl, sel_cnt, tid);
  // Between NBW and kSelCand / 64 batches of 64 candidates, the candidates are first narrowed by several
  // waves at once: wave w finds the kk-th best key among its own NBW batches (chunks 64 NBW w ..), and
  // since the row's kk-th best is at least the largest of these local values L, only keys >= L can be
  // kept.  Those are compacted into LDS in chunk order (so ties keep their order), and wave 0 selects
  // among them exactly as among all: the same kept set.
  constexpr int NBW = 4;
  const bool narrow = kk > 0 && kk < nc && nc > 64 * NBW && nc <= sel::kSelCand;
  uint32_t* cbits = reinterpret_cast<uint32_t*>(scores);           // (the scores are no longer read
  int32_t* cidx = reinterpret_cast<int32_t*>(scores + sel::kSelCand);  // once narrowing has begun)
  int ncand = 0;
  if (narrow) {                                   // block-uniform
    uint32_t x[NBW];
    int nw = 0;
#pragma unroll
    for (int bt = 0; bt < NBW; ++bt) {
      const int j = 64 * (NBW * wv + bt) + lane;
      x[bt] = j < nc ? sel::ordered_bits(scores[j]) : 0u;
      nw += __popcll(__ballot(x[bt] != 0u));
    }
    uint32_t lw = 0u;                             // this wave's kk-th best key (0: fewer than kk here)
    if (nw > kk) {
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t t = lw | (1u << bit);
        int c = 0;
#pragma unroll
        for (int bt = 0; bt < NBW; ++bt) c += __popcll(__ballot(x[bt] >= t));
        if (c >= kk) lw = t;
      }
    }
    if (lane == 0) sel_cnt[0][wv] = (int)lw;
    __syncthreads();
    uint32_t Lb = 0u;
#pragma unroll
    for (int w = 0; w < kRouteWaves; ++w) Lb = max(Lb, (uint32_t)sel_cnt[0][w]);
    uint64_t km[NBW];
    int cw = 0;
#pragma unroll
    for (int bt = 0; bt < NBW; ++bt) {
      km[bt] = __ballot(x[bt] != 0u && x[bt] >= Lb);
      cw += __popcll(km[bt]);
    }
    if (lane == 0) sel_cnt[1][wv] = cw;
    __syncthreads();                              // every wave has read slot 0 and the scores
    int base = 0;
#pragma unroll
    for (int w = 0; w < kRouteWaves; ++w) {
      const int c = sel_cnt[1][w];
      base += w < wv ? c : 0;
      ncand += c;
    }
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int bt = 0; bt < NBW; ++bt) {
      if ((km[bt] >> lane) & 1ull) {
        const int pos = base + __popcll(km[bt] & below);
        cbits[pos] = x[bt];
        cidx[pos] = 64 * (NBW * wv + bt) + lane;
      }
      base += __popcll(km[bt]);
    }
    __syncthreads();
  }
  if (tid < 64) {                                 // wave 0 selects (or finds kl written) and lays out spans
    if (kk == nc) {
      for (int x = lane; x < nc; x += 64) kl[x] = x;
    } else if (kk > 0 && nc <= 64 * NBW) {          // few candidates: wave 0 selects among all directly
      uint32_t ob[sel::kSelBatches];
      const int nb = (nc + 63) >> 6;
#pragma unroll
      for (int bt = 0; bt < sel::kSelBatches; ++bt) {
        const int j = 64 * bt + lane;
        ob[bt] = (bt < nb && j < nc) ? sel::ordered_bits(scores[j]) : 0u;
      }
      sel::select_dispatch<1>(nb, ob, kk, 0, lane, kl);
    } else if (narrow) {
      uint32_t ob[sel::kSelBatches];
      const int nb = (ncand + 63) >> 6;
#pragma unroll
      for (int bt = 0; bt < sel::kSelBatches; ++bt) {
        const int p = 64 * bt + lane;
        ob[bt] = (bt < nb && p < ncand) ? cbits[p] : 0u;
      }
      sel::select_dispatch<1>(nb, ob, kk, 0, lane, kl);   // positions in the candidate list
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      for (int x = lane; x < kk; x += 64) kl[x] = cidx[kl[x]];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // spans with exclusive token offsets (a wave scan per 64 spans, carried across batches)
    int carry = 0;
    for (int base = 0; base <= kk; base += 64) {
      const int i = base + lane;
      int start = 0, len = 0;
      if (i < kk) {                               // closed chunk j: its span from the chunk table;
        const int j = kl[i];                      // the chunk this token closes (j == nc0) ends at t
        start = cs[j];
        len = (j < nc0 ? cs[j + 1] : c0) - start;
      } else if (i == kk) {
        start = c0;
        len = t_end - c0;
      }
      int incl = len;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const int o = __shfl_up(incl, m);
        if (lane >= m) incl += o;
      }
      if (i <= kk) span_lds[i] = make_int3(start, len, carry + incl - len);
      carry += __shfl(incl, 63);
    }
    if (lane == 0) ntok[row] = carry;
  }
  __syncthreads();
  // each span's tokens get their cache rows in the row array, in kept order (a wave per span)
  for (int i = tid >> 6; i <= kk; i += kRouteThreads / 64) {
    const int3 sp3 = span_lds[i];
    for (int y = lane; y < sp3.y; y += 64) ur[sp3.z + y] = sp3.x + y;
  }
  if (tid >= 64) return;
  if (kept_out != nullptr) {                      // the kept closed chunks of every q head of the row
    const int h0 = GROUPED ? g * G : r, nh = GROUPED ? G : 1;
    for (int hh = 0; hh < nh; ++hh)
      for (int x = lane; x < topk; x += 64)
        kept_out[((size_t)b * Hq + h0 + hh) * topk + x] = x < kk ? kl[x] : -1;
  }
}

// ---------------------------------------------------------------------------------------------- attend
// Sum over the LPR consecutive lanes that read one key row (LPR in {8, 16, 32}) on the DPP paths:
// quad permutes, the half-row mirror (8 lanes), the row mirror (16 lanes), then the broadcast of each
// row's lane 15 into the next row (32 lanes: rows 1 and 3).  Lane LPR - 1 of each group holds the sum.
template <int LPR>
__device__ inline float group_sum(float x) {
  x += dpp_get<0xB1, 0xF>(x, 0.f);
  x += dpp_get<0x4E, 0xF>(x, 0.f);
  x += dpp_get<0x141, 0xF>(x, 0.f);
  if constexpr (LPR >= 16) x += dpp_get<0x140, 0xF>(x, 0.f);
  if constexpr (LPR >= 32) x += dpp_get<0x142, 0xA>(x, 0.f);
  return x;
}

// A row of n kept tokens as 64-token blocks, dealt to the grid's nsg >= 1 waves per row in equal runs:
// attend_run blocks per wave, the fewest any split over nsg waves can give the busiest one, and
// attend_waves waves, the fewest that take that run length (the last may take fewer blocks); a row
// with no kept token (a stopped sequence) has none.
__device__ inline int attend_run(int nsg, int n) {
  const int nblk = (n + 63) / 64;
  return (nblk + nsg - 1) / nsg;
}
__device__ inline int attend_waves(int nsg, int n) {
  if (n <= 0) return 0;
  const int nblk = (n + 63) / 64, run = attend_run(nsg, n);
  return (nblk + run - 1) / run;
}

// Split-K attention.  A wave owns (sequence, block of GH q heads sharing a kept row, one contiguous
// range of the row's kept tokens): GH = the group when routing per KV head (its heads read each K/V
// row once), else 1.  The row's n kept tokens, as 64-token blocks, are dealt in equal runs of
// consecutive blocks over at most S waves (S = the grid's waves per row, which the host sizes so that
// the whole grid is resident at once): the busiest wave has as few blocks as S waves allow, and the
// waves end together (fixed slices dealt round robin left the last of several rounds of waves partly
// empty).  A wave takes its range kDecodeSlice tokens at a time.  The kept tokens' cache rows come
// from the routing kernel's row array, loaded once per slice.  Per block of 64 tokens:
//   scores  K rows read across lanes (LPR lanes x 16 bytes per row, RPI rows per instruction, all of
//           a block's loads in flight, the next block's issued with this block's values), each lane's
//           partial dot products summed over its row's lanes on the DPP paths, the row's scores
//           handed through LDS to the token's lane.  bf16: packed dot products of the unscaled
//           queries with the keys as loaded (exact products, fp32 sums), the scale applied to the
//           score, as the prefill kernel does;
//   softmax online per head in base 2, one token per lane; bf16: weights rounded to bf16, and the
//           normaliser sums the rounded weights;
//   PV      16-byte value loads, RPV rows per instruction, each lane 8 columns of one row; bf16: two
//           rows' values repacked into per-column pairs against the two tokens' weights.
// One partial state per (sequence, q head, wave): (m, l, two unused floats, o[D]) over all of the
// wave's slices, o not normalised (o starts 16 bytes into the row, so it is read with 16-byte loads).
template <typename T, int D, bool GROUPED, int GH>
__global__ __launch_bounds__(64) void decode_attend_kernel(
    const T* __restrict__ q, const T* __restrict__ k_cache, const T* __restrict__ v_cache,
    const int32_t* __restrict__ urow, const int32_t* __restrict__ ntok, int Hq, int Hkv, int L, int NSg, int NS,
    float scale_log2, float* __restrict__ part) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int EPL = 16 / sizeof(T);             // elements per 16-byte load
  constexpr int LPR = D / EPL;                    // lanes per key row
  constexpr int RPI = 64 / LPR;                   // key rows per load instruction
  constexpr int NI = 64 / RPI;                    // load instructions per 64-row block
  constexpr int KB = NI < 16 ? NI : 16;           // key loads in flight
  constexpr int PARTS = D / 8;                    // 8-element parts of a value row
  constexpr int RPV = 64 / PARTS;                 // value rows per load instruction
  constexpr int NJV = 64 / RPV;                   // value row steps per 64-row block
  constexpr int VW = 8 / EPL;                     // 16-byte loads per lane and value row (8 columns)
  constexpr int VJB = NJV * VW <= 16 ? NJV : 16 / VW;   // value row steps in flight
  constexpr int NB = kDecodeSlice / 64;           // blocks per slice
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "key rows of 128, 256 or 512 bytes");
  static_assert(VJB % 2 == 0, "value rows are taken in pairs");
  __shared__ float qs[BF ? 1 : GH][D];
  __shared__ float pbuf[GH][64];
  __shared__ __attribute__((aligned(16))) float scb[64][GH];
  __shared__ int rowbuf[NB][64];
  __shared__ float ored[64][9];
  const int lane = threadIdx.x;
  const int s0 = blockIdx.x % NSg;
  const int bhb = blockIdx.x / NSg;
  const int nhb = Hq / GH;
  const int b = bhb / nhb, h0 = (bhb % nhb) * GH;
  const int G = Hq / Hkv, g = h0 / G;
  const size_t row = (size_t)b * (GROUPED ? Hkv : Hq) + (GROUPED ? g : h0);
  const int n = ntok[row];
  if (s0 >= attend_waves(NSg, n)) return;         // the combine reads only those waves' states
  const int run = 64 * attend_run(NSg, n);        // tokens per wave
  const int r_lo = s0 * run, r_hi = min(n, r_lo + run);
  const T* kb = k_cache + ((size_t)b * L * Hkv + g) * D;      // row u at kb + u * Hkv * D
  const T* vb = v_cache + ((size_t)b * L * Hkv + g) * D;
  const size_t rs = (size_t)Hkv * D;
  const uint32_t rsb = (uint32_t)(rs * sizeof(T));            // bytes between consecutive tokens' rows
  // a cache row's key (value) address: one 32 x 32 -> 64-bit multiply-add
  auto row_ptr = [rsb](const T* base, int u) __attribute__((always_inline)) {
    return reinterpret_cast<const uint8_t*>(base) + (uint64_t)(uint32_t)u * rsb;
  };
  const int32_t* ur = urow + row * (size_t)L;
  const int kr = lane / LPR, kp = lane % LPR;     // key row within an instruction, piece of the row
  const int vg = lane / PARTS, vp = lane % PARTS; // value row within an instruction, part of the row
  // this lane's slice of the queries, elements kp * EPL .. + EPL of every head: bf16 pairs as
  // stored (bf16), or scaled floats (fp32)
  uint32_t qpk[GH][4];
  float qreg[GH][EPL];
  if constexpr (BF) {
#pragma unroll
    for (int hh = 0; hh < GH; ++hh) {
      const uint4 w = *reinterpret_cast<const uint4*>(q + ((size_t)b * Hq + h0 + hh) * D + kp * EPL);
      qpk[hh][0] = w.x; qpk[hh][1] = w.y; qpk[hh][2] = w.z; qpk[hh][3] = w.w;
    }
  } else {
    for (int x = lane; x < GH * D; x += 64)
      qs[x / D][x % D] = to_f(q[((size_t)b * Hq + h0 + x / D) * D + x % D]) * scale_log2;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
    for (int hh = 0; hh < GH; ++hh)
#pragma unroll
      for (int e = 0; e < EPL; ++e) qreg[hh][e] = qs[hh][kp * EPL + e];
  }

  // one running softmax state per head across all of this wave's range
  float m[GH], l[GH], o[GH][8];
#pragma unroll
  for (int hh = 0; hh < GH; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
  }
  for (int lo_tok = r_lo; lo_tok < r_hi; lo_tok += kDecodeSlice) {
    const int hi_tok = min(r_hi, lo_tok + kDecodeSlice);
    // the slice's cache rows (-1 past its end), one load per block
#pragma unroll
    for (int bk = 0; bk < NB; ++bk) {
      const int t = lo_tok + 64 * bk + lane;
      rowbuf[bk][lane] = t < hi_tok ? ur[t] : -1;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const int nblk = (hi_tok - lo_tok + 63) / 64;
    uint4 kraw[KB];
    // Loads are unconditional (a load under a per-lane condition costs an exec-mask branch): a row
    // past the slice's end loads the block's first row instead, a kept token, so finite wherever the
    // result is; its score is replaced by -inf and its weight is 0.
    auto issue_k = [&](int bk, int j0) __attribute__((always_inline)) {
      const int r0 = rowbuf[bk][0];
      int uu[KB];
#pragma unroll
      for (int jj = 0; jj < KB; ++jj) uu[jj] = rowbuf[bk][(j0 + jj) * RPI + kr];
#pragma unroll
      for (int jj = 0; jj < KB; ++jj)
        kraw[jj] = *reinterpret_cast<const uint4*>(row_ptr(kb, uu[jj] >= 0 ? uu[jj] : r0) + kp * 16);
    };
    auto score_k = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
      for (int jj = 0; jj < KB; ++jj) {
        float acc[GH];
        if constexpr (BF) {
          const uint32_t kw[4] = {kraw[jj].x, kraw[jj].y, kraw[jj].z, kraw[jj].w};
#pragma unroll
          for (int hh = 0; hh < GH; ++hh) {
            float a = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kw[e]), __builtin_bit_cast(bf16x2, qpk[hh][e]),
                                                  a, false);
            acc[hh] = a;
          }
        } else {
          const float kf[4] = {__uint_as_float(kraw[jj].x), __uint_as_float(kraw[jj].y),
                               __uint_as_float(kraw[jj].z), __uint_as_float(kraw[jj].w)};
#pragma unroll
          for (int hh = 0; hh < GH; ++hh) {
            float a = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) a = fmaf(qreg[hh][e], kf[e], a);
            acc[hh] = a;
          }
        }
#pragma unroll
        for (int hh = 0; hh < GH; ++hh) acc[hh] = group_sum<LPR>(acc[hh]);
        if (kp == LPR - 1) {
          float* dst = &scb[(j0 + jj) * RPI + kr][0];
          if constexpr (GH % 4 == 0) {
#pragma unroll
            for (int hh = 0; hh < GH; hh += 4)
              *reinterpret_cast<float4*>(dst + hh) = make_float4(acc[hh], acc[hh + 1], acc[hh + 2], acc[hh + 3]);
          } else {
#pragma unroll
            for (int hh = 0; hh < GH; ++hh) dst[hh] = acc[hh];
          }
        }
      }
    };
    // value loads: rows j * RPV + vg, VJB row steps in flight (one or two 16-byte loads each)
    uint4 vraw[VJB][VW];
    auto issue_v = [&](int bk, int j0) __attribute__((always_inline)) {
      const int r0 = rowbuf[bk][0];
      int vv[VJB];
#pragma unroll
      for (int jj = 0; jj < VJB; ++jj) vv[jj] = rowbuf[bk][(j0 + jj) * RPV + vg];
#pragma unroll
      for (int jj = 0; jj < VJB; ++jj) {
        const int vr = vv[jj] >= 0 ? vv[jj] : r0;
#pragma unroll
        for (int x = 0; x < VW; ++x)
          vraw[jj][x] = *reinterpret_cast<const uint4*>(row_ptr(vb, vr) + vp * 8 * sizeof(T) + x * 16);
      }
    };
    auto accum_v = [&](int j0) __attribute__((always_inline)) {
      if constexpr (BF) {
#pragma unroll
        for (int jj = 0; jj < VJB; jj += 2) {   // rows ta, tb: column pairs (value of ta, value of tb)
          const int ta = (j0 + jj) * RPV + vg, tb = ta + RPV;
          const uint32_t wa[4] = {vraw[jj][0].x, vraw[jj][0].y, vraw[jj][0].z, vraw[jj][0].w};
          const uint32_t wb[4] = {vraw[jj + 1][0].x, vraw[jj + 1][0].y, vraw[jj + 1][0].z, vraw[jj + 1][0].w};
          uint32_t cp[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            cp[2 * e] = (wa[e] & 0xffffu) | (wb[e] << 16);
            cp[2 * e + 1] = (wa[e] >> 16) | (wb[e] & 0xffff0000u);
          }
#pragma unroll
          for (int hh = 0; hh < GH; ++hh) {
            const bf16x2 pk = {(__bf16)pbuf[hh][ta], (__bf16)pbuf[hh][tb]};   // exact: already bf16 values
#pragma unroll
            for (int e = 0; e < 8; ++e)
              o[hh][e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, cp[e]), pk, o[hh][e], false);
          }
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < VJB; ++jj) {
          const int tt = (j0 + jj) * RPV + vg;
          const float vf[8] = {__uint_as_float(vraw[jj][0].x), __uint_as_float(vraw[jj][0].y),
                               __uint_as_float(vraw[jj][0].z), __uint_as_float(vraw[jj][0].w),
                               __uint_as_float(vraw[jj][1].x), __uint_as_float(vraw[jj][1].y),
                               __uint_as_float(vraw[jj][1].z), __uint_as_float(vraw[jj][1].w)};
#pragma unroll
          for (int hh = 0; hh < GH; ++hh) {
            const float pw = pbuf[hh][tt];       // 0 for rows past the slice
#pragma unroll
            for (int e = 0; e < 8; ++e) o[hh][e] = fmaf(pw, vf[e], o[hh][e]);
          }
        }
      }
    };
    constexpr bool PREF = NI == KB;               // a block's key loads fit in one batch: prefetch them
    if constexpr (PREF) issue_k(0, 0);
    for (int bk = 0; bk < nblk; ++bk) {
      // ---- scores: key rows across lanes
      if constexpr (PREF) {
        score_k(0);
      } else {
#pragma unroll
        for (int j0 = 0; j0 < NI; j0 += KB) {
          issue_k(bk, j0);
          score_k(j0);
        }
      }
      // this block's first value loads and the next block's key loads go out before the softmax
      issue_v(bk, 0);
      if constexpr (PREF) {
        if (bk + 1 < nblk) issue_k(bk + 1, 0);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      // ---- online softmax, one token per lane
      const bool valid = rowbuf[bk][lane] >= 0;
      float scl[GH];
      if constexpr (GH % 4 == 0) {
#pragma unroll
        for (int hh = 0; hh < GH; hh += 4) {
          const float4 v4 = *reinterpret_cast<const float4*>(&scb[lane][hh]);
          scl[hh] = v4.x; scl[hh + 1] = v4.y; scl[hh + 2] = v4.z; scl[hh + 3] = v4.w;
        }
      } else {
#pragma unroll
        for (int hh = 0; hh < GH; ++hh) scl[hh] = scb[lane][hh];
      }
#pragma unroll
      for (int hh = 0; hh < GH; ++hh) {
        const float sc = valid ? (BF ? scl[hh] * scale_log2 : scl[hh]) : -INFINITY;
        const float m_new = fmaxf(m[hh], wave_max(sc));
        const float alpha = exp2f(m[hh] - m_new);   // m = -inf on the first block: alpha = 0
        float p = valid ? exp2f(sc - m_new) : 0.f;
        if constexpr (BF) p = to_f(bf16_rne(p));
        l[hh] = l[hh] * alpha + wave_add(p);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] *= alpha;
        m[hh] = m_new;
        pbuf[hh][lane] = p;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      // ---- PV
      accum_v(0);
#pragma unroll
      for (int j0 = VJB; j0 < NJV; j0 += VJB) {
        issue_v(bk, j0);
        accum_v(j0);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
  }
  // per head: sum the RPV row groups of each 8-element part; the wave's partial state goes to slot s0
#pragma unroll
  for (int hh = 0; hh < GH; ++hh) {
#pragma unroll
    for (int e = 0; e < 8; ++e) ored[lane][e] = o[hh][e];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    float* dst = part + (((size_t)b * Hq + h0 + hh) * NS + s0) * (D + kPartHead);
    for (int x = lane; x < D; x += 64) {
      const int p8 = x / 8, e = x % 8;
      float acc = 0.f;
      for (int r2 = 0; r2 < RPV; ++r2) acc += ored[r2 * PARTS + p8][e];
      dst[kPartHead + x] = acc;
    }
    if (lane == 0) { dst[0] = m[hh]; dst[1] = l[hh]; }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
}

// ---------------------------------------------------------------------------------------------- combine
// Per (sequence, q head), one workgroup of 256 threads: the slices' (m_s, l_s), one slice per thread,
// their weights exp2(m_s - M) by block reductions; then out = sum_s w_s o_s / sum_s w_s l_s, each thread
// summing one 4-column group of o over every (256 / (D / 4))-th slice with 16-byte loads, the groups'
// row sums added through LDS.
constexpr int kCombineThreads = 256;
template <typename T, int D, bool GROUPED>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ ntok, int Hq, int Hkv, int NS, int NSg,
    T* __restrict__ out,
    const T* __restrict__ q, const T* __restrict__ k, const int4* __restrict__ pend, int Cmax,
    int32_t* __restrict__ seq_len, int32_t* __restrict__ num_closed, int32_t* __restrict__ chunk_start,
    float* __restrict__ q_run, float* __restrict__ k_run, int32_t* __restrict__ status) {
  constexpr int NT = kCombineThreads, NWV = NT / 64;
  constexpr int C4 = D / 4;                       // 4-column groups of a row
  constexpr int SPR = NT / C4;                    // slices summed side by side
  constexpr int RS = D + kPartHead;               // floats per partial state
  static_assert(kDecodeGridSlices <= NT, "one slice per thread for the weights");
  __shared__ float wgt[kDecodeGridSlices];
  __shared__ float red[2][NWV];
  __shared__ float4 acc4[SPR][C4];
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int b = bh / Hq, h = bh % Hq;
  const int G = Hq / Hkv;
  const size_t row = (size_t)b * (GROUPED ? Hkv : Hq) + (GROUPED ? h / G : h);
  const int n = ntok[row];
  T* op = out + (size_t)bh * D;
  // The partial states are loaded before the row's token count is known: the grid's NSg slots of the
  // row, of which only the first attend_waves(NSg, n) were written this step.  The others hold stale
  // (or, before a first step, arbitrary) values, which are selected away below, never used in
  // arithmetic.  Thread (r, c) sums columns 4c .. 4c + 3 of slots r, r + SPR, ..., four in flight.
  const float* pp = part + (size_t)bh * NS * RS;
  const float m_raw = tid < NSg ? pp[(size_t)tid * RS] : -INFINITY;
  const float l_raw = tid < NSg ? pp[(size_t)tid * RS + 1] : 0.f;
  const int c = tid % C4, r = tid / C4;
  float4 v[4];
  auto load_o = [&](int s0, int lim) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sl = s0 + j * SPR;
      v[j] = sl < lim ? *reinterpret_cast<const float4*>(pp + (size_t)sl * RS + kPartHead + 4 * c)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  load_o(r, NSg);
  // commit the token's append to the state (no other kernel of the step reads these fields after the
  // routing launch): this head's query sum, the KV head's key sum (first head of its group), the
  // sequence's counters (head 0)
  const int4 pd = pend[b];
  if (pd.x == 0) {
    const bool cut = pd.y != 0;
    float* qr = q_run + (size_t)bh * D;
    const T* qn = q + (size_t)bh * D;
    for (int x = tid; x < D; x += NT) qr[x] = cut ? to_f(qn[x]) : qr[x] + to_f(qn[x]);
    if (h % G == 0) {
      float* kr = k_run + ((size_t)b * Hkv + h / G) * D;
      const T* kn = k + ((size_t)b * Hkv + h / G) * D;
      for (int x = tid; x < D; x += NT) kr[x] = cut ? to_f(kn[x]) : kr[x] + to_f(kn[x]);
    }
    if (h == 0 && tid == 0) {
      seq_len[b] = pd.z + 1;
      if (cut) {
        num_closed[b] = pd.w + 1;
        chunk_start[(size_t)b * (Cmax + 1) + pd.w + 1] = pd.z;
      }
    }
  } else if (pd.x > 0 && h == 0 && tid == 0) {
    status[b] = pd.x;
  }
  if (n == 0) {                                   // stopped sequence (no kept token): zeros
    for (int x = tid; x < D; x += NT) from_f(0.f, op[x]);
    return;
  }
  // partial states: one per attention wave with tokens (the row's first attend_waves(NSg, n) waves)
  const int nsl = attend_waves(NSg, n);           // <= NSg <= NS <= kDecodeGridSlices
  const float m0 = tid < nsl ? m_raw : -INFINITY;
  const float l0 = tid < nsl ? l_raw : 0.f;
  float M = wave_max(m0);
  if (lane == 0) red[0][wv] = M;
  __syncthreads();
#pragma unroll
  for (int x = 0; x < NWV; ++x) M = fmaxf(M, red[0][x]);
  const float w = tid < nsl ? exp2f(m0 - M) : 0.f;
  if (tid < nsl) wgt[tid] = w;
  float Ls = wave_add(w * l0);
  if (lane == 0) red[1][wv] = Ls;
  __syncthreads();
  Ls = 0.f;
#pragma unroll
  for (int x = 0; x < NWV; ++x) Ls += red[1][x];     // same order in every thread
  const float inv = 1.0f / Ls;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = r; s0 < nsl; s0 += 4 * SPR) {
    if (s0 != r) load_o(s0, nsl);
    float ww[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sl = s0 + j * SPR;
      ww[j] = sl < nsl ? wgt[sl] : 0.f;
      if (sl >= nsl) v[j] = make_float4(0.f, 0.f, 0.f, 0.f);   // a stale slot of the first batch
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a.x = fmaf(ww[j], v[j].x, a.x);
      a.y = fmaf(ww[j], v[j].y, a.y);
      a.z = fmaf(ww[j], v[j].z, a.z);
      a.w = fmaf(ww[j], v[j].w, a.w);
    }
  }
  acc4[r][c] = a;
  __syncthreads();
  if (tid < C4) {
    float4 t = acc4[0][tid];
#pragma unroll
    for (int x = 1; x < SPR; ++x) {
      const float4 u = acc4[x][tid];
      t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
    }
    from_f(t.x * inv, op[4 * tid]);
    from_f(t.y * inv, op[4 * tid + 1]);
    from_f(t.z * inv, op[4 * tid + 2]);
    from_f(t.w * inv, op[4 * tid + 3]);
  }
}

// ---------------------------------------------------------------------------------------------- load
// Prefix of a chunked batch (THD, global chunk ids) into the state: cache rows, then per chunk its key
// summary (closed chunks) or the running sums (a sequence's last chunk, which stays open).
template <typename T>
__global__ __launch_bounds__(256) void decode_load_rows_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ cu_seqlens, int B, int T_tok,
    int W, int L, T* __restrict__ k_cache, T* __restrict__ v_cache) {
  const size_t total = (size_t)T_tok * W;
  for (size_t x = (size_t)blockIdx.x * 256 + threadIdx.x; x < total; x += (size_t)gridDim.x * 256) {
    const int t = (int)(x / W), c = (int)(x % W);
    int lo = 0, hi = B - 1;                       // the sequence of token t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cu_seqlens[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const size_t dst = ((size_t)lo * L + (t - cu_seqlens[lo])) * W + c;
    k_cache[dst] = k[x];
    v_cache[dst] = v[x];
  }
}

template <typename T>
__global__ __launch_bounds__(256) void decode_load_sums_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const int32_t* __restrict__ cu_chunks,
    const int32_t* __restrict__ seq_chunk_start, int B, int Wq, int Wk, int Cmax, float* __restrict__ k_sum,
    float* __restrict__ q_run, float* __restrict__ k_run) {
  const int c = blockIdx.y;                       // global chunk id
  int lo = 0, hi = B - 1;                         // its sequence (the last b with seq_chunk_start[b] <= c)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seq_chunk_start[mid] <= c) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int j = c - seq_chunk_start[b];
  const bool open = c == seq_chunk_start[b + 1] - 1;
  const int s = cu_chunks[c], e = cu_chunks[c + 1];
  const int x = blockIdx.x * 256 + threadIdx.x;   // column over Wk (k) then Wq (q, open chunks only)
  if (x < Wk) {
    float acc = 0.f;
    for (int t = s; t < e; ++t) acc += to_f(k[(size_t)t * Wk + x]);
    if (open) k_run[(size_t)b * Wk + x] = acc;
    else k_sum[((size_t)b * Cmax + j) * Wk + x] = acc * (1.0f / sqrtf((float)(e - s)));
  } else if (open && x < Wk + Wq) {
    const int y = x - Wk;
    float acc = 0.f;
    for (int t = s; t < e; ++t) acc += to_f(q[(size_t)t * Wq + y]);
    q_run[(size_t)b * Wq + y] = acc;
  }
}

__global__ __launch_bounds__(64) void decode_load_counters_kernel(
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ cu_chunks,
    const int32_t* __restrict__ seq_chunk_start, int B, int Cmax, int Wq, int Wk, int32_t* __restrict__ seq_len,
    int32_t* __restrict__ num_closed, int32_t* __restrict__ chunk_start, float* __restrict__ q_run,
    float* __restrict__ k_run, int32_t* __restrict__ status) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int nch = seq_chunk_start[b + 1] - seq_chunk_start[b];
  const int closed = nch > 0 ? nch - 1 : 0;
  for (int j = lane; j <= closed; j += 64)
    chunk_start[(size_t)b * (Cmax + 1) + j] = nch > 0 ? cu_chunks[seq_chunk_start[b] + j] - cu_seqlens[b] : 0;
  if (nch == 0) {                                 // empty prefix: no open chunk yet, zero sums
    for (int x = lane; x < Wq; x += 64) q_run[(size_t)b * Wq + x] = 0.f;
    for (int x = lane; x < Wk; x += 64) k_run[(size_t)b * Wk + x] = 0.f;
  }
  if (lane == 0) {
    seq_len[b] = cu_seqlens[b + 1] - cu_seqlens[b];
    num_closed[b] = closed;
    status[b] = 0;
  }
}

// Single-wave workgroups of the attention kernel <T, D, GROUPED, GH> that the current GPU holds at once
// (its compute units times the occupancy the kernel's registers and LDS allow), looked up once per GPU;
// 0 when the runtime cannot say.
template <typename T, int D, bool GROUPED, int GH>
int attend_resident_waves() {
  static std::mutex mu;
  static int cache[kNoAllocMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocMaxDevices) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_attend_kernel<T, D, GROUPED, GH>, 64, 0) !=
        hipSuccess)
      return 0;
    cache[dev] = std::max(0, cus * per_cu);
  }
  return cache[dev];
}

template <typename T, int D, bool GROUPED>
hipError_t step_d(const DecodeDims& p, const DecodePtrs& s, const void* q, const void* k, const void* v, int lo,
                  int hi, float tau, int topk, float scale, void* out, int32_t* kept, const DecodeWork& w,
                  hipStream_t stream) {
  const int R = GROUPED ? p.Hkv : p.Hq;
  hipLaunchKernelGGL((decode_route_kernel<T, D, GROUPED>), dim3(p.B * R), dim3(kRouteThreads), 0, stream,
                     (const T*)q, (const T*)k, (const T*)v, (T*)s.k_cache, (T*)s.v_cache, s.k_sum, s.q_run, s.k_run,
                     s.seq_len, s.num_closed, s.chunk_start, s.status, p.Hq, p.Hkv, p.Cmax, p.L, topk, lo, hi, tau,
                     w.urow, w.ntok, kept, (int4*)w.pend);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // heads per attention wave: the whole group when routing per KV head (each K/V row read once for it)
  const int G = p.Hq / p.Hkv;
  const int gh = !GROUPED ? 1 : (G == 8 ? 8 : G == 4 ? 4 : G == 2 ? 2 : 1);
  // Waves per row: as many as the GPU holds at once over all rows (one round of waves, each with an
  // equal share of its row), but no more than 64-token blocks in a row of kept chunks of up to hi
  // tokens, nor than the workspace's partial states per row.  (Rows longer than that bound, e.g. from
  // a prefix chunked otherwise, only give each wave a longer range.)
  const long long need = ((long long)(topk + 1) * hi + 63) / 64;
  int NSg = 1;
  auto waves_per_row = [&](int gh_v, int resident) {
    const long long rows = (long long)p.B * (p.Hq / gh_v);
    const long long fit = resident > 0 ? resident / rows : need;
    return (int)std::max(1LL, std::min<long long>({(long long)w.NS, need, fit}));
  };
#define DHSA_ATTEND(GHV)                                                                                         \
  do {                                                                                                           \
    NSg = waves_per_row(GHV, attend_resident_waves<T, D, GROUPED, GHV>());                                      \
    hipLaunchKernelGGL((decode_attend_kernel<T, D, GROUPED, GHV>), dim3(p.B * (p.Hq / GHV) * NSg), dim3(64), 0, \
                       stream, (const T*)q, (const T*)s.k_cache, (const T*)s.v_cache, w.urow, w.ntok, p.Hq,     \
                       p.Hkv, p.L, NSg, w.NS, scale * kLog2e, w.part);                                          \
  } while (0)
  if constexpr (GROUPED) {
    if (gh == 8) DHSA_ATTEND(8);
    else if (gh == 4) DHSA_ATTEND(4);
    else if (gh == 2) DHSA_ATTEND(2);
    else DHSA_ATTEND(1);
  } else {
    DHSA_ATTEND(1);
  }
#undef DHSA_ATTEND
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL((decode_combine_kernel<T, D, GROUPED>), dim3(p.B * p.Hq), dim3(kCombineThreads), 0, stream,
                     w.part, w.ntok,
                     p.Hq, p.Hkv, w.NS, NSg, (T*)out, (const T*)q, (const T*)k, (const int4*)w.pend, p.Cmax,
                     s.seq_len,
                     s.num_closed, s.chunk_start, s.q_run, s.k_run, s.status);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t step_g(const DecodeDims& p, const DecodePtrs& s, const void* q, const void* k, const void* v, int lo,
                  int hi, float tau, int topk, bool grouped, float scale, void* out, int32_t* kept,
                  const DecodeWork& w, hipStream_t stream) {
  return grouped ? step_d<T, D, true>(p, s, q, k, v, lo, hi, tau, topk, scale, out, kept, w, stream)
                 : step_d<T, D, false>(p, s, q, k, v, lo, hi, tau, topk, scale, out, kept, w, stream);
}

template <typename T>
hipError_t load_t(const DecodeDims& p, const DecodePtrs& s, const Plan& pl, const void* q, const void* k,
                  const void* v, hipStream_t stream) {
  const int Wk = p.Hkv * p.d, Wq = p.Hq * p.d;
  hipLaunchKernelGGL(decode_load_counters_kernel, dim3(p.B), dim3(64), 0, stream, pl.cu_seqlens, pl.cu_chunks,
                     pl.seq_chunk_start, p.B, p.Cmax, Wq, Wk, s.seq_len, s.num_closed, s.chunk_start, s.q_run,
                     s.k_run, s.status);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || pl.T == 0) return err;
  const size_t total = (size_t)pl.T * Wk;
  const unsigned grid = (unsigned)std::min<size_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(decode_load_rows_kernel<T>, dim3(grid), dim3(256), 0, stream, (const T*)k, (const T*)v,
                     pl.cu_seqlens, p.B, pl.T, Wk, p.L, (T*)s.k_cache, (T*)s.v_cache);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(decode_load_sums_kernel<T>, dim3((Wk + Wq + 255) / 256, pl.C), dim3(256), 0, stream,
                     (const T*)q, (const T*)k, pl.cu_chunks, pl.seq_chunk_start, p.B, Wq, Wk, p.Cmax, s.k_sum,
                     s.q_run, s.k_run);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_step(const DecodeDims& p, const DecodePtrs& s, const void* q, const void* k, const void* v,
                              int lo, int hi, float tau, int topk, bool grouped, float scale, void* out,
                              int32_t* kept, const DecodeWork& w, hipStream_t stream) {
  if (p.dtype == 1) {
    switch (p.d) {
      case 64: return step_g<uint16_t, 64>(p, s, q, k, v, lo, hi, tau, topk, grouped, scale, out, kept, w, stream);
      case 128: return step_g<uint16_t, 128>(p, s, q, k, v, lo, hi, tau, topk, grouped, scale, out, kept, w, stream);
      case 256: return step_g<uint16_t, 256>(p, s, q, k, v, lo, hi, tau, topk, grouped, scale, out, kept, w, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (p.d) {
    case 64: return step_g<float, 64>(p, s, q, k, v, lo, hi, tau, topk, grouped, scale, out, kept, w, stream);
    case 128: return step_g<float, 128>(p, s, q, k, v, lo, hi, tau, topk, grouped, scale, out, kept, w, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_load(const DecodeDims& p, const DecodePtrs& s, const Plan& pl, const void* q, const void* k,
                              const void* v, hipStream_t stream) {
  return p.dtype == 1 ? load_t<uint16_t>(p, s, pl, q, k, v, stream) : load_t<float>(p, s, pl, q, k, v, stream);
}

hipError_t decode_noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kNoAllocMaxDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void* addr[kNoAllocMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {                     // first use on this GPU, which is current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace dhsa
