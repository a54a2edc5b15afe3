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
// Kernels, in stream order: append (one workgroup per sequence: similarity with
// the previous key row by a block reduction, the cut, the running sums, the
// cache rows); route (one wave per (sequence, row): scores of up to 1024 closed
// chunks in registers, the shared radix top-k, then the kept spans with their
// token offsets); attend (split-K: one wave per (sequence, q head, slice of
// kDecodeSlice kept tokens), or per (sequence, KV group, slice) when routing per
// KV head, so the group's heads read each K/V row once; QK^T with one token per lane reading its key row, online softmax in base
// 2, PV with 16-byte value loads, four rows per instruction for d = 128); combine
// (per (sequence, q head): the slices' partial softmax states).
#include <math.h>

#include <algorithm>

#include "dhsa_internal.hpp"
#include "select.hpp"

namespace dhsa {
namespace {

constexpr int kAppendThreads = 256;
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

// ---------------------------------------------------------------------------------------------- append
template <typename T>
__global__ __launch_bounds__(kAppendThreads) void decode_append_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ k_cache,
    T* __restrict__ v_cache, int32_t* __restrict__ seq_len, int32_t* __restrict__ num_closed,
    int32_t* __restrict__ chunk_start, float* __restrict__ k_sum, float* __restrict__ q_run,
    float* __restrict__ k_run, int32_t* __restrict__ status, int Hq, int Hkv, int d, int L, int Cmax, int lo,
    int hi, float tau) {
  __shared__ float red[3][kAppendThreads / 64];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Wk = Hkv * d, Wq = Hq * d;
  if (status[b] != 0) return;                     // block-uniform: a stopped sequence stays stopped
  const int t = seq_len[b];
  const int nc = num_closed[b];
  const int c0 = chunk_start[(size_t)b * (Cmax + 1) + nc];
  if (t >= L) {                                   // the cache is full
    if (tid == 0) status[b] = 1;
    return;
  }
  const T* kn = k + (size_t)b * Wk;
  const T* vn = v + (size_t)b * Wk;
  const T* qn = q + (size_t)b * Wq;
  T* kc = k_cache + (size_t)b * L * Wk;
  T* vc = v_cache + (size_t)b * L * Wk;
  // cosine with the previous key row
  float dot = 0.f, na = 0.f, nb = 0.f;
  if (t > 0) {
    for (int x = tid; x < Wk; x += kAppendThreads) {
      const float a = to_f(kc[(size_t)(t - 1) * Wk + x]), c = to_f(kn[x]);
      dot = fmaf(a, c, dot);
      na = fmaf(a, a, na);
      nb = fmaf(c, c, nb);
    }
  }
  dot = wave_add(dot);
  na = wave_add(na);
  nb = wave_add(nb);
  if (lane == 0) { red[0][wave] = dot; red[1][wave] = na; red[2][wave] = nb; }
  __syncthreads();
  dot = na = nb = 0.f;
#pragma unroll
  for (int w = 0; w < kAppendThreads / 64; ++w) { dot += red[0][w]; na += red[1][w]; nb += red[2][w]; }
  const float s = (t > 0 && na > 0.f && nb > 0.f) ? dot / (sqrtf(na) * sqrtf(nb)) : 1.0f;
  const int n_open = t - c0;
  const bool cut = t > 0 && ((n_open >= lo && s < tau) || n_open >= hi);
  if (cut && nc + 1 > Cmax) {                     // no room for another closed chunk
    if (tid == 0) status[b] = 2;
    return;
  }
  float* kr = k_run + (size_t)b * Wk;
  float* qr = q_run + (size_t)b * Wq;
  if (cut) {
    const float inv = 1.0f / sqrtf((float)n_open);
    float* ks = k_sum + ((size_t)b * Cmax + nc) * Wk;
    for (int x = tid; x < Wk; x += kAppendThreads) {
      ks[x] = kr[x] * inv;
      kr[x] = to_f(kn[x]);
    }
    for (int x = tid; x < Wq; x += kAppendThreads) qr[x] = to_f(qn[x]);
    if (tid == 0) {
      num_closed[b] = nc + 1;
      chunk_start[(size_t)b * (Cmax + 1) + nc + 1] = t;
    }
  } else {
    for (int x = tid; x < Wk; x += kAppendThreads) kr[x] += to_f(kn[x]);
    for (int x = tid; x < Wq; x += kAppendThreads) qr[x] += to_f(qn[x]);
  }
  for (int x = tid; x < Wk; x += kAppendThreads) {
    kc[(size_t)t * Wk + x] = kn[x];
    vc[(size_t)t * Wk + x] = vn[x];
  }
  if (tid == 0) seq_len[b] = t + 1;
}

// ---------------------------------------------------------------------------------------------- route
// One workgroup (kRouteThreads) per (sequence, row); a row is a q head, or a KV head when routing per
// KV head.  Every thread scores closed chunks (stride kRouteThreads) into LDS; wave 0 then holds the
// scores in registers, selects the top-k and writes the row's kept spans (closed chunks ascending, then
// the open chunk) as int4 (first token, length, tokens before this span, 0), their count and the row's
// total kept tokens.
constexpr int kRouteThreads = 256;

template <int D, bool GROUPED>
__global__ __launch_bounds__(kRouteThreads) void decode_route_kernel(
    const float* __restrict__ q_run, const float* __restrict__ k_sum, const int32_t* __restrict__ seq_len,
    const int32_t* __restrict__ num_closed, const int32_t* __restrict__ chunk_start,
    const int32_t* __restrict__ status, int Hq, int Hkv, int Cmax, int topk, int4* __restrict__ spans,
    int32_t* __restrict__ nspan, int32_t* __restrict__ ntok, int32_t* __restrict__ kept_out) {
  __shared__ __attribute__((aligned(16))) float qv[D];
  __shared__ float scores[sel::kSelCand];
  __shared__ int32_t kl[sel::kSelCand];
  const int R = GROUPED ? Hkv : Hq;
  const int b = blockIdx.x / R, r = blockIdx.x % R, tid = threadIdx.x, lane = tid & 63;
  const int G = Hq / Hkv;
  const int g = GROUPED ? r : r / G;
  const size_t row = (size_t)b * R + r;
  int4* sp = spans + row * (topk + 1);
  if (status[b] != 0) {                           // stopped sequence: nothing to attend (block-uniform)
    if (tid == 0) { nspan[row] = 0; ntok[row] = 0; }
    return;
  }
  const int t_end = seq_len[b];                   // tokens in the cache, the new one included
  const int nc = num_closed[b];
  const int32_t* cs = chunk_start + (size_t)b * (Cmax + 1);
  const int c0 = cs[nc];
  const float inv = 1.0f / sqrtf((float)(t_end - c0));
  for (int x = tid; x < D; x += kRouteThreads) {
    float a;
    if constexpr (GROUPED) {
      a = 0.f;
      for (int hh = 0; hh < G; ++hh) a += q_run[((size_t)b * Hq + g * G + hh) * D + x] * inv;
    } else {
      a = q_run[((size_t)b * Hq + r) * D + x] * inv;
    }
    qv[x] = a;
  }
  __syncthreads();
  const int kk = min(topk, nc);
  if (kk < nc && kk > 0) {
    for (int j = tid; j < nc; j += kRouteThreads) {
      const float4* kr = reinterpret_cast<const float4*>(k_sum + (((size_t)b * Cmax + j) * Hkv + g) * D);
      float acc = 0.f;
#pragma unroll 8
      for (int x = 0; x < D / 4; ++x) {
        const float4 kv = kr[x];
        const float4 q4 = *reinterpret_cast<const float4*>(&qv[4 * x]);
        acc = fmaf(q4.x, kv.x, acc);
        acc = fmaf(q4.y, kv.y, acc);
        acc = fmaf(q4.z, kv.z, acc);
        acc = fmaf(q4.w, kv.w, acc);
      }
      scores[j] = acc;
    }
  }
  __syncthreads();
  if (tid >= 64) return;                          // wave 0 selects and writes
  if (kk == nc) {
    for (int x = lane; x < nc; x += 64) kl[x] = x;
  } else if (kk > 0) {
    uint32_t ob[sel::kSelBatches];
    const int nb = (nc + 63) >> 6;
#pragma unroll
    for (int bt = 0; bt < sel::kSelBatches; ++bt) {
      const int j = 64 * bt + lane;
      ob[bt] = (bt < nb && j < nc) ? sel::ordered_bits(scores[j]) : 0u;
    }
    sel::select_dispatch<1>(nb, ob, kk, 0, lane, kl);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  // spans with exclusive token offsets (a wave scan per 64 spans, carried across batches)
  int carry = 0;
  for (int base = 0; base <= kk; base += 64) {
    const int i = base + lane;
    int start = 0, len = 0;
    if (i < kk) {
      const int j = kl[i];
      start = cs[j];
      len = cs[j + 1] - start;
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
    if (i <= kk) sp[i] = make_int4(start, len, carry + incl - len, 0);
    carry += __shfl(incl, 63);
  }
  if (lane == 0) { nspan[row] = kk + 1; ntok[row] = carry; }
  if (kept_out != nullptr) {                      // the kept closed chunks of every q head of the row
    const int h0 = GROUPED ? g * G : r, nh = GROUPED ? G : 1;
    for (int hh = 0; hh < nh; ++hh)
      for (int x = lane; x < topk; x += 64)
        kept_out[((size_t)b * Hq + h0 + hh) * topk + x] = x < kk ? kl[x] : -1;
  }
}

// ---------------------------------------------------------------------------------------------- attend
// One wave per (sequence, block of GH q heads sharing a kept row, slice of kDecodeSlice kept tokens):
// GH = the group when routing per KV head (its heads read each K/V row once), else 1.  Per 64 tokens
// (one per lane): the lane's key row against the GH queries, an online softmax per head in base 2,
// then PV with 16-byte value loads (RPI rows per instruction, each lane 8 columns of one row).
// Partial state per (sequence, q head, slice): (m, l, o[D]), o not normalised.
template <typename T, int D, bool GROUPED, int GH>
__global__ __launch_bounds__(64) void decode_attend_kernel(
    const T* __restrict__ q, const T* __restrict__ k_cache, const T* __restrict__ v_cache,
    const int4* __restrict__ spans, const int32_t* __restrict__ nspan, const int32_t* __restrict__ ntok,
    int Hq, int Hkv, int L, int topk, int NS, float scale_log2, float* __restrict__ part) {
  constexpr int VEC = 16 / sizeof(T);             // elements per 16-byte load
  constexpr int PARTS = D / 8;                    // 8-element parts of a value row
  constexpr int RPI = 64 / PARTS;                 // value rows per load instruction
  __shared__ float qs[GH][D];
  __shared__ float pbuf[GH][64];
  __shared__ int rowbuf[64];
  __shared__ float ored[64][9];
  const int lane = threadIdx.x;
  const int s = blockIdx.x % NS;
  const int bhb = blockIdx.x / NS;
  const int nhb = Hq / GH;
  const int b = bhb / nhb, h0 = (bhb % nhb) * GH;
  const int G = Hq / Hkv, g = h0 / G;
  const size_t row = (size_t)b * (GROUPED ? Hkv : Hq) + (GROUPED ? g : h0);
  const int n = ntok[row];
  const int lo_tok = s * kDecodeSlice;
  if (lo_tok >= n) return;                        // the combine reads only slices below n
  const int hi_tok = min(n, lo_tok + kDecodeSlice);
  const int ns = nspan[row];
  const int4* sp = spans + row * (topk + 1);
  for (int x = lane; x < GH * D; x += 64)
    qs[x / D][x % D] = to_f(q[((size_t)b * Hq + h0 + x / D) * D + x % D]) * scale_log2;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  const T* kb = k_cache + ((size_t)b * L * Hkv + g) * D;      // row u at kb + u * Hkv * D
  const T* vb = v_cache + ((size_t)b * L * Hkv + g) * D;
  const size_t rs = (size_t)Hkv * D;
  float m[GH], l[GH], o[GH][8];
#pragma unroll
  for (int hh = 0; hh < GH; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
  }
  const int rg = lane / PARTS, pt = lane % PARTS;
  int span_hint = 0;
  for (int blk = lo_tok; blk < hi_tok; blk += 64) {
    const int tok = blk + lane;
    const bool valid = tok < hi_tok;
    // the span holding tok: the last span whose offset is <= tok (binary search from the block's first)
    int lo_s = span_hint, hi_s = ns - 1;
    while (lo_s < hi_s) {
      const int mid = (lo_s + hi_s + 1) >> 1;
      if (sp[mid].z <= tok) lo_s = mid; else hi_s = mid - 1;
    }
    const int4 spn = sp[lo_s];
    const int u = spn.x + (tok - spn.z);
    span_hint = __builtin_amdgcn_readfirstlane(lo_s);   // lane 0 holds the block's lowest token
    float sc[GH];
#pragma unroll
    for (int hh = 0; hh < GH; ++hh) sc[hh] = -INFINITY;
    if (valid) {
      const uint4* kr = reinterpret_cast<const uint4*>(kb + (size_t)u * rs);
      float acc[GH];
#pragma unroll
      for (int hh = 0; hh < GH; ++hh) acc[hh] = 0.f;
#pragma unroll 4
      for (int x = 0; x < D / VEC; ++x) {
        const uint4 raw = kr[x];
        float kf[VEC];
        if constexpr (VEC == 8) {
          const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kf[2 * e] = __uint_as_float(w[e] << 16);
            kf[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
          }
        } else {
          kf[0] = __uint_as_float(raw.x); kf[1] = __uint_as_float(raw.y);
          kf[2] = __uint_as_float(raw.z); kf[3] = __uint_as_float(raw.w);
        }
#pragma unroll
        for (int hh = 0; hh < GH; ++hh)
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[hh] = fmaf(qs[hh][x * VEC + e], kf[e], acc[hh]);
      }
#pragma unroll
      for (int hh = 0; hh < GH; ++hh) sc[hh] = acc[hh];
    }
    rowbuf[lane] = valid ? u : -1;
#pragma unroll
    for (int hh = 0; hh < GH; ++hh) {
      const float m_new = fmaxf(m[hh], wave_max(sc[hh]));
      const float alpha = exp2f(m[hh] - m_new);   // m = -inf on the first block: alpha = 0
      const float p = valid ? exp2f(sc[hh] - m_new) : 0.f;
      l[hh] = l[hh] * alpha + wave_add(p);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[hh][e] *= alpha;
      m[hh] = m_new;
      pbuf[hh][lane] = p;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll 4
    for (int j = 0; j < 64 / RPI; ++j) {
      const int tt = j * RPI + rg;
      const int vr = rowbuf[tt];
      if (vr >= 0) {
        const T* vp = vb + (size_t)vr * rs + pt * 8;
        float vf[8];
        if constexpr (VEC == 8) {
          const uint4 raw = *reinterpret_cast<const uint4*>(vp);
          const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vf[2 * e] = __uint_as_float(w[e] << 16);
            vf[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
          }
        } else {
          const uint4 r0 = *reinterpret_cast<const uint4*>(vp);
          const uint4 r1 = *reinterpret_cast<const uint4*>(vp + 4);
          vf[0] = __uint_as_float(r0.x); vf[1] = __uint_as_float(r0.y); vf[2] = __uint_as_float(r0.z);
          vf[3] = __uint_as_float(r0.w); vf[4] = __uint_as_float(r1.x); vf[5] = __uint_as_float(r1.y);
          vf[6] = __uint_as_float(r1.z); vf[7] = __uint_as_float(r1.w);
        }
#pragma unroll
        for (int hh = 0; hh < GH; ++hh) {
          const float pw = pbuf[hh][tt];
#pragma unroll
          for (int e = 0; e < 8; ++e) o[hh][e] = fmaf(pw, vf[e], o[hh][e]);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
  // per head: sum the RPI row groups of each 8-element part
#pragma unroll
  for (int hh = 0; hh < GH; ++hh) {
#pragma unroll
    for (int e = 0; e < 8; ++e) ored[lane][e] = o[hh][e];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    float* dst = part + (((size_t)b * Hq + h0 + hh) * NS + s) * (D + 2);
    for (int x = lane; x < D; x += 64) {
      const int p8 = x / 8, e = x % 8;
      float acc = 0.f;
      for (int r2 = 0; r2 < RPI; ++r2) acc += ored[r2 * PARTS + p8][e];
      dst[2 + x] = acc;
    }
    if (lane == 0) { dst[0] = m[hh]; dst[1] = l[hh]; }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
}

// ---------------------------------------------------------------------------------------------- combine
// Per (sequence, q head): the slices' weights exp2(m_s - M) from one pass over (m_s, l_s) with wave
// reductions (64 slices at a time), then out = sum_s w_s o_s / sum_s w_s l_s, eight slices' loads in flight.
template <typename T, int D, bool GROUPED>
__global__ __launch_bounds__(64) void decode_combine_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ ntok, const int32_t* __restrict__ status,
    int Hq, int Hkv, int NS, T* __restrict__ out) {
  __shared__ float wgt[kDecodeMaxSlices];
  const int bh = blockIdx.x, lane = threadIdx.x;
  const int b = bh / Hq, h = bh % Hq;
  const int G = Hq / Hkv;
  const size_t row = (size_t)b * (GROUPED ? Hkv : Hq) + (GROUPED ? h / G : h);
  const int n = ntok[row];
  T* op = out + (size_t)bh * D;
  if (status[b] != 0 || n == 0) {                 // stopped sequence: zeros
    for (int x = lane; x < D; x += 64) from_f(0.f, op[x]);
    return;
  }
  const int nsl = (n + kDecodeSlice - 1) / kDecodeSlice;   // <= NS <= kDecodeMaxSlices
  const float* pp = part + (size_t)bh * NS * (D + 2);
  float M = -INFINITY;
  for (int s0 = 0; s0 < nsl; s0 += 64) {
    const int s = s0 + lane;
    M = fmaxf(M, wave_max(s < nsl ? pp[(size_t)s * (D + 2)] : -INFINITY));
  }
  float Lsum = 0.f;
  for (int s0 = 0; s0 < nsl; s0 += 64) {
    const int s = s0 + lane;
    float w = 0.f, l = 0.f;
    if (s < nsl) {
      w = exp2f(pp[(size_t)s * (D + 2)] - M);
      l = pp[(size_t)s * (D + 2) + 1];
      wgt[s] = w;
    }
    Lsum += wave_add(w * l);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  const float inv = 1.0f / Lsum;
  for (int x = lane; x < D; x += 64) {
    float acc = 0.f;
#pragma unroll 8
    for (int s = 0; s < nsl; ++s) acc = fmaf(wgt[s], pp[(size_t)s * (D + 2) + 2 + x], acc);
    from_f(acc * inv, op[x]);
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

template <typename T, int D, bool GROUPED>
hipError_t step_d(const DecodeDims& p, const DecodePtrs& s, const void* q, const void* k, const void* v, int lo,
                  int hi, float tau, int topk, float scale, void* out, int32_t* kept, const DecodeWork& w,
                  hipStream_t stream) {
  hipLaunchKernelGGL(decode_append_kernel<T>, dim3(p.B), dim3(kAppendThreads), 0, stream, (const T*)q, (const T*)k,
                     (const T*)v, (T*)s.k_cache, (T*)s.v_cache, s.seq_len, s.num_closed, s.chunk_start, s.k_sum,
                     s.q_run, s.k_run, s.status, p.Hq, p.Hkv, D, p.L, p.Cmax, lo, hi, tau);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int R = GROUPED ? p.Hkv : p.Hq;
  hipLaunchKernelGGL((decode_route_kernel<D, GROUPED>), dim3(p.B * R), dim3(kRouteThreads), 0, stream, s.q_run, s.k_sum,
                     s.seq_len, s.num_closed, s.chunk_start, s.status, p.Hq, p.Hkv, p.Cmax, topk, w.spans, w.nspan,
                     w.ntok, kept);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // heads per attention wave: the whole group when routing per KV head (each K/V row read once for it)
  const int G = p.Hq / p.Hkv;
  const int gh = !GROUPED ? 1 : (G == 8 ? 8 : G == 4 ? 4 : G == 2 ? 2 : 1);
#define DHSA_ATTEND(GHV)                                                                                         \
  hipLaunchKernelGGL((decode_attend_kernel<T, D, GROUPED, GHV>), dim3(p.B * (p.Hq / GHV) * w.NS), dim3(64), 0,  \
                     stream, (const T*)q, (const T*)s.k_cache, (const T*)s.v_cache, w.spans, w.nspan, w.ntok,     \
                     p.Hq, p.Hkv, p.L, topk, w.NS, scale * kLog2e, w.part)
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
  hipLaunchKernelGGL((decode_combine_kernel<T, D, GROUPED>), dim3(p.B * p.Hq), dim3(64), 0, stream, w.part, w.ntok,
                     s.status, p.Hq, p.Hkv, w.NS, (T*)out);
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

}  // namespace dhsa
