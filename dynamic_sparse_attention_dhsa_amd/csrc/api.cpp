// C ABI of the DHSA sparse-prefill library: host-side validation, planning
// and dispatch to the gfx950 kernels.  Nothing here allocates device memory or
// synchronises; every failure is reported before any kernel is enqueued.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "dhsa_internal.hpp"

using dhsa::Plan;

namespace {

bool head_dim_supported(int32_t dtype, int32_t d) {
  if (dtype == DHSA_BF16) return d == 64 || d == 128 || d == 256;
  if (dtype == DHSA_F32) return d == 32 || d == 64 || d == 128;
  return false;
}

// Validates the layout from its host mirrors and fills `plan`.
dhsa_status check_layout(const dhsa_layout* L, Plan* plan) {
  if (L == nullptr) return DHSA_ERR_NULL_ARG;
  if (L->num_seqs < 0 || L->total_tokens < 0 || L->total_chunks < 0 || L->num_q_heads < 1 ||
      L->num_kv_heads < 1 || L->head_dim < 1)
    return DHSA_ERR_BAD_SHAPE;
  if (L->num_q_heads % L->num_kv_heads != 0) return DHSA_ERR_BAD_SHAPE;
  if (L->dtype != DHSA_F32 && L->dtype != DHSA_BF16) return DHSA_ERR_UNSUPPORTED;
  if (!head_dim_supported(L->dtype, L->head_dim)) return DHSA_ERR_UNSUPPORTED;
  if (L->h_cu_seqlens == nullptr || L->h_cu_chunks == nullptr || L->h_seq_chunk_start == nullptr)
    return DHSA_ERR_NULL_ARG;
  if (L->cu_seqlens == nullptr || L->cu_chunks == nullptr || L->seq_chunk_start == nullptr)
    return DHSA_ERR_NULL_ARG;
  const int32_t B = L->num_seqs, C = L->total_chunks, T = L->total_tokens;
  const int32_t* cs = L->h_cu_seqlens;
  const int32_t* cc = L->h_cu_chunks;
  const int32_t* sc = L->h_seq_chunk_start;
  if (cs[0] != 0 || sc[0] != 0 || cc[0] != 0) return DHSA_ERR_BAD_LAYOUT;
  if (cs[B] != T || sc[B] != C || cc[C] != T) return DHSA_ERR_BAD_LAYOUT;
  int32_t max_len = 0, max_per_seq = 0;
  for (int32_t c = 0; c < C; ++c) {
    const int32_t n = cc[c + 1] - cc[c];
    if (n < 1) return DHSA_ERR_BAD_LAYOUT;
    if (n > max_len) max_len = n;
  }
  for (int32_t b = 0; b < B; ++b)    // monotone, so every seq_chunk_start entry lies in [0, C]
    if (cs[b + 1] < cs[b] || sc[b + 1] < sc[b]) return DHSA_ERR_BAD_LAYOUT;
  for (int32_t b = 0; b < B; ++b) {
    if (cc[sc[b]] != cs[b] || cc[sc[b + 1]] != cs[b + 1]) return DHSA_ERR_BAD_LAYOUT;
    const int32_t nc = sc[b + 1] - sc[b];
    if (nc > max_per_seq) max_per_seq = nc;
  }
  if (max_per_seq > DHSA_MAX_CHUNKS_PER_SEQ) return DHSA_ERR_UNSUPPORTED;
  if (plan != nullptr) {
    *plan = Plan{B, T, C, L->num_q_heads, L->num_kv_heads, L->head_dim, L->dtype,
                 L->cu_seqlens, L->cu_chunks, L->seq_chunk_start, max_len, max_per_seq, cc};
  }
  return DHSA_OK;
}

// Row pointers must be the plan of some budget: row i holds between 1 and i_loc + 1 entries.
// Sets *wide when a row with more than kRouteRegCand earlier chunks keeps some but not all of them.
dhsa_status check_row_ptr(const dhsa_layout* L, const int32_t* h_row_ptr, int64_t nnz, bool* wide) {
  if (h_row_ptr == nullptr) return DHSA_ERR_NULL_ARG;
  const int32_t* sc = L->h_seq_chunk_start;
  if (h_row_ptr[0] != 0) return DHSA_ERR_BAD_SHAPE;
  *wide = false;
  for (int32_t b = 0; b < L->num_seqs; ++b) {
    for (int32_t c = sc[b]; c < sc[b + 1]; ++c) {
      const int64_t len = (int64_t)h_row_ptr[c + 1] - h_row_ptr[c];
      const int32_t i_loc = c - sc[b];
      if (len < 1 || len > (int64_t)i_loc + 1) return DHSA_ERR_BAD_SHAPE;
      if (len - 1 > 0 && len - 1 < i_loc && i_loc > dhsa::kRouteRegCand) *wide = true;
    }
  }
  if ((int64_t)h_row_ptr[L->total_chunks] != nnz) return DHSA_ERR_BAD_SHAPE;
  return DHSA_OK;
}

dhsa_status launched(hipError_t e) { return e == hipSuccess ? DHSA_OK : DHSA_ERR_LAUNCH; }

// Tensors the kernels read or write with 16-byte vector or buffer accesses: base pointers 16-byte
// aligned (NULL passes here; the null checks come first).
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }
template <typename... P>
bool all_aligned16(const P*... p) { return (aligned16(p) && ...); }

// Decode state: shapes, capacities and pointers (host-side view only).
dhsa_status check_decode_state(const dhsa_decode_state* st, dhsa::DecodeDims* dims, dhsa::DecodePtrs* ptrs) {
  if (st == nullptr) return DHSA_ERR_NULL_ARG;
  if (st->num_seqs < 1 || st->num_q_heads < 1 || st->num_kv_heads < 1 || st->max_tokens < 1 ||
      st->max_chunks < 1)
    return DHSA_ERR_BAD_SHAPE;
  if (st->num_q_heads % st->num_kv_heads != 0) return DHSA_ERR_BAD_SHAPE;
  if (st->dtype == DHSA_BF16) {
    if (st->head_dim != 64 && st->head_dim != 128 && st->head_dim != 256) return DHSA_ERR_UNSUPPORTED;
  } else if (st->dtype == DHSA_F32) {
    if (st->head_dim != 64 && st->head_dim != 128) return DHSA_ERR_UNSUPPORTED;
  } else {
    return DHSA_ERR_UNSUPPORTED;
  }
  if (st->max_chunks > dhsa::kDecodeMaxChunks) return DHSA_ERR_UNSUPPORTED;
  if (st->max_tokens > dhsa::kDecodeMaxTokens) return DHSA_ERR_UNSUPPORTED;
  const int64_t elem = st->dtype == DHSA_BF16 ? 2 : 4;
  if ((int64_t)st->max_tokens * st->num_kv_heads * st->head_dim * elem > ((int64_t)1 << 40)) return DHSA_ERR_UNSUPPORTED;
  if (st->k_cache == nullptr || st->v_cache == nullptr || st->seq_len == nullptr || st->num_closed == nullptr ||
      st->chunk_start == nullptr || st->k_sum == nullptr || st->q_run == nullptr || st->k_run == nullptr ||
      st->status == nullptr)
    return DHSA_ERR_NULL_ARG;
  if (!all_aligned16(st->k_cache, st->v_cache, st->k_sum, st->q_run, st->k_run)) return DHSA_ERR_BAD_SHAPE;
  *dims = dhsa::DecodeDims{st->num_seqs, st->num_q_heads, st->num_kv_heads, st->head_dim, st->dtype,
                           st->max_tokens, st->max_chunks};
  *ptrs = dhsa::DecodePtrs{st->k_cache, st->v_cache, st->seq_len, st->num_closed, st->chunk_start,
                           st->k_sum, st->q_run, st->k_run, st->status};
  return DHSA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout of a decode step: the kept tokens' cache rows, token counts, split-K partial states,
// each sequence's pending append record.
size_t decode_workspace(const dhsa::DecodeDims& p, int topk, bool grouped, dhsa::DecodeWork* w, void* base) {
  const size_t rows = (size_t)p.B * (grouped ? p.Hkv : p.Hq);
  // one split-K partial state per attention wave of a row: the grid has at most kDecodeGridSlices
  const int NS = std::min((p.L + dhsa::kDecodeSlice - 1) / dhsa::kDecodeSlice, dhsa::kDecodeGridSlices);
  const size_t o_urow = 0;
  const size_t o_ntok = align256(o_urow + rows * (size_t)p.L * sizeof(int32_t));
  const size_t o_part = align256(o_ntok + rows * sizeof(int32_t));
  const size_t o_pend = align256(o_part + (size_t)p.B * p.Hq * NS * (p.d + dhsa::kPartHead) * sizeof(float));
  const size_t total = align256(o_pend + (size_t)p.B * 4 * sizeof(int32_t));
  if (w != nullptr) {
    char* c = (char*)base;
    *w = dhsa::DecodeWork{(int32_t*)(c + o_urow), (int32_t*)(c + o_ntok), (float*)(c + o_part),
                          (int32_t*)(c + o_pend), NS};
  }
  return total;
}


// Token offsets of a batch (host mirror): start at 0, monotone, end at T.
dhsa_status check_seqlens(int32_t B, int32_t T, const int32_t* cu_seqlens, const int32_t* h_cu_seqlens) {
  if (B < 0 || T < 0) return DHSA_ERR_BAD_SHAPE;
  if (cu_seqlens == nullptr || h_cu_seqlens == nullptr) return DHSA_ERR_NULL_ARG;
  if (h_cu_seqlens[0] != 0 || h_cu_seqlens[B] != T) return DHSA_ERR_BAD_LAYOUT;
  for (int32_t b = 0; b < B; ++b)
    if (h_cu_seqlens[b + 1] < h_cu_seqlens[b]) return DHSA_ERR_BAD_LAYOUT;
  return DHSA_OK;
}


// Row capacities under a token budget: row i holds 1 + the number of the shortest earlier chunks
// of its sequence whose lengths fit in h_tb[i] (the most any ranking could keep).  A Fenwick tree
// over chunk lengths (counts and token sums) answers each row in O(log max_len).  Writes
// h_row_ptr, or (h_row_ptr == nullptr) compares against h_check.  *too_wide: some row with more
// candidates than the routing registers hold keeps some but not all of them (the general kernel
// selects those rows).
dhsa_status plan_tokens(const dhsa_layout* L, const int32_t* h_tb, int32_t* h_row_ptr, const int32_t* h_check,
                        int64_t* nnz, bool* too_wide) {
  const int32_t* sc = L->h_seq_chunk_start;
  const int32_t* cc = L->h_cu_chunks;
  for (int32_t c = 0; c < L->total_chunks; ++c)
    if (h_tb[c] < 0) return DHSA_ERR_BAD_BUDGET;
  int32_t maxlen = 1;
  for (int32_t c = 0; c < L->total_chunks; ++c) maxlen = std::max(maxlen, cc[c + 1] - cc[c]);
  int LOG = 1;
  while ((1 << LOG) <= maxlen) ++LOG;
  const int N = 1 << LOG;                         // tree positions 1..N-1 hold lengths 1..N-1
  std::vector<int64_t> fcnt(N, 0), fsum(N, 0);
  int64_t acc = 0;
  if (h_row_ptr != nullptr) h_row_ptr[0] = 0;
  else if (h_check[0] != 0) return DHSA_ERR_BAD_SHAPE;
  *too_wide = false;
  for (int32_t b = 0; b < L->num_seqs; ++b) {
    std::fill(fcnt.begin(), fcnt.end(), 0);
    std::fill(fsum.begin(), fsum.end(), 0);
    int64_t total = 0;                            // tokens of the earlier chunks
    for (int32_t c = sc[b]; c < sc[b + 1]; ++c) {
      const int32_t i_loc = c - sc[b];
      const int64_t budget = h_tb[c];
      int64_t fit;
      if (budget >= total) {
        fit = i_loc;
      } else {
        // largest length bound v with sum(lengths <= v) <= budget, then part of the next length
        int pos = 0;
        int64_t cnt = 0, sum = 0;
        for (int step = N >> 1; step > 0; step >>= 1) {
          const int nx = pos + step;
          if (nx < N && sum + fsum[nx] <= budget) {
            pos = nx;
            sum += fsum[nx];
            cnt += fcnt[nx];
          }
        }
        // chunks of length pos + 1 that still fit (all of that length would exceed the budget)
        const int64_t v = pos + 1;
        fit = cnt + (v < N ? (budget - sum) / v : 0);
        if (i_loc > dhsa::kRouteRegCand) *too_wide = true;
      }
      acc += fit + 1;
      if (acc > 0x7fffffffLL) return DHSA_ERR_BAD_SHAPE;
      if (h_row_ptr != nullptr) h_row_ptr[c + 1] = (int32_t)acc;
      else if (h_check[c + 1] != (int32_t)acc) return DHSA_ERR_BAD_SHAPE;
      const int32_t len = cc[c + 1] - cc[c];
      total += len;
      for (int x = len; x < N; x += x & -x) {
        fcnt[x] += 1;
        fsum[x] += len;
      }
    }
  }
  *nnz = acc;
  return DHSA_OK;
}

// Arguments of a decode step other than its scratch (shared by the workspace and static-scratch entries).
dhsa_status check_decode_step(const dhsa_decode_state* state, const void* q, const void* k, const void* v, int32_t lo,
                              int32_t hi, float tau, int32_t topk, float softmax_scale, const void* out,
                              dhsa::DecodeDims* p, dhsa::DecodePtrs* s) {
  dhsa_status st = check_decode_state(state, p, s);
  if (st != DHSA_OK) return st;
  if (lo < 1 || hi < lo || !isfinite(tau)) return DHSA_ERR_BAD_SHAPE;
  if (topk < 0 || topk >= dhsa::kDecodeMaxTopk) return DHSA_ERR_BAD_BUDGET;
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return DHSA_ERR_BAD_SHAPE;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return DHSA_ERR_NULL_ARG;
  if (!all_aligned16(q, k, v, out)) return DHSA_ERR_BAD_SHAPE;
  return DHSA_OK;
}

}  // namespace

extern "C" {

int32_t dhsa_abi_version(void) { return DHSA_ABI_VERSION; }

const char* dhsa_status_str(int32_t status) {
  switch (status) {
    case DHSA_OK: return "DHSA_OK";
    case DHSA_ERR_NULL_ARG: return "DHSA_ERR_NULL_ARG: a required pointer is NULL";
    case DHSA_ERR_BAD_SHAPE: return "DHSA_ERR_BAD_SHAPE: inconsistent sizes or row pointers";
    case DHSA_ERR_BAD_LAYOUT: return "DHSA_ERR_BAD_LAYOUT: chunk/sequence offsets are invalid";
    case DHSA_ERR_BAD_BUDGET: return "DHSA_ERR_BAD_BUDGET: negative key-chunk budget";
    case DHSA_ERR_UNSUPPORTED: return "DHSA_ERR_UNSUPPORTED: dtype, head_dim or chunk count not supported";
    case DHSA_ERR_LAUNCH: return "DHSA_ERR_LAUNCH: kernel launch failed";
    case DHSA_ERR_WORKSPACE:
      return "DHSA_ERR_WORKSPACE: the step needs more scratch than the library's static device array holds";
    default: return "unknown dhsa_status";
  }
}

dhsa_status dhsa_validate_layout(const dhsa_layout* layout) { return check_layout(layout, nullptr); }

dhsa_status dhsa_route_plan(const dhsa_layout* layout, const int32_t* h_topk, int32_t* h_row_ptr,
                            int64_t* nnz) {
  dhsa_status st = check_layout(layout, nullptr);
  if (st != DHSA_OK) return st;
  if (h_topk == nullptr || h_row_ptr == nullptr || nnz == nullptr) return DHSA_ERR_NULL_ARG;
  const int32_t* sc = layout->h_seq_chunk_start;
  for (int32_t c = 0; c < layout->total_chunks; ++c)
    if (h_topk[c] < 0) return DHSA_ERR_BAD_BUDGET;
  int64_t acc = 0;
  h_row_ptr[0] = 0;
  for (int32_t b = 0; b < layout->num_seqs; ++b) {
    for (int32_t c = sc[b]; c < sc[b + 1]; ++c) {
      const int32_t i_loc = c - sc[b];
      acc += (int64_t)(h_topk[c] < i_loc ? h_topk[c] : i_loc) + 1;
      if (acc > 0x7fffffffLL) return DHSA_ERR_BAD_SHAPE;
      h_row_ptr[c + 1] = (int32_t)acc;
    }
  }
  *nnz = acc;
  return DHSA_OK;
}

dhsa_status dhsa_route_plan_tokens(const dhsa_layout* layout, const int32_t* h_token_budget, int32_t* h_row_ptr,
                                   int64_t* nnz) {
  dhsa_status st = check_layout(layout, nullptr);
  if (st != DHSA_OK) return st;
  if (h_token_budget == nullptr || h_row_ptr == nullptr || nnz == nullptr) return DHSA_ERR_NULL_ARG;
  bool too_wide = false;
  return plan_tokens(layout, h_token_budget, h_row_ptr, nullptr, nnz, &too_wide);
}

dhsa_status dhsa_chunk_summarize(const dhsa_layout* layout, const void* q, const void* k, float* q_sum,
                                 float* k_sum, void* stream) {
  Plan p;
  dhsa_status st = check_layout(layout, &p);
  if (st != DHSA_OK) return st;
  if (p.C == 0) return DHSA_OK;
  if (q == nullptr || k == nullptr || q_sum == nullptr || k_sum == nullptr) return DHSA_ERR_NULL_ARG;
  if (!all_aligned16(q, k, q_sum, k_sum)) return DHSA_ERR_BAD_SHAPE;
  return launched(dhsa::launch_summarize(p, q, k, q_sum, k_sum, (hipStream_t)stream));
}

static dhsa_status route_common(const dhsa_layout* layout, const float* q_sum, const float* k_sum,
                                const int32_t* row_ptr, const int32_t* h_row_ptr, int64_t nnz,
                                int32_t* block_idx, bool grouped, void* stream) {
  Plan p;
  dhsa_status st = check_layout(layout, &p);
  if (st != DHSA_OK) return st;
  bool wide = false;
  st = check_row_ptr(layout, h_row_ptr, nnz, &wide);
  if (st != DHSA_OK) return st;
  if (p.C == 0) return DHSA_OK;
  if (q_sum == nullptr || k_sum == nullptr || row_ptr == nullptr || block_idx == nullptr)
    return DHSA_ERR_NULL_ARG;
  if (!all_aligned16(q_sum, k_sum)) return DHSA_ERR_BAD_SHAPE;
  return launched(dhsa::launch_route(p, q_sum, k_sum, row_ptr, nnz, block_idx, wide, grouped,
                                     (hipStream_t)stream));
}

dhsa_status dhsa_route(const dhsa_layout* layout, const float* q_sum, const float* k_sum,
                       const int32_t* row_ptr, const int32_t* h_row_ptr, int64_t nnz, int32_t* block_idx,
                       void* stream) {
  return route_common(layout, q_sum, k_sum, row_ptr, h_row_ptr, nnz, block_idx, false, stream);
}

dhsa_status dhsa_route_grouped(const dhsa_layout* layout, const float* q_sum, const float* k_sum,
                               const int32_t* row_ptr, const int32_t* h_row_ptr, int64_t nnz,
                               int32_t* block_idx, void* stream) {
  return route_common(layout, q_sum, k_sum, row_ptr, h_row_ptr, nnz, block_idx, true, stream);
}

dhsa_status dhsa_route_tokens(const dhsa_layout* layout, const float* q_sum, const float* k_sum,
                              const int32_t* token_budget, const int32_t* h_token_budget, const int32_t* row_ptr,
                              const int32_t* h_row_ptr, int64_t nnz, int32_t grouped, int32_t* block_idx,
                              void* stream) {
  Plan p;
  dhsa_status st = check_layout(layout, &p);
  if (st != DHSA_OK) return st;
  if (h_token_budget == nullptr || h_row_ptr == nullptr) return DHSA_ERR_NULL_ARG;
  int64_t planned = 0;
  bool too_wide = false;
  st = plan_tokens(layout, h_token_budget, nullptr, h_row_ptr, &planned, &too_wide);
  if (st != DHSA_OK) return st;
  if (planned != nnz) return DHSA_ERR_BAD_SHAPE;
  if (p.C == 0) return DHSA_OK;
  if (q_sum == nullptr || k_sum == nullptr || token_budget == nullptr || row_ptr == nullptr || block_idx == nullptr)
    return DHSA_ERR_NULL_ARG;
  if (!all_aligned16(q_sum, k_sum)) return DHSA_ERR_BAD_SHAPE;
  return launched(dhsa::launch_route_tokens(p, q_sum, k_sum, token_budget, row_ptr, nnz, block_idx, too_wide,
                                            grouped != 0, (hipStream_t)stream));
}

dhsa_status dhsa_sparse_prefill(const dhsa_layout* layout, const void* q, const void* k, const void* v,
                                const int32_t* row_ptr, const int32_t* h_row_ptr, int64_t nnz,
                                const int32_t* block_idx, float softmax_scale, void* out, float* lse,
                                void* stream) {
  Plan p;
  dhsa_status st = check_layout(layout, &p);
  if (st != DHSA_OK) return st;
  bool wide = false;
  st = check_row_ptr(layout, h_row_ptr, nnz, &wide);
  if (st != DHSA_OK) return st;
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return DHSA_ERR_BAD_SHAPE;
  if (p.C == 0) return DHSA_OK;
  if (q == nullptr || k == nullptr || v == nullptr || row_ptr == nullptr || block_idx == nullptr ||
      out == nullptr)
    return DHSA_ERR_NULL_ARG;
  if (!all_aligned16(q, k, v, out)) return DHSA_ERR_BAD_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  // the bf16 kernel addresses one KV head's rows with 32-bit buffer offsets
  if (p.dtype == DHSA_BF16 && (int64_t)p.T * p.Hkv * p.d * 2 > (int64_t)INT32_MAX) return DHSA_ERR_UNSUPPORTED;
  if (p.dtype == DHSA_BF16)
    return launched(dhsa::launch_prefill_bf16(p, q, k, v, row_ptr, nnz, block_idx, softmax_scale, out, lse, s));
  return launched(dhsa::launch_prefill_f32(p, q, k, v, row_ptr, nnz, block_idx, softmax_scale, out, lse, s));
}


dhsa_status dhsa_adjacent_similarity(int32_t num_seqs, int32_t total_tokens, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t dtype, const int32_t* cu_seqlens,
                                     const int32_t* h_cu_seqlens, const void* k, float tau, float* sim,
                                     uint64_t* cut_bits, void* stream) {
  dhsa_status st = check_seqlens(num_seqs, total_tokens, cu_seqlens, h_cu_seqlens);
  if (st != DHSA_OK) return st;
  if (num_kv_heads < 1 || head_dim < 1 || (int64_t)num_kv_heads * head_dim > INT32_MAX / 4) return DHSA_ERR_BAD_SHAPE;
  if (dtype != DHSA_F32 && dtype != DHSA_BF16) return DHSA_ERR_UNSUPPORTED;
  const int32_t W = num_kv_heads * head_dim;
  if (W % (dtype == DHSA_BF16 ? 8 : 4) != 0) return DHSA_ERR_UNSUPPORTED;
  if (W / (dtype == DHSA_BF16 ? 8 : 4) > dhsa::kSimMaxPieces) return DHSA_ERR_UNSUPPORTED;
  if (!isfinite(tau)) return DHSA_ERR_BAD_SHAPE;
  if (total_tokens == 0) return DHSA_OK;
  if (k == nullptr || sim == nullptr || cut_bits == nullptr) return DHSA_ERR_NULL_ARG;
  if (!all_aligned16(k)) return DHSA_ERR_BAD_SHAPE;
  return launched(dhsa::launch_adjacent_similarity(num_seqs, total_tokens, W, dtype, cu_seqlens, k, tau, sim,
                                                   cut_bits, (hipStream_t)stream));
}

dhsa_status dhsa_chunk_boundaries(int32_t num_seqs, int32_t total_tokens, const int32_t* cu_seqlens,
                                  const int32_t* h_cu_seqlens, const uint64_t* cut_bits, int32_t lo, int32_t hi,
                                  int32_t* cu_chunks, int32_t* seq_chunk_start, int32_t* num_chunks,
                                  void* stream) {
  dhsa_status st = check_seqlens(num_seqs, total_tokens, cu_seqlens, h_cu_seqlens);
  if (st != DHSA_OK) return st;
  if (lo < 1 || hi < lo) return DHSA_ERR_BAD_SHAPE;
  if (cu_chunks == nullptr || seq_chunk_start == nullptr || num_chunks == nullptr) return DHSA_ERR_NULL_ARG;
  if (total_tokens > 0 && cut_bits == nullptr) return DHSA_ERR_NULL_ARG;
  // Limits past the longest sequence change nothing; clamping keeps c0 + hi inside int range.
  const int32_t cap = total_tokens > 0 ? total_tokens : 1;
  const int32_t hi_c = hi < cap ? hi : cap;
  const int32_t lo_c = lo < hi_c ? lo : hi_c;
  return launched(dhsa::launch_chunk_walk(num_seqs, total_tokens, cu_seqlens, cut_bits, lo_c, hi_c, cu_chunks,
                                          seq_chunk_start, num_chunks, (hipStream_t)stream));
}


size_t dhsa_decode_workspace_bytes(const dhsa_decode_state* state, int32_t topk, int32_t grouped) {
  dhsa::DecodeDims p;
  dhsa::DecodePtrs s;
  if (check_decode_state(state, &p, &s) != DHSA_OK || topk < 0 || topk >= dhsa::kDecodeMaxTopk) return 0;
  return decode_workspace(p, topk, grouped != 0, nullptr, nullptr);
}

dhsa_status dhsa_decode_load_prefix(const dhsa_decode_state* state, const dhsa_layout* prefix, const void* q,
                                    const void* k, const void* v, void* stream) {
  dhsa::DecodeDims p;
  dhsa::DecodePtrs s;
  dhsa_status st = check_decode_state(state, &p, &s);
  if (st != DHSA_OK) return st;
  Plan pl;
  if ((st = check_layout(prefix, &pl)) != DHSA_OK) return st;
  if (pl.B != p.B || pl.Hq != p.Hq || pl.Hkv != p.Hkv || pl.d != p.d || pl.dtype != p.dtype) return DHSA_ERR_BAD_SHAPE;
  for (int32_t b = 0; b < pl.B; ++b) {
    if (prefix->h_cu_seqlens[b + 1] - prefix->h_cu_seqlens[b] > p.L) return DHSA_ERR_BAD_SHAPE;
    if (prefix->h_seq_chunk_start[b + 1] - prefix->h_seq_chunk_start[b] > p.Cmax + 1) return DHSA_ERR_BAD_SHAPE;
  }
  if (pl.T > 0 && (q == nullptr || k == nullptr || v == nullptr)) return DHSA_ERR_NULL_ARG;
  if (!all_aligned16(q, k, v)) return DHSA_ERR_BAD_SHAPE;
  return launched(dhsa::launch_decode_load(p, s, pl, q, k, v, (hipStream_t)stream));
}

dhsa_status dhsa_decode_step(const dhsa_decode_state* state, const void* q, const void* k, const void* v,
                             int32_t lo, int32_t hi, float tau, int32_t topk, int32_t grouped,
                             float softmax_scale, void* out, int32_t* kept, void* workspace,
                             size_t workspace_bytes, void* stream) {
  dhsa::DecodeDims p;
  dhsa::DecodePtrs s;
  dhsa_status st = check_decode_step(state, q, k, v, lo, hi, tau, topk, softmax_scale, out, &p, &s);
  if (st != DHSA_OK) return st;
  if (workspace == nullptr) return DHSA_ERR_NULL_ARG;
  if (((uintptr_t)workspace & 255) != 0) return DHSA_ERR_BAD_SHAPE;
  dhsa::DecodeWork w;
  if (decode_workspace(p, topk, grouped != 0, &w, workspace) > workspace_bytes) return DHSA_ERR_BAD_SHAPE;
  return launched(dhsa::launch_decode_step(p, s, q, k, v, lo, hi, tau, topk, grouped != 0, softmax_scale, out, kept,
                                           w, (hipStream_t)stream));
}

dhsa_status dhsa_decode_step_noalloc(const dhsa_decode_state* state, const void* q, const void* k, const void* v,
                                     int32_t lo, int32_t hi, float tau, int32_t topk, int32_t grouped,
                                     float softmax_scale, void* out, int32_t* kept, void* stream) {
  dhsa::DecodeDims p;
  dhsa::DecodePtrs s;
  dhsa_status st = check_decode_step(state, q, k, v, lo, hi, tau, topk, softmax_scale, out, &p, &s);
  if (st != DHSA_OK) return st;
  if (decode_workspace(p, topk, grouped != 0, nullptr, nullptr) > dhsa::kNoAllocScratchBytes)
    return DHSA_ERR_WORKSPACE;
  // the scratch is the current GPU's copy of the static array, so the stream must belong to that GPU
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return DHSA_ERR_LAUNCH;
  if (stream != nullptr) {
    hipDevice_t sd = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sd) != hipSuccess) return DHSA_ERR_LAUNCH;
    if (sd != cur) return DHSA_ERR_UNSUPPORTED;
  }
  void* scratch = nullptr;
  if (dhsa::decode_noalloc_scratch(&scratch) != hipSuccess) return DHSA_ERR_LAUNCH;
  dhsa::DecodeWork w;
  decode_workspace(p, topk, grouped != 0, &w, scratch);
  return launched(dhsa::launch_decode_step(p, s, q, k, v, lo, hi, tau, topk, grouped != 0, softmax_scale, out, kept,
                                           w, (hipStream_t)stream));
}

}  // extern "C"
