/*
 * dhsa.h - C ABI of the MI355X (gfx950) DHSA chunk-routed sparse causal prefill.
 *
 * Dynamic Hierarchical Sparse Attention splits each sequence into
 * variable-length chunks, represents every chunk by the average of its token
 * vectors times sqrt(n) for a chunk of n tokens, scores chunk pairs
 * causally, upsamples the chunk scores to token level and runs exact softmax
 * attention over the token interactions that survive ("Long-Context Modeling
 * with Dynamic Hierarchical Sparse Attention for On-Device LLMs", Abstract and
 * Innovation; "... for Memory-Constrained LLM Inference", ICML 2026 spotlight
 * page, Abstract).  The pages leave the chunk rule, the keep budget and the
 * diagonal open; here they are explicit: boundaries are an input, each query
 * chunk keeps its top-k earlier key chunks plus itself, ties go to the lower
 * chunk index.  Because the budget is counted in chunks, the token-level
 * importance obtained by broadcasting chunk scores keeps exactly the union of
 * the kept chunks' tokens (causally masked), so routing is decided per chunk.
 *
 * Conventions shared by every call
 *  - Layout "THD": tokens of all sequences packed back to back.
 *      q   [T, Hq,  d]   k, v [T, Hkv, d]   out [T, Hq, d]   (row-major, contiguous)
 *      q_sum [C, Hq, d], k_sum [C, Hkv, d]  float32
 *    q/k/v/out are float32 (DHSA_F32) or bfloat16 (DHSA_BF16).  Base pointers
 *    of tensors must be 16-byte aligned (checked: DHSA_ERR_BAD_SHAPE otherwise).
 *  - GQA: query head h reads KV head h / (Hq / Hkv); Hq % Hkv == 0.
 *  - Chunk ids are global (0..C-1); the chunks of sequence b are
 *    seq_chunk_start[b] .. seq_chunk_start[b+1]-1 and tile its tokens exactly.
 *  - Pointers without the h_ prefix are HIP device memory; h_ pointers are
 *    host memory.  Everything is OWNED BY THE CALLER: the library allocates
 *    no device memory, never synchronises, and enqueues its kernels on
 *    `stream` (a hipStream_t; NULL = default stream).  Its only mutable global
 *    state is the scratch of dhsa_decode_step_noalloc (see there).
 *  - Errors: every argument, shape and layout problem is detected on the host
 *    (from the h_ mirrors) and returned BEFORE anything is launched; outputs
 *    are then untouched.  A failed launch returns DHSA_ERR_LAUNCH.  The device
 *    arrays must hold the same values as their host mirrors; if they do not,
 *    behaviour is undefined.
 *  - Supported: DHSA_BF16 with d in {64, 128, 256}; DHSA_F32 with d in
 *    {32, 64, 128}.  At most DHSA_MAX_CHUNKS_PER_SEQ chunks per sequence.
 *  - Empty batches (T == 0 or C == 0) are valid and launch nothing.
 */
#ifndef DHSA_H
#define DHSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DHSA_ABI_VERSION 1
#define DHSA_MAX_CHUNKS_PER_SEQ 8192

typedef enum dhsa_status {
  DHSA_OK = 0,
  DHSA_ERR_NULL_ARG = 1,     /* a required pointer is NULL                          */
  DHSA_ERR_BAD_SHAPE = 2,    /* negative sizes, Hq % Hkv != 0, nnz mismatch          */
  DHSA_ERR_BAD_LAYOUT = 3,   /* offsets not monotone, empty chunk, chunk crosses seq */
  DHSA_ERR_BAD_BUDGET = 4,   /* negative top-k                                       */
  DHSA_ERR_UNSUPPORTED = 5,  /* dtype / head_dim / chunk count outside the support   */
  DHSA_ERR_LAUNCH = 6,       /* hipGetLastError after a launch was not hipSuccess    */
  DHSA_ERR_WORKSPACE = 7     /* dhsa_decode_step_noalloc: more scratch than the      */
                             /* library's static device array holds                  */
} dhsa_status;

typedef enum dhsa_dtype { DHSA_F32 = 0, DHSA_BF16 = 1 } dhsa_dtype;

/* Packed varlen batch description.  Device arrays feed the kernels; the host
 * mirrors (required, same contents) are used for validation and launch
 * sizing. */
typedef struct dhsa_layout {
  int32_t num_seqs;                  /* B >= 0                                   */
  int32_t total_tokens;              /* T = cu_seqlens[B]                        */
  int32_t total_chunks;              /* C = seq_chunk_start[B]                   */
  int32_t num_q_heads;               /* Hq >= 1                                  */
  int32_t num_kv_heads;              /* Hkv >= 1, Hq % Hkv == 0                  */
  int32_t head_dim;                  /* d                                        */
  int32_t dtype;                     /* dhsa_dtype of q, k, v, out               */
  const int32_t* cu_seqlens;         /* device [B+1] token offsets, [0] = 0      */
  const int32_t* cu_chunks;          /* device [C+1] global chunk starts, [C]=T  */
  const int32_t* seq_chunk_start;    /* device [B+1] first chunk of each seq     */
  const int32_t* h_cu_seqlens;       /* host mirror of cu_seqlens                */
  const int32_t* h_cu_chunks;        /* host mirror of cu_chunks                 */
  const int32_t* h_seq_chunk_start;  /* host mirror of seq_chunk_start           */
} dhsa_layout;

/* ABI version (DHSA_ABI_VERSION). */
int32_t dhsa_abi_version(void);

/* Static, human-readable name of a status code. */
const char* dhsa_status_str(int32_t status);

/* Host-only check of a layout (the same check every call below performs):
 * offsets start at 0 and are monotone, every chunk has >= 1 token, the chunks
 * of each sequence tile its token range, and the shape fields are supported. */
dhsa_status dhsa_validate_layout(const dhsa_layout* layout);

/* Routing plan (host only, pure).  Row i of the compressed block list keeps
 * min(h_topk[i], i_loc) + 1 key chunks, i_loc = i - first chunk of i's
 * sequence: the top-k earlier chunks plus the diagonal.  The pages leave the
 * keep budget open (they say importance decides which token interactions are
 * kept, not how many: "Long-Context Modeling with Dynamic Hierarchical Sparse
 * Attention for On-Device LLMs", Abstract); this library makes it an explicit
 * parameter: a count of earlier chunks per query chunk, the diagonal chunk
 * always kept on top of it, ties broken toward the lower chunk index (the rule
 * dhsa_route applies).
 *   h_topk     host [C]   off-diagonal key-chunk budget per query chunk (>= 0)
 *   h_row_ptr  host [C+1] written: CSR row offsets, shared by all q heads
 *   nnz        written: h_row_ptr[C], the entries per q head */
dhsa_status dhsa_route_plan(const dhsa_layout* layout, const int32_t* h_topk,
                            int32_t* h_row_ptr, int64_t* nnz);

/* Stage 1: length-normalised chunk summaries ("Long-Context Modeling with
 * Dynamic Hierarchical Sparse Attention for On-Device LLMs", Abstract and
 * Innovation: the average of the chunk's token vectors times
 * sqrt(chunk size)), for Q and K:
 *   q_sum[c, h, :] = (sum_{t in chunk c} q[t, h, :]) / sqrt(n_c),
 *   k_sum[c, g, :] likewise from k.
 * fp32 accumulation.  q_sum and k_sum are written completely. */
dhsa_status dhsa_chunk_summarize(const dhsa_layout* layout, const void* q, const void* k,
                                 float* q_sum, float* k_sum, void* stream);

/* Stage 2: causal chunk routing (same page, Abstract: chunk-level similarity
 * upsampled to token level decides the kept interactions; ICML 2026 page,
 * Abstract: routing is causal).  For q head h and query chunk i, every earlier
 * chunk j of the same sequence is scored s_j = q_sum[i, h, :] . k_sum[j, h/G, :]
 * (fp32); the top (row length - 1) by (s_j descending, j ascending) are kept,
 * then i itself.  Row (h, i) is written to
 *   block_idx[h * nnz + row_ptr[i] .. h * nnz + row_ptr[i+1] - 1]
 * in ascending chunk order (so the diagonal is last).
 *   row_ptr    device [C+1] from dhsa_route_plan (its host copy h_row_ptr is
 *              used for validation)
 *   block_idx  device [Hq, nnz] int32, written completely */
dhsa_status dhsa_route(const dhsa_layout* layout, const float* q_sum, const float* k_sum,
                       const int32_t* row_ptr, const int32_t* h_row_ptr, int64_t nnz,
                       int32_t* block_idx, void* stream);

/* Stage 2, routed once per KV head (same pages; the granularity at which
 * grouped-query heads are routed is left open there).  For KV head g and query
 * chunk i, every earlier chunk j of the same sequence is scored
 *   s_j = (sum over the query heads h of g's group of q_sum[i, h, :]) . k_sum[j, g, :]
 * (fp32; the group sum in ascending head order), selected like dhsa_route, and
 * the group's row is written to the rows of all of its query heads, so
 * block_idx has the same layout and dhsa_sparse_prefill takes it unchanged.
 * Arguments, validation and errors as dhsa_route. */
dhsa_status dhsa_route_grouped(const dhsa_layout* layout, const float* q_sum, const float* k_sum,
                               const int32_t* row_ptr, const int32_t* h_row_ptr, int64_t nnz,
                               int32_t* block_idx, void* stream);

/* ---- Routing under a token budget (an extension: the pages keep the
 * important token interactions - "Long-Context Modeling with Dynamic
 * Hierarchical Sparse Attention for On-Device LLMs", Abstract - and report the
 * memory saved, without fixing how much is kept; a budget in tokens is the
 * other plain reading beside the chunk count).  Query chunk i ranks the earlier
 * chunks of its sequence exactly as dhsa_route (score descending, chunk
 * ascending) and keeps the longest prefix of that ranking whose chunk lengths
 * sum to at most token_budget[i] (the first chunk that does not fit ends it),
 * plus itself. */

/* Plan (host only, pure).  The kept count depends on the scores, so row i gets
 * the most any ranking could keep: 1 + how many of the shortest earlier chunks
 * of the sequence fit in h_token_budget[i].
 *   h_token_budget  host [C] tokens per query chunk (>= 0, else BAD_BUDGET)
 *   h_row_ptr       host [C+1] written: CSR row offsets, shared by all q heads
 *   nnz             written: h_row_ptr[C] */
dhsa_status dhsa_route_plan_tokens(const dhsa_layout* layout, const int32_t* h_token_budget,
                                   int32_t* h_row_ptr, int64_t* nnz);

/* Routing under a token budget, per q head (grouped = 0) or per KV head with
 * the group sum of the query summaries (grouped != 0, as dhsa_route_grouped).
 * Row (h, i) gets its kept chunks ascending, then i, then -1 up to the row's
 * capacity; dhsa_sparse_prefill skips the -1 entries.
 *   token_budget    device [C], equal to its host mirror h_token_budget
 *   row_ptr         device [C+1] from dhsa_route_plan_tokens with the same
 *                   budgets; h_row_ptr its host mirror (checked against the plan:
 *                   BAD_SHAPE if it differs, or if nnz does)
 *   block_idx       device [Hq, nnz] int32, written completely */
dhsa_status dhsa_route_tokens(const dhsa_layout* layout, const float* q_sum, const float* k_sum,
                              const int32_t* token_budget, const int32_t* h_token_budget,
                              const int32_t* row_ptr, const int32_t* h_row_ptr, int64_t nnz,
                              int32_t grouped, int32_t* block_idx, void* stream);

/* Stage 3: block-sparse causal prefill (ICML 2026 page, Abstract: tiled
 * backend; exact softmax over the kept token interactions).  Query token t of
 * chunk i, head h attends to every key u <= t lying in a kept chunk of row
 * (h, i):
 *   out[t, h, :] = sum_u softmax_u(softmax_scale * q[t,h,:] . k[u,g,:]) v[u,g,:]
 *   lse[h, t]    = log sum_u exp(softmax_scale * q[t,h,:] . k[u,g,:])   (natural log)
 * fp32 accumulation; out is rounded to its dtype (bf16: to nearest even).
 *   row_ptr, block_idx  device CSR as written by dhsa_route (or any list in the
 *              same format: ascending, inside the query chunk's sequence, j <= i,
 *              with the diagonal present; entries outside the sequence's chunks
 *              up to i, such as the -1 padding of dhsa_route_tokens, are skipped)
 *   lse        device [Hq, T] float32 or NULL
 * out (and lse) are written completely.  bf16 additionally needs k and v below
 * 2 GiB each (T * Hkv * head_dim * 2 bytes): larger returns UNSUPPORTED. */
dhsa_status dhsa_sparse_prefill(const dhsa_layout* layout, const void* q, const void* k,
                                const void* v, const int32_t* row_ptr, const int32_t* h_row_ptr,
                                int64_t nnz, const int32_t* block_idx, float softmax_scale,
                                void* out, float* lse, void* stream);

/* ---- Online chunking (this library's own rule, an extension: the pages
 * claim online variable-length chunking as the step before the summaries -
 * "Long-Context Modeling with Dynamic Hierarchical Sparse Attention for
 * On-Device LLMs", Abstract and Innovation; ICML 2026 page, Abstract - but
 * state no rule).  The rule: a cut may fall between adjacent tokens whose key
 * rows point in different directions, and chunks hold between lo and hi
 * tokens.  Its output feeds dhsa_layout (copy cu_chunks / seq_chunk_start to
 * the host for the mirrors). */

/* Step 1, adjacent key similarity.  For every token t of sequence b:
 *   sim[t] = cos(k[t-1, :, :], k[t, :, :])    over all KV heads of the two rows
 *            (fp32 accumulation), or 1 when t is the first token of its
 *            sequence or either row is all zeros;
 *   bit (t mod 64) of cut_bits[t / 64] = (sim[t] < tau).
 *   cu_seqlens    device [B+1] token offsets; h_cu_seqlens its host mirror
 *                 (required: validated like dhsa_layout's)
 *   k             device [T, Hkv, d], dtype DHSA_BF16 or DHSA_F32, 16-byte aligned;
 *                 Hkv * d must be a multiple of 8 (bf16) or 4 (fp32) and at most
 *                 4096 (bf16) or 2048 (fp32): a row is 16-byte loads, at most 8 per lane
 *   tau           finite cut threshold
 *   sim           device float[T], written completely
 *   cut_bits      device uint64[ceil(T / 64)], written completely (bits past T are 0)
 * T == 0 launches nothing.  Errors as for the stage calls. */
dhsa_status dhsa_adjacent_similarity(int32_t num_seqs, int32_t total_tokens, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t dtype, const int32_t* cu_seqlens,
                                     const int32_t* h_cu_seqlens, const void* k, float tau, float* sim,
                                     uint64_t* cut_bits, void* stream);

/* Step 2, greedy cut.  Per sequence, from its first token c0: the chunk ends at
 * the first t in [c0 + lo, min(c0 + hi, end of sequence)) whose cut bit is set,
 * else at min(c0 + hi, end); the next chunk starts there.  So every chunk but a
 * sequence's last holds between lo and hi tokens, the last at most hi.
 *   cut_bits         device uint64[ceil(T / 64)] from dhsa_adjacent_similarity
 *   lo, hi           1 <= lo <= hi
 *   cu_chunks        device int32[T + 1] (capacity): entries 0..C written,
 *                    cu_chunks[0] = 0, cu_chunks[C] = T
 *   seq_chunk_start  device int32[B + 1], written
 *   num_chunks       device int32[1]: C
 * One workgroup walks the sequences in order (the cut is sequential by nature);
 * it stages the bitmap in 64 KB of LDS at a time. */
dhsa_status dhsa_chunk_boundaries(int32_t num_seqs, int32_t total_tokens, const int32_t* cu_seqlens,
                                  const int32_t* h_cu_seqlens, const uint64_t* cut_bits, int32_t lo, int32_t hi,
                                  int32_t* cu_chunks, int32_t* seq_chunk_start, int32_t* num_chunks,
                                  void* stream);

/* ---- Decode: one new token per sequence, against the kept structure (an
 * extension; the pages evaluate prefill only - "Long-Context Modeling with
 * Dynamic Hierarchical Sparse Attention for On-Device LLMs", Abstract; ICML 2026
 * page, Abstract - and describe the method as online).  This library's reading:
 * the new token joins the open (last) chunk unless the chunking rule above cuts
 * before it ((t - c0 >= lo and cos(K[t-1], K[t]) < tau) or t - c0 >= hi); a
 * chunk's key summary (sum of its key rows / sqrt(size)) is kept when it closes;
 * the open chunk's query summary so far, (sum of q over c0..t) / sqrt(t - c0 + 1),
 * scores the closed chunks; the top-k by (score desc, chunk asc) plus the open
 * chunk are kept; the token attends exactly to their tokens up to itself.  At a
 * chunk's last token this equals prefill at that token.
 *
 * The state is the caller's (device memory, sizes as shown; B sequences,
 * capacity L tokens and C closed chunks each). */
typedef struct dhsa_decode_state {
  int32_t num_seqs;          /* B >= 1                                            */
  int32_t num_q_heads;       /* Hq                                                */
  int32_t num_kv_heads;      /* Hkv, Hq % Hkv == 0                                */
  int32_t head_dim;          /* d: 64, 128, 256 (bf16) or 64, 128 (fp32)          */
  int32_t dtype;             /* dhsa_dtype of the cache, q, k, v, out             */
  int32_t max_tokens;        /* 1 <= L <= 2^20: cache capacity per sequence       */
  int32_t max_chunks;        /* C, 1 <= C <= 8192: closed chunks per sequence     */
  void* k_cache;             /* [B, L, Hkv, d]                                    */
  void* v_cache;             /* [B, L, Hkv, d]                                    */
  int32_t* seq_len;          /* [B] tokens in the cache                           */
  int32_t* num_closed;       /* [B] closed chunks                                 */
  int32_t* chunk_start;      /* [B, C + 1] chunk starts (token offsets in the
                                sequence); entry num_closed is the open chunk's   */
  float* k_sum;              /* [B, C, Hkv, d] key summaries of closed chunks     */
  float* q_run;              /* [B, Hq, d] sum of q over the open chunk           */
  float* k_run;              /* [B, Hkv, d] sum of k over the open chunk          */
  int32_t* status;           /* [B] 0; 1 once the cache was full, 2 once the chunk
                                table was full: that sequence then stays as it was
                                and its outputs are zeros                          */
} dhsa_decode_state;

/* Workspace bytes dhsa_decode_step needs for this state and budget (host only). */
size_t dhsa_decode_workspace_bytes(const dhsa_decode_state* state, int32_t topk, int32_t grouped);

/* Load the prefix of each sequence from a chunked batch (the layout of the
 * prefill calls; B equal to the state's): key/value rows into the cache, key
 * summaries of every chunk but each sequence's last, which becomes the open
 * chunk (its q and k sums are kept), counters set, status cleared.  q [T, Hq, d],
 * k, v [T, Hkv, d] as in prefill.  The chunks should come from the same rule
 * (dhsa_chunk_boundaries with the lo, hi, tau later given to dhsa_decode_step)
 * for decode to continue it.  Errors: shapes or dtypes differing from the
 * state's, a sequence longer than L or with more than C + 1 chunks. */
dhsa_status dhsa_decode_load_prefix(const dhsa_decode_state* state, const dhsa_layout* prefix, const void* q,
                                    const void* k, const void* v, void* stream);

/* One decode step for every sequence: append token (q [B, Hq, d], k, v [B, Hkv, d]),
 * then write out [B, Hq, d] (its attention output, dtype of the state).
 *   lo, hi, tau     the chunking rule (1 <= lo <= hi, tau finite)
 *   topk            closed chunks kept per row, 0 <= topk <= 1023 (a row may
 *                   have up to max_chunks closed chunks to choose from)
 *   grouped         0: routing per query head; 1: once per KV head (group-summed
 *                   query summaries, the same kept chunks for the group)
 *   softmax_scale   > 0
 *   kept            optional device int32 [B, Hq, topk]: the kept closed chunks,
 *                   ascending, -1 padded (NULL: not written)
 *   workspace       device, >= dhsa_decode_workspace_bytes(state, topk, grouped),
 *                   256-byte aligned; contents are scratch between calls */
dhsa_status dhsa_decode_step(const dhsa_decode_state* state, const void* q, const void* k, const void* v,
                             int32_t lo, int32_t hi, float tau, int32_t topk, int32_t grouped,
                             float softmax_scale, void* out, int32_t* kept, void* workspace,
                             size_t workspace_bytes, void* stream);

/* The decode step above for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): same arguments, results and errors as dhsa_decode_step, but the
 * step's scratch is a static device array inside the library, of
 * DHSA_NOALLOC_SCRATCH_BYTES, instead of a caller workspace.  Every GPU the
 * library runs on holds its own copy of that array from the first call there
 * until the process ends; the call allocates nothing (no hipMalloc, no
 * allocating library routine) and never synchronises.
 *   Errors, besides those of dhsa_decode_step: DHSA_ERR_WORKSPACE when this
 *   state and budget need more scratch than the array holds (the bytes
 *   dhsa_decode_workspace_bytes reports must not exceed
 *   DHSA_NOALLOC_SCRATCH_BYTES); DHSA_ERR_UNSUPPORTED when `stream` belongs to
 *   a GPU other than the current one (the scratch used is the current GPU's).
 *   Calls on one GPU share its array: calls that may overlap in time (on
 *   different streams or from different threads) race and must not be made;
 *   calls in one stream's order are safe.  Nothing in the array needs to start
 *   at zero: every value a step uses was written earlier in the same step (the
 *   combine also loads partial-state slots that no attention wave wrote in this
 *   step, and discards them unused).  The first call on a GPU looks up the
 *   array's address and the attention kernel's occupancy there; a graph capture
 *   should come after a first call made outside it. */
#define DHSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
dhsa_status dhsa_decode_step_noalloc(const dhsa_decode_state* state, const void* q, const void* k,
                                     const void* v, int32_t lo, int32_t hi, float tau, int32_t topk,
                                     int32_t grouped, float softmax_scale, void* out, int32_t* kept,
                                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DHSA_H */
