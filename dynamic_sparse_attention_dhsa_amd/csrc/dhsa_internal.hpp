// Internal declarations shared by the C-ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dhsa.h"

#define DHSA_MAX_WORDS (DHSA_MAX_CHUNKS_PER_SEQ / 32)

namespace dhsa {

// Layout facts derived on the host from the validated host mirrors.
struct Plan {
  int32_t B, T, C, Hq, Hkv, d, dtype;
  const int32_t* cu_seqlens;       // device
  const int32_t* cu_chunks;        // device
  const int32_t* seq_chunk_start;  // device
  int32_t max_chunk_len;           // longest chunk (tokens)
  int32_t max_chunks_per_seq;      // most chunks in one sequence
  const int32_t* h_cu_chunks;      // host mirror of cu_chunks (valid during the call)
};

// Stage 1: q_sum / k_sum (fp32).
hipError_t launch_summarize(const Plan& p, const void* q, const void* k, float* q_sum, float* k_sum,
                            hipStream_t stream);

// Stage 2: kept key-chunk lists.  The main routing kernel holds up to kRouteRegCand candidates
// of a row in registers; `wide_rows` tells whether some row with more candidates than that keeps
// some but not all of them (those rows take the general sorting kernel).
constexpr int kRouteRegCand = 1024;
hipError_t launch_route(const Plan& p, const float* q_sum, const float* k_sum, const int32_t* row_ptr,
                        int64_t nnz, int32_t* block_idx, bool wide_rows, bool grouped, hipStream_t stream);

// Stage 2 under a token budget (device token_budget [C]); rows sized by dhsa_route_plan_tokens.
// `wide_rows`: some row with more candidates than the registers hold keeps some but not all of them.
hipError_t launch_route_tokens(const Plan& p, const float* q_sum, const float* k_sum, const int32_t* token_budget,
                               const int32_t* row_ptr, int64_t nnz, int32_t* block_idx, bool wide_rows, bool grouped,
                               hipStream_t stream);

// Stage 3: block-sparse causal prefill.
hipError_t launch_prefill_bf16(const Plan& p, const void* q, const void* k, const void* v,
                               const int32_t* row_ptr, int64_t nnz, const int32_t* block_idx,
                               float softmax_scale, void* out, float* lse, hipStream_t stream);
hipError_t launch_prefill_f32(const Plan& p, const void* q, const void* k, const void* v,
                              const int32_t* row_ptr, int64_t nnz, const int32_t* block_idx,
                              float softmax_scale, void* out, float* lse, hipStream_t stream);

// Online chunking (this library's own boundary rule).  A key row is read in at most kSimMaxPieces
// 16-byte pieces (8 per lane).
constexpr int kSimMaxPieces = 512;
hipError_t launch_adjacent_similarity(int B, int ntok, int W, int dtype, const int32_t* cu_seqlens, const void* k,
                                      float tau, float* sim, uint64_t* cut_bits, hipStream_t stream);
hipError_t launch_chunk_walk(int B, int ntok, const int32_t* cu_seqlens, const uint64_t* cut_bits, int lo, int hi,
                             int32_t* cu_chunks, int32_t* seq_chunk_start, int32_t* num_chunks, hipStream_t stream);

// Decode (one new token per sequence against the kept structure).
constexpr int kDecodeSlice = 128;                 // kept tokens a split-K attention wave stages at a time
constexpr int kDecodeMaxChunks = DHSA_MAX_CHUNKS_PER_SEQ;   // closed chunks per sequence (scores in LDS)
constexpr int kDecodeMaxTopk = 1024;              // topk < this: the kept list of a row
constexpr int kDecodeMaxTokens = 1 << 20;         // cache capacity per sequence, at most
constexpr int kDecodeGridSlices = 128;            // attention waves (split-K partial states) per row, at most
constexpr int kPartHead = 4;                       // floats before o in a split-K partial state (m, l, unused)
struct DecodeDims {
  int32_t B, Hq, Hkv, d, dtype, L, Cmax;
};
struct DecodePtrs {                               // the caller's state (device)
  void* k_cache;
  void* v_cache;
  int32_t* seq_len;
  int32_t* num_closed;
  int32_t* chunk_start;
  float* k_sum;
  float* q_run;
  float* k_run;
  int32_t* status;
};
struct DecodeWork {                               // carved from the caller's workspace
  int32_t* urow;                                  // [B * rows, L]: cache row of each kept token, kept order
  int32_t* ntok;                                  // [B * rows]
  float* part;                                    // [B * Hq * NS, d + 2]: one partial state per attention wave
  int32_t* pend;                                  // [B, 4]: the token's append, committed by the combine
  int NS;                                         // partial states per (sequence, q head)
};
hipError_t launch_decode_step(const DecodeDims& p, const DecodePtrs& s, const void* q, const void* k, const void* v,
                              int lo, int hi, float tau, int topk, bool grouped, float scale, void* out,
                              int32_t* kept, const DecodeWork& w, hipStream_t stream);
hipError_t launch_decode_load(const DecodeDims& p, const DecodePtrs& s, const Plan& pl, const void* q, const void* k,
                              const void* v, hipStream_t stream);

// Scratch of the decode step that allocates nothing: a static device array of kNoAllocScratchBytes in
// decode.hip, one copy per GPU.  Returns the device address of the current GPU's copy (looked up with
// hipGetSymbolAddress on the first call on that GPU, then cached).
constexpr size_t kNoAllocScratchBytes = DHSA_NOALLOC_SCRATCH_BYTES;
constexpr int kNoAllocMaxDevices = 64;
hipError_t decode_noalloc_scratch(void** ptr);

// Device helpers ----------------------------------------------------------------------------

// Index of the sequence containing chunk c: the last b with seq_chunk_start[b] <= c.
__device__ inline int seq_of_chunk(const int32_t* __restrict__ seq_chunk_start, int B, int c) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (seq_chunk_start[mid] <= c) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace dhsa
