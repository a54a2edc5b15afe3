"""CPU oracle for routing with a token budget (instead of a chunk count).

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of bench.py may import this module; the product path never
imports, links or calls it, and it imports nothing from the product path.

The pages keep "token-level interactions" chosen by importance ([P2] "Long-
Context Modeling with Dynamic Hierarchical Sparse Attention for On-Device
LLMs", Abstract) and report memory savings ([P2] Abstract; [P3] ICML 2026
page, Abstract) without fixing how much is kept.  Besides the chunk-count
budget of the main path, a budget in tokens is the other plain reading; this
module is that reading, stated in full:

  * query chunk i with token budget b_i ranks the earlier chunks of its
    sequence by (score desc, chunk asc), exactly as the chunk-count rule, and
    keeps the longest prefix of that ranking whose chunk lengths sum to at
    most b_i (it stops at the first chunk that does not fit), plus itself;
  * the number kept then depends on the scores, so the CSR rows of the block
    list get the largest count any ranking could keep, m_max(i) + 1, where
    m_max(i) is how many of the shortest earlier chunks fit in b_i; a row's
    kept chunks come first, ascending, the diagonal after them, and -1 pads
    the rest.
"""
from __future__ import annotations

import numpy as np

from .dhsa_oracle import chunk_scores, chunk_sequence, group_chunk_scores


def route_plan_tokens(cu_chunks, seq_chunk_start, token_budget):
    """Row capacities for a token budget: ``(row_ptr [C+1] int32, nnz)``."""
    cc = np.asarray(cu_chunks, np.int64)
    sc = np.asarray(seq_chunk_start, np.int64)
    tb = np.asarray(token_budget, np.int64)
    C = int(sc[-1])
    if tb.shape != (C,) or np.any(tb < 0):
        raise ValueError("token_budget needs one non-negative entry per chunk")
    lens = np.diff(cc)
    seq = chunk_sequence(sc)
    counts = np.empty(C, np.int64)
    for i in range(C):
        earlier = np.sort(lens[sc[seq[i]]:i])
        counts[i] = int(np.searchsorted(np.cumsum(earlier), tb[i], side="right")) + 1
    row_ptr = np.zeros(C + 1, np.int64)
    row_ptr[1:] = np.cumsum(counts)
    return row_ptr.astype(np.int32), int(row_ptr[-1])


def select_key_chunks_tokens(scores_row, lens, first: int, i: int, budget: int) -> np.ndarray:
    """Kept chunks of query chunk i under a token budget, ascending, the diagonal last."""
    cand = np.arange(first, i, dtype=np.int64)
    s = np.asarray(scores_row, np.float32)[first:i]
    order = np.lexsort((cand, -s))              # ranking: score desc, then chunk asc
    cum = np.cumsum(np.asarray(lens, np.int64)[cand[order]])
    m = int(np.searchsorted(cum, budget, side="right"))   # longest prefix with sum <= budget
    return np.concatenate([np.sort(cand[order[:m]]), [i]]).astype(np.int32)


def route_tokens(q_sum, k_sum, cu_chunks, seq_chunk_start, token_budget, grouped: bool = False):
    """Routing under a token budget: ``(row_ptr, block_idx [Hq, nnz] with -1 padding, scores)``."""
    cc = np.asarray(cu_chunks, np.int64)
    lens = np.diff(cc)
    S = (group_chunk_scores if grouped else chunk_scores)(q_sum, k_sum, seq_chunk_start)
    Hq = np.asarray(q_sum).shape[1]
    R, C, _ = S.shape
    G = Hq // R
    row_ptr, nnz = route_plan_tokens(cc, seq_chunk_start, token_budget)
    sc = np.asarray(seq_chunk_start, np.int64)
    seq = chunk_sequence(sc)
    block_idx = np.full((Hq, nnz), -1, np.int32)
    for r in range(R):
        for i in range(C):
            kept = select_key_chunks_tokens(S[r, i], lens, int(sc[seq[i]]), i, int(token_budget[i]))
            block_idx[r * G:(r + 1) * G, row_ptr[i]:row_ptr[i] + kept.size] = kept
    return row_ptr, block_idx, S
