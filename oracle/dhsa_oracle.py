"""CPU oracle for DHSA chunk-routed sparse causal prefill.

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of bench.py may import this module.  The product path
(the ``dynamic_sparse_attention_dhsa_amd`` package and its HIP library) never
imports, links or calls it, and it imports nothing from the product path.

What it follows (the pages are two versions of one paper):
  [P2] "Long-Context Modeling with Dynamic Hierarchical Sparse Attention for
       On-Device LLMs" (newx.sg paper page): Abstract, AI Summary, Innovation.
  [P3] "Long-Context Modeling with Dynamic Hierarchical Sparse Attention for
       Memory-Constrained LLM Inference" (ICML 2026 spotlight page): Abstract.
The steps, in the pages' order: the sequence is split into variable-length
chunks; each chunk gets a representation by aggregating its token vectors,
the mean times sqrt(n) for a chunk of n tokens [P2 Abstract,
Innovation]; chunk-level similarity is computed [P2 Abstract] causally
[P3 Abstract]; the chunk scores are upsampled to token level and the
resulting importance decides which token interactions are kept [P2 Abstract,
AI Summary; P3 Abstract]; softmax attention runs over the kept interactions.

Parameters the pages leave open are explicit inputs: chunk boundaries
(``cu_chunks``), a per-query-chunk budget of top-k earlier key chunks
(``topk``), the diagonal chunk always kept, ties to the lower chunk index.

Precision: float64 arithmetic, except where floating point decides an
integer.  Summaries are computed in float64 and stored as float32, and chunk
scores are rounded to float32 before ranking, because the GPU path stores
summaries and takes the top-k decision in float32.

Every function here is pinned by tests in tests/oracle_pins.py against
closed forms, brute force, library routines and hand-worked examples.
"""
from __future__ import annotations

from typing import Iterable, Optional, Tuple

import numpy as np


# ----------------------------------------------------------------------------- layout

def validate_layout(cu_seqlens, cu_chunks, seq_chunk_start) -> None:
    """Chunks must tile each sequence exactly, with at least one token each."""
    cs = np.asarray(cu_seqlens, np.int64)
    cc = np.asarray(cu_chunks, np.int64)
    sc = np.asarray(seq_chunk_start, np.int64)
    if cs.ndim != 1 or cc.ndim != 1 or sc.ndim != 1 or cs.size < 1 or cc.size < 1:
        raise ValueError("layout arrays must be 1-D and non-empty")
    if cs.size != sc.size:
        raise ValueError("cu_seqlens and seq_chunk_start need B+1 entries each")
    if cs[0] != 0 or cc[0] != 0 or sc[0] != 0:
        raise ValueError("offsets must start at 0")
    if sc[-1] != cc.size - 1 or cc[-1] != cs[-1]:
        raise ValueError("chunk layout does not cover the tokens")
    if np.any(np.diff(cs) < 0) or np.any(np.diff(sc) < 0):
        raise ValueError("sequence offsets must be non-decreasing")
    if np.any(np.diff(cc) < 1):
        raise ValueError("every chunk needs at least one token")
    for b in range(cs.size - 1):
        if cc[sc[b]] != cs[b] or cc[sc[b + 1]] != cs[b + 1]:
            raise ValueError(f"chunks of sequence {b} do not match its token range")


def chunk_sequence(seq_chunk_start) -> np.ndarray:
    """Sequence id of every chunk."""
    sc = np.asarray(seq_chunk_start, np.int64)
    return np.repeat(np.arange(sc.size - 1), np.diff(sc))


# ----------------------------------------------------------------------------- step 1: summaries

def chunk_summaries(x, cu_chunks) -> np.ndarray:
    """Length-normalised chunk representation, one per (chunk, head).

    [P2 Abstract, Innovation]: the token vectors of a chunk are averaged and
    the average is multiplied by sqrt(chunk size), so that chunk length does
    not bias the scores.  ``x`` is ``[T, H, d]``; returns float32 ``[C, H, d]``.
    """
    x = np.asarray(x)
    cc = np.asarray(cu_chunks, np.int64)
    C = cc.size - 1
    out = np.empty((C,) + x.shape[1:], np.float64)
    for c in range(C):
        s, e = cc[c], cc[c + 1]
        n = e - s
        mean = x[s:e].astype(np.float64).sum(axis=0) / n
        out[c] = mean * np.sqrt(n)
    return out.astype(np.float32)


# ----------------------------------------------------------------------------- step 2: chunk scores

def chunk_scores(q_sum, k_sum, seq_chunk_start) -> np.ndarray:
    """Causal chunk-to-chunk similarity, ``[Hq, C, C]`` float32.

    [P2 Abstract] chunk-level similarity; [P3 Abstract] routing is causal.
    The similarity of query chunk i and key chunk j is the dot product of
    their representations, for j <= i in the same sequence; the KV head of
    query head h is ``h // (Hq // Hkv)``.  Entries outside the causal
    same-sequence region are NaN.  Products are summed in float64 and the
    result rounded to float32, the precision the top-k decision is taken in.
    """
    qs = np.asarray(q_sum, np.float64)
    ks = np.asarray(k_sum, np.float64)
    C, Hq, _ = qs.shape
    Hkv = ks.shape[1]
    G = Hq // Hkv
    sc = np.asarray(seq_chunk_start, np.int64)
    S = np.full((Hq, C, C), np.nan, np.float32)
    for b in range(sc.size - 1):
        c0, c1 = sc[b], sc[b + 1]
        for h in range(Hq):
            full = qs[c0:c1, h, :] @ ks[c0:c1, h // G, :].T
            causal = np.tril(np.ones((c1 - c0, c1 - c0), bool))
            S[h, c0:c1, c0:c1] = np.where(causal, full, np.nan).astype(np.float32)
    return S


def group_chunk_scores(q_sum, k_sum, seq_chunk_start) -> np.ndarray:
    """Causal chunk similarity of each GQA group, ``[Hkv, C, C]`` float32.

    The pages do not fix the granularity at which grouped-query heads are
    routed.  This variant routes once per KV head: the score of query chunk i
    and key chunk j for KV head g is the sum, over the query heads h of g's
    group, of their similarities q_sum[i,h] . k_sum[j,g] [P2 Abstract:
    chunk-level similarity; P3 Abstract: causal].  Summed in float64, rounded
    once to float32; NaN outside the causal same-sequence region.
    """
    qs = np.asarray(q_sum, np.float64)
    ks = np.asarray(k_sum, np.float64)
    C, Hq, _ = qs.shape
    Hkv = ks.shape[1]
    G = Hq // Hkv
    sc = np.asarray(seq_chunk_start, np.int64)
    S = np.full((Hkv, C, C), np.nan, np.float32)
    for b in range(sc.size - 1):
        c0, c1 = sc[b], sc[b + 1]
        lower = np.tri(c1 - c0, dtype=bool)         # j <= i
        for g in range(Hkv):
            full = np.zeros((c1 - c0, c1 - c0))
            for h in range(g * G, (g + 1) * G):
                full += qs[c0:c1, h, :] @ ks[c0:c1, g, :].T
            S[g, c0:c1, c0:c1] = np.where(lower, full, np.nan).astype(np.float32)
    return S


# ----------------------------------------------------------------------------- step 3: keep decision

def route_plan(seq_chunk_start, topk) -> Tuple[np.ndarray, int]:
    """CSR row pointers shared by all heads: row i keeps min(topk[i], i_loc) + 1 chunks."""
    sc = np.asarray(seq_chunk_start, np.int64)
    tk = np.asarray(topk, np.int64)
    C = int(sc[-1])
    if tk.shape != (C,) or np.any(tk < 0):
        raise ValueError("topk needs one non-negative entry per chunk")
    seq = chunk_sequence(sc)
    i_loc = np.arange(C) - sc[seq] if C else np.zeros(0, np.int64)
    counts = np.minimum(tk, i_loc) + 1
    row_ptr = np.zeros(C + 1, np.int64)
    row_ptr[1:] = np.cumsum(counts)
    return row_ptr.astype(np.int32), int(row_ptr[-1])


def select_key_chunks(scores_row, first: int, i: int, k: int) -> np.ndarray:
    """Kept key chunks of query chunk i: the diagonal plus the top-k earlier chunks.

    Candidates are the chunks ``first..i-1`` of i's sequence.  They are ranked
    by score (descending), equal scores by chunk id (ascending), and the first
    ``min(k, i - first)`` are kept.  The diagonal chunk i is always kept.
    Returned ascending, so the diagonal comes last.
    """
    cand = np.arange(first, i, dtype=np.int64)
    s = np.asarray(scores_row, np.float32)[first:i]
    order = np.lexsort((cand, -s))          # primary key: -score; secondary: chunk id
    kept = cand[order[:min(k, cand.size)]]
    return np.concatenate([np.sort(kept), [i]]).astype(np.int32)


def route(q_sum, k_sum, seq_chunk_start, topk):
    """Full routing: returns ``(row_ptr [C+1], block_idx [Hq, nnz], scores [Hq, C, C])``."""
    S = chunk_scores(q_sum, k_sum, seq_chunk_start)
    Hq, C, _ = S.shape
    row_ptr, nnz = route_plan(seq_chunk_start, topk)
    sc = np.asarray(seq_chunk_start, np.int64)
    seq = chunk_sequence(sc)
    block_idx = np.empty((Hq, nnz), np.int32)
    for h in range(Hq):
        for i in range(C):
            kept = select_key_chunks(S[h, i], int(sc[seq[i]]), i, int(topk[i]))
            block_idx[h, row_ptr[i]:row_ptr[i + 1]] = kept
    return row_ptr, block_idx, S


def route_grouped(q_sum, k_sum, seq_chunk_start, topk):
    """Routing once per KV head (see ``group_chunk_scores``): every query head of a
    group keeps its group's chunks.  Returns ``(row_ptr [C+1], block_idx [Hq, nnz],
    scores [Hkv, C, C])``, with the same row layout and selection rule as ``route``."""
    S = group_chunk_scores(q_sum, k_sum, seq_chunk_start)
    Hkv, C, _ = S.shape
    Hq = np.asarray(q_sum).shape[1]
    G = Hq // Hkv
    row_ptr, nnz = route_plan(seq_chunk_start, topk)
    sc = np.asarray(seq_chunk_start, np.int64)
    seq = chunk_sequence(sc)
    block_idx = np.empty((Hq, nnz), np.int32)
    for g in range(Hkv):
        for i in range(C):
            kept = select_key_chunks(S[g, i], int(sc[seq[i]]), i, int(topk[i]))
            block_idx[g * G:(g + 1) * G, row_ptr[i]:row_ptr[i + 1]] = kept
    return row_ptr, block_idx, S


def token_importance(scores_h, cu_chunks) -> np.ndarray:
    """Upsample one head's chunk scores to token level, ``[T, T]``.

    [P2 AI Summary, Abstract]: block-level similarity is upsampled to token
    level.  The upsampling is the nearest-neighbour broadcast: token pair
    (t, u) takes the score of (chunk(t), chunk(u)).  Small T only; the
    routing above decides at chunk level, which this broadcast makes
    equivalent (pinned in the tests).
    """
    cc = np.asarray(cu_chunks, np.int64)
    tok_chunk = np.repeat(np.arange(cc.size - 1), np.diff(cc))
    return np.asarray(scores_h)[np.ix_(tok_chunk, tok_chunk)]


def kept_token_mask(row_ptr, block_idx_h, cu_chunks) -> np.ndarray:
    """Token-level keep mask ``[T, T]`` of one head: kept key chunk and causal (u <= t)."""
    cc = np.asarray(cu_chunks, np.int64)
    C = cc.size - 1
    T = int(cc[-1])
    keep_chunk = np.zeros((C, C), bool)
    for i in range(C):
        row = np.asarray(block_idx_h[row_ptr[i]:row_ptr[i + 1]])
        keep_chunk[i, row[row >= 0]] = True     # -1 entries pad rows of variable length
    tok_chunk = np.repeat(np.arange(C), np.diff(cc))
    mask = keep_chunk[np.ix_(tok_chunk, tok_chunk)]
    return mask & (np.arange(T)[None, :] <= np.arange(T)[:, None])


# ----------------------------------------------------------------------------- step 4: attention

def attend(q, k, v, cu_chunks, row_ptr, block_idx, softmax_scale: float,
           heads: Optional[Iterable[int]] = None, chunks: Optional[Iterable[int]] = None):
    """Exact causal softmax attention over the kept token interactions.

    Query token t of chunk i, head h, attends to every key token u <= t that
    lies in a kept key chunk of (h, i); the KV head is ``h // (Hq // Hkv)``.
    Two-pass softmax: logits ``z = scale * q.k``, ``p = exp(z - max z)``,
    ``O = sum(p v) / sum(p)``, ``LSE = max z + log(sum p)``.
    Returns float64 ``O [T, Hq, d]`` and ``LSE [Hq, T]``; rows not requested
    through ``heads``/``chunks`` are NaN.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    cc = np.asarray(cu_chunks, np.int64)
    T, Hq, d = q.shape
    G = Hq // k.shape[1]
    C = cc.size - 1
    O = np.full((T, Hq, d), np.nan)
    LSE = np.full((Hq, T), np.nan)
    heads = range(Hq) if heads is None else heads
    chunks = range(C) if chunks is None else chunks
    for h in heads:
        g = h // G
        for i in chunks:
            s_i, e_i = cc[i], cc[i + 1]
            kept = block_idx[h, row_ptr[i]:row_ptr[i + 1]]
            kept = kept[kept >= 0]              # -1 entries pad rows of variable length
            keys = np.concatenate([np.arange(cc[j], cc[j + 1]) for j in kept])
            qi = q[s_i:e_i, h, :].astype(np.float64)
            Z = softmax_scale * (qi @ k[keys, g, :].astype(np.float64).T)
            visible = keys[None, :] <= np.arange(s_i, e_i)[:, None]
            Z = np.where(visible, Z, -np.inf)
            m = Z.max(axis=1, keepdims=True)
            P = np.exp(Z - m)
            lsum = P.sum(axis=1, keepdims=True)
            O[s_i:e_i, h, :] = (P @ v[keys, g, :].astype(np.float64)) / lsum
            LSE[h, s_i:e_i] = m[:, 0] + np.log(lsum[:, 0])
    return O, LSE


def dense_attention(q, k, v, cu_seqlens, softmax_scale: float):
    """Plain causal GQA attention per sequence (every earlier key kept)."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    cs = np.asarray(cu_seqlens, np.int64)
    T, Hq, d = q.shape
    G = Hq // k.shape[1]
    O = np.zeros((T, Hq, d))
    LSE = np.zeros((Hq, T))
    for b in range(cs.size - 1):
        s, e = cs[b], cs[b + 1]
        if e == s:
            continue
        causal = np.tril(np.ones((e - s, e - s), bool))
        for h in range(Hq):
            Z = softmax_scale * (q[s:e, h].astype(np.float64) @ k[s:e, h // G].astype(np.float64).T)
            Z = np.where(causal, Z, -np.inf)
            m = Z.max(axis=1, keepdims=True)
            P = np.exp(Z - m)
            lsum = P.sum(axis=1, keepdims=True)
            O[s:e, h] = (P @ v[s:e, h // G].astype(np.float64)) / lsum
            LSE[h, s:e] = m[:, 0] + np.log(lsum[:, 0])
    return O, LSE


# ----------------------------------------------------------------------------- whole path

def prefill(q, k, v, cu_seqlens, cu_chunks, seq_chunk_start, topk, softmax_scale: float,
            heads=None, chunks=None, grouped: bool = False):
    """Summaries, routing (per query head, or per KV head when ``grouped``) and sparse
    attention in the pages' order.

    Returns a dict with ``q_sum, k_sum, scores, row_ptr, block_idx, out, lse``.
    """
    validate_layout(cu_seqlens, cu_chunks, seq_chunk_start)
    q_sum = chunk_summaries(q, cu_chunks)
    k_sum = chunk_summaries(k, cu_chunks)
    row_ptr, block_idx, S = (route_grouped if grouped else route)(q_sum, k_sum, seq_chunk_start, topk)
    out, lse = attend(q, k, v, cu_chunks, row_ptr, block_idx, softmax_scale, heads, chunks)
    return dict(q_sum=q_sum, k_sum=k_sum, scores=S, row_ptr=row_ptr, block_idx=block_idx,
                out=out, lse=lse)
