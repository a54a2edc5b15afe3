"""CPU oracle for an online chunk-boundary rule (a design of this project, not of the pages).

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of bench.py may import this module; the product path never
imports, links or calls it, and it imports nothing from the product path.

The pages claim online variable-length chunking of the sequence as the step
before chunk summaries ([P2] "Long-Context Modeling with Dynamic Hierarchical
Sparse Attention for On-Device LLMs", Abstract and Innovation: the sequence is
split into variable-length chunks; [P3] the ICML 2026 page, Abstract: dynamic
chunking) but state no rule.  The rule here is our own plain one, labelled as
such everywhere it appears:

  * adjacent similarity: sim[t] = cos(K[t-1], K[t]) over the concatenation of
    all KV heads of the two key rows, for t inside a sequence; sim = 1 at a
    sequence's first token (there is no predecessor) and where either row is
    all zeros (no direction to compare);
  * greedy cut: a chunk starting at c0 in a sequence ending at e ends at the
    first t in [c0 + lo, min(c0 + hi, e)) with sim[t] < tau (a new chunk
    starts at t); if there is none it ends at min(c0 + hi, e).  So every chunk
    but a sequence's last has between lo and hi tokens, and the last has at
    most hi.

Precision: sim is computed in float64 and rounded to float32, and the
comparison with tau is taken in float32, because the GPU path computes sim in
float32 and takes the cut decision on it.
"""
from __future__ import annotations

import numpy as np


def adjacent_similarity(k, cu_seqlens) -> np.ndarray:
    """sim[t] for every token, float32 ``[T]`` (see the module docstring).  ``k`` is ``[T, Hkv, d]``."""
    k = np.asarray(k)
    T = k.shape[0]
    rows = k.reshape(T, -1).astype(np.float64)
    sim = np.ones(T, np.float64)
    cs = np.asarray(cu_seqlens, np.int64)
    for b in range(cs.size - 1):
        for t in range(int(cs[b]) + 1, int(cs[b + 1])):
            a, c = rows[t - 1], rows[t]
            na, nc = float(np.dot(a, a)), float(np.dot(c, c))
            if na > 0.0 and nc > 0.0:
                sim[t] = float(np.dot(a, c)) / np.sqrt(na * nc)
    return sim.astype(np.float32)


def chunk_boundaries(sim, cu_seqlens, lo: int, hi: int, tau: float):
    """Greedy cut of every sequence; returns ``(cu_chunks [C+1], seq_chunk_start [B+1])`` int32."""
    if not (1 <= lo <= hi):
        raise ValueError("need 1 <= lo <= hi")
    sim = np.asarray(sim, np.float32)
    tau32 = np.float32(tau)
    cs = np.asarray(cu_seqlens, np.int64)
    cu_chunks, seq_chunk_start = [0], [0]
    for b in range(cs.size - 1):
        s, e = int(cs[b]), int(cs[b + 1])
        c0 = s
        while c0 < e:
            end = min(c0 + hi, e)
            cut = end
            for t in range(c0 + lo, end):
                if sim[t] < tau32:
                    cut = t
                    break
            cu_chunks.append(cut)
            c0 = cut
        seq_chunk_start.append(len(cu_chunks) - 1)
    return np.array(cu_chunks, np.int32), np.array(seq_chunk_start, np.int32)
