"""Comparison helpers for GPU-vs-oracle parity (test infrastructure).

Kept-set rule: a GPU row must be ascending, unique, inside the query chunk's
sequence, end with the diagonal, and have the oracle row's length.  Where the
sets differ, the chunks only the oracle keeps and the chunks only the GPU
keeps are each sorted by ORACLE score and paired in order; every pair must
score within 1e-4 relative of each other (the GPU sums the fp32 dot product in
another order, so near-equal scores may swap).
"""
from __future__ import annotations

import numpy as np

REL_TIE = 1e-4
ATOL_BF16 = 2e-2
ATOL_F32 = 1e-4


def chunk_seq_first(seq_chunk_start) -> np.ndarray:
    sc = np.asarray(seq_chunk_start, np.int64)
    seq = np.repeat(np.arange(sc.size - 1), np.diff(sc))
    return sc[seq]


def compare_kept_sets(gpu_bidx: np.ndarray, ora_bidx: np.ndarray, row_ptr: np.ndarray, scores: np.ndarray,
                      seq_chunk_start, heads=None, rel: float = REL_TIE):
    """Returns (rows_equal, rows_tolerated, failures) over the requested heads (all by default)."""
    first = chunk_seq_first(seq_chunk_start)
    Hq = gpu_bidx.shape[0]
    C = row_ptr.size - 1
    equal = tolerated = 0
    failures = []
    for h in (range(Hq) if heads is None else heads):
        for i in range(C):
            g = gpu_bidx[h, row_ptr[i]:row_ptr[i + 1]]
            o = ora_bidx[h, row_ptr[i]:row_ptr[i + 1]]
            if np.array_equal(g, o):
                equal += 1
                continue
            gl = g.tolist()
            if gl != sorted(set(gl)) or gl[-1] != i or min(gl) < first[i] or max(gl) > i:
                failures.append((h, i, "malformed row", gl, o.tolist()))
                continue
            only_o = sorted(set(o.tolist()) - set(gl), key=lambda j: -scores[h, i, j])
            only_g = sorted(set(gl) - set(o.tolist()), key=lambda j: -scores[h, i, j])
            ok = len(only_o) == len(only_g)
            for a, b in zip(only_o, only_g):
                sa, sb = float(scores[h, i, a]), float(scores[h, i, b])
                if not abs(sa - sb) <= rel * max(abs(sa), abs(sb)):
                    ok = False
            if ok:
                tolerated += 1
            else:
                failures.append((h, i, "swap outside tie band", gl, o.tolist(),
                                 [(j, float(scores[h, i, j])) for j in only_o + only_g]))
    return equal, tolerated, failures


def rows_with_swaps(gpu_bidx, ora_bidx, row_ptr):
    """(h, i) rows whose kept sets differ (after a tolerated swap)."""
    out = []
    for h in range(gpu_bidx.shape[0]):
        for i in range(row_ptr.size - 1):
            if not np.array_equal(gpu_bidx[h, row_ptr[i]:row_ptr[i + 1]], ora_bidx[h, row_ptr[i]:row_ptr[i + 1]]):
                out.append((h, i))
    return out


def compare_token_rows(gpu_bidx: np.ndarray, ora_bidx: np.ndarray, row_ptr: np.ndarray, scores: np.ndarray,
                       seq_chunk_start, cu_chunks, token_budget, heads=None, rel: float = REL_TIE):
    """Kept lists under a token budget.  A GPU row must hold its kept chunks ascending inside the
    query chunk's sequence, then the diagonal, then -1 up to the row's capacity.  Where it differs
    from the oracle row, the GPU set must still be one the prefix rule could give under a ranking
    that reorders only scores within ``rel`` of each other: it fits the budget, no chunk it drops
    scores clearly above one it keeps, and (unless it keeps every candidate) some chunk that could
    come next in such a ranking does not fit.  Returns (rows_equal, rows_tolerated, failures)."""
    first = chunk_seq_first(seq_chunk_start)
    lens = np.diff(np.asarray(cu_chunks, np.int64))
    Hq = gpu_bidx.shape[0]
    C = row_ptr.size - 1
    equal = tolerated = 0
    failures = []

    def close(a, b):
        return abs(a - b) <= rel * max(abs(a), abs(b))

    for h in (range(Hq) if heads is None else heads):
        for i in range(C):
            g = gpu_bidx[h, row_ptr[i]:row_ptr[i + 1]].tolist()
            o = ora_bidx[h, row_ptr[i]:row_ptr[i + 1]].tolist()
            if g == o:
                equal += 1
                continue
            if i not in g:
                failures.append((h, i, "no diagonal", g, o))
                continue
            p = g.index(i)
            kept, pad = g[:p], g[p + 1:]
            if (kept != sorted(set(kept)) or any(j < first[i] or j >= i for j in kept)
                    or any(x != -1 for x in pad)):
                failures.append((h, i, "malformed row", g, o))
                continue
            s = scores[h, i]
            dropped = [j for j in range(int(first[i]), i) if j not in set(kept)]
            ok = int(lens[kept].sum()) <= int(token_budget[i])
            if ok and kept and dropped:
                a = min(kept, key=lambda j: s[j])
                b = max(dropped, key=lambda j: s[j])
                ok = s[a] >= s[b] or close(float(s[a]), float(s[b]))
            if ok and dropped:
                top = max(float(s[j]) for j in dropped)
                nxt = [j for j in dropped if float(s[j]) >= top or close(float(s[j]), top)]
                ok = any(int(lens[kept].sum()) + int(lens[j]) > int(token_budget[i]) for j in nxt)
            if ok:
                tolerated += 1
            else:
                failures.append((h, i, "not a prefix of a tie-band ranking", g, o))
    return equal, tolerated, failures
