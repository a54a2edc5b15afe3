"""The parity comparator (tests/parity.py) against planted disagreements (CPU).

The GPU tests accept a kept set that differs from the oracle's only by swaps of chunks whose oracle
scores lie within the tie band, and reject everything else.  Here the comparator is fed the oracle's
own lists with planted changes: a swap inside the band, a swap outside it, a row out of order, a row
without its diagonal, a chunk of another sequence, a row of the wrong length; and, under a token budget,
a list that exceeds the budget, one that drops a clearly better chunk and one that stops while a
candidate still fits.  Each must be classed as planted.
"""
import numpy as np

import oracle
from parity import compare_kept_sets, compare_token_rows, rows_with_swaps

C_SEQ = (9, 7)                                   # chunks per sequence


def _routing(topk=3, seed=0):
    rng = np.random.default_rng(seed)
    C = sum(C_SEQ)
    Hq, Hkv, d = 4, 2, 8
    qs = rng.standard_normal((C, Hq, d)).astype(np.float32)
    ks = rng.standard_normal((C, Hkv, d)).astype(np.float32)
    sc = np.array([0, C_SEQ[0], C], np.int64)
    rp, bidx, S = oracle.route(qs, ks, sc, np.full(C, topk, np.int32))
    return rp, bidx, S.copy(), sc


def _row_with_dropped(rp, bidx, sc, h=1):
    """A row of head h in the first sequence that keeps some earlier chunks and drops others."""
    for i in range(C_SEQ[0]):
        kept = [j for j in bidx[h, rp[i]:rp[i + 1]] if j != i]
        if kept and len(kept) < i:
            return h, i
    raise AssertionError("no row with dropped chunks")


def _swap(bidx, rp, S, h, i):
    """Replace the row's lowest-scoring kept chunk by its best dropped one; returns both."""
    row = bidx[h, rp[i]:rp[i + 1]].tolist()
    kept = [j for j in row if j != i]
    dropped = [j for j in range(0, i) if j not in kept]
    lo = min(kept, key=lambda j: S[h, i, j])
    hi = max(dropped, key=lambda j: S[h, i, j])
    new = sorted([j for j in kept if j != lo] + [hi]) + [i]
    g = bidx.copy()
    g[h, rp[i]:rp[i + 1]] = new
    return g, lo, hi


def test_identical_lists_are_equal():
    rp, bidx, S, sc = _routing()
    eq, tol, fails = compare_kept_sets(bidx, bidx, rp, S, sc)
    assert (tol, fails) == (0, []) and eq == bidx.shape[0] * (rp.size - 1)
    assert rows_with_swaps(bidx, bidx, rp) == []


def test_swap_inside_the_tie_band_is_tolerated():
    rp, bidx, S, sc = _routing()
    h, i = _row_with_dropped(rp, bidx, sc)
    g, lo, hi = _swap(bidx, rp, S, h, i)
    S[h, i, hi] = S[h, i, lo] * (1 + 2e-5)       # within 1e-4 relative of each other
    eq, tol, fails = compare_kept_sets(g, bidx, rp, S, sc)
    assert fails == [] and tol == 1
    assert rows_with_swaps(g, bidx, rp) == [(h, i)]


def test_swap_outside_the_tie_band_fails():
    rp, bidx, S, sc = _routing()
    h, i = _row_with_dropped(rp, bidx, sc)
    g, lo, hi = _swap(bidx, rp, S, h, i)
    S[h, i, hi] = S[h, i, lo] - 1e-2 * (abs(S[h, i, lo]) + 1.0)
    _, tol, fails = compare_kept_sets(g, bidx, rp, S, sc)
    assert tol == 0 and len(fails) == 1 and fails[0][:3] == (h, i, "swap outside tie band")


def test_malformed_rows_fail():
    rp, bidx, S, sc = _routing()
    h, i = _row_with_dropped(rp, bidx, sc)
    row = bidx[h, rp[i]:rp[i + 1]].tolist()
    cases = {
        "out of order": row[::-1],
        "no diagonal last": row[1:] + [row[0]],
        "repeated chunk": [row[0]] * (len(row) - 1) + [i],
    }
    for name, bad in cases.items():
        g = bidx.copy()
        g[h, rp[i]:rp[i + 1]] = bad
        _, _, fails = compare_kept_sets(g, bidx, rp, S, sc)
        assert len(fails) == 1 and fails[0][2] == "malformed row", name
    # a chunk of the other sequence in a second-sequence row
    i2 = C_SEQ[0] + C_SEQ[1] - 1
    row2 = bidx[h, rp[i2]:rp[i2 + 1]].tolist()
    g = bidx.copy()
    g[h, rp[i2]:rp[i2 + 1]] = [0] + row2[1:]
    _, _, fails = compare_kept_sets(g, bidx, rp, S, sc)
    assert len(fails) == 1 and fails[0][2] == "malformed row"


def test_two_swaps_one_outside_the_band_fails():
    rp, bidx, S, sc = _routing()
    h = 1
    for i in range(C_SEQ[0]):                    # a row with at least two kept and two dropped chunks
        kept = [j for j in bidx[h, rp[i]:rp[i + 1]] if j != i]
        dropped = [j for j in range(i) if j not in kept]
        if len(kept) >= 2 and len(dropped) >= 2:
            break
    else:
        raise AssertionError("no row with two kept and two dropped chunks")
    lo2 = sorted(kept, key=lambda j: S[h, i, j])[:2]            # the two weakest kept
    hi2 = sorted(dropped, key=lambda j: -S[h, i, j])[:2]        # the two strongest dropped
    g = bidx.copy()
    g[h, rp[i]:rp[i + 1]] = sorted([j for j in kept if j not in lo2] + hi2) + [i]
    S[h, i, hi2[0]] = S[h, i, lo2[1]]            # one pair scores the same
    S[h, i, hi2[1]] = S[h, i, lo2[0]] - 1.0      # the other far apart
    _, tol, fails = compare_kept_sets(g, bidx, rp, S, sc)
    assert tol == 0 and len(fails) == 1 and fails[0][2] == "swap outside tie band"


def _token_routing(seed=1):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 12, size=sum(C_SEQ))
    cc = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    C = lens.size
    Hq, Hkv, d = 2, 1, 8
    qs = rng.standard_normal((C, Hq, d)).astype(np.float32)
    ks = rng.standard_normal((C, Hkv, d)).astype(np.float32)
    sc = np.array([0, C_SEQ[0], C], np.int64)
    budget = np.full(C, 20, np.int32)
    rp, bidx, S = oracle.route_tokens(qs, ks, cc, sc, budget)
    return rp, bidx, S.copy(), sc, cc, budget


def test_token_rows_identical_and_planted():
    rp, bidx, S, sc, cc, budget = _token_routing()
    eq, tol, fails = compare_token_rows(bidx, bidx, rp, S, sc, cc, budget)
    assert (tol, fails) == (0, [])
    lens = np.diff(cc)
    # a row that keeps some but not all of its earlier chunks, with room after them (-1 padding) and a
    # dropped chunk that does not fit beside the kept ones
    found = None
    for h in range(bidx.shape[0]):
        for i in range(2, C_SEQ[0]):
            row = bidx[h, rp[i]:rp[i + 1]].tolist()
            kept = row[:row.index(i)]
            dropped = [j for j in range(i) if j not in kept]
            over = [j for j in dropped if int(lens[kept].sum() + lens[j]) > int(budget[i])]
            if kept and over and len(kept) + 2 <= len(row):
                found = (h, i, row, kept, dropped, over)
                break
        if found:
            break
    assert found, "no row to plant in"
    h, i, row, kept, dropped, over = found
    pad = len(row) - len(kept) - 1

    def planted(new_kept):
        g = bidx.copy()
        g[h, rp[i]:rp[i + 1]] = sorted(new_kept) + [i] + [-1] * (len(row) - len(new_kept) - 1)
        return g

    # over the budget: the kept chunks plus a dropped one that does not fit beside them
    _, _, fails = compare_token_rows(planted(kept + [over[0]]), bidx, rp, S, sc, cc, budget)
    assert len(fails) == 1
    # dropping the best kept chunk for nothing: the best dropped one would still fit -> not a prefix
    best = max(kept, key=lambda j: S[h, i, j])
    _, _, fails = compare_token_rows(planted([j for j in kept if j != best]), bidx, rp, S, sc, cc, budget)
    assert len(fails) == 1
    # a missing diagonal
    g = bidx.copy()
    g[h, rp[i]:rp[i + 1]] = kept + [-1] * (pad + 1)
    _, _, fails = compare_token_rows(g, bidx, rp, S, sc, cc, budget)
    assert len(fails) == 1 and fails[0][2] == "no diagonal"
