"""Pins that tie the CPU oracle to something other than itself.

Every ``pin_*`` function takes the oracle module as its argument and raises
AssertionError when the oracle disagrees with a closed form, a brute-force
enumeration, a library routine, an invariant or a hand-worked example.
tests/test_oracle_pins.py runs them against the oracle; the mutation test
runs them against deliberately broken copies of it and requires that every
copy fails at least one pin.
"""
from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

from dynamic_sparse_attention_dhsa_amd.workloads import SeqSpec, make_workload

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------- helpers (independent of the oracle)

def _layout_from_lengths(seq_chunk_lens):
    """cu_seqlens, cu_chunks, seq_chunk_start from per-sequence chunk length lists."""
    cu_seqlens, cu_chunks, scs = [0], [0], [0]
    for lens in seq_chunk_lens:
        for n in lens:
            cu_chunks.append(cu_chunks[-1] + n)
        cu_seqlens.append(cu_chunks[-1])
        scs.append(scs[-1] + len(lens))
    return (np.array(cu_seqlens, np.int32), np.array(cu_chunks, np.int32), np.array(scs, np.int32))


def _tok_chunk(cu_chunks):
    out = []
    for c in range(len(cu_chunks) - 1):
        out += [c] * int(cu_chunks[c + 1] - cu_chunks[c])
    return np.array(out, np.int64)


def _chunk_seq(seq_chunk_start):
    out = []
    for b in range(len(seq_chunk_start) - 1):
        out += [b] * int(seq_chunk_start[b + 1] - seq_chunk_start[b])
    return np.array(out, np.int64)


def _small_workload(seed, lens_per_seq=((5, 9, 3, 12, 7, 1, 6),), Hq=4, Hkv=2, d=8, topk=2, dtype="f32"):
    seqs = [SeqSpec(sum(l), ("explicit", list(l)), topk, 0) for l in lens_per_seq]
    return make_workload(seqs, Hq, Hkv, d, dtype, seed=seed)


def _sdpa_causal_fp64(q, k, v, scale):
    """torch's scaled_dot_product_attention on one sequence, KV heads repeated, float64 on the CPU."""
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    qt = torch.from_numpy(np.ascontiguousarray(q, np.float64)).permute(1, 0, 2)
    kt = torch.from_numpy(np.ascontiguousarray(k, np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)
    vt = torch.from_numpy(np.ascontiguousarray(v, np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)
    o = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None], is_causal=True,
                                                         scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def _parse(x):
    if x is None:
        return float("nan")
    if isinstance(x, str):
        if x == "sqrt2":
            return math.sqrt(2.0)
        return float(Fraction(x))
    return float(x)


def _parse_nested(a):
    if isinstance(a, list):
        return [_parse_nested(b) for b in a]
    return _parse(a)


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        g = json.load(f)
    g["scale"] = math.log(2.0) if g["softmax_scale"] == "ln2" else float(g["softmax_scale"])
    for key in ("q", "k", "v"):
        g[key] = np.array(g[key], np.float32)
    return g


GOLDEN_FILES = ("g1_length_norm_two_heads.json", "g2_tie_lower_index.json", "g3_ragged_no_cross_sequence.json")


# ----------------------------------------------------------------------------- pins

def pin_golden(O):
    """Hand-worked examples (tests/golden): every intermediate and final value."""
    for name in GOLDEN_FILES:
        g = load_golden(name)
        ex = g["expected"]
        r = O.prefill(g["q"], g["k"], g["v"], g["cu_seqlens"], g["cu_chunks"], g["seq_chunk_start"],
                      np.array(g["topk"]), g["scale"])
        np.testing.assert_allclose(r["q_sum"], np.array(_parse_nested(ex["q_sum"])), rtol=1e-6, err_msg=name)
        np.testing.assert_allclose(r["k_sum"], np.array(_parse_nested(ex["k_sum"])), rtol=1e-6, err_msg=name)
        np.testing.assert_allclose(r["scores"], np.array(_parse_nested(ex["scores"])), rtol=1e-6,
                                   equal_nan=True, err_msg=name)
        assert list(r["row_ptr"]) == ex["row_ptr"], name
        assert r["block_idx"].tolist() == ex["block_idx"], name
        np.testing.assert_allclose(r["out"], np.array(_parse_nested(ex["out"])), rtol=0, atol=1e-12,
                                   err_msg=name)
        lse_exp = np.log(np.array(_parse_nested(ex["sum_exp"])))
        np.testing.assert_allclose(r["lse"], lse_exp, rtol=0, atol=1e-12, err_msg=name)


def pin_summary_closed_forms(O):
    """n = 1 is the identity; a constant chunk x gives sqrt(n) x; integer inputs match a library segment sum."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((9, 3, 4)).astype(np.float32)
    assert np.array_equal(O.chunk_summaries(x, np.arange(10)), x)
    for n in (1, 2, 3, 4, 9, 16, 100):
        c = rng.integers(-5, 6, size=(1, 2, 4)).astype(np.float32)
        xs = np.repeat(c, n, axis=0)
        got = O.chunk_summaries(xs, np.array([0, n]))
        np.testing.assert_allclose(got[0], (math.sqrt(n) * c[0].astype(np.float64)).astype(np.float32),
                                   rtol=2e-7, atol=0)
    lens = np.array([1, 4, 7, 2, 16, 5, 9])
    cu = np.concatenate([[0], np.cumsum(lens)])
    xi = rng.integers(-8, 9, size=(cu[-1], 2, 6)).astype(np.float32)
    seg = torch.segment_reduce(torch.from_numpy(xi.astype(np.float64)), "sum",
                               lengths=torch.from_numpy(lens), axis=0).numpy()
    ref = seg / np.sqrt(lens)[:, None, None]
    np.testing.assert_allclose(O.chunk_summaries(xi, cu), ref.astype(np.float32), rtol=2e-7, atol=0)


def pin_scores_bruteforce(O):
    """Chunk score = (1/sqrt(n_i n_j)) * sum over token pairs of q.k, from the full token matrix; causal only."""
    w = _small_workload(7, lens_per_seq=((3, 5, 1, 4, 6), (2, 7, 3)), Hq=4, Hkv=2, d=5)
    q, k = w.q_f32().astype(np.float64), w.k_f32().astype(np.float64)
    S = O.chunk_scores(O.chunk_summaries(w.q, w.cu_chunks), O.chunk_summaries(w.k, w.cu_chunks),
                       w.seq_chunk_start)
    tc = _tok_chunk(w.cu_chunks)
    cseq = _chunk_seq(w.seq_chunk_start)
    C = w.total_chunks
    G = w.num_q_heads // w.num_kv_heads
    for h in range(w.num_q_heads):
        full = q[:, h, :] @ k[:, h // G, :].T
        for i in range(C):
            for j in range(C):
                if cseq[i] != cseq[j] or j > i:
                    assert np.isnan(S[h, i, j]), (h, i, j)
                    continue
                ni, nj = (tc == i).sum(), (tc == j).sum()
                ref = full[np.ix_(tc == i, tc == j)].sum() / math.sqrt(ni * nj)
                assert abs(S[h, i, j] - ref) <= 1e-5 * max(1.0, abs(ref)), (h, i, j, S[h, i, j], ref)


def pin_topk_bruteforce(O):
    """Kept set = the best-sum k-subset of earlier chunks, lexicographically smallest among equal sums.

    Summaries are integer-valued, so scores and subset sums are exact; half the rows carry forced ties.
    """
    rng = np.random.default_rng(3)
    for trial in range(6):
        lens = [[1] * int(rng.integers(2, 10)) for _ in range(int(rng.integers(1, 3)))]
        cu_seqlens, cu_chunks, scs = _layout_from_lengths(lens)
        C = int(scs[-1])
        Hq, Hkv, d = 2, 1, 3
        lo, hi = (-1, 2) if trial % 2 else (-4, 5)          # narrow range -> many exact ties
        qs = rng.integers(lo, hi, size=(C, Hq, d)).astype(np.float32)
        ks = rng.integers(lo, hi, size=(C, Hkv, d)).astype(np.float32)
        topk = rng.integers(0, 5, size=C).astype(np.int32)
        row_ptr, bidx, _ = O.route(qs, ks, scs, topk)
        cseq = _chunk_seq(scs)
        for h in range(Hq):
            for i in range(C):
                first = int(scs[cseq[i]])
                cand = list(range(first, i))
                kk = min(int(topk[i]), len(cand))
                sc = {j: int(np.dot(qs[i, h].astype(np.int64), ks[j, 0].astype(np.int64))) for j in cand}
                best = None
                for sub in itertools.combinations(cand, kk):
                    key = (-sum(sc[j] for j in sub), sub)
                    if best is None or key < best:
                        best = key
                want = sorted(best[1]) + [i]
                got = bidx[h, row_ptr[i]:row_ptr[i + 1]].tolist()
                assert got == want, (trial, h, i, got, want, sc)


def pin_kept_invariants(O):
    """|kept| = min(k, available) + 1, diagonal present and last, ascending, same sequence, causal."""
    w = _small_workload(11, lens_per_seq=((4,) * 9, (2, 3, 5, 1, 1, 8), (6,)), Hq=4, Hkv=2, d=6, topk=3)
    tk = np.array([0, 1, 2, 3, 5, 9, 2, 0, 4, 1, 3, 3, 2, 7, 3, 1], np.int32)
    row_ptr, bidx, _ = O.route(O.chunk_summaries(w.q, w.cu_chunks), O.chunk_summaries(w.k, w.cu_chunks),
                               w.seq_chunk_start, tk)
    cseq = _chunk_seq(w.seq_chunk_start)
    for h in range(w.num_q_heads):
        for i in range(w.total_chunks):
            row = bidx[h, row_ptr[i]:row_ptr[i + 1]].tolist()
            first = int(w.seq_chunk_start[cseq[i]])
            assert len(row) == min(int(tk[i]), i - first) + 1, (h, i, row)
            assert row[-1] == i and row == sorted(set(row)), (h, i, row)
            assert all(first <= j <= i for j in row), (h, i, row)


def pin_dense_special_case(O):
    """Keeping every earlier chunk gives causal dense attention (torch SDPA, float64), GQA included."""
    w = _small_workload(5, lens_per_seq=((3, 8, 2, 5, 9), (4, 4, 1), (1,)), Hq=6, Hkv=2, d=8, topk=0)
    big = np.full(w.total_chunks, 1000, np.int32)
    r = O.prefill(w.q, w.k, w.v, w.cu_seqlens, w.cu_chunks, w.seq_chunk_start, big, w.softmax_scale)
    dense_o, _ = O.dense_attention(w.q, w.k, w.v, w.cu_seqlens, w.softmax_scale)
    for b in range(w.num_seqs):
        s, e = w.cu_seqlens[b], w.cu_seqlens[b + 1]
        ref = _sdpa_causal_fp64(w.q[s:e], w.k[s:e], w.v[s:e], w.softmax_scale)
        np.testing.assert_allclose(r["out"][s:e], ref, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dense_o[s:e], ref, rtol=1e-10, atol=1e-12)


def pin_token_level_bruteforce(O):
    """Upsampled token importance and the kept token mask, built by loops, drive a masked dense softmax."""
    w = _small_workload(13, lens_per_seq=((3, 6, 2, 7, 4, 5),), Hq=2, Hkv=1, d=4, topk=2)
    r = O.prefill(w.q, w.k, w.v, w.cu_seqlens, w.cu_chunks, w.seq_chunk_start, w.topk, w.softmax_scale)
    T = w.total_tokens
    tc = _tok_chunk(w.cu_chunks)
    q, k, v = (x.astype(np.float64) for x in (w.q, w.k, w.v))
    for h in range(w.num_q_heads):
        imp = O.token_importance(r["scores"][h], w.cu_chunks)
        for t in range(T):
            for u in range(T):
                sv = r["scores"][h, tc[t], tc[u]]
                assert (np.isnan(imp[t, u]) and np.isnan(sv)) or imp[t, u] == sv
        # kept mask from the kept chunk lists, by loops
        mask = np.zeros((T, T), bool)
        for t in range(T):
            kept = set(r["block_idx"][h, r["row_ptr"][tc[t]]:r["row_ptr"][tc[t] + 1]].tolist())
            for u in range(t + 1):
                mask[t, u] = tc[u] in kept
        assert np.array_equal(mask, O.kept_token_mask(r["row_ptr"], r["block_idx"][h], w.cu_chunks))
        logits = torch.from_numpy(w.softmax_scale * (q[:, h] @ k[:, 0].T))
        logits = logits.masked_fill(~torch.from_numpy(mask), float("-inf"))
        ref = (torch.softmax(logits, dim=1) @ torch.from_numpy(v[:, 0])).numpy()
        np.testing.assert_allclose(r["out"][:, h], ref, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(r["lse"][h], torch.logsumexp(logits, dim=1).numpy(), rtol=1e-12, atol=1e-12)


def pin_row_sum_and_lse(O):
    """V = 1 gives O = 1; LSE equals torch.logsumexp of the kept logits."""
    w = _small_workload(17, lens_per_seq=((5, 2, 9, 3, 6, 4),), Hq=2, Hkv=2, d=8, topk=1)
    ones = np.ones_like(w.v)
    r = O.prefill(w.q, w.k, ones, w.cu_seqlens, w.cu_chunks, w.seq_chunk_start, w.topk, w.softmax_scale)
    np.testing.assert_allclose(r["out"], 1.0, rtol=0, atol=1e-14)
    q, k = w.q.astype(np.float64), w.k.astype(np.float64)
    for h in range(2):
        mask = O.kept_token_mask(r["row_ptr"], r["block_idx"][h], w.cu_chunks)
        z = torch.from_numpy(w.softmax_scale * (q[:, h] @ k[:, h].T)).masked_fill(~torch.from_numpy(mask),
                                                                                    float("-inf"))
        np.testing.assert_allclose(r["lse"][h], torch.logsumexp(z, 1).numpy(), rtol=1e-12, atol=1e-12)


def pin_causality(O):
    """Changing K, V after token t and Q in later chunks leaves outputs up to t bit-identical."""
    w = _small_workload(19, lens_per_seq=((4, 6, 3, 8, 5, 2),), Hq=2, Hkv=1, d=6, topk=2)
    base = O.prefill(w.q, w.k, w.v, w.cu_seqlens, w.cu_chunks, w.seq_chunk_start, w.topk, w.softmax_scale)
    tc = _tok_chunk(w.cu_chunks)
    rng = np.random.default_rng(0)
    for t in (3, 9, 12, 19):
        q2, k2, v2 = w.q.copy(), w.k.copy(), w.v.copy()
        k2[t + 1:] += rng.standard_normal(k2[t + 1:].shape).astype(np.float32) * 5
        v2[t + 1:] += rng.standard_normal(v2[t + 1:].shape).astype(np.float32) * 5
        later = tc > tc[t]
        q2[later] += rng.standard_normal(q2[later].shape).astype(np.float32) * 5
        r = O.prefill(q2, k2, v2, w.cu_seqlens, w.cu_chunks, w.seq_chunk_start, w.topk, w.softmax_scale)
        assert np.array_equal(r["out"][:t + 1], base["out"][:t + 1]), t
        assert np.array_equal(r["lse"][:, :t + 1], base["lse"][:, :t + 1]), t


def pin_gqa_and_permutation(O):
    """Repeating KV heads to G = 1 changes nothing; permuting whole head groups permutes outputs."""
    w = _small_workload(23, lens_per_seq=((3, 7, 2, 5, 6),), Hq=4, Hkv=2, d=6, topk=1)
    base = O.prefill(w.q, w.k, w.v, w.cu_seqlens, w.cu_chunks, w.seq_chunk_start, w.topk, w.softmax_scale)
    k_rep, v_rep = np.repeat(w.k, 2, axis=1), np.repeat(w.v, 2, axis=1)
    rep = O.prefill(w.q, k_rep, v_rep, w.cu_seqlens, w.cu_chunks, w.seq_chunk_start, w.topk, w.softmax_scale)
    assert np.array_equal(rep["out"], base["out"]) and np.array_equal(rep["block_idx"], base["block_idx"])
    perm_kv = [1, 0]
    perm_q = [2, 3, 0, 1]
    pr = O.prefill(w.q[:, perm_q], w.k[:, perm_kv], w.v[:, perm_kv], w.cu_seqlens, w.cu_chunks,
                   w.seq_chunk_start, w.topk, w.softmax_scale)
    assert np.array_equal(pr["out"], base["out"][:, perm_q])
    assert np.array_equal(pr["block_idx"], base["block_idx"][perm_q])


def pin_ragged_equals_separate(O):
    """A packed batch gives, sequence by sequence, what each sequence gives alone."""
    lens = ((4, 2, 7, 3), (5,), (1, 1, 6, 2, 3, 4))
    w = _small_workload(29, lens_per_seq=lens, Hq=2, Hkv=1, d=5, topk=2)
    packed = O.prefill(w.q, w.k, w.v, w.cu_seqlens, w.cu_chunks, w.seq_chunk_start, w.topk, w.softmax_scale)
    for b, l in enumerate(lens):
        s, e = w.cu_seqlens[b], w.cu_seqlens[b + 1]
        c0, c1 = w.seq_chunk_start[b], w.seq_chunk_start[b + 1]
        cs1, cc1, sc1 = _layout_from_lengths([l])
        alone = O.prefill(w.q[s:e], w.k[s:e], w.v[s:e], cs1, cc1, sc1, w.topk[c0:c1], w.softmax_scale)
        assert np.array_equal(alone["out"], packed["out"][s:e]), b
        for i in range(c1 - c0):
            a = alone["block_idx"][:, alone["row_ptr"][i]:alone["row_ptr"][i + 1]] + c0
            p = packed["block_idx"][:, packed["row_ptr"][c0 + i]:packed["row_ptr"][c0 + i + 1]]
            assert np.array_equal(a, p), (b, i)


def pin_grouped_routing(O):
    """Routing per KV head: with one query head per KV head it is the per-head routing; the kept set
    of every (group, row) is the best-sum k-subset under the group-summed integer scores (exact, with
    the lower-index tie rule); every head of a group gets the group's row; and it equals per-head
    routing of the group-summed queries (chunks of 4 tokens: the sqrt(4) normalisation is exact)."""
    rng = np.random.default_rng(21)
    # (1) one query head per KV head
    w = _small_workload(23, lens_per_seq=((3, 5, 2, 6, 4, 1, 7),), Hq=3, Hkv=3, d=6, topk=3)
    qs, ks = O.chunk_summaries(w.q, w.cu_chunks), O.chunk_summaries(w.k, w.cu_chunks)
    a, b = O.route(qs, ks, w.seq_chunk_start, w.topk), O.route_grouped(qs, ks, w.seq_chunk_start, w.topk)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(a[2], b[2], equal_nan=True)
    # (2) brute force over subsets, integer summaries, G = 2 or 3
    for trial in range(6):
        lens = [[1] * int(rng.integers(2, 9)) for _ in range(int(rng.integers(1, 3)))]
        _, _, scs = _layout_from_lengths(lens)
        C = int(scs[-1])
        Hkv, G, d = 2, 2 + trial % 2, 3
        lo, hi = (-1, 2) if trial % 2 else (-3, 4)
        q_s = rng.integers(lo, hi, size=(C, Hkv * G, d)).astype(np.float32)
        k_s = rng.integers(lo, hi, size=(C, Hkv, d)).astype(np.float32)
        topk = rng.integers(0, 4, size=C).astype(np.int32)
        row_ptr, bidx, _ = O.route_grouped(q_s, k_s, scs, topk)
        cseq = _chunk_seq(scs)
        for g in range(Hkv):
            for i in range(C):
                first = int(scs[cseq[i]])
                cand = list(range(first, i))
                kk = min(int(topk[i]), len(cand))
                sc = {j: sum(int(np.dot(q_s[i, h].astype(np.int64), k_s[j, g].astype(np.int64)))
                             for h in range(g * G, (g + 1) * G)) for j in cand}
                best = None
                for sub in itertools.combinations(cand, kk):
                    key = (-sum(sc[j] for j in sub), sub)
                    if best is None or key < best:
                        best = key
                want = sorted(best[1]) + [i]
                for h in range(g * G, (g + 1) * G):
                    got = bidx[h, row_ptr[i]:row_ptr[i + 1]].tolist()
                    assert got == want, (trial, g, h, i, got, want)
    # (3) the group-summed query, routed per head
    Hkv, G, d, n = 2, 3, 4, 4
    lens = [[n] * 7, [n] * 5]
    cu_seqlens, cu_chunks, scs = _layout_from_lengths(lens)
    T = int(cu_seqlens[-1])
    q = rng.integers(-2, 3, size=(T, Hkv * G, d)).astype(np.float32)
    k = rng.integers(-2, 3, size=(T, Hkv, d)).astype(np.float32)
    topk = rng.integers(0, 5, size=int(scs[-1])).astype(np.int32)
    grouped = O.route_grouped(O.chunk_summaries(q, cu_chunks), O.chunk_summaries(k, cu_chunks), scs, topk)
    qg = q.reshape(T, Hkv, G, d).sum(axis=2)
    single = O.route(O.chunk_summaries(qg, cu_chunks), O.chunk_summaries(k, cu_chunks), scs, topk)
    assert np.array_equal(grouped[2], single[2], equal_nan=True)
    for g in range(Hkv):
        for h in range(g * G, (g + 1) * G):
            assert np.array_equal(grouped[1][h], single[1][g]), (g, h)


# ----------------------------------------------------------------------------- online chunking rule (our design)

def _num(x):
    x = str(x).strip()
    neg = x.startswith("-")
    x = x.lstrip("-")
    v = math.sqrt(float(Fraction(x[5:-1]))) if x.startswith("sqrt(") else float(Fraction(x))
    return -v if neg else v


def pin_chunking_golden(O):
    g = json.load(open(os.path.join(GOLDEN, "g4_chunk_boundaries.json")))
    k = np.array(g["k"], np.float32)
    sim = O.adjacent_similarity(k, g["cu_seqlens"])
    want = np.array([_num(x) for x in g["expected_sim"]], np.float64).astype(np.float32)
    assert sim.dtype == np.float32 and np.array_equal(sim, want), (sim, want)
    for case in g["cases"]:
        cc, sc = O.chunk_boundaries(want, g["cu_seqlens"], case["lo"], case["hi"], case["tau"])
        assert cc.tolist() == case["cu_chunks"] and sc.tolist() == case["seq_chunk_start"], (case, cc, sc)


def pin_chunking_closed_forms(O):
    rng = np.random.default_rng(11)
    # equal rows: similarity 1 everywhere, so chunks are hi long (the last one what remains)
    row = rng.standard_normal((1, 2, 8)).astype(np.float32)
    k = np.repeat(row, 23, axis=0)
    sim = O.adjacent_similarity(k, [0, 23])
    assert np.allclose(sim, 1.0, atol=1e-6)
    cc, sc = O.chunk_boundaries(sim, [0, 23], 2, 5, 0.9)
    assert cc.tolist() == [0, 5, 10, 15, 20, 23] and sc.tolist() == [0, 5]
    # rows alternating between two orthogonal directions: similarity 0, so chunks are lo long
    e = np.zeros((2, 2, 8), np.float32)
    e[0, 0, 0] = 3.0
    e[1, 1, 5] = -2.0
    k = np.concatenate([e] * 9, axis=0)[:17]
    sim = O.adjacent_similarity(k, [0, 17])
    assert sim[0] == 1.0 and np.all(sim[1:] == 0.0)
    cc, _ = O.chunk_boundaries(sim, [0, 17], 3, 7, 0.5)
    assert cc.tolist() == [0, 3, 6, 9, 12, 15, 17]
    # lo == hi: fixed-length chunks whatever the similarity
    sim = rng.uniform(-1, 1, 40).astype(np.float32)
    cc, sc = O.chunk_boundaries(sim, [0, 13, 13, 40], 4, 4, 0.0)
    assert cc.tolist() == [0, 4, 8, 12, 13, 17, 21, 25, 29, 33, 37, 40] and sc.tolist() == [0, 4, 4, 11]


def pin_chunking_rule_invariants(O):
    """Property check of the greedy cut, independent of how it is computed: the chunks tile every
    sequence, lengths respect [lo, hi] (the last chunk of a sequence may be shorter), no position a
    chunk could have been cut at earlier has a drop, and a chunk shorter than its limit ends at a drop."""
    rng = np.random.default_rng(12)
    for trial in range(200):
        lens = rng.integers(0, 40, size=rng.integers(1, 4))
        cs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        sim = rng.choice(np.array([-0.5, 0.2, 0.5, 0.9, 1.0], np.float32), size=int(cs[-1]))
        lo = int(rng.integers(1, 6))
        hi = int(rng.integers(lo, 12))
        tau = float(rng.choice([0.2, 0.5, 0.95]))
        cc, sc = O.chunk_boundaries(sim, cs, lo, hi, tau)
        assert sc.size == cs.size and sc[0] == 0 and cc[0] == 0 and cc[-1] == cs[-1]
        for b in range(cs.size - 1):
            bounds = cc[sc[b]:sc[b + 1] + 1]
            assert bounds[0] == cs[b] and bounds[-1] == cs[b + 1]
            for c0, c1 in zip(bounds[:-1], bounds[1:]):
                n = c1 - c0
                assert 1 <= n <= hi
                last = c1 == cs[b + 1]
                if not last:
                    assert n >= lo
                assert all(sim[t] >= np.float32(tau) for t in range(c0 + lo, c1))
                if n < hi and not last:
                    assert sim[c1] < np.float32(tau)


def pin_similarity_library(O):
    """sim against torch's cosine_similarity in float64 on random keys, two sequences."""
    rng = np.random.default_rng(13)
    k = rng.standard_normal((50, 3, 16)).astype(np.float32)
    cs = [0, 21, 50]
    sim = O.adjacent_similarity(k, cs)
    rows = torch.from_numpy(k.reshape(50, -1).astype(np.float64))
    ref = torch.nn.functional.cosine_similarity(rows[:-1], rows[1:], dim=1).numpy()
    for t in range(50):
        if t in (0, 21):
            assert sim[t] == 1.0
        else:
            assert abs(float(sim[t]) - ref[t - 1]) <= 1e-6, t
    # positive per-row scale leaves every similarity unchanged
    scale = rng.uniform(0.1, 10.0, size=(50, 1, 1)).astype(np.float64)
    sim2 = O.adjacent_similarity(k.astype(np.float64) * scale, cs)
    assert np.allclose(sim2, sim, atol=1e-6)


# ----------------------------------------------------------------------------- decode against the kept structure

def _decode_inputs(seed, T=90, Hq=4, Hkv=2, d=8, shift_every=None):
    """Random q/k/v; keys drift within stretches so the cut rule sees both high and low similarity."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, Hq, d))
    base = rng.standard_normal((T // 7 + 1, Hkv, d))
    k = np.repeat(base, 7, axis=0)[:T] + 0.4 * rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    return q, k, v


def pin_decode_cuts_match_offline(O):
    for seed, (lo, hi, tau) in enumerate([(2, 9, 0.6), (1, 4, 0.9), (5, 5, 0.0), (3, 40, 0.3)]):
        q, k, v = _decode_inputs(100 + seed)
        _, starts, _ = O.decode_sequence(q, k, v, lo, hi, tau, 2, 0.3, first_output=len(q) - 1)
        cc, _ = O.chunk_boundaries(O.adjacent_similarity(k, [0, len(q)]), [0, len(q)], lo, hi, tau)
        assert starts + [len(q)] == cc.tolist(), (starts, cc)


def pin_decode_chunk_end_equals_prefill(O):
    """At the last token of every chunk the open summary is the chunk's prefill summary, so the decode
    output equals the prefill oracle's output at that token (same boundaries, same budget)."""
    for grouped in (False, True):
        q, k, v = _decode_inputs(110 + grouped)
        T = len(q)
        lo, hi, tau, topk, scale = 3, 12, 0.6, 2, 0.37
        out, starts, kept = O.decode_sequence(q, k, v, lo, hi, tau, topk, scale, grouped=grouped)
        cu = np.array(starts + [T], np.int32)
        scs = np.array([0, len(starts)], np.int32)
        tk = np.full(len(starts), topk, np.int32)
        qs = O.chunk_summaries(q, cu)
        ks = O.chunk_summaries(k, cu)
        rp, bi, _ = (O.route_grouped if grouped else O.route)(qs, ks, scs, tk)
        o_pre, _ = O.attend(q, k, v, cu, rp, bi, scale)
        for i in range(len(starts)):
            t = int(cu[i + 1]) - 1
            for h in range(q.shape[1]):
                assert kept[t][h] == bi[h, rp[i]:rp[i + 1] - 1].tolist(), (t, h)
            assert np.abs(out[t] - o_pre[t]).max() < 1e-10, t


def pin_decode_dense_equals_causal_attention(O):
    q, k, v = _decode_inputs(120, T=50)
    T, Hq, d = q.shape
    G = Hq // k.shape[1]
    out, _, _ = O.decode_sequence(q, k, v, 2, 6, 0.5, 10 ** 6, 0.41)
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(np.repeat(k, G, axis=1)).permute(1, 0, 2)
    vt = torch.from_numpy(np.repeat(v, G, axis=1)).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=0.41)
    assert np.abs(out - ref.permute(1, 0, 2).numpy()).max() < 1e-10


def pin_decode_first_output_and_groups(O):
    """Outputs do not depend on where output starts; grouped routing with one head per group is per-head."""
    q, k, v = _decode_inputs(130, Hq=2, Hkv=2)
    a, sa, ka = O.decode_sequence(q, k, v, 2, 9, 0.6, 2, 0.3)
    b, sb, kb = O.decode_sequence(q, k, v, 2, 9, 0.6, 2, 0.3, first_output=40)
    assert sa == sb and np.array_equal(a[40:], b) and ka[40:] == kb
    c, sc, kc = O.decode_sequence(q, k, v, 2, 9, 0.6, 2, 0.3, grouped=True)
    assert sc == sa and kc == ka and np.array_equal(c, a)


def pin_decode_ties_to_lower_index(O):
    """Identical key rows: no cut before hi, every closed chunk has the same summary, every score ties
    exactly, so the kept chunks are the lowest indices."""
    rng = np.random.default_rng(140)
    T, Hq, Hkv, d, hi, topk = 60, 2, 1, 8, 5, 2
    q = rng.standard_normal((T, Hq, d))
    k = np.repeat(rng.standard_normal((1, Hkv, d)), T, axis=0)
    v = rng.standard_normal((T, Hkv, d))
    _, starts, kept = O.decode_sequence(q, k, v, 2, hi, 0.5, topk, 0.3)
    assert starts == list(range(0, T, hi))
    for t in range(T):
        closed = t // hi
        for h in range(Hq):
            assert kept[t][h] == list(range(min(topk, closed))), (t, h, kept[t][h])


# ----------------------------------------------------------------------------- token budget

def _budget_workload(seed, lens_per_seq, Hq=4, Hkv=2, d=8):
    cs, cc, scs = _layout_from_lengths(lens_per_seq)
    rng = np.random.default_rng(seed)
    T = int(cs[-1])
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    return cs, cc, scs, q, k, v


def pin_budget_equal_lengths_is_topk(O):
    """All chunks of length L: a budget of b tokens keeps exactly the top floor(b / L) chunks."""
    L = 3
    cs, cc, scs, q, k, v = _budget_workload(150, [[L] * 9, [L] * 6])
    qs, ks = O.chunk_summaries(q, cc), O.chunk_summaries(k, cc)
    rng = np.random.default_rng(151)
    budget = rng.integers(0, 8 * L, size=int(scs[-1])).astype(np.int32)
    for grouped in (False, True):
        rp_t, bi_t, _ = O.route_tokens(qs, ks, cc, scs, budget, grouped=grouped)
        rp_k, bi_k, _ = (O.route_grouped if grouped else O.route)(qs, ks, scs, budget // L)
        assert np.array_equal(rp_t, rp_k) and np.array_equal(bi_t, bi_k)


def pin_budget_prefix_bruteforce(O):
    """Each row is the longest prefix of the (score desc, chunk asc) ranking that fits, checked with
    Python's sorted() on the chunk scores; -1 pads the row after the diagonal; the capacity equals the
    count of the shortest earlier chunks that fit."""
    rng = np.random.default_rng(152)
    for trial in range(12):
        lens = [rng.integers(1, 9, size=rng.integers(1, 9)).tolist() for _ in range(rng.integers(1, 3))]
        cs, cc, scs, q, k, v = _budget_workload(153 + trial, lens)
        C = int(scs[-1])
        budget = rng.integers(0, 25, size=C).astype(np.int32)
        qs, ks = O.chunk_summaries(q, cc), O.chunk_summaries(k, cc)
        rp, bi, S = O.route_tokens(qs, ks, cc, scs, budget)
        L = np.diff(cc)
        for i in range(C):
            b = max(x for x in range(len(scs) - 1) if scs[x] <= i)
            first = int(scs[b])
            cap, tot = 0, 0
            for n in sorted(L[first:i]):
                if tot + n > budget[i]:
                    break
                tot += n
                cap += 1
            assert rp[i + 1] - rp[i] == cap + 1
            for h in range(q.shape[1]):
                rank = sorted(range(first, i), key=lambda j: (-float(S[h, i, j]), j))
                want, tot = [], 0
                for j in rank:
                    if tot + L[j] > budget[i]:
                        break
                    tot += L[j]
                    want.append(j)
                row = bi[h, rp[i]:rp[i + 1]].tolist()
                m = len(want)
                assert row[:m + 1] == sorted(want) + [i] and all(x == -1 for x in row[m + 1:]), (i, h, row, want)


def pin_budget_extremes_and_padding(O):
    cs, cc, scs, q, k, v = _budget_workload(160, [[2, 5, 3, 4, 1, 6]])
    qs, ks = O.chunk_summaries(q, cc), O.chunk_summaries(k, cc)
    C = int(scs[-1])
    rp, bi, _ = O.route_tokens(qs, ks, cc, scs, np.zeros(C, np.int32))
    assert np.array_equal(rp, np.arange(C + 1)) and np.array_equal(bi[0], np.arange(C))
    rp, bi, _ = O.route_tokens(qs, ks, cc, scs, np.full(C, 10 ** 6, np.int32))
    for i in range(C):
        assert bi[0, rp[i]:rp[i + 1]].tolist() == list(range(i + 1))
    # attention ignores the padding: a padded list gives the same output as the same list compacted
    budget = np.array([0, 3, 4, 6, 2, 9], np.int32)
    rp, bi, _ = O.route_tokens(qs, ks, cc, scs, budget)
    rows = [[[x for x in bi[h, rp[i]:rp[i + 1]] if x >= 0] for i in range(C)] for h in range(q.shape[1])]
    a, la = O.attend(q, k, v, cc, rp, bi, 0.3)
    for h in range(q.shape[1]):
        rp_c = np.concatenate([[0], np.cumsum([len(r) for r in rows[h]])]).astype(np.int32)
        bi_c = np.concatenate(rows[h]).astype(np.int32)[None, :].repeat(q.shape[1], axis=0)
        b_, lb = O.attend(q, k, v, cc, rp_c, bi_c, 0.3, heads=[h])
        assert np.allclose(a[:, h], b_[:, h], atol=1e-12) and np.allclose(la[h], lb[h], atol=1e-12)


def _raises_value_error(fn, *args) -> bool:
    """True when fn(*args) raises ValueError; any other outcome (no error, another exception) is False."""
    try:
        fn(*args)
    except ValueError:
        return True
    except Exception:  # noqa: BLE001 - a malformed layout must be refused by the check, not crash later
        return False
    return False


# Layouts as (cu_seqlens, cu_chunks, seq_chunk_start).  Each malformed one breaks exactly one rule of
# the chunk layout: the chunks of every sequence tile its token range exactly, each with >= 1 token
# ("Long-Context Modeling with Dynamic Hierarchical Sparse Attention for On-Device LLMs", Abstract:
# each sequence is split into variable-length chunks).  The same cases are fed to the C ABI's check.
GOOD_LAYOUTS = {
    "two sequences": ([0, 10, 17], [0, 4, 10, 13, 17], [0, 2, 4]),
    "empty sequences inside a batch": ([0, 0, 5, 5], [0, 2, 5], [0, 0, 2, 2]),
    "empty batch": ([0], [0], [0]),
    "one-token chunks": ([0, 3], [0, 1, 2, 3], [0, 3]),
}
BAD_LAYOUTS = {
    "chunk crosses a sequence boundary": ([0, 10, 17], [0, 4, 11, 13, 17], [0, 2, 4]),
    "empty chunk": ([0, 10, 17], [0, 4, 4, 10, 17], [0, 3, 4]),
    "chunk offsets do not start at 0": ([0, 10, 17], [1, 4, 10, 13, 17], [0, 2, 4]),
    "token offsets do not start at 0": ([2, 10, 17], [0, 4, 10, 13, 17], [0, 2, 4]),
    "sequence chunk starts out of order": ([0, 10, 17], [0, 4, 10, 13, 17], [0, 5, 4]),
    "chunks stop short of the tokens": ([0, 10, 18], [0, 4, 10, 13, 17], [0, 2, 4]),
    "a sequence ends inside a chunk": ([0, 9, 17], [0, 4, 10, 13, 17], [0, 2, 4]),
    "chunk offsets go backwards": ([0, 10, 17], [0, 6, 4, 10, 13, 17], [0, 3, 5]),
    "sequence offsets go backwards": ([0, 10, 4, 17], [0, 4, 10, 13, 17], [0, 2, 2, 4]),
    "chunk count differs from the sequence table": ([0, 10, 17], [0, 4, 10, 13, 17], [0, 2, 3]),
    "sequence tables of different lengths": ([0, 10, 17], [0, 4, 10, 13, 17], [0, 4]),
}


def pin_layout_validation(O):
    """Every well-formed layout passes the oracle's layout check and the whole path runs on it; every
    malformed one is refused with ValueError, both by the check and by the whole path (which validates
    before anything else).  A negative chunk budget is refused by the plan and the whole path."""
    rng = np.random.default_rng(5)
    for name, (cs, cc, sc) in GOOD_LAYOUTS.items():
        O.validate_layout(cs, cc, sc)
        T, C = int(cc[-1]), len(cc) - 1
        q, k, v = (rng.standard_normal((T, 2, 4)) for _ in range(3))
        r = O.prefill(q, k, v, cs, cc, sc, np.ones(C, np.int32), 0.5)
        assert r["out"].shape == (T, 2, 4) and not np.isnan(r["out"]).any(), name
    for name, (cs, cc, sc) in BAD_LAYOUTS.items():
        assert _raises_value_error(O.validate_layout, cs, cc, sc), f"layout check accepts: {name}"
        T = max(int(max(cs)), int(max(cc)), 1)
        C = max(len(cc) - 1, 1)
        q, k, v = (rng.standard_normal((T, 2, 4)) for _ in range(3))
        assert _raises_value_error(O.prefill, q, k, v, cs, cc, sc, np.ones(C, np.int32), 0.5), \
            f"whole path accepts: {name}"
    cs, cc, sc = GOOD_LAYOUTS["two sequences"]
    q, k, v = (rng.standard_normal((17, 2, 4)) for _ in range(3))
    for tk in ([1, 1, -1, 1], [1, 1, 1], [1, 1, 1, 1, 1]):      # a negative budget, too few and too many entries
        assert _raises_value_error(O.route_plan, sc, np.array(tk, np.int32)), tk
        assert _raises_value_error(O.prefill, q, k, v, cs, cc, sc, np.array(tk, np.int32), 0.5), tk


ALL_PINS = [pin_layout_validation, pin_golden, pin_summary_closed_forms, pin_scores_bruteforce, pin_topk_bruteforce,
            pin_kept_invariants, pin_dense_special_case, pin_token_level_bruteforce, pin_row_sum_and_lse,
            pin_causality, pin_gqa_and_permutation, pin_ragged_equals_separate, pin_grouped_routing,
            pin_chunking_golden, pin_chunking_closed_forms, pin_chunking_rule_invariants, pin_similarity_library,
            pin_decode_cuts_match_offline, pin_decode_chunk_end_equals_prefill,
            pin_decode_dense_equals_causal_attention, pin_decode_first_output_and_groups,
            pin_decode_ties_to_lower_index, pin_budget_equal_lengths_is_topk, pin_budget_prefix_bruteforce,
            pin_budget_extremes_and_padding]
