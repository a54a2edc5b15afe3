"""GPU parity of decode (dhsa_decode_load_prefix + dhsa_decode_step) against the decode oracle.

A prefix of every sequence is chunked by the GPU chunking calls and loaded; the remaining tokens are
decoded one step at a time.  Checks per step: outputs within the bf16 / fp32 bar of the prefill
tests; kept closed chunks equal to the oracle's, except a swap of two chunks whose oracle scores
are within 1e-4 relative (the routing decision is fp32 on both sides, from summaries that differ
by rounding only); after the last step the chunk table equals the oracle's boundaries exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import dynamic_sparse_attention_dhsa_amd as D
from dynamic_sparse_attention_dhsa_amd import workloads as W
from dynamic_sparse_attention_dhsa_amd.workloads import SeqSpec

pytestmark = pytest.mark.gpu

OUT_ATOL = {"bf16": 2e-2, "f32": 1e-4}
REL_TIE = 1e-4


def _dev(a, dt):
    a = np.ascontiguousarray(a)
    if dt == "bf16":
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def _oracle_scores(qf, kf, starts, t, h, Hkv, grouped):
    """fp64 scores of the closed chunks for output token t (test-side, from the oracle's boundaries)."""
    Hq, d = qf.shape[1], qf.shape[2]
    G = Hq // Hkv
    g = h // G
    closed = [s for s in starts if s <= t]
    c0 = closed[-1]
    ks = []
    for j in range(len(closed) - 1):
        a, b = closed[j], closed[j + 1]
        ks.append((kf[a:b, g].astype(np.float64).sum(0) / np.sqrt(b - a)).astype(np.float32))
    qo = (qf[c0:t + 1].astype(np.float64).sum(0) / np.sqrt(t + 1 - c0)).astype(np.float32).astype(np.float64)
    qv = qo[g * G:(g + 1) * G].sum(0) if grouped else qo[h]
    return np.array([float(np.dot(qv, x.astype(np.float64))) for x in ks])


def _run(seqs, Hq, Hkv, d, dt, seed, P, lo, hi, tau, topk, grouped, L=None, C=256, steps=None):
    w = W.make_workload(seqs, Hq, Hkv, d, dt, seed=seed, name="decode")
    B = w.num_seqs
    cs = w.cu_seqlens
    lens = np.diff(cs)
    assert np.all(lens == lens[0])
    T_seq = int(lens[0])
    S = T_seq - P if steps is None else steps
    qf, kf, vf = w.q_f32(), w.k_f32(), w.v_f32()
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    scale = 1.0 / np.sqrt(d)
    # prefix: first P tokens of every sequence, chunked on the GPU by the same rule
    rows = np.concatenate([np.arange(cs[b], cs[b] + P) for b in range(B)]) if P else np.zeros(0, np.int64)
    cu_p = np.arange(B + 1, dtype=np.int32) * P
    state = D.DecodeState(B, Hq, Hkv, d, tdt, L or T_seq, C)
    if P:
        kp = _dev(w.k[rows], dt)
        cc, scs = D.online_chunks(kp, cu_p, lo, hi, tau)
        lay = D.Layout(cu_p, cc, scs, Hq, Hkv, d, tdt)
        state.load_prefix(lay, _dev(w.q[rows], dt), kp, _dev(w.v[rows], dt))
    else:
        lay = D.Layout(cu_p, np.zeros(1, np.int32), np.zeros(B + 1, np.int32), Hq, Hkv, d, tdt)
        state.load_prefix(lay, torch.empty((0, Hq, d), dtype=tdt, device="cuda"),
                          torch.empty((0, Hkv, d), dtype=tdt, device="cuda"),
                          torch.empty((0, Hkv, d), dtype=tdt, device="cuda"))
    outs, kepts = [], []
    kept_buf = torch.empty((B, Hq, max(topk, 1)), dtype=torch.int32, device="cuda")
    for s in range(S):
        idx = cs[:-1] + P + s
        o = state.step(_dev(w.q[idx], dt), _dev(w.k[idx], dt), _dev(w.v[idx], dt), lo, hi, tau, topk, grouped,
                       scale, kept=kept_buf if topk > 0 else None)
        outs.append(o.float().cpu().numpy())
        kepts.append(kept_buf.cpu().numpy().copy())
    torch.cuda.synchronize()
    outs = np.array(outs)                       # [S, B, Hq, d]
    status = state.status.cpu().numpy()
    return w, outs, kepts, state, status, (qf, kf, vf, scale, P, S, T_seq)


def _check(seqs, Hq, Hkv, d, dt, seed, P, lo, hi, tau, topk, grouped=False, C=256):
    w, outs, kepts, state, status, (qf, kf, vf, scale, P, S, T_seq) = _run(seqs, Hq, Hkv, d, dt, seed, P, lo, hi,
                                                                              tau, topk, grouped, C=C)
    assert np.all(status == 0)
    cs = w.cu_seqlens
    swaps = 0
    for b in range(w.num_seqs):
        sl = slice(cs[b], cs[b + 1])
        o_out, starts, o_kept = oracle.decode_sequence(qf[sl], kf[sl], vf[sl], lo, hi, tau, topk, scale,
                                                       first_output=P, grouped=grouped)
        err = np.abs(outs[:, b] - o_out).max()
        assert err <= OUT_ATOL[dt], f"seq {b}: out max-abs err {err:.3e}"
        for n in range(S):
            t = P + n
            for h in range(Hq):
                g_list = [x for x in kepts[n][b, h].tolist() if x >= 0] if topk > 0 else []
                o_list = o_kept[n][h]
                if g_list != o_list:
                    sc = _oracle_scores(qf[sl], kf[sl], starts, t, h, Hkv, grouped)
                    only_g = sorted(set(g_list) - set(o_list), key=lambda j: -sc[j])
                    only_o = sorted(set(o_list) - set(g_list), key=lambda j: -sc[j])
                    assert len(only_g) == len(only_o), (t, h, g_list, o_list)
                    for a, c in zip(only_g, only_o):
                        assert abs(sc[a] - sc[c]) <= REL_TIE * max(abs(sc[a]), abs(sc[c])), (t, h, a, c, sc[a], sc[c])
                        swaps += 1
        nc = int(state.num_closed[b].item())
        g_starts = state.chunk_start[b, :nc + 1].cpu().numpy().tolist()
        assert g_starts == starts, (g_starts[:10], starts[:10])
        assert int(state.seq_len[b].item()) == T_seq
    return swaps


CASES = {
    # name: (seqs, Hq, Hkv, d, dtype, seed, P, lo, hi, tau, topk)
    "bf16_d128_gqa4": ([SeqSpec(700, ("uniform", 24, 120), 0, 0), SeqSpec(700, ("uniform", 24, 120), 0, 0)],
                       8, 2, 128, "bf16", 51, 560, 16, 160, 0.5, 4),
    "bf16_d64_mha": ([SeqSpec(500, ("uniform", 16, 90), 0, 0)], 4, 4, 64, "bf16", 52, 400, 8, 100, 0.5, 3),
    "bf16_d256_gqa2": ([SeqSpec(400, ("uniform", 32, 100), 0, 0)], 8, 4, 256, "bf16", 53, 330, 16, 128, 0.5, 2),
    "f32_d64": ([SeqSpec(300, ("uniform", 16, 60), 0, 0), SeqSpec(300, ("uniform", 16, 60), 0, 0)],
                2, 1, 64, "f32", 54, 240, 8, 80, 0.5, 3),
    "dense_budget": ([SeqSpec(400, ("uniform", 24, 80), 0, 0)], 4, 2, 128, "bf16", 55, 330, 16, 100, 0.5, 1000),
    "no_budget": ([SeqSpec(300, ("uniform", 24, 80), 0, 0)], 4, 2, 128, "bf16", 56, 250, 16, 100, 0.5, 0),
    "from_empty": ([SeqSpec(160, ("uniform", 16, 40), 0, 0)], 4, 2, 64, "bf16", 57, 0, 8, 48, 0.5, 2),
    "long_slices": ([SeqSpec(5000, ("uniform", 400, 1000), 0, 0)], 4, 1, 128, "bf16", 58, 4970, 64, 1024, 0.5, 3),
    # group sizes outside {1, 2, 4, 8} (one q head per attention wave when routing per KV head) and 8
    "bf16_d128_g3": ([SeqSpec(600, ("uniform", 24, 100), 0, 0)], 6, 2, 128, "bf16", 60, 480, 16, 120, 0.5, 3),
    "bf16_d128_g8": ([SeqSpec(600, ("uniform", 24, 100), 0, 0)], 16, 2, 128, "bf16", 61, 480, 16, 120, 0.5, 3),
    # more than eight query heads per KV head (the routing kernel sums the heads past eight separately)
    "bf16_d64_g16": ([SeqSpec(500, ("uniform", 24, 100), 0, 0)], 32, 2, 64, "bf16", 62, 400, 16, 120, 0.5, 3),
}


@pytest.mark.parametrize("grouped", [False, True])
@pytest.mark.parametrize("name", sorted(CASES))
def test_decode_matches_oracle(name, grouped):
    if grouped and CASES[name][1] == CASES[name][2]:
        pytest.skip("one head per group: grouped routing is per-head routing")
    _check(*CASES[name], grouped=grouped)


def test_full_cache_stops_the_sequence():
    seqs = [SeqSpec(120, ("uniform", 16, 40), 0, 0)]
    w, outs, _, state, status, meta = _run(seqs, 4, 2, 64, "bf16", 59, 100, 8, 48, 0.5, 2, False, L=110, steps=15)
    assert status.tolist() == [1]
    assert int(state.seq_len[0].item()) == 110
    assert np.all(outs[10:] == 0.0) and np.any(outs[:10] != 0.0)
    qf, kf, vf, scale, P, S, T_seq = meta
    o_out, _, _ = oracle.decode_sequence(qf[:110], kf[:110], vf[:110], 8, 48, 0.5, 2, scale, first_output=100)
    assert np.abs(outs[:10, 0] - o_out).max() <= OUT_ATOL["bf16"]


@pytest.mark.parametrize("grouped", [False, True])
def test_full_chunk_table_stops_only_that_sequence(grouped):
    """Two sequences, table of C closed chunks: C is the first sequence's final count (it fills the table
    exactly and goes on), the second reaches a (C + 1)-th cut mid-run and stops there (status 2): its
    outputs are zeros from that token on, its state stays as it was; the first is unaffected."""
    seqs = [SeqSpec(220, ("uniform", 8, 30), 0, 0), SeqSpec(220, ("uniform", 8, 30), 0, 0)]
    Hq, Hkv, d, seed, P, lo, hi, tau, topk = 4, 2, 64, 68, 120, 8, 32, 0.5, 2
    w = W.make_workload(seqs, Hq, Hkv, d, "bf16", seed=seed, name="decode")
    qf, kf, vf = w.q_f32(), w.k_f32(), w.v_f32()
    cs = w.cu_seqlens
    scale = 1.0 / np.sqrt(d)
    ref = [oracle.decode_sequence(qf[cs[b]:cs[b + 1]], kf[cs[b]:cs[b + 1]], vf[cs[b]:cs[b + 1]], lo, hi, tau,
                                  topk, scale, first_output=P, grouped=grouped) for b in range(2)]
    starts = [r[1] for r in ref]
    C = len(starts[0]) - 1
    assert len(starts[1]) - 1 > C and starts[1][C + 1] >= P, "the seed must give a mid-run stop"
    t_stop = starts[1][C + 1]                   # the token whose cut would close chunk C + 1
    w2, outs, _, state, status, _ = _run(seqs, Hq, Hkv, d, "bf16", seed, P, lo, hi, tau, topk, grouped, C=C)
    assert status.tolist() == [0, 2]
    n_ok = t_stop - P
    assert np.abs(outs[:, 0] - ref[0][0]).max() <= OUT_ATOL["bf16"]
    assert np.abs(outs[:n_ok, 1] - ref[1][0][:n_ok]).max() <= OUT_ATOL["bf16"]
    assert np.all(outs[n_ok:, 1] == 0.0)
    assert int(state.seq_len[0].item()) == 220 and int(state.seq_len[1].item()) == t_stop
    assert [int(x) for x in state.num_closed.cpu()] == [C, C]
    for b in range(2):
        assert state.chunk_start[b, :C + 1].cpu().numpy().tolist() == starts[b][:C + 1]


def _draw_decode_case(i: int):
    """Seeded random decode setting: 1-3 equal-length sequences, head layout, head dim and dtype, the
    chunking rule, the prefix length (0 included) and the budget (0 to past every closed chunk)."""
    rng = np.random.default_rng(8000 + i)
    B = int(rng.integers(1, 4))
    length = int(rng.integers(60, 400))
    lo = int(rng.integers(1, 24))
    hi = int(rng.integers(lo, lo + 80))
    seqs = [SeqSpec(length, ("uniform", lo, hi), 0, 0) for _ in range(B)]
    Hkv = int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 3, 4, 8]))
    dt = "f32" if rng.random() < 0.25 else "bf16"
    d = int(rng.choice([64, 128] if dt == "f32" else [64, 128, 256]))
    P = 0 if rng.random() < 0.2 else int(rng.integers(1, length - 8))
    topk = int(rng.integers(0, 12))
    tau = float(rng.choice([0.3, 0.5, 0.7]))
    grouped = bool(rng.random() < 0.5) and G > 1
    return (seqs, Hkv * G, Hkv, d, dt, 8100 + i, P, lo, hi, tau, topk), grouped


@pytest.mark.parametrize("i", range(8))
def test_random_decode_settings(i):
    args, grouped = _draw_decode_case(i)
    seqs, Hq, Hkv, d, dt, seed, P, lo, hi, tau, topk = args
    print(f"[decode sweep {i}] B={len(seqs)} len={seqs[0].length} Hq/Hkv={Hq}/{Hkv} d={d} {dt} P={P} "
          f"lo={lo} hi={hi} tau={tau} topk={topk} grouped={grouped}", flush=True)
    _check(*args, grouped=grouped)


@pytest.mark.slow
def test_decode_32k_context():
    seqs = [SeqSpec(32768 + 24, ("uniform", 64, 512), 0, 0)]
    _check(seqs, 32, 8, 128, "bf16", 60, 32768, 32, 1024, 0.5, 32, grouped=False)


@pytest.mark.parametrize("grouped", [False, True])
def test_decode_narrowed_selection(grouped):
    """A 16K-token context in chunks of 24..40 tokens: about 500 closed chunks, between the direct and
    the workgroup-wide selections, so routing first narrows the candidates across waves (each wave's
    own top-k bound) and then selects among the survivors.  Outputs, kept lists and the final chunk
    table against the decode oracle."""
    seqs = [SeqSpec(16384 + 12, ("uniform", 24, 40), 0, 0)]
    _check(seqs, 4, 2, 64, "bf16", 64, 16384, 16, 64, 0.5, 32, grouped=grouped, C=1024)


@pytest.mark.slow
@pytest.mark.parametrize("grouped", [False, True])
def test_decode_128k_context_beyond_1024_chunks(grouped):
    """A 131072-token context in chunks of 24..40 tokens: about 4100 closed chunks, more than one wave
    holds in registers, so the whole routing workgroup selects the top-k.  Outputs, kept lists and the
    final chunk table against the decode oracle."""
    seqs = [SeqSpec(131072 + 12, ("uniform", 24, 40), 0, 0)]
    _check(seqs, 4, 2, 64, "bf16", 63, 131072, 16, 64, 0.5, 32, grouped=grouped, C=8192)


def test_rows_longer_than_the_slice_grid():
    """The attention grid covers (topk + 1) * hi kept tokens per row; a prefix chunked with longer chunks
    keeps more, and the waves then loop over slices.  Each step's output must equal exact attention
    over the kept closed chunks the step reports plus the open chunk, from the state's own chunk table
    (self-consistency: the decode oracle would chunk the prefix by the step's rule instead)."""
    Hq, Hkv, d, dt = 4, 2, 64, "bf16"
    T_seq, P = 1400, 1380
    w = W.make_workload([SeqSpec(T_seq, ("uniform", 300, 500), 0, 0)], Hq, Hkv, d, dt, seed=62, name="longrows")
    qf, kf, vf = w.q_f32(), w.k_f32(), w.v_f32()
    tdt = torch.bfloat16
    scale = 1.0 / np.sqrt(d)
    kp = _dev(w.k[:P], dt)
    cu_p = np.array([0, P], np.int32)
    cc, scs = D.online_chunks(kp, cu_p, 64, 512, 0.5)
    assert np.diff(cc).max() > 256
    state = D.DecodeState(1, Hq, Hkv, d, tdt, T_seq, 64)
    state.load_prefix(D.Layout(cu_p, cc, scs, Hq, Hkv, d, tdt), _dev(w.q[:P], dt), kp, _dev(w.v[:P], dt))
    lo, hi, tau, topk = 8, 16, 0.5, 6
    kept_buf = torch.empty((1, Hq, topk), dtype=torch.int32, device="cuda")
    G = Hq // Hkv
    longest = 0
    for t in range(P, P + 12):
        o = state.step(_dev(w.q[t:t + 1], dt), _dev(w.k[t:t + 1], dt), _dev(w.v[t:t + 1], dt), lo, hi, tau, topk,
                       False, scale, kept=kept_buf)
        out = o.float().cpu().numpy()[0]
        kept = kept_buf.cpu().numpy()[0]
        nc = int(state.num_closed[0].item())
        starts = state.chunk_start[0, :nc + 1].cpu().numpy().tolist()
        for h in range(Hq):
            rows = []
            for j in kept[h].tolist():
                if j >= 0:
                    rows += list(range(starts[j], starts[j + 1]))
            rows += list(range(starts[nc], t + 1))
            longest = max(longest, len(rows))
            kk = kf[rows, h // G].astype(np.float64)
            z = scale * (kk @ qf[t, h].astype(np.float64))
            p = np.exp(z - z.max())
            ref = (p / p.sum()) @ vf[rows, h // G].astype(np.float64)
            err = np.abs(out[h] - ref).max()
            assert err <= OUT_ATOL[dt], (t, h, err)
    assert longest > (topk + 1) * hi and longest > 2 * 256     # several slices for one wave


def test_decode_more_rows_than_resident_waves():
    """More (sequence, q head) rows than attention waves the GPU holds at once (routing per query head at
    d = 64: 272 x 16 = 4352 rows, against 4096 resident waves of that kernel on a 256-CU part): the grid
    then gives each row one wave, which takes all of the row's kept tokens (several 64-token blocks,
    128 at a time), and the combine reads one partial state per row.  Every sequence against the oracle."""
    seqs = [SeqSpec(404, ("uniform", 48, 160), 0, 0)] * 272
    _check(seqs, 16, 4, 64, "bf16", 63, 400, 48, 256, 0.5, 3, grouped=False)
