"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Stage by stage:
  * summaries  -- GPU fp32 vs oracle (fp64 sums rounded to fp32), relative 2e-5 of the row scale;
  * routing    -- GPU kept sets vs oracle kept sets, equal except swaps within 1e-4 relative
                  oracle score (tests/parity.py);
  * attention  -- GPU sparse prefill fed the ORACLE's block list vs oracle attention on that
                  list: max-abs 2e-2 (bf16 out) / 1e-4 (fp32 out); LSE 2e-3 / 1e-4;
  * end to end -- GPU routing + attention vs the oracle's whole path; a row whose kept set holds a
                  tolerated tie swap is compared with the oracle's attention over the GPU's list.
Full-size workloads (8K..164K tokens) are checked on sampled rows the oracle computes one by one.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from parity import ATOL_BF16, ATOL_F32, compare_kept_sets, rows_with_swaps

pytestmark = pytest.mark.gpu

import dynamic_sparse_attention_dhsa_amd as D  # noqa: E402
from dynamic_sparse_attention_dhsa_amd import workloads as W  # noqa: E402
from dynamic_sparse_attention_dhsa_amd.workloads import SeqSpec  # noqa: E402

LSE_ATOL = {"bf16": 2e-3, "f32": 1e-4}
OUT_ATOL = {"bf16": ATOL_BF16, "f32": ATOL_F32}


def _dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class Case:
    """A workload with its device tensors, the GPU path's results and the oracle's."""

    def __init__(self, w: W.Workload, topk=None, grouped: bool = False):
        self.w = w
        self.grouped = grouped
        self.topk = w.topk if topk is None else np.asarray(topk, np.int32)
        print(f"[case] {w.name} seed={w.seed} T={w.total_tokens} C={w.total_chunks} Hq={w.num_q_heads} "
              f"Hkv={w.num_kv_heads} d={w.head_dim} {w.dtype}", flush=True)
        self.q, self.k, self.v = (_dev(a, w.dtype) for a in (w.q, w.k, w.v))
        self.qf, self.kf, self.vf = w.q_f32(), w.k_f32(), w.v_f32()
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.layout = D.Layout(w.cu_seqlens, w.cu_chunks, w.seq_chunk_start, w.num_q_heads, w.num_kv_heads,
                               w.head_dim, tdt)
        self.plan = D.RoutePlan(self.layout, self.topk)
        # oracle: summaries and routing for every row
        self.o_qs = oracle.chunk_summaries(self.qf, w.cu_chunks)
        self.o_ks = oracle.chunk_summaries(self.kf, w.cu_chunks)
        if grouped:     # one selection per KV head; its scores stand for every head of the group
            self.o_rp, self.o_bidx, s_g = oracle.route_grouped(self.o_qs, self.o_ks, w.seq_chunk_start, self.topk)
            self.o_scores = np.repeat(s_g, w.num_q_heads // w.num_kv_heads, axis=0)
        else:
            self.o_rp, self.o_bidx, self.o_scores = oracle.route(self.o_qs, self.o_ks, w.seq_chunk_start,
                                                                 self.topk)
        assert np.array_equal(self.o_rp, self.plan.h_row_ptr)

    # GPU stages ---------------------------------------------------------------------------
    def gpu_summaries(self):
        qs, ks = D.chunk_summarize(self.layout, self.q, self.k)
        torch.cuda.synchronize()
        return qs.cpu().numpy(), ks.cpu().numpy()

    def gpu_route(self, q_sum=None, k_sum=None):
        if q_sum is None:
            q_sum, k_sum = D.chunk_summarize(self.layout, self.q, self.k)
        else:
            q_sum, k_sum = torch.from_numpy(q_sum).cuda(), torch.from_numpy(k_sum).cuda()
        b = D.route(self.layout, self.plan, q_sum, k_sum, grouped=self.grouped)
        torch.cuda.synchronize()
        return b.cpu().numpy()

    def gpu_attend(self, bidx: np.ndarray):
        out, lse = D.sparse_prefill(self.layout, self.plan, self.q, self.k, self.v,
                                    torch.from_numpy(np.ascontiguousarray(bidx)).cuda(), self.w.softmax_scale,
                                    return_lse=True)
        torch.cuda.synchronize()
        return out.float().cpu().numpy(), lse.cpu().numpy()

    def gpu_prefill(self):
        r = D.prefill(self.q, self.k, self.v, self.w.cu_seqlens, self.w.cu_chunks, self.w.seq_chunk_start,
                      self.topk, self.w.softmax_scale, return_lse=True, grouped=self.grouped)
        torch.cuda.synchronize()
        return r["block_idx"].cpu().numpy(), r["out"].float().cpu().numpy(), r["lse"].cpu().numpy()

    # oracle attention on chosen rows ------------------------------------------------------------
    def oracle_attend(self, bidx, heads=None, chunks=None):
        return oracle.attend(self.qf, self.kf, self.vf, self.w.cu_chunks, self.o_rp, bidx, self.w.softmax_scale,
                             heads=heads, chunks=chunks)


def check_summaries(case: Case):
    g_qs, g_ks = case.gpu_summaries()
    for g, o in ((g_qs, case.o_qs), (g_ks, case.o_ks)):
        scale = np.abs(o).max(axis=-1, keepdims=True) + 1e-30
        err = np.abs(g.astype(np.float64) - o.astype(np.float64)) / scale
        assert err.max() <= 2e-5, f"summary rel err {err.max():.3e}"


def check_routing(case: Case, q_sum=None, k_sum=None, heads=None):
    g_b = case.gpu_route(q_sum, k_sum)
    eq, tol, fails = compare_kept_sets(g_b, case.o_bidx, case.o_rp, case.o_scores, case.w.seq_chunk_start,
                                       heads=heads)
    assert not fails, f"{len(fails)} routing failures, first: {fails[:3]}"
    return g_b, eq, tol


def check_attention(case: Case, heads=None, chunks=None):
    """GPU attention and oracle attention on the oracle's block list, on the requested rows."""
    g_o, g_l = case.gpu_attend(case.o_bidx)
    # the output does not depend on whether the LSE is requested
    bidx = torch.from_numpy(np.ascontiguousarray(case.o_bidx)).cuda()
    g_o2 = D.sparse_prefill(case.layout, case.plan, case.q, case.k, case.v, bidx, case.w.softmax_scale)
    torch.cuda.synchronize()
    assert np.array_equal(g_o2.float().cpu().numpy(), g_o)
    o_o, o_l = case.oracle_attend(case.o_bidx, heads, chunks)
    sel = ~np.isnan(o_o)
    assert sel.any()
    err = np.abs(g_o[sel] - o_o[sel]).max()
    assert err <= OUT_ATOL[case.w.dtype], f"out max-abs err {err:.3e}"
    lsel = ~np.isnan(o_l)
    lerr = np.abs(g_l[lsel] - o_l[lsel]).max()
    assert lerr <= LSE_ATOL[case.w.dtype], f"lse max-abs err {lerr:.3e}"
    return err, lerr


def check_end_to_end(case: Case, heads=None, chunks=None):
    g_b, g_o, g_l = case.gpu_prefill()
    eq, tol, fails = compare_kept_sets(g_b, case.o_bidx, case.o_rp, case.o_scores, case.w.seq_chunk_start)
    assert not fails, fails[:3]
    swapped = set(rows_with_swaps(g_b, case.o_bidx, case.o_rp))
    o_o, o_l = case.oracle_attend(case.o_bidx, heads, chunks)
    cc = case.w.cu_chunks
    worst = 0.0
    for h in (range(case.w.num_q_heads) if heads is None else heads):
        for i in (range(case.w.total_chunks) if chunks is None else chunks):
            s, e = cc[i], cc[i + 1]
            if (h, i) in swapped:
                # a tolerated tie swap: the output is unique given the kept set, so the row is checked
                # against the oracle's attention over the list the GPU kept
                ref, _ = case.oracle_attend(g_b, heads=[h], chunks=[i])
            else:
                ref = o_o
            worst = max(worst, float(np.abs(g_o[s:e, h] - ref[s:e, h]).max()))
    assert worst <= OUT_ATOL[case.w.dtype], f"end-to-end max-abs err {worst:.3e}"
    return len(swapped)


def small(seqs, Hq, Hkv, d, dtype, seed, name, **kw):
    return W.make_workload(seqs, Hq, Hkv, d, dtype, seed=seed, name=name, **kw)


# ------------------------------------------------------------------------------------------ small cases
SMALL = {
    "cfg0_full": lambda: W.make_config(0),
    "bf16_d128_g4_ragged": lambda: small([SeqSpec(700, ("uniform", 20, 150), 5, 2), SeqSpec(333, ("uniform", 1, 40), 3, 1),
                                          SeqSpec(1, ("fixed", 1), 2, 0), SeqSpec(0, ("fixed", 8), 2, 0),
                                          SeqSpec(517, ("explicit", [517]), 1, 0)], 8, 2, 128, "bf16", 11, "ragged_g4"),
    "bf16_d64_g1": lambda: small([SeqSpec(900, ("uniform", 30, 200), 4, 2)], 3, 3, 64, "bf16", 12, "d64_g1"),
    "bf16_d256_g2": lambda: small([SeqSpec(1200, ("lognormal", 128, 16, 700), "tenth", 3)], 4, 2, 256, "bf16", 13,
                                  "d256_g2"),
    "bf16_d128_g8_long_chunks": lambda: small([SeqSpec(2600, ("uniform", 300, 1024), 2, 1)], 16, 2, 128, "bf16", 14,
                                              "g8_long"),
    "bf16_d128_len1_chunks": lambda: small([SeqSpec(150, ("fixed", 1), 6, 4)], 4, 1, 128, "bf16", 15, "len1"),
    "bf16_divergent_heads": lambda: small([SeqSpec(1500, ("uniform", 16, 96), 7, 5)], 8, 2, 128, "bf16", 16,
                                          "divergent", topics_per_head=True),
    "f32_d128_g2": lambda: small([SeqSpec(400, ("uniform", 10, 90), 3, 1), SeqSpec(250, ("uniform", 40, 60), 1, 0)],
                                 4, 2, 128, "f32", 17, "f32_d128"),
    "f32_d32": lambda: small([SeqSpec(300, ("uniform", 5, 50), 2, 1)], 2, 1, 32, "f32", 18, "f32_d32"),
    # group sizes that are not a power of two (one head per workgroup slot) and larger than four
    "bf16_d128_g3": lambda: small([SeqSpec(800, ("uniform", 20, 130), 4, 2), SeqSpec(200, ("uniform", 8, 40), 2, 0)],
                                  6, 2, 128, "bf16", 19, "g3"),
    "bf16_d128_g16": lambda: small([SeqSpec(900, ("uniform", 24, 200), 5, 2)], 32, 2, 128, "bf16", 20, "g16",
                                   topics_per_head=True),
    # chunk lengths on both sides of the key tile (64 keys at d = 64 and 128, 32 at d = 256) and of the
    # staging group (8, 4 and 2 rows): tiles that lie inside one chunk, tiles that pack the ends of
    # several, short groups at chunk ends, chunks that some heads of a group keep and others do not
    "bf16_d128_tile_edges": lambda: small(
        [SeqSpec(1303, ("explicit", [63, 64, 65, 1, 127, 128, 129, 3, 4, 5, 66, 130, 62, 200, 64, 64, 31, 97]), 7, 2)],
        8, 2, 128, "bf16", 22, "tile_edges_d128", topics_per_head=True),
    "bf16_d256_tile_edges": lambda: small(
        [SeqSpec(838, ("explicit", [31, 32, 33, 1, 63, 64, 65, 2, 3, 95, 96, 97, 34, 30, 160, 32]), 6, 2)],
        4, 2, 256, "bf16", 23, "tile_edges_d256", topics_per_head=True),
    "bf16_d64_tile_edges": lambda: small(
        [SeqSpec(713, ("explicit", [7, 8, 9, 63, 64, 65, 1, 15, 16, 17, 127, 128, 129, 64]), 5, 2)],
        8, 2, 64, "bf16", 24, "tile_edges_d64", topics_per_head=True),
}


@pytest.fixture(scope="module", params=sorted(SMALL))
def small_case(request):
    return Case(SMALL[request.param]())


def test_small_summaries(small_case):
    check_summaries(small_case)


def test_small_routing_from_oracle_summaries(small_case):
    check_routing(small_case, small_case.o_qs, small_case.o_ks)


def test_small_routing_from_gpu_summaries(small_case):
    check_routing(small_case)


def test_small_attention(small_case):
    check_attention(small_case)


def test_small_end_to_end(small_case):
    check_end_to_end(small_case)


# routing once per KV head: the group's row, checked against the oracle's grouped routing, and the
# whole path end to end with it
GROUPED = ("bf16_d128_g4_ragged", "bf16_d128_g8_long_chunks", "bf16_d256_g2", "bf16_d64_g1", "bf16_divergent_heads",
           "f32_d128_g2", "bf16_d128_g3", "bf16_d128_g16", "bf16_d128_tile_edges", "bf16_d256_tile_edges")


@pytest.mark.parametrize("name", GROUPED)
def test_small_grouped_routing_and_end_to_end(name):
    case = Case(SMALL[name](), grouped=True)
    g_b, eq, tol = check_routing(case)
    G = case.w.num_q_heads // case.w.num_kv_heads
    for h in range(case.w.num_q_heads):      # every head of a group carries the group's row
        assert np.array_equal(g_b[h], g_b[(h // G) * G]), h
    check_routing(case, case.o_qs, case.o_ks)
    check_end_to_end(case)


def test_many_groups_take_the_padded_block_numbering():
    """More than 2048 (KV head, chunk) groups per XCD: the prefill kernel numbers its blocks with every
    group padded to the longest chunk's row tiles instead of compacting each XCD's real row tiles (the
    per-block scan over an XCD's groups would grow too long).  Whole path against the oracle."""
    w = small([SeqSpec(2100, ("uniform", 1, 7), 3, 0) for _ in range(8)], 4, 4, 64, "bf16", 21, "many_groups")
    assert (w.num_kv_heads * w.total_chunks + 7) // 8 > 2048
    case = Case(w)
    check_attention(case)
    check_end_to_end(case)


def test_binding_refuses_mis_sized_buffers():
    """Caller-supplied tensors the kernels read or write in full are checked for shape, dtype and device
    before any launch: a short output, a wrong-dtype LSE, short summaries, a mis-sized block list or
    decode kept array raise DhsaError."""
    case = Case(SMALL["bf16_d64_g1"]())
    L, plan, w = case.layout, case.plan, case.w
    bidx = torch.from_numpy(np.ascontiguousarray(case.o_bidx)).cuda()
    short_out = torch.empty((w.total_tokens - 1, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(D.DhsaError):
        D.sparse_prefill(L, plan, case.q, case.k, case.v, bidx, w.softmax_scale, out=short_out)
    with pytest.raises(D.DhsaError):
        D.sparse_prefill(L, plan, case.q, case.k, case.v, bidx, w.softmax_scale, return_lse=True,
                         lse=torch.empty((w.num_q_heads, w.total_tokens), dtype=torch.float64, device="cuda"))
    with pytest.raises(D.DhsaError):
        D.sparse_prefill(L, plan, case.q, case.k, case.v, bidx[:, :-1].contiguous(), w.softmax_scale)
    qs, ks = D.chunk_summarize(L, case.q, case.k)
    with pytest.raises(D.DhsaError):
        D.route(L, plan, qs[:-1].contiguous(), ks)
    with pytest.raises(D.DhsaError):
        D.route(L, plan, qs, ks, block_idx=torch.empty((w.num_q_heads, plan.nnz + 1), dtype=torch.int32,
                                                       device="cuda"))
    # the chunk walk reads cut_bits as dense 64-bit words: a strided or stride-0 view is refused
    nw = (w.total_tokens + 63) // 64
    sl = D.SeqLayout(w.cu_seqlens)
    with pytest.raises(D.DhsaError):
        D.chunk_boundaries(torch.zeros(2 * nw, dtype=torch.int64, device="cuda")[::2], sl, 4, 64)
    with pytest.raises(D.DhsaError):
        D.chunk_boundaries(torch.zeros(1, dtype=torch.int64, device="cuda").expand(nw), sl, 4, 64)
    st = D.DecodeState(1, 4, 2, 64, torch.bfloat16, 64, 8)
    q1 = torch.zeros((1, 4, 64), dtype=torch.bfloat16, device="cuda")
    k1 = torch.zeros((1, 2, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(D.DhsaError):
        st.step(q1, k1, k1, 4, 16, 0.5, 3, kept=torch.empty((1, 4, 2), dtype=torch.int32, device="cuda"))
    with pytest.raises(D.DhsaError):
        st.step(q1, k1, k1, 4, 16, 0.5, 3, out=torch.empty((1, 4, 64), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_lists_with_entries_outside_the_sequence_are_cleaned(dtype):
    """A caller's block list may hold entries that are not chunks of the query chunk's sequence up to
    the chunk itself (a chunk of an earlier sequence, a later chunk, -1 padding); both dtypes skip them,
    so the output equals oracle attention over the list without them, and the GPU's own output on
    that clean list, bit for bit."""
    seqs = [SeqSpec(400, ("uniform", 16, 64), 2, 1), SeqSpec(500, ("uniform", 16, 64), 2, 1),
            SeqSpec(300, ("uniform", 16, 64), 3, 0)]
    w = small(seqs, 4, 2, 64, dtype, 26, f"foreign_entries_{dtype}")
    case = Case(w)
    C, Hq = w.total_chunks, w.num_q_heads
    first = np.repeat(w.seq_chunk_start[:-1], np.diff(w.seq_chunk_start))
    rows = [[] for _ in range(Hq)]
    rp = [0]
    n_foreign = 0
    for i in range(C):
        kept = [case.o_bidx[h, case.o_rp[i]:case.o_rp[i + 1]].tolist() for h in range(Hq)]
        room = (i - first[i] + 1) - len(kept[0])          # a row holds at most i_loc + 1 entries
        extra = []
        if first[i] > 0:
            extra.append(int(first[i]) - 1)               # the last chunk of the previous sequence
        if i + 1 < C:
            extra.append(i + 1)                           # a later chunk
        extra.append(-1)
        extra = extra[:max(room, 0)]
        n_foreign += len(extra)
        for h in range(Hq):
            rows[h].append(sorted(kept[h] + extra))
        rp.append(rp[-1] + len(rows[0][-1]))
    assert n_foreign > C // 2
    plan = D.RoutePlan.from_row_ptr(case.layout, np.array(rp, np.int32))
    bidx = np.array([[x for r in rows[h] for x in r] for h in range(Hq)], np.int32)
    out, lse = D.sparse_prefill(case.layout, plan, case.q, case.k, case.v, torch.from_numpy(bidx).cuda(),
                                w.softmax_scale, return_lse=True)
    torch.cuda.synchronize()
    g_o, g_l = out.float().cpu().numpy(), lse.cpu().numpy()
    c_o, c_l = case.gpu_attend(case.o_bidx)
    assert np.array_equal(g_o, c_o) and np.array_equal(g_l, c_l)
    o_o, o_l = case.oracle_attend(case.o_bidx)
    assert np.abs(g_o - o_o).max() <= OUT_ATOL[dtype]
    assert np.abs(g_l - o_l).max() <= LSE_ATOL[dtype]


def test_budget_extremes():
    w = small([SeqSpec(800, ("uniform", 20, 80), 0, 2), SeqSpec(500, ("uniform", 10, 60), 0, 0)], 4, 2, 128, "bf16",
              21, "extremes")
    C = w.total_chunks
    for tk in (np.zeros(C, np.int32), np.full(C, 10000, np.int32), np.arange(C, dtype=np.int32) % 5):
        case = Case(w, topk=tk)
        check_routing(case)
        check_attention(case)


def test_dense_budget_equals_dense_attention():
    w = small([SeqSpec(600, ("uniform", 16, 120), 10000, 2), SeqSpec(300, ("uniform", 16, 120), 10000, 0)], 8, 2, 128,
              "bf16", 22, "dense")
    case = Case(w)
    g_b, g_o, _ = case.gpu_prefill()
    dense, _ = oracle.dense_attention(case.qf, case.kf, case.vf, w.cu_seqlens, w.softmax_scale)
    assert np.abs(g_o - dense).max() <= ATOL_BF16


def test_rows_keeping_more_than_a_wave_of_chunks():
    # rows keep 70..100 of up to ~300 earlier chunks: more kept chunks than lanes in a wave
    w = small([SeqSpec(2400, ("uniform", 4, 12), 0, 4)], 4, 1, 64, "bf16", 23, "wide")
    tk = 70 + (np.arange(w.total_chunks) % 31).astype(np.int32)
    case = Case(w, topk=tk)
    assert max(np.diff(case.o_rp) - 1) > 64 and case.w.total_chunks > 200
    check_routing(case)
    check_routing(case, case.o_qs, case.o_ks)
    check_attention(case, heads=[0, 3], chunks=list(range(0, case.w.total_chunks, 7)))


def test_rows_beyond_register_candidates_use_general_selection():
    # one sequence of ~1250 short chunks: late rows have more than 1024 candidates, which the main
    # routing kernel does not hold in registers, so the general sorting kernel selects them
    w = small([SeqSpec(6200, ("uniform", 2, 8), 0, 0)], 4, 4, 64, "bf16", 25, "very_wide")
    tk = np.where(np.arange(w.total_chunks) % 3 == 0, 40, 700).astype(np.int32)
    case = Case(w, topk=tk)
    assert w.total_chunks > 1100
    check_routing(case)
    check_routing(case, case.o_qs, case.o_ks)
    check_attention(case, heads=[1], chunks=list(range(1030, case.w.total_chunks, 37)))


def test_exact_ties_break_to_lower_index():
    # equal-length chunks with identical integer-valued tokens: every score is exactly equal
    T, n, d = 640, 16, 128
    w = small([SeqSpec(T, ("fixed", n), 5, 0)], 4, 2, d, "bf16", 24, "ties")
    rng = np.random.default_rng(0)
    proto_q = rng.integers(-2, 3, size=(1, 4, d)).astype(np.float32)
    proto_k = rng.integers(-2, 3, size=(1, 2, d)).astype(np.float32)
    w.q = W.f32_to_bf16_bits(np.repeat(proto_q, T, axis=0))
    w.k = W.f32_to_bf16_bits(np.repeat(proto_k, T, axis=0))
    case = Case(w)
    g_b = case.gpu_route()
    assert np.array_equal(g_b, case.o_bidx)
    for i in range(6, w.total_chunks):
        assert case.o_bidx[0, case.o_rp[i]:case.o_rp[i + 1]].tolist() == [0, 1, 2, 3, 4, i]


def test_deterministic_and_ragged_equals_separate():
    seqs = [SeqSpec(500, ("uniform", 16, 128), 3, 1), SeqSpec(900, ("uniform", 64, 200), 4, 2),
            SeqSpec(300, ("fixed", 64), 2, 0)]
    w = small(seqs, 8, 2, 128, "bf16", 25, "ragged")
    case = Case(w)
    b1, o1, l1 = case.gpu_prefill()
    b2, o2, l2 = case.gpu_prefill()
    assert np.array_equal(b1, b2) and np.array_equal(o1, o2) and np.array_equal(l1, l2)
    for b in range(3):
        s, e = w.cu_seqlens[b], w.cu_seqlens[b + 1]
        c0, c1 = w.seq_chunk_start[b], w.seq_chunk_start[b + 1]
        cc = (w.cu_chunks[c0:c1 + 1] - s).astype(np.int32)
        r = D.prefill(case.q[s:e].contiguous(), case.k[s:e].contiguous(), case.v[s:e].contiguous(), [0, e - s], cc,
                      [0, c1 - c0], w.topk[c0:c1], w.softmax_scale, return_lse=True)
        assert np.array_equal(r["out"].float().cpu().numpy(), o1[s:e])
        bi = r["block_idx"].cpu().numpy() + c0
        for i in range(c1 - c0):
            rs, re_ = r["plan"].h_row_ptr[i], r["plan"].h_row_ptr[i + 1]
            assert np.array_equal(bi[:, rs:re_], b1[:, case.o_rp[c0 + i]:case.o_rp[c0 + i + 1]])


def test_empty_batch():
    for dt in (torch.bfloat16, torch.float32):
        q = torch.empty((0, 4, 128), dtype=dt, device="cuda")
        k = torch.empty((0, 2, 128), dtype=dt, device="cuda")
        r = D.prefill(q, k, k, [0], [0], [0], np.zeros(0, np.int32), 0.1, return_lse=True)
        assert r["out"].shape == (0, 4, 128) and r["block_idx"].shape == (4, 0)


# ------------------------------------------------------------------------------------------ full-size configs
def _sample_rows(case: Case, n_heads=4, n_chunks=12, seed=0):
    rng = np.random.default_rng(seed)
    w = case.w
    lens = np.diff(w.cu_chunks)
    C = w.total_chunks
    heads = sorted(set([0, w.num_q_heads - 1] + rng.choice(w.num_q_heads, n_heads, replace=False).tolist()))
    chunks = {0, C - 1, int(np.argmax(lens)), int(np.argmin(lens))}
    chunks |= {int(nd[0]) for nd in w.needles[:3]}
    chunks |= set(rng.choice(C, n_chunks, replace=False).tolist())
    chunks |= {int(c) for c in w.seq_chunk_start[1:-1]}          # first chunk of later sequences
    chunks |= {int(c) - 1 for c in w.seq_chunk_start[1:]}         # last chunk of every sequence
    return heads, sorted(c for c in chunks if 0 <= c < C)


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_full_config_sampled(cfg):
    case = Case(W.make_config(cfg))
    check_summaries(case)
    _, eq, tol = check_routing(case)
    print(f"[cfg{cfg}] kept sets: {eq} equal rows, {tol} tolerated swaps", flush=True)
    heads, chunks = _sample_rows(case)
    err, lerr = check_attention(case, heads, chunks)
    print(f"[cfg{cfg}] sampled {len(heads)}x{len(chunks)} rows: out err {err:.3e}, lse err {lerr:.3e}", flush=True)
    # the whole path on a second, independent sample of rows
    heads, chunks = _sample_rows(case, seed=1)
    check_end_to_end(case, heads, chunks)


@pytest.mark.slow
def test_full_config_grouped_sampled():
    """The 128K workload routed once per KV head: every row's kept set against the oracle's grouped
    routing, and the whole path on sampled rows."""
    case = Case(W.make_config(3), grouped=True)
    _, eq, tol = check_routing(case)
    print(f"[cfg3 grouped] kept sets: {eq} equal rows, {tol} tolerated swaps", flush=True)
    heads, chunks = _sample_rows(case, seed=2)
    check_end_to_end(case, heads, chunks)


@pytest.mark.slow
def test_maximum_chunks_per_sequence():
    """8192 chunks in one sequence (the supported maximum): rows past 1024 candidates take the general
    sorting kernel, the prefill's chunk bitmaps are at their largest; every row's kept set against
    the oracle, attention on sampled rows, among them the last chunk's (8191 candidates)."""
    n, C = 4, 8192
    w = small([SeqSpec(n * C, ("fixed", n), 0, 0)], 2, 1, 64, "bf16", 43, "max_chunks")
    assert w.total_chunks == C
    i_loc = np.arange(C)
    tk = np.where(i_loc % 5 == 0, 100, np.where(i_loc % 5 == 1, 1500, 7)).astype(np.int32)
    case = Case(w, topk=tk)
    _, eq, tol = check_routing(case)
    print(f"[max chunks] kept sets: {eq} equal rows, {tol} tolerated swaps", flush=True)
    check_attention(case, heads=[0, 1], chunks=[0, 1, 1023, 1024, 1025, 4000, 8190, 8191])
