"""GPU parity of routing under a token budget (dhsa_route_plan_tokens + dhsa_route_tokens) against
the token-budget oracle, and of the sparse prefill on the padded block lists it writes.

  * routing   -- every row against the oracle's, equal except where near-equal fp32 scores
                 (within 1e-4 relative) reorder the ranking (tests/parity.py compare_token_rows);
                 from the oracle's summaries and from the GPU's;
  * equal chunk lengths -- a budget of b tokens must give exactly the GPU's own top-(b // L)
                 routing, entry for entry (both select from the same fp32 scores);
  * attention -- the GPU prefill fed the oracle's padded list against oracle attention on it
                 (max-abs 2e-2 bf16 / 1e-4 fp32, LSE 2e-3 / 1e-4), and end to end on rows whose
                 kept lists are identical.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from parity import ATOL_BF16, ATOL_F32, compare_token_rows

pytestmark = pytest.mark.gpu

import dynamic_sparse_attention_dhsa_amd as D  # noqa: E402
from dynamic_sparse_attention_dhsa_amd import workloads as W  # noqa: E402
from dynamic_sparse_attention_dhsa_amd.workloads import SeqSpec  # noqa: E402

OUT_ATOL = {"bf16": ATOL_BF16, "f32": ATOL_F32}
LSE_ATOL = {"bf16": 2e-3, "f32": 1e-4}


def _dev(a, dt):
    a = np.ascontiguousarray(a)
    if dt == "bf16":
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


class TokenCase:
    def __init__(self, w: W.Workload, budget, grouped=False):
        self.w, self.grouped = w, grouped
        self.budget = np.asarray(budget, np.int32)
        print(f"[case] {w.name} seed={w.seed} T={w.total_tokens} C={w.total_chunks} Hq={w.num_q_heads} "
              f"Hkv={w.num_kv_heads} d={w.head_dim} {w.dtype} grouped={grouped}", flush=True)
        self.q, self.k, self.v = (_dev(a, w.dtype) for a in (w.q, w.k, w.v))
        self.qf, self.kf, self.vf = w.q_f32(), w.k_f32(), w.v_f32()
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.layout = D.Layout(w.cu_seqlens, w.cu_chunks, w.seq_chunk_start, w.num_q_heads, w.num_kv_heads,
                               w.head_dim, tdt)
        self.plan = D.TokenPlan(self.layout, self.budget)
        self.o_qs = oracle.chunk_summaries(self.qf, w.cu_chunks)
        self.o_ks = oracle.chunk_summaries(self.kf, w.cu_chunks)
        self.o_rp, self.o_bidx, S = oracle.route_tokens(self.o_qs, self.o_ks, w.cu_chunks, w.seq_chunk_start,
                                                        self.budget, grouped=grouped)
        self.o_scores = np.repeat(S, w.num_q_heads // S.shape[0], axis=0)
        assert np.array_equal(self.o_rp, self.plan.h_row_ptr)

    def gpu_route(self, from_oracle=False):
        if from_oracle:
            qs, ks = torch.from_numpy(self.o_qs).cuda(), torch.from_numpy(self.o_ks).cuda()
        else:
            qs, ks = D.chunk_summarize(self.layout, self.q, self.k)
        b = D.route_tokens(self.layout, self.plan, qs, ks, grouped=self.grouped)
        torch.cuda.synchronize()
        return b.cpu().numpy()

    def check_routing(self, from_oracle=False, heads=None):
        g = self.gpu_route(from_oracle)
        eq, tol, fails = compare_token_rows(g, self.o_bidx, self.o_rp, self.o_scores, self.w.seq_chunk_start,
                                            self.w.cu_chunks, self.budget, heads=heads)
        assert not fails, f"{len(fails)} routing failures, first: {fails[:3]}"
        return g, eq, tol

    def check_attention(self, heads=None, chunks=None):
        bidx = torch.from_numpy(np.ascontiguousarray(self.o_bidx)).cuda()
        out, lse = D.sparse_prefill(self.layout, self.plan, self.q, self.k, self.v, bidx, self.w.softmax_scale,
                                    return_lse=True)
        torch.cuda.synchronize()
        g_o, g_l = out.float().cpu().numpy(), lse.cpu().numpy()
        o_o, o_l = oracle.attend(self.qf, self.kf, self.vf, self.w.cu_chunks, self.o_rp, self.o_bidx,
                                 self.w.softmax_scale, heads=heads, chunks=chunks)
        sel = ~np.isnan(o_o)
        assert sel.any()
        err = float(np.abs(g_o[sel] - o_o[sel]).max())
        lerr = float(np.abs(g_l[~np.isnan(o_l)] - o_l[~np.isnan(o_l)]).max())
        assert err <= OUT_ATOL[self.w.dtype], f"out max-abs err {err:.3e}"
        assert lerr <= LSE_ATOL[self.w.dtype], f"lse max-abs err {lerr:.3e}"
        return err, lerr

    def check_end_to_end(self, heads=None, chunks=None):
        r = D.prefill(self.q, self.k, self.v, self.w.cu_seqlens, self.w.cu_chunks, self.w.seq_chunk_start,
                      token_budget=self.budget, softmax_scale=self.w.softmax_scale, grouped=self.grouped)
        torch.cuda.synchronize()
        g_b, g_o = r["block_idx"].cpu().numpy(), r["out"].float().cpu().numpy()
        _, _, fails = compare_token_rows(g_b, self.o_bidx, self.o_rp, self.o_scores, self.w.seq_chunk_start,
                                         self.w.cu_chunks, self.budget, heads=heads)
        assert not fails, fails[:3]
        o_o, _ = oracle.attend(self.qf, self.kf, self.vf, self.w.cu_chunks, self.o_rp, self.o_bidx,
                               self.w.softmax_scale, heads=heads, chunks=chunks)
        cc, rp = self.w.cu_chunks, self.o_rp
        worst, compared = 0.0, 0
        for h in (range(self.w.num_q_heads) if heads is None else heads):
            for i in (range(self.w.total_chunks) if chunks is None else chunks):
                if not np.array_equal(g_b[h, rp[i]:rp[i + 1]], self.o_bidx[h, rp[i]:rp[i + 1]]):
                    continue
                s, e = cc[i], cc[i + 1]
                worst = max(worst, float(np.abs(g_o[s:e, h] - o_o[s:e, h]).max()))
                compared += 1
        assert compared > 0
        assert worst <= OUT_ATOL[self.w.dtype], f"end-to-end max-abs err {worst:.3e}"


def _budgets(w, seed, scale):
    """Per-chunk budgets from 0 to about ``scale`` mean chunk lengths, with a few that keep everything."""
    rng = np.random.default_rng(seed)
    C = w.total_chunks
    mean = max(1.0, w.total_tokens / max(C, 1))
    b = rng.integers(0, int(scale * mean) + 2, size=C)
    b[rng.random(C) < 0.1] = 1 << 30
    return b.astype(np.int32)


SMALL = {
    "bf16_d128_g4_ragged": lambda: W.make_workload(
        [SeqSpec(900, ("uniform", 10, 150), 0, 2), SeqSpec(333, ("uniform", 1, 40), 0, 1), SeqSpec(1, ("fixed", 1), 0, 0),
         SeqSpec(0, ("fixed", 8), 0, 0)], 8, 2, 128, "bf16", seed=31, name="tok_ragged"),
    "bf16_d64_g1": lambda: W.make_workload([SeqSpec(1100, ("uniform", 30, 200), 0, 2)], 3, 3, 64, "bf16", seed=32,
                                           name="tok_d64"),
    "bf16_d256_lognormal": lambda: W.make_workload([SeqSpec(1500, ("lognormal", 128, 16, 700), 0, 3)], 4, 2, 256,
                                                   "bf16", seed=33, name="tok_d256"),
    "bf16_divergent_heads": lambda: W.make_workload([SeqSpec(1600, ("uniform", 8, 96), 0, 5)], 8, 2, 128, "bf16",
                                                    seed=34, name="tok_divergent", topics_per_head=True),
    "f32_d128": lambda: W.make_workload([SeqSpec(500, ("uniform", 10, 90), 0, 1), SeqSpec(250, ("uniform", 3, 60), 0, 0)],
                                        4, 2, 128, "f32", seed=35, name="tok_f32"),
}


@pytest.mark.parametrize("grouped", [False, True])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_token_routing_and_attention(name, grouped):
    w = SMALL[name]()
    case = TokenCase(w, _budgets(w, 40 + len(name), 6), grouped=grouped)
    assert (np.diff(case.o_rp) > 1).any()
    case.check_routing(from_oracle=True)
    _, eq, tol = case.check_routing()
    print(f"[{name}] kept lists: {eq} equal rows, {tol} tolerated", flush=True)
    pad = (case.o_bidx == -1).sum()
    print(f"[{name}] -1 padding entries in the oracle lists: {pad}", flush=True)
    case.check_attention()
    case.check_end_to_end()


@pytest.mark.parametrize("grouped", [False, True])
def test_equal_lengths_budget_is_topk_exactly(grouped):
    L = 48
    w = W.make_workload([SeqSpec(48 * 40, ("fixed", L), 0, 2), SeqSpec(48 * 17, ("fixed", L), 0, 1)], 8, 2, 128, "bf16",
                        seed=36, name="tok_equal")
    rng = np.random.default_rng(5)
    budget = rng.integers(0, 12 * L, size=w.total_chunks).astype(np.int32)
    case = TokenCase(w, budget, grouped=grouped)
    g_tok = case.gpu_route()
    plan_k = D.RoutePlan(case.layout, budget // L)
    assert np.array_equal(plan_k.h_row_ptr, case.plan.h_row_ptr)
    qs, ks = D.chunk_summarize(case.layout, case.q, case.k)
    g_k = D.route(case.layout, plan_k, qs, ks, grouped=grouped).cpu().numpy()
    assert np.array_equal(g_tok, g_k)
    assert not (g_tok == -1).any()
    case.check_routing()


def test_budget_extremes_and_padding():
    w = W.make_workload([SeqSpec(1200, ("uniform", 5, 120), 0, 2), SeqSpec(700, ("uniform", 20, 60), 0, 0)], 4, 2, 128,
                        "bf16", seed=37, name="tok_extremes")
    C = w.total_chunks
    lens = np.diff(w.cu_chunks)
    for budget in (np.zeros(C, np.int32), np.full(C, 1 << 30, np.int32), np.full(C, int(lens.min()) - 1, np.int32),
                   (lens * 3).astype(np.int32)):
        case = TokenCase(w, budget)
        g, _, _ = case.check_routing()
        if not budget.any():
            # nothing fits: every row is its diagonal alone
            assert np.array_equal(np.diff(case.o_rp), np.ones(C, np.int32))
        case.check_attention()


def test_beyond_register_candidates_with_full_rows():
    # ~1250 short chunks in one sequence: rows past 1024 candidates are supported when their budget
    # keeps every earlier chunk; the others select in registers
    w = W.make_workload([SeqSpec(6200, ("uniform", 2, 8), 0, 0)], 4, 4, 64, "bf16", seed=38, name="tok_wide")
    C = w.total_chunks
    assert C > 1100
    cc = w.cu_chunks
    rng = np.random.default_rng(9)
    budget = rng.integers(0, 600, size=C).astype(np.int32)
    budget[1025:] = (cc[1025:C] - cc[0]).astype(np.int32)
    case = TokenCase(w, budget)
    case.check_routing()
    case.check_routing(from_oracle=True)
    case.check_attention(heads=[2], chunks=list(range(0, C, 41)))


@pytest.mark.parametrize("grouped", [False, True])
def test_budget_over_register_candidates_takes_the_general_kernel(grouped):
    """~1250 short chunks in one sequence, budgets that keep some but not all earlier chunks: rows past
    1024 candidates select in the general kernel (sorted keys, then the longest fitting prefix of the
    ranking by a block scan of the lengths); every row against the oracle, attention on sampled rows."""
    w = W.make_workload([SeqSpec(6200, ("uniform", 2, 8), 0, 0)], 4, 4, 64, "bf16", seed=38, name="tok_wide")
    C = w.total_chunks
    assert C > 1100
    rng = np.random.default_rng(10)
    budget = rng.integers(0, 2000, size=C).astype(np.int32)
    budget[rng.random(C) < 0.05] = 0
    case = TokenCase(w, budget, grouped=grouped)
    first = 0
    assert any(i - first > 1024 and 0 < budget[i] < w.cu_chunks[i] for i in range(C))
    case.check_routing()
    case.check_routing(from_oracle=True)
    case.check_attention(heads=[1], chunks=list(range(1000, C, 29)))
    case.check_end_to_end(heads=[0, 3], chunks=[1030, 1100, C - 1])


@pytest.mark.slow
def test_128k_short_chunks_token_budget():
    """131072 tokens in chunks of 16..48 tokens (about 4100 chunks): most rows have more than 1024
    candidates and a budget of about 32 mean chunks, so they select in the general kernel; every row's
    kept list against the oracle, attention on sampled rows."""
    w = W.make_workload([SeqSpec(131072, ("uniform", 16, 48), 0, 16)], 4, 2, 64, "bf16", seed=44,
                        name="tok_128k_short")
    C = w.total_chunks
    assert C > 3500
    rng = np.random.default_rng(11)
    budget = rng.integers(600, 1500, size=C).astype(np.int32)
    case = TokenCase(w, budget)
    _, eq, tol = case.check_routing()
    print(f"[128K short chunks] kept lists: {eq} equal rows, {tol} tolerated", flush=True)
    case.check_end_to_end(heads=[0, 3], chunks=[0, 1500, 3000, C - 1])


@pytest.mark.parametrize("grouped", [False, True])
def test_exact_ties_break_to_lower_index_tokens(grouped):
    """Identical integer-valued tokens with q equal to its KV head's k: a chunk's score is
    sqrt(n_i n_j) |k|^2, so chunks of equal length tie exactly and longer ones rank first; the kept
    lists (many exact ties at the budget boundary) must equal the oracle's entry for entry."""
    lens = [16, 32] * 12
    T, d = sum(lens), 128
    w = W.make_workload([SeqSpec(T, ("explicit", lens), 0, 0)], 4, 2, d, "bf16", seed=39, name="tok_ties")
    rng = np.random.default_rng(3)
    proto_k = rng.integers(-2, 3, size=(1, 2, d)).astype(np.float32)
    proto_q = np.repeat(proto_k, 2, axis=1)
    w.q = W.f32_to_bf16_bits(np.repeat(proto_q, T, axis=0))
    w.k = W.f32_to_bf16_bits(np.repeat(proto_k, T, axis=0))
    budget = rng.integers(0, 400, size=w.total_chunks).astype(np.int32)
    case = TokenCase(w, budget, grouped=grouped)
    g = case.gpu_route()
    assert np.array_equal(g, case.o_bidx)
    # a row whose budget ends inside the 32-token class keeps the lowest-index 32-token chunks
    i = w.total_chunks - 1
    row = case.o_bidx[0, case.o_rp[i]:case.o_rp[i + 1]]
    kept = [j for j in row.tolist() if 0 <= j < i]
    m32 = int(budget[i]) // 32                   # the row has 11 earlier 32-token chunks
    want = [2 * x + 1 for x in range(m32)] if m32 < 11 else None
    if want is not None:
        assert kept == want, (kept, want, int(budget[i]))


@pytest.mark.slow
@pytest.mark.parametrize("grouped", [False, True])
def test_full_128k_token_budget(grouped):
    """The 128K workload (32 q / 8 KV heads, d 128) with an 8192-token budget per row (32 chunks of
    the mean length): every row's kept list against the oracle, attention on sampled rows."""
    w = W.make_config(3)
    budget = np.full(w.total_chunks, 8192, np.int32)
    case = TokenCase(w, budget, grouped=grouped)
    _, eq, tol = case.check_routing()
    print(f"[128K tokens grouped={grouped}] kept lists: {eq} equal rows, {tol} tolerated", flush=True)
    C = w.total_chunks
    chunks = sorted({0, 1, 40, 200, C // 2, C - 2, C - 1})
    case.check_end_to_end(heads=[0, 13, 31], chunks=chunks)
