"""GPU parity on a seeded sweep of small random layouts, through the same checks as the named cases.

Each case draws, from its own seed: 1-4 sequences of 0-1200 tokens (empty and one-token sequences
included), a chunk-length range, a per-sequence chunk budget (0 to past every earlier chunk), needles,
the head layout (Hkv 1-4, group sizes 1, 2, 3, 4, 5, 8), the head dimension and dtype (bf16: 64, 128,
256; fp32: 32, 64, 128), head-specific topics or shared ones, and routing per query head or per KV head.
Checks per case: summaries, routing from the GPU summaries, attention on the oracle's block list (output
and LSE), and the whole path end to end.  A second sweep routes under a token budget instead, with a
budget drawn per query chunk (0 to about eight mean chunk lengths), through the token-budget checks.
"""
from __future__ import annotations

import numpy as np
import pytest

from dynamic_sparse_attention_dhsa_amd import workloads as W
from dynamic_sparse_attention_dhsa_amd.workloads import SeqSpec
from test_gpu_parity import Case, check_attention, check_end_to_end, check_routing, check_summaries
from test_gpu_token_budget import TokenCase

pytestmark = pytest.mark.gpu

N_CASES = 16
N_TOKEN_CASES = 12


def draw_case(i: int, base: int = 7000):
    rng = np.random.default_rng(base + i)
    B = int(rng.integers(1, 5))
    seqs = []
    for _ in range(B):
        kind = rng.random()
        length = 0 if kind < 0.08 else 1 if kind < 0.14 else int(rng.integers(2, 1201))
        lo = int(rng.integers(1, 33))
        hi = int(rng.integers(lo, lo + 97))
        budget = int(rng.integers(0, 12))
        seqs.append(SeqSpec(length, ("uniform", lo, hi), budget, int(rng.integers(0, 3))))
    if sum(s.length for s in seqs) == 0:
        seqs[0] = SeqSpec(257, ("uniform", 8, 64), 3, 1)
    Hkv = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 3, 4, 5, 8]))
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    d = int(rng.choice([32, 64, 128] if dtype == "f32" else [64, 128, 256]))
    grouped = bool(rng.random() < 0.4) and G > 1
    topics_per_head = bool(rng.random() < 0.3)
    w = W.make_workload(seqs, Hkv * G, Hkv, d, dtype, seed=base + 100 + i, name=f"sweep{base}_{i}",
                        topics_per_head=topics_per_head)
    return w, grouped, rng


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_layout(i):
    w, grouped, _ = draw_case(i)
    print(f"[sweep {i}] B={w.num_seqs} lens={np.diff(w.cu_seqlens).tolist()} chunks={w.total_chunks} "
          f"Hq/Hkv={w.num_q_heads}/{w.num_kv_heads} d={w.head_dim} {w.dtype} grouped={grouped} "
          f"topk={sorted(set(w.topk.tolist()))}", flush=True)
    case = Case(w, grouped=grouped)
    check_summaries(case)
    check_routing(case)
    check_attention(case)
    check_end_to_end(case)


@pytest.mark.parametrize("i", range(N_TOKEN_CASES))
def test_random_layout_token_budget(i):
    w, grouped, rng = draw_case(i, base=7500)
    mean_len = max(1.0, w.total_tokens / max(1, w.total_chunks))
    budget = rng.integers(0, int(8 * mean_len) + 2, size=w.total_chunks).astype(np.int32)
    print(f"[sweep tokens {i}] B={w.num_seqs} lens={np.diff(w.cu_seqlens).tolist()} chunks={w.total_chunks} "
          f"Hq/Hkv={w.num_q_heads}/{w.num_kv_heads} d={w.head_dim} {w.dtype} grouped={grouped} "
          f"budget max={int(budget.max()) if budget.size else 0}", flush=True)
    case = TokenCase(w, budget, grouped=grouped)
    case.check_routing()
    case.check_attention()
    case.check_end_to_end()
