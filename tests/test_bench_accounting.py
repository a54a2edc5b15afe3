"""The benchmark's bookkeeping (CPU): the kept-FLOP count behind the roofline fraction, the stage
byte counts against the sizes of the arrays they stand for, and the refusal of a multi-GPU run.

bench.kept_flops counts 4·d FLOPs (QK^T and PV, a multiply-add each) per kept (query, key) pair from a
block list, per chunk row.  It is checked against the token-level keep mask the oracle builds by
broadcasting kept chunks to token pairs and masking u <= t, summed pair by pair, under a chunk count,
under a token budget (rows padded with -1) and with every chunk kept (all causal pairs, a closed form).
"""
import subprocess
import sys
import os

import numpy as np

import bench
import oracle
from dynamic_sparse_attention_dhsa_amd import workloads as W
from dynamic_sparse_attention_dhsa_amd.workloads import SeqSpec

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _layout(seed):
    w = W.make_workload([SeqSpec(300, ("uniform", 8, 40), 0, 0), SeqSpec(0, ("fixed", 8), 0, 0),
                         SeqSpec(170, ("uniform", 4, 30), 0, 0)], 4, 2, 16, "f32", seed=seed, name="acct")
    qs = oracle.chunk_summaries(w.q_f32(), w.cu_chunks)
    ks = oracle.chunk_summaries(w.k_f32(), w.cu_chunks)
    return w, qs, ks


def _bruteforce(rp, bidx, cu_chunks, d):
    return 4.0 * d * sum(int(oracle.kept_token_mask(rp, bidx[h], cu_chunks).sum()) for h in range(bidx.shape[0]))


def test_kept_flops_chunk_budget():
    w, qs, ks = _layout(11)
    for topk in (0, 2, 5):
        rp, bidx, _ = oracle.route(qs, ks, w.seq_chunk_start, np.full(w.total_chunks, topk, np.int32))
        assert bench.kept_flops(bidx, rp, w.cu_chunks, w.head_dim) == _bruteforce(rp, bidx, w.cu_chunks, w.head_dim)


def test_kept_flops_token_budget_with_padding():
    w, qs, ks = _layout(12)
    budget = np.full(w.total_chunks, 60, np.int32)
    rp, bidx, _ = oracle.route_tokens(qs, ks, w.cu_chunks, w.seq_chunk_start, budget)
    assert (bidx < 0).any(), "the budget should leave padded rows"
    assert bench.kept_flops(bidx, rp, w.cu_chunks, w.head_dim) == _bruteforce(rp, bidx, w.cu_chunks, w.head_dim)


def test_kept_flops_dense_is_all_causal_pairs():
    w, qs, ks = _layout(13)
    rp, bidx, _ = oracle.route(qs, ks, w.seq_chunk_start, np.full(w.total_chunks, 10 ** 6, np.int32))
    n = np.diff(w.cu_seqlens).astype(np.int64)
    pairs = int((n * (n + 1) // 2).sum())
    assert bench.kept_flops(bidx, rp, w.cu_chunks, w.head_dim) == 4.0 * w.head_dim * w.num_q_heads * pairs


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr and r.stdout.strip() == ""


def test_stage_bytes_match_the_arrays_moved():
    """Stage 1 reads Q and K once and writes both summaries; stage 2 reads the summaries, the row
    pointers and the per-chunk sequence starts and writes the block list: the formula against the
    sizes of those arrays for a bf16 and an fp32 workload."""
    for dtype in ("bf16", "f32"):
        w = W.make_workload([SeqSpec(200, ("uniform", 8, 40), 0, 0), SeqSpec(90, ("uniform", 4, 30), 0, 0)],
                            8, 2, 32, dtype, seed=14, name="acct")
        qs = oracle.chunk_summaries(w.q_f32(), w.cu_chunks).astype(np.float32)
        ks = oracle.chunk_summaries(w.k_f32(), w.cu_chunks).astype(np.float32)
        rp, bidx, _ = oracle.route(qs, ks, w.seq_chunk_start, np.full(w.total_chunks, 2, np.int32))
        bidx = bidx.astype(np.int32)
        s = 2 if dtype == "bf16" else 4
        b1, b2 = bench.stage_bytes(w.total_tokens, w.total_chunks, w.num_q_heads, w.num_kv_heads, w.head_dim, s,
                                   bidx.shape[1])
        assert w.q.dtype.itemsize == s and w.k.dtype.itemsize == s
        assert b1 == w.q.nbytes + w.k.nbytes + qs.nbytes + ks.nbytes
        per_chunk_seq_start = np.zeros(w.total_chunks, np.int32)        # one int per chunk
        assert b2 == qs.nbytes + ks.nbytes + rp.astype(np.int32).nbytes + per_chunk_seq_start.nbytes + bidx.nbytes
