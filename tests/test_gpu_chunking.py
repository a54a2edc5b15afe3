"""GPU parity of the online chunking calls (this library's own boundary rule) against the CPU oracle.

Similarity: the GPU accumulates in fp32, the oracle in fp64 rounded to fp32; they must agree within
SIM_ATOL.  Cut bits: exactly the GPU's own decisions sim < tau, and the oracle's wherever the oracle's
similarity is farther than SIM_ATOL from tau (only there can the two precisions decide differently).
Boundaries: integer work, so bit-exact: the GPU walk equals the oracle's walk over the GPU's own
similarity array, and equals the oracle end to end when no similarity lies within SIM_ATOL of tau.
"""
import numpy as np
import pytest
import torch

import oracle
from dynamic_sparse_attention_dhsa_amd import binding as Bd
from dynamic_sparse_attention_dhsa_amd import workloads as W
from dynamic_sparse_attention_dhsa_amd.workloads import SeqSpec

pytestmark = pytest.mark.gpu

SIM_ATOL = 1e-5


def _dev_k(w):
    if w.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(w.k).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(w.k)).cuda()


def _check(w, lo, hi, tau):
    T = w.total_tokens
    k = _dev_k(w)
    sim, bits = Bd.adjacent_similarity(k, w.cu_seqlens, tau)
    cu, scs, nch = Bd.chunk_boundaries(bits, w.cu_seqlens, lo, hi)
    torch.cuda.synchronize()
    g_sim = sim.cpu().numpy()
    g_bits = bits.cpu().numpy().view(np.uint64)
    C = int(nch.cpu().item())
    g_cu = cu.cpu().numpy()[:C + 1]
    g_scs = scs.cpu().numpy()
    o_sim = oracle.adjacent_similarity(w.k_f32(), w.cu_seqlens)
    err = np.abs(g_sim - o_sim).max() if T else 0.0
    assert err <= SIM_ATOL, f"sim max-abs err {err:.3e}"
    # cut bits: the GPU's own decisions, exactly; zero past T
    dec = np.zeros(((T + 63) // 64) * 64, bool)
    dec[:T] = g_sim < np.float32(tau)
    want = np.packbits(dec.reshape(-1, 64)[:, ::-1], axis=1).view(">u8").ravel().astype(np.uint64)
    assert np.array_equal(g_bits, want)
    far = np.abs(o_sim - np.float32(tau)) > SIM_ATOL
    assert np.array_equal((o_sim < np.float32(tau))[far], (g_sim < np.float32(tau))[far])
    # boundaries: bit-exact against the oracle's walk over the GPU similarity
    o_cu, o_scs = oracle.chunk_boundaries(g_sim, w.cu_seqlens, lo, hi, tau)
    assert np.array_equal(g_cu, o_cu) and np.array_equal(g_scs, o_scs), (g_cu[:20], o_cu[:20])
    if far.all():
        e_cu, e_scs = oracle.chunk_boundaries(o_sim, w.cu_seqlens, lo, hi, tau)
        assert np.array_equal(g_cu, e_cu) and np.array_equal(g_scs, e_scs)
    return g_cu, g_scs, int((~far).sum())


SMALL = [
    # (seqs, Hkv, d, dtype, seed)
    ([SeqSpec(700, ("uniform", 24, 160), 4, 2), SeqSpec(0, ("uniform", 8, 8), 1, 0),
      SeqSpec(301, ("uniform", 16, 64), 3, 0)], 2, 128, "bf16", 31),
    ([SeqSpec(1, ("fixed", 1), 0, 0), SeqSpec(65, ("uniform", 4, 20), 2, 0),
      SeqSpec(64, ("fixed", 64), 0, 0)], 1, 64, "bf16", 32),
    ([SeqSpec(2000, ("lognormal", 100, 8, 600), 4, 4)], 8, 128, "bf16", 33),
    ([SeqSpec(513, ("uniform", 16, 64), 2, 1), SeqSpec(127, ("uniform", 16, 64), 2, 0)], 1, 64, "f32", 34),
    ([SeqSpec(900, ("uniform", 32, 256), 4, 2)], 4, 256, "bf16", 35),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("lo,hi,tau", [(1, 1, 0.5), (16, 64, 0.5), (3, 500, 0.3), (64, 512, 0.5), (8, 40, 0.95)])
def test_small_chunking(case, lo, hi, tau):
    seqs, hkv, d, dt, seed = SMALL[case]
    w = W.make_workload(seqs, hkv, hkv, d, dt, seed=seed, name=f"chunk{case}")
    _check(w, lo, hi, tau)


def test_constant_and_zero_rows():
    # equal rows: no cuts, chunks of hi; all-zero rows: similarity 1, no cuts either
    T = 300
    w = W.make_workload([SeqSpec(T, ("fixed", 300), 0, 0)], 1, 1, 64, "bf16", seed=36, name="const")
    row = W.f32_to_bf16_bits(np.linspace(-1, 1, 64, dtype=np.float32).reshape(1, 1, 64))
    w.k = np.repeat(row, T, axis=0)
    cu, _, _ = _check(w, 10, 64, 0.99)
    assert cu.tolist() == list(range(0, T, 64)) + [T]
    w.k = np.zeros_like(w.k)
    cu, _, _ = _check(w, 10, 64, 0.99)
    assert cu.tolist() == list(range(0, T, 64)) + [T]


def test_topic_segments_are_recovered():
    """On the topic-plus-noise generator (adjacent keys of one chunk share a topic, cos ~ 0.84; across a
    chunk boundary the topics are independent, cos ~ 0), tau = 0.5 with limits that bracket the
    generator's lengths recovers its chunk boundaries, except next to planted needles."""
    w = W.make_workload([SeqSpec(20000, ("uniform", 64, 512), 4, 0)], 8, 8, 128, "bf16", seed=37, name="recover")
    cu, _, near = _check(w, 32, 1024, 0.5)
    gen = set(w.cu_chunks.tolist())
    assert near == 0
    assert len(gen & set(cu.tolist())) == len(gen)       # every generator boundary is found (no needles)


@pytest.mark.slow
def test_full_size_chunking_128k():
    w = W.make_config(3)
    cu, scs, _ = _check(w, 32, 1024, 0.5)
    gen = set(w.cu_chunks.tolist())
    assert len(gen & set(cu.tolist())) >= 0.85 * len(gen)   # a needle can hide the boundary after it


@pytest.mark.slow
def test_walk_restages_the_bitmap():
    # 600K tokens: the cut bitmap (9375 words) is longer than one 8192-word LDS segment
    w = W.make_workload([SeqSpec(350000, ("uniform", 32, 400), 0, 0), SeqSpec(250000, ("uniform", 16, 100), 0, 0)],
                        1, 1, 64, "bf16", seed=38, name="long")
    _check(w, 8, 300, 0.5)


def test_walk_segments_that_never_merge_and_dropped_lists():
    """The walk runs its segments speculatively from their first tokens and stitches them; the result
    must be the sequential walk's also where the speculative walks never meet the true chain and where
    a segment holds more cuts than its list keeps."""
    # constant rows: no cut bits, chunks of hi = 100; the 16 segments start at multiples of 320, most of
    # them between two true cuts, and walks from there stay offset (every chunk is hi long)
    T = 5000
    w = W.make_workload([SeqSpec(T, ("fixed", T), 0, 0)], 1, 1, 64, "bf16", seed=41, name="nomerge")
    row = W.f32_to_bf16_bits(np.linspace(-1, 1, 64, dtype=np.float32).reshape(1, 1, 64))
    w.k = np.repeat(row, T, axis=0)
    cu, _, _ = _check(w, 10, 100, 0.99)
    assert cu.tolist() == list(range(0, T, 100)) + [T]
    # one-token chunks over 40000 tokens: 2500 cuts per segment, more than a list keeps
    T = 40000
    w = W.make_workload([SeqSpec(T - 1, ("fixed", 64), 0, 0), SeqSpec(1, ("fixed", 1), 0, 0)], 1, 1, 64, "bf16",
                        seed=42, name="dropped")
    cu, scs, _ = _check(w, 1, 1, 0.5)
    assert cu.tolist() == list(range(T + 1)) and scs.tolist() == [0, T - 1, T]
