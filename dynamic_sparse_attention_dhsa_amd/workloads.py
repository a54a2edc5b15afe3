"""Seeded synthetic inputs for chunk-routed sparse causal prefill.

This module holds random draws and input layout only: chunk boundaries,
Q/K/V tensors, planted needles and per-chunk key-chunk budgets.  It contains
none of the method's arithmetic (no summaries, scores, selection or
attention), so both the HIP path and the CPU oracle can consume what it
produces without sharing any computation.

The workloads stand in for the long-context suites the DHSA pages evaluate on
(Needle-in-a-Haystack, LongBench, RULER; "Long-Context Modeling with Dynamic
Hierarchical Sparse Attention for Memory-Constrained LLM Inference", ICML 2026
spotlight page, Abstract): each chunk draws a topic vector, queries and keys
of a chunk are that topic plus noise, and a few "needle" keys are planted that
align with queries of chunks at least eight chunks later.  No item of any
suite is used or reproduced.

Draw order per workload (numpy PCG64, ``default_rng(seed)``):
  1. chunk lengths, sequence by sequence;
  2. topic vectors ``[C, d]`` (shared by all heads);
  3. Q noise ``[T, Hq, d]``;  4. K noise ``[T, Hkv, d]``;  5. V ``[T, Hkv, d]``;
  6. needles (target chunk, source chunk, token, noise), one after another.

Chunking: lengths are drawn one after another until their sum reaches the
sequence length; the last chunk is cut to fit (it may fall below the
distribution's minimum, which exercises short chunks).  The lognormal
distribution uses sigma = 1 (natural log) and rounds ``median * exp(z)`` to the
nearest integer before clipping.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple, Union

import numpy as np

ChunkDist = Tuple  # ("uniform", lo, hi) | ("lognormal", median, lo, hi) | ("fixed", n) | ("explicit", [n...])
Budget = Union[int, str, Sequence[int]]  # int k for every chunk | "tenth" | explicit per-chunk list


@dataclasses.dataclass
class SeqSpec:
    length: int
    chunks: ChunkDist
    budget: Budget
    needles: int = 0


@dataclasses.dataclass
class Workload:
    """One packed varlen batch in THD layout (tokens, heads, head_dim)."""

    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                      # "f32" or "bf16"
    cu_seqlens: np.ndarray          # int32 [B+1]
    cu_chunks: np.ndarray           # int32 [C+1], global token offsets
    seq_chunk_start: np.ndarray     # int32 [B+1], first chunk id of each sequence
    topk: np.ndarray                # int32 [C], off-diagonal key-chunk budget per query chunk
    q: np.ndarray                   # f32 [T,Hq,d]  or  uint16 bf16 bits
    k: np.ndarray                   # f32 [T,Hkv,d] or  uint16 bf16 bits
    v: np.ndarray                   # f32 [T,Hkv,d] or  uint16 bf16 bits
    softmax_scale: float
    seed: int
    needles: List[Tuple[int, int, int]] = dataclasses.field(default_factory=list)  # (target chunk, source chunk, token)

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def total_chunks(self) -> int:
        return int(self.cu_chunks.shape[0] - 1)

    @property
    def num_seqs(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    def q_f32(self) -> np.ndarray:
        return self.q if self.dtype == "f32" else bf16_bits_to_f32(self.q)

    def k_f32(self) -> np.ndarray:
        return self.k if self.dtype == "f32" else bf16_bits_to_f32(self.k)

    def v_f32(self) -> np.ndarray:
        return self.v if self.dtype == "f32" else bf16_bits_to_f32(self.v)

    def chunk_lengths(self) -> np.ndarray:
        return np.diff(self.cu_chunks)

    def max_chunks_per_seq(self) -> int:
        return int(np.diff(self.seq_chunk_start).max()) if self.num_seqs else 0


# ----------------------------------------------------------------------------- bf16 bits

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    flat_in = x.reshape(-1).view(np.uint32)
    flat_out = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_in.size, step):
        u = flat_in[s:s + step]
        bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
        flat_out[s:s + step] = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------- chunking

def _draw_length(rng: np.random.Generator, dist: ChunkDist) -> int:
    kind = dist[0]
    if kind == "uniform":
        return int(rng.integers(dist[1], dist[2] + 1))
    if kind == "lognormal":
        median, lo, hi = dist[1], dist[2], dist[3]
        z = rng.standard_normal()
        return int(min(max(math.floor(median * math.exp(z) + 0.5), lo), hi))
    if kind == "fixed":
        return int(dist[1])
    raise ValueError(f"unknown chunk distribution {dist!r}")


def draw_chunk_lengths(rng: np.random.Generator, length: int, dist: ChunkDist) -> List[int]:
    if dist[0] == "explicit":
        lens = [int(n) for n in dist[1]]
        if sum(lens) != length or any(n < 1 for n in lens):
            raise ValueError("explicit chunk lengths must be >= 1 and sum to the sequence length")
        return lens
    lens: List[int] = []
    total = 0
    while total < length:
        n = _draw_length(rng, dist)
        n = min(n, length - total)
        lens.append(n)
        total += n
    return lens


def chunk_budget(budget: Budget, num_chunks: int) -> List[int]:
    """Off-diagonal key-chunk budget for each query chunk of one sequence.

    ``"tenth"``: the row keeps 10% of its causal chunk pairs (i_loc + 1 of
    them, diagonal included), rounded half up, at least one (the diagonal);
    the off-diagonal budget is that count minus one.
    """
    if isinstance(budget, str):
        if budget != "tenth":
            raise ValueError(f"unknown budget rule {budget!r}")
        return [max(1, (i + 1 + 5) // 10) - 1 for i in range(num_chunks)]
    if isinstance(budget, (int, np.integer)):
        return [int(budget)] * num_chunks
    lst = [int(x) for x in budget]
    if len(lst) != num_chunks:
        raise ValueError("explicit budget needs one entry per chunk")
    return lst


# ----------------------------------------------------------------------------- generator

def make_workload(seqs: Sequence[SeqSpec], num_q_heads: int, num_kv_heads: int, head_dim: int,
                  dtype: str, seed: int, name: str = "custom",
                  topic_weight: float = 0.7, noise_weight: float = 0.3,
                  needle_snr: float = 3.0, topics_per_head: bool = False,
                  layout_only: bool = False) -> Workload:
    """Topic-plus-noise Q/K with planted needles; V ~ N(0, 1).

    ``Q[t, h] = 0.7 * topic[chunk(t)] + 0.3 * N(0, I)``, K the same per KV
    head.  A needle picks a target query chunk i (local index >= 8), a source
    key chunk j (local index <= i - 8) and a token u in j, and overwrites
    ``K[u, every KV head] = 0.7 * g_j * topic[i] + 0.3 * N(0, I)`` with
    ``g_j = needle_snr * n_j / sqrt(d)``, which lifts chunk j's summary score
    against chunk i by about ``needle_snr`` standard deviations of the
    off-topic scores.  Sequences with fewer than nine chunks get no needles.
    With ``topics_per_head`` every Q head and KV head draws its own topics,
    which makes the key-chunk lists of a GQA group diverge.  With
    ``layout_only`` only draw 1 happens (the layout is identical to the full
    workload's) and q, k, v are None.
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError("dtype must be 'f32' or 'bf16'")
    rng = np.random.default_rng(seed)
    d = head_dim
    cu_seqlens = [0]
    cu_chunks = [0]
    seq_chunk_start = [0]
    topk: List[int] = []
    for spec in seqs:                                  # draw 1: chunk lengths
        lens = draw_chunk_lengths(rng, spec.length, spec.chunks) if spec.length > 0 else []
        for n in lens:
            cu_chunks.append(cu_chunks[-1] + n)
        cu_seqlens.append(cu_seqlens[-1] + spec.length)
        seq_chunk_start.append(seq_chunk_start[-1] + len(lens))
        topk.extend(chunk_budget(spec.budget, len(lens)))
    T = cu_seqlens[-1]
    C = len(cu_chunks) - 1
    cu_chunks_a = np.asarray(cu_chunks, np.int32)
    if layout_only:
        return Workload(name=name, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=d,
                        dtype=dtype, cu_seqlens=np.asarray(cu_seqlens, np.int32), cu_chunks=cu_chunks_a,
                        seq_chunk_start=np.asarray(seq_chunk_start, np.int32),
                        topk=np.asarray(topk, np.int32), q=None, k=None, v=None,
                        softmax_scale=1.0 / math.sqrt(d), seed=seed)
    tok_chunk = np.repeat(np.arange(C), np.diff(cu_chunks_a)) if C else np.zeros(0, np.int64)

    n_topic_sets = max(num_q_heads, num_kv_heads) if topics_per_head else 1
    topics = rng.standard_normal((n_topic_sets, C, d), dtype=np.float32)   # draw 2

    def _mix(noise: np.ndarray, heads: int) -> np.ndarray:
        noise *= np.float32(noise_weight)
        for h in range(heads):
            tp = topics[h % n_topic_sets] if topics_per_head else topics[0]
            noise[:, h, :] += np.float32(topic_weight) * tp[tok_chunk]
        return noise

    q = _mix(rng.standard_normal((T, num_q_heads, d), dtype=np.float32), num_q_heads)    # draw 3
    k = _mix(rng.standard_normal((T, num_kv_heads, d), dtype=np.float32), num_kv_heads)  # draw 4
    v = rng.standard_normal((T, num_kv_heads, d), dtype=np.float32)                        # draw 5

    needles = []
    for b, spec in enumerate(seqs):                    # draw 6: needles
        c0, c1 = seq_chunk_start[b], seq_chunk_start[b + 1]
        nc = c1 - c0
        if nc < 9:
            continue
        for _ in range(spec.needles):
            i_loc = int(rng.integers(8, nc))
            j_loc = int(rng.integers(0, i_loc - 7))
            i, j = c0 + i_loc, c0 + j_loc
            u = int(rng.integers(cu_chunks[j], cu_chunks[j + 1]))
            noise = rng.standard_normal((num_kv_heads, d), dtype=np.float32)
            gamma = needle_snr * (cu_chunks[j + 1] - cu_chunks[j]) / math.sqrt(d)
            for g in range(num_kv_heads):
                tp = topics[g % n_topic_sets] if topics_per_head else topics[0]
                k[u, g, :] = np.float32(topic_weight * gamma) * tp[i] + np.float32(noise_weight) * noise[g]
            needles.append((i, j, u))

    if dtype == "bf16":
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    return Workload(name=name, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=d,
                    dtype=dtype, cu_seqlens=np.asarray(cu_seqlens, np.int32), cu_chunks=cu_chunks_a,
                    seq_chunk_start=np.asarray(seq_chunk_start, np.int32),
                    topk=np.asarray(topk, np.int32), q=q, k=k, v=v,
                    softmax_scale=1.0 / math.sqrt(d), seed=seed, needles=needles)


# ----------------------------------------------------------------------------- named workloads

def _cfg(i: int):
    if i == 0:   # 1 head, d=64, fp32, L=1024, U[16,64], top-4 + diagonal, 3 needles
        return dict(name="L1K-h1-d64-f32", Hq=1, Hkv=1, d=64, dtype="f32",
                    seqs=[SeqSpec(1024, ("uniform", 16, 64), 4, 3)])
    if i == 1:   # LLaMA-3.1-8B attention shape at L=8192
        return dict(name="llama3-8b-attn-L8K", Hq=32, Hkv=8, d=128, dtype="bf16",
                    seqs=[SeqSpec(8192, ("uniform", 32, 256), 16, 16)])
    if i == 2:   # Gemma2-2B-like, d=256, lognormal chunks, 10% of causal chunk pairs
        return dict(name="gemma2-2b-attn-L32K", Hq=8, Hkv=4, d=256, dtype="bf16",
                    seqs=[SeqSpec(32768, ("lognormal", 128, 16, 1024), "tenth", 64)])
    if i == 3:   # LLaMA-3.1-8B attention shape at L=131072 (the headline shape)
        return dict(name="llama3-8b-attn-L128K", Hq=32, Hkv=8, d=128, dtype="bf16",
                    seqs=[SeqSpec(131072, ("uniform", 64, 512), 32, 256)])
    if i == 4:   # ragged batch of four sequences, one needle per 512 tokens
        return dict(name="ragged4-llama3-8b-attn", Hq=32, Hkv=8, d=128, dtype="bf16",
                    seqs=[SeqSpec(16384, ("uniform", 16, 128), 8, 32),
                          SeqSpec(32768, ("uniform", 64, 512), 16, 64),
                          SeqSpec(49152, ("lognormal", 256, 16, 1024), 24, 96),
                          SeqSpec(65536, ("fixed", 128), 32, 128)])
    raise ValueError(f"no workload {i}")


NUM_CONFIGS = 5


def config_name(i: int) -> str:
    return _cfg(i)["name"]


def make_config(i: int, seed: Optional[int] = None, layout_only: bool = False) -> Workload:
    """Named workload ``i`` (0..4); the default seed is ``1000 + i``."""
    c = _cfg(i)
    return make_workload(c["seqs"], c["Hq"], c["Hkv"], c["d"], c["dtype"],
                         seed=1000 + i if seed is None else seed, name=c["name"],
                         layout_only=layout_only)
