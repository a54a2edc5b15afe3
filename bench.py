#!/usr/bin/env python3
"""Throughput of the DHSA chunk-routed sparse prefill on one MI355X.

One step = the whole hot path on one batch: chunk summaries (stage 1), causal
chunk routing (stage 2) and block-sparse causal prefill (stage 3), each a
gfx950 kernel launched through the C ABI on torch's current stream.  Inputs
are resident in HBM before the timed region starts; the routing plan (CSR
row pointers, a pure function of the chunk layout and the budget) is built
on the host once, with the inputs.

Default workload: the LLaMA-3.1-8B attention-layer shape at L = 131072
(32 query heads, 8 KV heads, head_dim 128, bf16), chunk lengths uniform in
[64, 512], top-32 earlier chunks plus the diagonal, 256 planted needles.

Prints one JSON line with the throughput, a roofline object for the
dominant kernel (stage 3, MFMA bf16 against the kept FLOPs), per-stage
figures, and the CPU oracle timed on a bounded sample on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-prefill tokens/s per attn layer at 128K (8B shape); % MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 vector ALU: 256 CUs x 4 SIMDs x 16 lanes x 2 (packed) x 2 FLOP x 2.4 GHz
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PREFILL_SRC = os.path.join(ROOT, "dynamic_sparse_attention_dhsa_amd", "csrc", "prefill_bf16.hip")


def kept_flops(block_idx: np.ndarray, row_ptr: np.ndarray, cu_chunks: np.ndarray, d: int) -> float:
    """Algorithmic FLOPs of stage 3: 4*d per kept (query, key) pair (QK^T and PV, 2 FLOPs per MAC).
    Entries of -1 (the padding of token-budget rows) keep nothing."""
    lens = np.diff(cu_chunks).astype(np.int64)
    C = lens.size
    total = 0
    row_of = np.repeat(np.arange(C), np.diff(row_ptr))
    for h in range(block_idx.shape[0]):
        kept = block_idx[h].astype(np.int64)
        diag = kept == row_of
        offd = ~diag & (kept >= 0)
        off = np.bincount(row_of[offd], weights=lens[kept[offd]], minlength=C)
        total += float((lens * off).sum() + (lens * (lens + 1) // 2).sum())
    return 4.0 * d * total


def stage_bytes(T, C, Hq, Hkv, d, s, nnz):
    """Algorithmic bytes of stage 1 (Q, K read once, summaries written) and stage 2 (summaries read,
    row pointers and per-chunk sequence starts read, block list written)."""
    b1 = T * (Hq + Hkv) * d * s + C * (Hq + Hkv) * d * 4
    b2 = C * (Hq + Hkv) * d * 4 + (C + 1) * 4 + C * 4 + Hq * nnz * 4
    return b1, b2


def memory_report(torch, D, w, q, k, v, grouped: bool, token_budget=None):
    """Device memory of one whole-path call (dhsa.prefill: plan upload, summaries, block list, output)
    measured with torch's allocator statistics (the library allocates nothing itself), beside the
    inputs and what dense attention over the same causal pairs would hold."""
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    if token_budget is None:
        r = D.prefill(q, k, v, w.cu_seqlens, w.cu_chunks, w.seq_chunk_start, w.topk, w.softmax_scale,
                      grouped=grouped)
    else:
        r = D.prefill(q, k, v, w.cu_seqlens, w.cu_chunks, w.seq_chunk_start, token_budget=token_budget,
                      softmax_scale=w.softmax_scale, grouped=grouped)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    out_b = r["out"].numel() * r["out"].element_size()
    parts = {"q_sum_k_sum": (r["q_sum"].numel() + r["k_sum"].numel()) * 4,
             "block_idx": r["block_idx"].numel() * 4}
    T, Hq = w.total_tokens, w.num_q_heads
    s = q.element_size()
    pairs = sum(int(n) * int(n) for n in np.diff(w.cu_seqlens))
    del r
    return {"peak_bytes_above_inputs_measured": int(peak), "output_bytes": int(out_b),
            "path_extra_bytes_measured": int(peak - out_b), "path_extra_parts": parts,
            "inputs_qkv_bytes": int(q.numel() * s + k.numel() * s + v.numel() * s),
            "dense_eager_score_bytes": int(Hq * pairs * s),
            "dense_fused_extra_bytes": int(Hq * T * 4),
            "note": "dense_eager = the [Hq, L, L] score matrix of unfused attention in the input dtype "
                    "(computed, not allocated); dense_fused = a fused kernel's fp32 row statistics"}


def achievable_peaks(torch):
    """Measured ceilings on this device, beside the published peaks the roofline fractions use:
    the hand-written dense bf16 MFMA loop and the streaming-read kernel of libdhsa_calib.so, plus a
    1 GiB device-to-device copy and a large bf16 GEMM (hipBLASLt through torch) for context."""
    import ctypes
    from dynamic_sparse_attention_dhsa_amd.build import CALIB_LIB
    if not os.path.exists(CALIB_LIB):
        raise RuntimeError(f"{CALIB_LIB} is missing: build it with dynamic_sparse_attention_dhsa_amd.build.build()")
    cal = ctypes.CDLL(CALIB_LIB)
    cal.dhsa_calib_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    cal.dhsa_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    mm_blocks, mm_iters = 2 * n_cu, 20000
    sink = torch.empty(max(mm_blocks, 8 * n_cu) * 256, device="cuda", dtype=torch.float32)
    x = torch.empty(512 * 1024 * 1024, device="cuda", dtype=torch.bfloat16)   # 1 GiB
    x.fill_(1.0)
    y = torch.empty_like(x)
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    def mfma():
        if cal.dhsa_calib_mfma_bf16(mm_blocks, mm_iters, ctypes.c_void_p(sink.data_ptr()), stream) != 0:
            raise RuntimeError("dhsa_calib_mfma_bf16 failed to launch")

    def read():
        if cal.dhsa_calib_read(ctypes.c_void_p(x.data_ptr()), x.numel() * 2, 8 * n_cu,
                               ctypes.c_void_p(sink.data_ptr()), stream) != 0:
            raise RuntimeError("dhsa_calib_read failed to launch")

    t_loop = timed(mfma, 3)
    t_read = timed(read, 10)
    t_copy = timed(lambda: y.copy_(x), 10)
    t_mm = timed(lambda: torch.matmul(a, b), 10)
    del a, b, x, y, sink
    return {"mfma_loop_TFLOPs": mm_blocks * 16.0 * mm_iters * 32768 / t_loop / 1e12,
            "read_1GiB_GBps": 1024 ** 3 / t_read / 1e9,
            "copy_1GiB_GBps": 2 * 1024 ** 3 / t_copy / 1e9,
            "bf16_gemm_8192_TFLOPs": 2 * 8192 ** 3 / t_mm / 1e12}


def stage_protocol(torch, stages, reps: int = 20):
    """Per-stage HIP-event times over `reps` repetitions, each after an untimed read of a 1 GiB buffer
    that evicts L2 and the 256 MB last-level cache with clean lines (a write would leave dirty lines
    whose write-back the next timed kernel would pay for), so every stage starts from HBM:
    (median, min) in s."""
    scratch = torch.ones(256 * 1024 * 1024, device="cuda", dtype=torch.float32)
    sink = scratch.sum()                          # the buffer's lines are clean from here on
    times = [[] for _ in stages]
    for _ in range(reps):
        sink = scratch.sum()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
        ev[0].record()
        for k, fn in enumerate(stages):
            fn()
            ev[k + 1].record()
        torch.cuda.synchronize()
        for k in range(len(stages)):
            times[k].append(ev[k].elapsed_time(ev[k + 1]) * 1e-3)
    del scratch, sink
    return [(float(np.median(t)), float(np.min(t))) for t in times]


def decode_measure(torch, D, w, q, k, v, batch: int, steps: int = 30, warmup: int = 5):
    """Decode against the kept structure (an extension, not part of the step): ``batch`` copies of the
    workload's first sequence as the context, chunked by this library's rule, loaded into a decode
    state; then one-token steps (routing once per KV head, top-k of the workload).  Algorithmic bytes per
    step: the kept K and V rows of every (sequence, KV head) plus the closed chunks' key summaries."""
    T = int(w.cu_seqlens[1])
    Hq, Hkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
    topk = int(w.topk.max())
    lo, hi, tau = 32, 1024, 0.5
    cc, scs = D.online_chunks(k[:T], w.cu_seqlens[:2], lo, hi, tau)
    C = len(cc) - 1
    cu_b = np.arange(batch + 1, dtype=np.int32) * T
    cc_b = np.concatenate([[0]] + [cc[1:] + b * T for b in range(batch)]).astype(np.int32)
    scs_b = np.arange(batch + 1, dtype=np.int32) * C
    lay = D.Layout(cu_b, cc_b, scs_b, Hq, Hkv, d, q.dtype)
    st = D.DecodeState(batch, Hq, Hkv, d, q.dtype, T + warmup + steps + 1, 1024)
    st.load_prefix(lay, q[:T].repeat(batch, 1, 1), k[:T].repeat(batch, 1, 1), v[:T].repeat(batch, 1, 1))
    # new tokens: rows of the sequence's last chunk, so the open chunk keeps growing with its topic;
    # every step's inputs are built (resident in HBM) before anything is timed
    src = torch.arange(T - 64, T, device=q.device)
    kept = torch.empty((batch, Hq, topk), dtype=torch.int32, device=q.device)
    out = torch.empty((batch, Hq, d), dtype=q.dtype, device=q.device)
    idx = src[torch.arange(warmup + steps, device=q.device) % 64]
    q_in = q[idx].unsqueeze(1).expand(-1, batch, -1, -1).contiguous()     # [steps, batch, Hq, d]
    k_in = k[idx].unsqueeze(1).expand(-1, batch, -1, -1).contiguous()
    v_in = v[idx].unsqueeze(1).expand(-1, batch, -1, -1).contiguous()

    def step(i):
        st.step(q_in[i], k_in[i], v_in[i], lo, hi, tau, topk, True, w.softmax_scale, out=out, kept=kept)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(warmup + i)
    e1.record()
    torch.cuda.synchronize()
    t_eager = e0.elapsed_time(e1) / steps * 1e-3
    # The same steps on a second state, captured in one HIP graph through the entry point that allocates
    # nothing (its scratch is the library's static device array), then replayed once: the launch cost
    # of the Python loop above is gone, so this is the step's device time.
    st2 = D.DecodeState(batch, Hq, Hkv, d, q.dtype, T + warmup + steps + 1, 1024)
    st2.load_prefix(lay, q[:T].repeat(batch, 1, 1), k[:T].repeat(batch, 1, 1), v[:T].repeat(batch, 1, 1))
    out2 = torch.empty_like(out)
    kept2 = torch.empty_like(kept)

    def step2(i):
        st2.step_noalloc(q_in[i], k_in[i], v_in[i], lo, hi, tau, topk, True, w.softmax_scale, out=out2, kept=kept2)

    for i in range(warmup):
        step2(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    capture = torch.cuda.Stream()
    capture.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=capture):
        for i in range(steps):
            step2(warmup + i)
    torch.cuda.synchronize()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    t_step = e0.elapsed_time(e1) / steps * 1e-3
    same = bool(torch.equal(out, out2) and torch.equal(kept, kept2))
    del graph, st2
    # bytes of the last step: kept closed chunks (per KV head: the same list for its query heads)
    starts = st.chunk_start.cpu().numpy()
    ncl = st.num_closed.cpu().numpy()
    seql = st.seq_len.cpu().numpy()
    kp = kept.cpu().numpy()
    G = Hq // Hkv
    kept_tok = 0
    for b in range(batch):
        lens = np.diff(starts[b, :ncl[b] + 1])
        open_len = int(seql[b] - starts[b, ncl[b]])
        for g in range(Hkv):
            ids = kp[b, g * G][kp[b, g * G] >= 0]
            kept_tok += int(lens[ids].sum()) + open_len
    b_step = kept_tok * d * 2 * 2 + int(ncl.sum()) * Hkv * d * 4 + batch * (Hq + 2 * Hkv) * d * 2 * 2
    return {"context_tokens": T, "batch": batch, "routing": "per_kv_head", "topk": topk,
            "chunk_rule": f"cosine < {tau}, lengths [{lo}, {hi}]", "closed_chunks": int(ncl[0]),
            "ms_per_step": t_step * 1e3, "timing": "one HIP graph of the steps (no-alloc entry point), replayed",
            "ms_per_step_eager_python": t_eager * 1e3, "graph_equals_eager": same,
            "tokens_per_s": batch / t_step,
            "kept_tokens_per_kv_head": kept_tok / (batch * Hkv), "bytes_per_step": b_step,
            "hbm_GBps": b_step / t_step / 1e9, "hbm_frac": b_step / t_step / 1e9 / PEAK_HBM_GBS}


def traffic_record(workload: str):
    """HBM traffic of stage 3 from committed rocprofv3 counter runs, if they match the kernel source."""
    path = os.path.join(ROOT, "profiles", f"prefill_bf16_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src_hash = hashlib.sha256(open(PREFILL_SRC, "rb").read()).hexdigest()[:16]
    if rec.get("kernel_source_sha256_16") != src_hash:
        return None
    return rec.get("bytes_per_launch")


_CPU = {}                          # the oracle's inputs, shared with forked workers (copy on write)


def _attend_rows(rows):
    """Oracle attention on (head, chunk) rows in a worker process, BLAS on one thread."""
    import oracle
    from threadpoolctl import threadpool_limits
    c = _CPU
    t0 = time.perf_counter()
    with threadpool_limits(1):
        for h, i in rows:
            oracle.attend(c["q"], c["k"], c["v"], c["cu_chunks"], c["row_ptr"], c["block_idx"], c["scale"],
                          heads=[h], chunks=[i])
    return time.perf_counter() - t0


def cpu_baseline(w, topk, fraction: float = 0.05, grouped: bool = False, workers: int = 16):
    """The CPU oracle (as it stands) on a bounded sample of the same workload: summaries and routing of
    the whole workload on one thread, then oracle attention on random (head, chunk) rows holding at
    least `fraction` of the kept (query, key) pairs, spread over `workers` processes with one BLAS
    thread each; the attention time is extrapolated by kept pairs."""
    import multiprocessing as mp

    import oracle
    from threadpoolctl import threadpool_limits
    workers = max(1, min(workers, len(os.sched_getaffinity(0))))
    qf, kf, vf = w.q_f32(), w.k_f32(), w.v_f32()
    with threadpool_limits(1):
        t0 = time.perf_counter()
        qs = oracle.chunk_summaries(qf, w.cu_chunks)
        ks = oracle.chunk_summaries(kf, w.cu_chunks)
        t_sum = time.perf_counter() - t0
        t0 = time.perf_counter()
        rp, bi, _ = (oracle.route_grouped if grouped else oracle.route)(qs, ks, w.seq_chunk_start, topk)
        t_route = time.perf_counter() - t0
    lens = np.diff(w.cu_chunks).astype(np.int64)
    C, Hq = w.total_chunks, w.num_q_heads
    # kept (query, key) pairs of each row: the causal half of the diagonal plus whole earlier chunks
    pairs = np.zeros((Hq, C))
    for h in range(Hq):
        for i in range(C):
            kept = bi[h, rp[i]:rp[i + 1]]
            kept = kept[(kept >= 0) & (kept != i)]
            pairs[h, i] = lens[i] * lens[kept].sum() + lens[i] * (lens[i] + 1) / 2
    total = pairs.sum()
    rng = np.random.default_rng(0)
    order = rng.permutation(Hq * C)
    take = np.searchsorted(np.cumsum(pairs.reshape(-1)[order]), fraction * total) + 1
    rows = [(int(x // C), int(x % C)) for x in order[:take]]
    sample_pairs = float(sum(pairs[h, i] for h, i in rows))
    # deal the rows to the workers longest first, so they finish together
    rows.sort(key=lambda r: -pairs[r])
    shards = [[] for _ in range(workers)]
    load = np.zeros(workers)
    for r in rows:
        j = int(np.argmin(load))
        shards[j].append(r)
        load[j] += pairs[r]
    _CPU.update(q=qf, k=kf, v=vf, cu_chunks=w.cu_chunks, row_ptr=rp, block_idx=bi, scale=w.softmax_scale)
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        busy = pool.map(_attend_rows, shards)
    t_att = time.perf_counter() - t0
    _CPU.clear()
    t_att_full = t_att * total / sample_pairs
    t_full = t_sum + t_route + t_att_full
    return {"value": w.total_tokens / t_full, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": (f"oracle summaries + routing of the whole workload on one thread ({t_sum + t_route:.1f} s); "
                       f"oracle attention on {len(rows)} random (head, chunk) rows holding "
                       f"{100 * sample_pairs / total:.1f}% of the kept (query, key) pairs, over {workers} worker "
                       f"processes with one BLAS thread each ({t_att:.1f} s wall), extrapolated by kept pairs; "
                       f"fp64 numpy"),
            "seconds_est_full_step": t_full, "cpu_model": _cpu_model(),
            "stage_seconds": {"summaries": t_sum, "routing": t_route, "attention_sample_wall": t_att,
                              "attention_sample_worker_busy": float(sum(busy))}}


def _cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo; empty where that is not readable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, help="named workload 0..4 (3 = 128K headline)")
    ap.add_argument("--routing", choices=("head", "kv-group"), default="head",
                    help="route per query head (default) or once per KV head")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-batch", type=int, default=8,
                    help="sequences in the decode measurement at the workload's context (0: skip it)")
    ap.add_argument("--cpu-fraction", type=float, default=0.05,
                    help="share of the kept (query, key) pairs the oracle baseline computes")
    ap.add_argument("--cpu-workers", type=int, default=16, help="worker processes of the oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for {args.gpus} GPUs).",
              file=sys.stderr)
        return 2

    import torch

    import dynamic_sparse_attention_dhsa_amd as D
    from dynamic_sparse_attention_dhsa_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    print(f"[bench] generating workload {args.config}", file=sys.stderr, flush=True)
    w = W.make_config(args.config)
    grouped = args.routing == "kv-group"
    bf16 = w.dtype == "bf16"
    tdt = torch.bfloat16 if bf16 else torch.float32

    def dev(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16) if bf16 else torch.from_numpy(a).cuda()

    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    T, C, Hq, Hkv, d = w.total_tokens, w.total_chunks, w.num_q_heads, w.num_kv_heads, w.head_dim
    layout = D.Layout(w.cu_seqlens, w.cu_chunks, w.seq_chunk_start, Hq, Hkv, d, tdt)
    plan = D.RoutePlan(layout, w.topk)
    q_sum = torch.empty((C, Hq, d), dtype=torch.float32, device="cuda")
    k_sum = torch.empty((C, Hkv, d), dtype=torch.float32, device="cuda")
    block_idx = torch.empty((Hq, plan.nnz), dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        D.chunk_summarize(layout, q, k, q_sum, k_sum)
        if ev is not None:
            ev[1].record(stream)
        D.route(layout, plan, q_sum, k_sum, block_idx, grouped=grouped)
        if ev is not None:
            ev[2].record(stream)
        D.sparse_prefill(layout, plan, q, k, v, block_idx, w.softmax_scale, out=out)
        if ev is not None:
            ev[3].record(stream)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    print(f"[bench] timed {args.steps} steps in {elapsed:.3f} s", file=sys.stderr, flush=True)

    t1 = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e-3
    t2 = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) * 1e-3
    t3 = float(np.mean([e[2].elapsed_time(e[3]) for e in evs])) * 1e-3

    bidx = block_idx.cpu().numpy()
    F3 = kept_flops(bidx, plan.h_row_ptr, w.cu_chunks, d)
    b1, b2 = stage_bytes(T, C, Hq, Hkv, d, 2 if bf16 else 4, plan.nnz)
    causal_pairs = float(sum(((n := int(w.cu_seqlens[b + 1] - w.cu_seqlens[b])) * (n + 1)) // 2
                             for b in range(w.num_seqs))) * Hq
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    achieved = F3 / t3 / 1e12
    ms_per_step = elapsed / args.steps * 1e3
    result = {
        "metric": METRIC,
        "value": T * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": T, "num_seqs": w.num_seqs, "num_q_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": d, "chunks": C,
                   "topk": int(w.topk.max()) if C else 0, "routing": "per_kv_head" if grouped else "per_q_head",
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma" if bf16 else "alu", "kernel": "prefill_bf16_kernel" if bf16 else "prefill_f32_kernel",
                     "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                     # the committed counter record is of the per-q-head lists (bench_traffic.py)
                     "traffic": traffic_record(w.name) if bf16 and not grouped else None,
                     # compulsory bytes: Q, K and V read once, the output written once
                     "compulsory_bytes": float(2 * q.numel() * q.element_size() + 2 * k.numel() * k.element_size()),
                     "algorithmic_flops_per_launch": F3},
        "stages": {
            "t_summarize_ms": t1 * 1e3, "t_route_ms": t2 * 1e3, "t_prefill_ms": t3 * 1e3,
            "summarize_GBps": b1 / t1 / 1e9, "route_GBps": b2 / t2 / 1e9,
            "stages12_hbm_frac": (b1 + b2) / (t1 + t2) / 1e9 / PEAK_HBM_GBS,
            "bytes_stage1": b1, "bytes_stage2": b2,
            "kept_density_vs_causal": F3 / (4.0 * d * causal_pairs),
        },
    }
    print("[bench] stage protocol (20 reps from a cold cache) and device ceilings", file=sys.stderr, flush=True)
    (p1, m1), (p2, m2), (p3, m3) = stage_protocol(torch, [
        lambda: D.chunk_summarize(layout, q, k, q_sum, k_sum),
        lambda: D.route(layout, plan, q_sum, k_sum, block_idx, grouped=grouped),
        lambda: D.sparse_prefill(layout, plan, q, k, v, block_idx, w.softmax_scale, out=out)])
    # online chunking (this library's own boundary rule; not part of the step, which takes the
    # workload's chunks): adjacent key similarity (HBM-bound) and the greedy cut walk
    tau, lo_c, hi_c = 0.5, 32, 1024
    seqs = D.SeqLayout(w.cu_seqlens)
    sim_t = torch.empty(T, dtype=torch.float32, device="cuda")
    bits_t = torch.empty((T + 63) // 64, dtype=torch.int64, device="cuda")
    cut_out = (torch.empty(T + 1, dtype=torch.int32, device="cuda"),
               torch.empty(w.num_seqs + 1, dtype=torch.int32, device="cuda"),
               torch.empty(1, dtype=torch.int32, device="cuda"))
    (p_s, m_s), (p_w, m_w) = stage_protocol(torch, [
        lambda: D.adjacent_similarity(k, seqs, tau, sim_t, bits_t),
        lambda: D.chunk_boundaries(bits_t, seqs, lo_c, hi_c, cut_out)])
    b_sim = T * Hkv * d * (2 if bf16 else 4) + T * 4 + ((T + 63) // 64) * 8
    result["stages"]["online_chunking"] = {
        "rule": f"cut where adjacent key cosine < {tau}, chunk length in [{lo_c}, {hi_c}]",
        "similarity_median_min_ms": [p_s * 1e3, m_s * 1e3], "walk_median_min_ms": [p_w * 1e3, m_w * 1e3],
        "similarity_bytes": b_sim, "similarity_GBps": b_sim / p_s / 1e9,
        "similarity_hbm_frac": b_sim / p_s / 1e9 / PEAK_HBM_GBS}
    # routing under a token budget: every row gets the mean kept tokens of the chunk budget
    # (top-k x mean chunk length), then the prefill on its padded lists
    tok = int(round(float(w.topk.mean()) * T / max(C, 1)))
    tplan = D.TokenPlan(layout, np.full(C, tok, np.int32))
    tb_idx = torch.empty((Hq, tplan.nnz), dtype=torch.int32, device="cuda")
    print("[bench] token-budget routing", file=sys.stderr, flush=True)
    (p_t, m_t), (p_tp, m_tp) = stage_protocol(torch, [
        lambda: D.route_tokens(layout, tplan, q_sum, k_sum, tb_idx, grouped=grouped),
        lambda: D.sparse_prefill(layout, tplan, q, k, v, tb_idx, w.softmax_scale, out=out)])
    F3t = kept_flops(tb_idx.cpu().numpy(), tplan.h_row_ptr, w.cu_chunks, d)
    result["stages"]["token_budget"] = {
        "tokens_per_row": tok, "row_capacity_entries": tplan.nnz, "route_median_min_ms": [p_t * 1e3, m_t * 1e3],
        "prefill_median_min_ms": [p_tp * 1e3, m_tp * 1e3], "prefill_TFLOPs": F3t / p_tp / 1e12,
        "kept_density_vs_causal": F3t / (4.0 * d * causal_pairs)}
    print("[bench] memory report", file=sys.stderr, flush=True)
    result["memory"] = memory_report(torch, D, w, q, k, v, grouped)
    result["stages"]["cold_cache_median_min_ms"] = {
        "summarize": [p1 * 1e3, m1 * 1e3], "route": [p2 * 1e3, m2 * 1e3], "prefill": [p3 * 1e3, m3 * 1e3],
        "stages12_hbm_frac_median": (b1 + b2) / (p1 + p2) / 1e9 / PEAK_HBM_GBS,
        "prefill_frac_median": F3 / p3 / 1e12 / peak,
        "protocol": "20 reps, each after an untimed 1 GiB read evicting L2 and the last-level cache with clean lines"}
    if bf16 and args.decode_batch > 0:
        print("[bench] decode at the workload's context", file=sys.stderr, flush=True)
        result["decode"] = decode_measure(torch, D, w, q, k, v, args.decode_batch)
    if bf16:
        peaks = achievable_peaks(torch)
        result["roofline"]["achievable_peak_measured"] = peaks["mfma_loop_TFLOPs"]
        result["roofline"]["achievable_peak_source"] = "hand-written dense bf16 MFMA loop (libdhsa_calib)"
        result["roofline"]["frac_of_achievable"] = achieved / peaks["mfma_loop_TFLOPs"]
        result["roofline"]["bf16_gemm_8192_TFLOPs"] = peaks["bf16_gemm_8192_TFLOPs"]
        result["stages"]["read_GBps_measured"] = peaks["read_1GiB_GBps"]
        result["stages"]["copy_GBps_measured"] = peaks["copy_1GiB_GBps"]
        result["stages"]["stages12_frac_of_read"] = (b1 + b2) / (t1 + t2) / 1e9 / peaks["read_1GiB_GBps"]
    if result["roofline"]["traffic"]:
        result["roofline"]["traffic_over_compulsory"] = result["roofline"]["traffic"] / result["roofline"]["compulsory_bytes"]
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, w.topk, args.cpu_fraction, grouped, args.cpu_workers)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
