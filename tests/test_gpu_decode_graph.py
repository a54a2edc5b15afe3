"""The decode step that allocates nothing (dhsa_decode_step_noalloc) captured in a HIP graph.

Two decode states are loaded with the same chunked prefix.  One is stepped eagerly through
dhsa_decode_step; the other by replaying a graph that holds one captured no-alloc step reading its
token from static input buffers.  Before each replay the next token is copied into those buffers
(eager work between replays), and after it the replay's output, kept list and the whole state must
equal the eager step's bit for bit.
"""
import numpy as np
import pytest
import torch

import dynamic_sparse_attention_dhsa_amd as D
from dynamic_sparse_attention_dhsa_amd import workloads as W
from dynamic_sparse_attention_dhsa_amd.workloads import SeqSpec

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


@pytest.mark.parametrize("grouped", [False, True])
def test_graph_replays_of_the_noalloc_step_equal_eager_steps(grouped):
    B, Hq, Hkv, d, P, steps = 2, 8, 2, 128, 900, 10
    lo, hi, tau, topk = 16, 128, 0.5, 5
    print(f"[decode graph] B={B} Hq={Hq} Hkv={Hkv} d={d} prefix={P} grouped={grouped}", flush=True)
    w = W.make_workload([SeqSpec(P + steps, ("uniform", 24, 100), 0, 0)] * B, Hq, Hkv, d, "bf16", seed=77,
                        name="decode_graph")
    cs = w.cu_seqlens
    rows = np.concatenate([np.arange(cs[b], cs[b] + P) for b in range(B)])
    cu_p = np.arange(B + 1, dtype=np.int32) * P
    kp = _dev(w.k[rows])
    cc, scs = D.online_chunks(kp, cu_p, lo, hi, tau)
    lay = D.Layout(cu_p, cc, scs, Hq, Hkv, d, torch.bfloat16)
    eager, graphed = (D.DecodeState(B, Hq, Hkv, d, torch.bfloat16, P + steps, 64) for _ in range(2))
    for st in (eager, graphed):
        st.load_prefix(lay, _dev(w.q[rows]), kp, _dev(w.v[rows]))
    scale = 1.0 / np.sqrt(d)
    q_buf = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    k_buf = torch.empty((B, Hkv, d), dtype=torch.bfloat16, device="cuda")
    v_buf = torch.empty_like(k_buf)
    out_buf = torch.empty_like(q_buf)
    kept_buf = torch.empty((B, Hq, topk), dtype=torch.int32, device="cuda")
    out_e = torch.empty_like(q_buf)
    kept_e = torch.empty_like(kept_buf)
    toks = [cs[:-1] + P + s for s in range(steps)]
    # the first token eagerly on both (the no-alloc path looks its scratch up here, outside capture)
    q0, k0, v0 = _dev(w.q[toks[0]]), _dev(w.k[toks[0]]), _dev(w.v[toks[0]])
    eager.step(q0, k0, v0, lo, hi, tau, topk, grouped, scale, out=out_e, kept=kept_e)
    graphed.step_noalloc(q0, k0, v0, lo, hi, tau, topk, grouped, scale, out=out_buf, kept=kept_buf)
    torch.cuda.synchronize()
    assert torch.equal(out_e, out_buf) and torch.equal(kept_e, kept_buf)
    g = torch.cuda.CUDAGraph()
    capture = torch.cuda.Stream()
    capture.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=capture):
        graphed.step_noalloc(q_buf, k_buf, v_buf, lo, hi, tau, topk, grouped, scale, out=out_buf, kept=kept_buf)
    torch.cuda.synchronize()
    for s in range(1, steps):
        qs, ks, vs = _dev(w.q[toks[s]]), _dev(w.k[toks[s]]), _dev(w.v[toks[s]])
        q_buf.copy_(qs)
        k_buf.copy_(ks)
        v_buf.copy_(vs)
        g.replay()
        eager.step(qs, ks, vs, lo, hi, tau, topk, grouped, scale, out=out_e, kept=kept_e)
        torch.cuda.synchronize()
        assert torch.equal(out_e, out_buf), f"replay {s}: outputs differ"
        assert torch.equal(kept_e, kept_buf), f"replay {s}: kept lists differ"
        for a, b in zip((eager.k_cache, eager.v_cache, eager.seq_len, eager.num_closed, eager.chunk_start,
                         eager.k_sum, eager.q_run, eager.k_run, eager.status),
                        (graphed.k_cache, graphed.v_cache, graphed.seq_len, graphed.num_closed, graphed.chunk_start,
                         graphed.k_sum, graphed.q_run, graphed.k_run, graphed.status)):
            assert torch.equal(a, b), f"replay {s}: decode states differ"
    assert int(graphed.seq_len[0].item()) == P + steps
