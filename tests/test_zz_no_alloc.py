"""dhsa_decode_step_noalloc (scratch in the library's static device array) against dhsa_decode_step
(scratch in a caller workspace), through the C ABI.

Two decode states are loaded with the same chunked prefix and fed the same tokens, one stepped by
each entry point.  The two share every kernel and differ only in where the scratch lives, so the
outputs, kept lists and the whole state must be bit-identical after every step; the no-alloc path's
outputs are also checked against the decode oracle (the bar of the other decode tests).  The two
settings run one after the other, the second with a smaller state, so the second call finds the
static array holding the first call's contents.
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

# (sequences, Hq, Hkv, d, dtype, seed, prefix tokens, lo, hi, tau, topk, grouped, steps); the second is
# the smaller one
SETTINGS = [
    ([SeqSpec(1400, ("uniform", 24, 120), 0, 0)] * 3, 8, 2, 128, "bf16", 71, 1200, 24, 160, 0.5, 6, True, 12),
    ([SeqSpec(400, ("uniform", 16, 64), 0, 0)], 4, 2, 64, "bf16", 72, 300, 16, 80, 0.5, 3, False, 8),
]


def _dev(a, dt):
    a = np.ascontiguousarray(a)
    if dt == "bf16":
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def _state_tensors(st):
    return [st.k_cache, st.v_cache, st.seq_len, st.num_closed, st.chunk_start, st.k_sum, st.q_run, st.k_run,
            st.status]


def _run_setting(seqs, Hq, Hkv, d, dt, seed, P, lo, hi, tau, topk, grouped, steps):
    print(f"[no-alloc] B={len(seqs)} Hq={Hq} Hkv={Hkv} d={d} {dt} prefix={P} topk={topk} grouped={grouped}",
          flush=True)
    w = W.make_workload(seqs, Hq, Hkv, d, dt, seed=seed, name="noalloc")
    B, cs = w.num_seqs, w.cu_seqlens
    T_seq = int(cs[1] - cs[0])
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    scale = 1.0 / np.sqrt(d)
    rows = np.concatenate([np.arange(cs[b], cs[b] + P) for b in range(B)])
    cu_p = np.arange(B + 1, dtype=np.int32) * P
    kp = _dev(w.k[rows], dt)
    cc, scs = D.online_chunks(kp, cu_p, lo, hi, tau)
    lay = D.Layout(cu_p, cc, scs, Hq, Hkv, d, tdt)
    states = [D.DecodeState(B, Hq, Hkv, d, tdt, T_seq, 64) for _ in range(2)]
    for st in states:
        st.load_prefix(lay, _dev(w.q[rows], dt), kp, _dev(w.v[rows], dt))
    need = D.load_library().dhsa_decode_workspace_bytes(__import__("ctypes").byref(states[0].struct), topk,
                                                         int(grouped))
    assert 0 < need <= 64 << 20
    out_ws = torch.empty((B, Hq, d), dtype=tdt, device="cuda")
    out_na = torch.empty_like(out_ws)
    kept_ws = torch.empty((B, Hq, topk), dtype=torch.int32, device="cuda")
    kept_na = torch.empty_like(kept_ws)
    outs = []
    for s in range(steps):
        idx = cs[:-1] + P + s
        q, k, v = _dev(w.q[idx], dt), _dev(w.k[idx], dt), _dev(w.v[idx], dt)
        states[0].step(q, k, v, lo, hi, tau, topk, grouped, scale, out=out_ws, kept=kept_ws)
        states[1].step_noalloc(q, k, v, lo, hi, tau, topk, grouped, scale, out=out_na, kept=kept_na)
        torch.cuda.synchronize()
        assert torch.equal(out_ws, out_na), f"step {s}: outputs differ"
        assert torch.equal(kept_ws, kept_na), f"step {s}: kept lists differ"
        for a, b in zip(_state_tensors(states[0]), _state_tensors(states[1])):
            assert torch.equal(a, b), f"step {s}: decode states differ"
        outs.append(out_na.float().cpu().numpy())
    assert int(states[1].status.abs().sum().item()) == 0
    qf, kf, vf = w.q_f32(), w.k_f32(), w.v_f32()
    outs = np.array(outs)
    for b in range(B):
        sl = slice(cs[b], cs[b] + P + steps)
        o_out, _, _ = oracle.decode_sequence(qf[sl], kf[sl], vf[sl], lo, hi, tau, topk, scale, first_output=P,
                                             grouped=grouped)
        err = np.abs(outs[:, b] - o_out).max()
        assert err <= OUT_ATOL[dt], f"seq {b}: no-alloc output max-abs err {err:.3e}"


def test_noalloc_step_equals_workspace_step_twice():
    for setting in SETTINGS:
        _run_setting(*setting)


def test_noalloc_step_refuses_without_out():
    st = D.DecodeState(1, 4, 2, 64, torch.bfloat16, 64, 8)
    q = torch.zeros((1, 4, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(D.DhsaError):
        st.step_noalloc(q, k, k, 4, 16, 0.5, 3)
