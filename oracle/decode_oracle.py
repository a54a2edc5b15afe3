"""CPU oracle for DHSA decode: tokens appended one at a time against the kept structure.

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of bench.py may import this module; the product path never
imports, links or calls it, and it imports nothing from the product path.

The pages evaluate prefill only ([P2] "Long-Context Modeling with Dynamic
Hierarchical Sparse Attention for On-Device LLMs", Abstract; [P3] ICML 2026
page, Abstract) and describe the method as online: chunks form as the sequence
streams in, each chunk is summarised by its mean scaled by sqrt(size), chunk
similarity is causal and decides the kept interactions.  Decode here is the
plain online reading of the same steps (a reading of this project, stated in
full so the GPU path and this oracle implement one definition):

  * chunking: token t joins the open (last) chunk, which starts at c0, unless
    the chunk-boundary rule of ``chunking_oracle`` cuts before it, i.e.
    (t - c0 >= lo and sim[t] < tau) or t - c0 >= hi; the rule only looks at
    tokens up to t, so the online cuts equal the offline ones;
  * a chunk closes when the next one starts; its key summary is then the sum
    of its key rows over sqrt(size) (float64, stored float32), as in prefill;
  * routing of token t: the open chunk's query summary so far,
    q_open = (sum of q over c0..t) / sqrt(t - c0 + 1) (stored float32), scores
    every closed chunk j of the sequence, s_j = q_open . k_sum[j] (float64,
    rounded to float32); the top-k by (s desc, j asc) are kept, plus the open
    chunk; routing is per query head, or once per KV head with the group's
    summed query summaries (as in prefill);
  * attention of token t: exact softmax over the tokens of the kept closed
    chunks and of the open chunk up to t.

At the last token of a chunk the open summary equals the chunk's prefill
summary, so decode there equals prefill at that token (pinned).
"""
from __future__ import annotations

import numpy as np

from .chunking_oracle import adjacent_similarity


def decode_sequence(q, k, v, lo: int, hi: int, tau: float, topk: int, softmax_scale: float,
                    first_output: int = 0, grouped: bool = False):
    """Process one sequence token by token.

    ``q`` [T, Hq, d], ``k``/``v`` [T, Hkv, d] (any float dtype; widened to float64).  Outputs are
    produced for tokens ``first_output .. T-1`` (earlier tokens are only appended).  Returns
    ``(out [T - first_output, Hq, d] float64, chunk_starts list, kept list)`` where ``kept[n][h]`` is
    the ascending list of closed chunks kept for output token ``first_output + n`` and head h (the
    open chunk, always kept, is not listed).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sim = adjacent_similarity(k, [0, T])
    tau32 = np.float32(tau)
    starts = [0]                  # chunk starts; the last one is the open chunk's
    k_sums = []                   # float32 [Hkv, d] per closed chunk
    q_run = np.zeros((Hq, d))
    k_run = np.zeros((Hkv, d))
    outs, kept_all = [], []
    for t in range(T):
        c0 = starts[-1]
        if t > 0 and ((t - c0 >= lo and sim[t] < tau32) or t - c0 >= hi):
            k_sums.append((k_run / np.sqrt(t - c0)).astype(np.float32))
            starts.append(t)
            c0 = t
            q_run[:] = 0.0
            k_run[:] = 0.0
        q_run += q[t]
        k_run += k[t]
        if t < first_output:
            continue
        n_open = t - c0 + 1
        q_open = (q_run / np.sqrt(n_open)).astype(np.float32).astype(np.float64)
        C = len(k_sums)
        ks = np.array(k_sums, np.float64).reshape(C, Hkv, d)
        out_t = np.empty((Hq, d))
        kept_t = []
        for h in range(Hq):
            g = h // G
            if grouped:
                qv = q_open[g * G:(g + 1) * G].sum(axis=0)
            else:
                qv = q_open[h]
            s = (ks[:, g, :] @ qv).astype(np.float32) if C else np.zeros(0, np.float32)
            order = np.lexsort((np.arange(C), -s.astype(np.float64)))
            chosen = np.sort(order[:min(topk, C)])
            kept_t.append(chosen.tolist())
            keys = [np.arange(starts[j], starts[j + 1]) for j in chosen] + [np.arange(c0, t + 1)]
            keys = np.concatenate(keys)
            z = softmax_scale * (k[keys, g, :] @ q[t, h])
            w = np.exp(z - z.max())
            out_t[h] = (w @ v[keys, g, :]) / w.sum()
        outs.append(out_t)
        kept_all.append(kept_t)
    out = np.array(outs).reshape(len(outs), Hq, d)
    return out, starts, kept_all
