"""Plant plausible mistakes in copies of the CPU oracle; each copy must fail at least one pin.

The mistakes are textual edits of oracle/dhsa_oracle.py or oracle/chunking_oracle.py applied to an
in-memory copy (the oracle on disk is never touched); the mutant module holds both files' functions,
one of them edited, so a pin of the other file cannot "catch" it by a missing name.  Each edit must
match exactly once, so the lists stay in step with the oracle's source.
"""
import os
import types

import pytest

import oracle_pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
SRC = os.path.join(ORACLE_DIR, "dhsa_oracle.py")
CHUNK_SRC = os.path.join(ORACLE_DIR, "chunking_oracle.py")
DECODE_SRC = os.path.join(ORACLE_DIR, "decode_oracle.py")
BUDGET_SRC = os.path.join(ORACLE_DIR, "budget_oracle.py")

MUTATIONS = {
    "layout_no_per_sequence_tiling": ("if cc[sc[b]] != cs[b] or cc[sc[b + 1]] != cs[b + 1]:", "if False:"),
    "layout_allows_empty_chunk": ("if np.any(np.diff(cc) < 1):", "if np.any(np.diff(cc) < 0):"),
    "plan_accepts_negative_budget": ("if tk.shape != (C,) or np.any(tk < 0):", "if tk.shape != (C,):"),
    "plain_mean": ("out[c] = mean * np.sqrt(n)", "out[c] = mean"),
    "plain_sum": ("out[c] = mean * np.sqrt(n)", "out[c] = mean * n"),
    "inverse_sqrt": ("out[c] = mean * np.sqrt(n)", "out[c] = mean / np.sqrt(n)"),
    "drop_last_token": ("mean = x[s:e].astype(np.float64).sum(axis=0) / n",
                        "mean = x[s:e - 1].astype(np.float64).sum(axis=0) / n"),
    "kv_head_modulo_in_scores": ("ks[c0:c1, h // G, :].T", "ks[c0:c1, h % Hkv, :].T"),
    "non_causal_scores": ("causal = np.tril(np.ones((c1 - c0, c1 - c0), bool))",
                          "causal = np.ones((c1 - c0, c1 - c0), bool)"),
    "tie_to_higher_index": ("order = np.lexsort((cand, -s))", "order = np.lexsort((-cand, -s))"),
    "ascending_scores": ("order = np.lexsort((cand, -s))", "order = np.lexsort((cand, s))"),
    "diagonal_competes": ("cand = np.arange(first, i, dtype=np.int64)",
                          "cand = np.arange(first, i + 1, dtype=np.int64)"),
    "budget_off_by_one": ("kept = cand[order[:min(k, cand.size)]]", "kept = cand[order[:min(k + 1, cand.size)]]"),
    "plan_without_diagonal": ("counts = np.minimum(tk, i_loc) + 1", "counts = np.minimum(tk, i_loc + 1)"),
    "global_chunk_index": ("i_loc = np.arange(C) - sc[seq] if C", "i_loc = np.arange(C) if C"),
    "candidates_cross_sequences": ("kept = select_key_chunks(S[h, i], int(sc[seq[i]]), i, int(topk[i]))",
                                   "kept = select_key_chunks(S[h, i], 0, i, int(topk[i]))"),
    "strict_causal_mask": ("visible = keys[None, :] <= np.arange(s_i, e_i)[:, None]",
                           "visible = keys[None, :] < np.arange(s_i, e_i)[:, None] + (e_i == s_i + 1)"),
    "no_causal_mask": ("Z = np.where(visible, Z, -np.inf)", "Z = Z"),
    "kv_head_modulo_in_attention": ("        g = h // G\n        for i in chunks:",
                                    "        g = h % k.shape[1]\n        for i in chunks:"),
    "missing_softmax_scale": ("Z = softmax_scale * (qi @ k[keys, g, :].astype(np.float64).T)",
                              "Z = (qi @ k[keys, g, :].astype(np.float64).T)"),
    "lse_without_max": ("LSE[h, s_i:e_i] = m[:, 0] + np.log(lsum[:, 0])", "LSE[h, s_i:e_i] = np.log(lsum[:, 0])"),
    "values_from_wrong_head": ("O[s_i:e_i, h, :] = (P @ v[keys, g, :].astype(np.float64)) / lsum",
                               "O[s_i:e_i, h, :] = (P @ v[keys, 0, :].astype(np.float64)) / lsum"),
    "group_max_instead_of_sum": ("full += qs[c0:c1, h, :] @ ks[c0:c1, g, :].T",
                                 "full = np.maximum(full, qs[c0:c1, h, :] @ ks[c0:c1, g, :].T)"),
    "group_wrong_heads": ("for h in range(g * G, (g + 1) * G):\n                full +=",
                          "for h in range(g, g + G):\n                full +="),
    "group_row_to_first_head_only": ("block_idx[g * G:(g + 1) * G, row_ptr[i]:row_ptr[i + 1]] = kept",
                                     "block_idx[g * G, row_ptr[i]:row_ptr[i + 1]] = kept"),
    "unnormalised_output": ("O[s_i:e_i, h, :] = (P @ v[keys, g, :].astype(np.float64)) / lsum",
                            "O[s_i:e_i, h, :] = (P @ v[keys, g, :].astype(np.float64))"),
}


CHUNK_MUTATIONS = {
    "chunk_lo_off_by_one": ("for t in range(c0 + lo, end):", "for t in range(c0 + lo + 1, end):"),
    "chunk_cut_at_equal": ("if sim[t] < tau32:", "if sim[t] <= tau32:"),
    "chunk_hi_exclusive": ("end = min(c0 + hi, e)", "end = min(c0 + hi - 1, e)"),
    "chunk_cut_after_drop": ("                    cut = t\n", "                    cut = t + 1\n"),
    "sim_unnormalised": ("sim[t] = float(np.dot(a, c)) / np.sqrt(na * nc)", "sim[t] = float(np.dot(a, c))"),
    "sim_across_sequences": ("for t in range(int(cs[b]) + 1, int(cs[b + 1])):",
                             "for t in range(max(int(cs[b]), 1), int(cs[b + 1])):"),
    "sim_zero_rows_compared": ("if na > 0.0 and nc > 0.0:", "if na > 0.0 or nc > 0.0:"),
    "sim_first_head_only": ("rows = k.reshape(T, -1).astype(np.float64)", "rows = k[:, 0, :].astype(np.float64)"),
}


DECODE_MUTATIONS = {
    "decode_routes_by_token_query": ("                qv = q_open[h]\n", "                qv = q[t, h]\n"),
    "decode_skips_current_token": ("[np.arange(c0, t + 1)]", "[np.arange(c0, max(t, c0 + 1))]"),
    "decode_cut_ignores_lo": ("if t > 0 and ((t - c0 >= lo and sim[t] < tau32) or t - c0 >= hi):",
                              "if t > 0 and (sim[t] < tau32 or t - c0 >= hi):"),
    "decode_no_query_reset": ("            q_run[:] = 0.0\n", ""),
    "decode_summary_mean": ("k_sums.append((k_run / np.sqrt(t - c0)).astype(np.float32))",
                            "k_sums.append((k_run / (t - c0)).astype(np.float32))"),
    "decode_budget_plus_one": ("chosen = np.sort(order[:min(topk, C)])", "chosen = np.sort(order[:min(topk + 1, C)])"),
    "decode_values_head0": ("out_t[h] = (w @ v[keys, g, :]) / w.sum()", "out_t[h] = (w @ v[keys, 0, :]) / w.sum()"),
    "decode_ties_to_higher": ("order = np.lexsort((np.arange(C), -s.astype(np.float64)))",
                              "order = np.lexsort((-np.arange(C), -s.astype(np.float64)))"),
}


BUDGET_MUTATIONS = {
    "budget_strict_fit": ('m = int(np.searchsorted(cum, budget, side="right"))',
                          'm = int(np.searchsorted(cum, budget, side="left"))'),
    "budget_skips_misfits": ('m = int(np.searchsorted(cum, budget, side="right"))',
                             'm = int(np.sum(np.asarray(lens, np.int64)[cand[order]] <= budget))'),
    "budget_rank_ascending": ("order = np.lexsort((cand, -s))              # ranking: score desc, then chunk asc",
                              "order = np.lexsort((cand, s))              # ranking: score desc, then chunk asc"),
    "budget_plan_longest_first": ("earlier = np.sort(lens[sc[seq[i]]:i])", "earlier = np.sort(lens[sc[seq[i]]:i])[::-1]"),
    "budget_pad_with_diagonal": ("block_idx = np.full((Hq, nnz), -1, np.int32)", "block_idx = np.full((Hq, nnz), 0, np.int32)"),
}


def _mutant(old, new, target=SRC):
    srcs = {}
    for path in (SRC, CHUNK_SRC, DECODE_SRC, BUDGET_SRC):
        with open(path) as f:
            srcs[path] = f.read()
    assert srcs[target].count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    srcs[target] = srcs[target].replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    for path, src in srcs.items():
        # one namespace holds every file, so the package-relative imports are dropped
        src = "\n".join(l for l in src.split("\n") if not l.startswith("from ."))
        exec(compile(src, os.path.basename(path), "exec"), mod.__dict__)
    return mod


ALL = {**{n: (m, SRC) for n, m in MUTATIONS.items()}, **{n: (m, CHUNK_SRC) for n, m in CHUNK_MUTATIONS.items()},
       **{n: (m, DECODE_SRC) for n, m in DECODE_MUTATIONS.items()},
       **{n: (m, BUDGET_SRC) for n, m in BUDGET_MUTATIONS.items()}}


@pytest.mark.parametrize("name", sorted(ALL))
def test_mutant_is_caught(name):
    (old, new), target = ALL[name]
    mod = _mutant(old, new, target)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure of a pin counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutant {name} survived every pin"
