"""Plant plausible mistakes in copies of the CPU oracle; each copy must fail at least one pin.

The mistakes are textual edits of oracle/dhsa_oracle.py applied to an
in-memory copy (the oracle on disk is never touched).  Each edit must match
exactly once, so the list stays in step with the oracle's source.
"""
import os
import types

import pytest

import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "dhsa_oracle.py")

MUTATIONS = {
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


def _mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    mod = types.ModuleType("dhsa_oracle_mutant")
    exec(compile(src.replace(old, new), "dhsa_oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_is_caught(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure of a pin counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutant {name} survived every pin"
