"""Plant plausible mistakes in copies of the oracle and check that the pins catch each one.

Every mutant is a one-line source substitution (a dropped term, a wrong sign or
index, a transposed or swapped operand, a reversed tie-break ...).  A mutant is
caught when at least one pin raises.  The mutants run on the CPU only.
"""
import importlib.util
import os
import types

import pytest

from tests import oracle_pins as pins

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "hs2_oracle.py")

MUTANTS = [
    ("dropped_scale", "s = scale * (q_g @ k_rows.T)", "s = (q_g @ k_rows.T)"),
    ("logits_from_values", "s = scale * (q_g @ k_rows.T)", "s = scale * (q_g @ v_rows.T)"),
    ("dropped_normaliser", "lse = m + np.log(l)", "lse = m"),
    ("output_from_keys", "out = probs @ v_rows", "out = probs @ k_rows"),
    ("mean_over_heads", "return probs.max(axis=0)", "return probs.mean(axis=0)"),
    ("sum_over_heads", "return probs.max(axis=0)", "return probs.sum(axis=0)"),
    ("min_over_heads", "return probs.max(axis=0)", "return probs.min(axis=0)"),
    ("window_one_too_wide", "first = max(0, pos - window + 1)", "first = max(0, pos - window)"),
    ("window_one_too_narrow", "first = max(0, pos - window + 1)", "first = max(0, pos - window + 2)"),
    ("ties_to_higher_index", "order = np.lexsort((cand, -score[cand]))",
     "order = np.lexsort((-cand, -score[cand]))"),
    ("smallest_scores", "order = np.lexsort((cand, -score[cand]))",
     "order = np.lexsort((cand, score[cand]))"),
    ("one_too_few_taken", "taken = cand[order[:n_take]]", "taken = cand[order[:max(0, n_take - 1)]]"),
    ("query_excludes_itself", "kk[: pos + 1], vv[: pos + 1], scale)", "kk[: pos], vv[: pos], scale)"),
    ("positions_shifted", "pos = S - T + t", "pos = S - T + t - 1"),
    ("sparse_ignores_index_k", "ks = k_rows[idx]", "ks = k_rows[: idx.size]"),
    ("sparse_ignores_index_v", "vs = v_rows[idx]", "vs = v_rows[: idx.size]"),
    ("sparse_unnormalised", "p = p / p.sum(axis=1, keepdims=True)", "p = p / p.shape[1]"),
    ("sparse_reuses_full_queries", "qn = widen_bf16(q_sparse[n, b, t, heads])",
     "qn = widen_bf16(q_full[b, t, heads])"),
    ("sparse_scale_dropped", "s = scale * (q_g @ ks.T)", "s = (q_g @ ks.T)"),
    ("widen_shift", "<< np.uint32(16)", "<< np.uint32(15)"),
    ("keys_from_wrong_head", "kk = widen_bf16(k[b, g])", "kk = widen_bf16(k[b, (g + 1) % k.shape[1]])"),
    ("queries_wrong_group", "heads = slice(g * G, (g + 1) * G)", "heads = slice(0, G)"),
    ("bridge_values_from_key_weights", "wv = widen_bf16(w_kv[1])", "wv = widen_bf16(w_kv[0])"),
    ("bridge_batch_and_head_swapped", 'k_new = np.einsum("gdm,btm->bgtd", wk, h)',
     'k_new = np.einsum("gdm,btm->gbtd", wk, h)'),
    ("bridge_tokens_reversed", "h = widen_bf16(hidden)", "h = widen_bf16(hidden)[:, ::-1]"),
    ("bridge_weight_transposed", 'v_new = np.einsum("gdm,btm->bgtd", wv, h)',
     'v_new = np.einsum("gdm,btm->bgtd", wv[:, ::-1], h)'),
    ("append_one_row_late", "k_out[:, :, pos0:pos0 + n] = k_new",
     "k_out[:, :, pos0 + 1:pos0 + n + 1] = k_new[:, :, : k_out.shape[2] - pos0 - 1]"),
    ("append_values_from_keys", "v_out[:, :, pos0:pos0 + n] = v_new",
     "v_out[:, :, pos0:pos0 + n] = k_new"),
    ("block_mean_not_max", "bscore = np.array([score[c * block:min((c + 1) * block, first)].max()",
     "bscore = np.array([score[c * block:min((c + 1) * block, first)].mean()"),
    ("block_ties_to_higher_index", "order = np.lexsort((blocks, -bscore))",
     "order = np.lexsort((-blocks, -bscore))"),
    ("block_last_partial_dropped", "n_blocks = (first + block - 1) // block",
     "n_blocks = first // block"),
    ("block_one_too_many", "n_take = min(top_k // block, n_blocks)",
     "n_take = min(top_k // block + 1, n_blocks)"),
    ("block_boundaries_shifted",
     "toks = [np.arange(c * block, min((c + 1) * block, first), dtype=np.int64) for c in taken]",
     "toks = [np.arange(c * block + 1, min((c + 1) * block + 1, first), dtype=np.int64) for c in taken]"),
    ("swa_branch_dropped", "+ attention_or_zero(q_g, kloc_rows, vloc_rows, scale))",
     "+ 0.0 * attention_or_zero(q_g, kloc_rows, vloc_rows, scale))"),
    ("swa_keeps_window_entries", "sel = lst[lst < first]", "sel = lst"),
    ("swa_local_rows_shifted", "rows = np.arange(first, pos + 1) - (S - Lc)",
     "rows = np.arange(first, pos + 1) - (S - Lc) - 1"),
    ("swa_local_from_shared_cache", "kl = widen_bf16(k_loc[n, b, g])[rows]", "kl = kk[first:pos + 1]"),
    ("swa_branch_unnormalised", "    p = p / p.sum(axis=1, keepdims=True)\n    return p @ v_rows",
     "    return p @ v_rows"),
]


def _load_mutant(name, old, new):
    with open(SRC_PATH, encoding="utf-8") as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutant {name}: pattern not found"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    mod.__file__ = SRC_PATH
    exec(compile(src.replace(old, new), SRC_PATH, "exec"), mod.__dict__)
    return mod


def test_unmutated_copy_passes_every_pin():
    mod = _load_mutant("identity", "import numpy as np", "import numpy as np")
    for pin in pins.ALL_PINS:
        pin(mod)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    mod = _load_mutant(name, old, new)
    failures = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError, or a crash the mistake causes
            failures.append((pin.__name__, type(e).__name__))
    assert failures, f"no pin caught mutant {name}"
