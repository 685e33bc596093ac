"""The pins bite: each plausible mistake planted in a copy of the oracle (on the CPU)
must make at least one pin fail.  The real oracle is never modified."""

import os
import types

import pytest

from tests import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "reference.py")

# (name, original text, mutated text)
MUTANTS = [
    ("indexer_relu_after_head_sum",
     "    relu = np.maximum(dots, 0.0)\n    return np.matmul(_f64(w), relu)",
     "    return np.maximum(np.matmul(_f64(w), dots), 0.0)"),
    ("indexer_weights_dropped", "return np.matmul(_f64(w), relu)", "return relu.sum(axis=0)"),
    ("indexer_key_off_by_one", "k = _f64(ki[b, : t + 1])", "k = _f64(ki[b, 1: t + 2])"),
    ("indexer_transposed_operand", "dots = np.matmul(q, k.T)", "dots = np.matmul(q[:, ::-1], k.T)"),
    ("topk_ties_to_higher", "ties = np.flatnonzero(s == kth)[:need]",
     "ties = np.flatnonzero(s == kth)[::-1][:need]"),
    ("topk_kth_smallest", "kth = np.partition(s, n - k)[n - k]", "kth = np.partition(s, k - 1)[k - 1]"),
    ("topk_unsorted_output", "sel = np.sort(np.concatenate([above, ties]))",
     "sel = np.concatenate([above, ties])"),
    ("topk_no_padding_when_short", "out[:n] = np.arange(n, dtype=np.int32)",
     "out[:n] = np.arange(n, dtype=np.int32)\n        out[n:] = 0"),
    ("attn_window_off_by_one", "m[max(0, t - window + 1): t + 1] = True",
     "m[max(0, t - window): t + 1] = True"),
    ("attn_window_excludes_self", "m[max(0, t - window + 1): t + 1] = True",
     "m[max(0, t - window + 1): t] = True"),
    ("attn_scale_dropped", "logits = scale * np.matmul(qh, kb[: t + 1, g].T)",
     "logits = np.matmul(qh, kb[: t + 1, g].T)"),
    ("attn_wrong_kv_head", "logits = scale * np.matmul(qh, kb[: t + 1, g].T)",
     "logits = scale * np.matmul(qh, kb[: t + 1, (g + 1) % Hkv].T)"),
    ("attn_negative_index_accepted", "ids = ids[(ids >= 0) & (ids <= t)]", "ids = ids[ids <= t]"),
    ("attn_lse_without_max", "lse = (mx + np.log(l))[:, 0]", "lse = np.log(l)[:, 0]"),
    ("attn_sum_not_normalised", "out = np.matmul(p, vals) / l if", "out = np.matmul(p, vals) if"),
    ("graph_clamp_not_drop", "return np.sort(t - o[o <= t])", "return np.unique(np.maximum(t - o, 0))"),
    ("graph_tau_sign", "logits = -tau * dist2 + bias[:, None]", "logits = tau * dist2 + bias[:, None]"),
    ("graph_bias_dropped", "logits = -tau * dist2 + bias[:, None]", "logits = -tau * dist2"),
    ("graph_extra_pow2", "{1 << j for j in range(n_pow2)}", "{1 << j for j in range(n_pow2 + 1)}"),
    ("graph_count_includes_local_pow2", "if (1 << j) > local and (1 << j) <= t)",
     "if (1 << j) <= t)"),
    ("graph_distance_not_squared", "dist2 = np.sum(diff * diff, axis=2).T",
     "dist2 = np.sqrt(np.sum(diff * diff, axis=2)).T"),
    ("decode_sum_not_mean", "kbar[b, :nfull] = kb.mean(axis=1)", "kbar[b, :nfull] = kb.sum(axis=1)"),
    ("decode_first_head_only", "scores = np.matmul(qg, kbar[b, :nfull, g].T).sum(axis=0)",
     "scores = np.matmul(qg, kbar[b, :nfull, g].T)[0]"),
    ("decode_window_off_by_one", "wstart = max(0, L - window)", "wstart = max(0, L - window + 1)"),
    ("decode_partial_block_scored", "nfull = int(lens[b]) // block\n        for g in range(Hkv):",
     "nfull = min(kbar.shape[1], (int(lens[b]) + block - 1) // block)\n        for g in range(Hkv):"),
    ("indexcache_indexes_every_layer", 'if kind == "F":', "if True:"),
    ("e4m3_bias_8", "np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    ("e4m3_subnormal_scale", "(m / 8.0) * 2.0 ** -6", "(m / 8.0) * 2.0 ** -7"),
    ("e4m3_mantissa_sixteenths", "(1.0 + m / 8.0) * np.exp2", "(1.0 + m / 16.0) * np.exp2"),
    ("e4m3_no_nan", "out[(e == 15) & ((c & 7) == 7)] = np.nan", "pass"),
    ("e4m3_sign_dropped", "out = np.where(negative, -magnitude, magnitude)", "out = magnitude"),
    ("cmp_partial_block_joins", "            nfull = (t + 1) // block\n            for g in range(Hkv):\n                qh",
     "            nfull = min(kbar.shape[1], (t + block) // block)\n            for g in range(Hkv):\n                qh"),
    ("cmp_scale_dropped", "logits = scale * np.matmul(qh, kb.T)                       # [G, nfull]",
     "logits = np.matmul(qh, kb.T)"),
    ("select_last_group_only", "scores += np.matmul(qg, _f64(kbar[b, :nfull, g]).T).sum(axis=0)",
     "scores = np.matmul(qg, _f64(kbar[b, :nfull, g]).T).sum(axis=0)"),
    ("block_tokens_shifted", "int(j) * block + i for j", "int(j) * block + i + 1 for j"),
    ("combine_gates_swapped", "g[..., 1:2] * o_slc + g[..., 2:3] * o_win",
     "g[..., 2:3] * o_slc + g[..., 1:2] * o_win"),
    ("nsa_decode_selected_before_window",
     "m_slc[int(j) * block: int(j) * block + block] = True",
     "m_slc[int(j) * block: min(int(j) * block + block, L - window)] = True"),
    ("bwd_delta_dropped", "ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "ds = p * dp"),
    ("bwd_dq_scale_dropped", "dQ[b, t, hs] = scale * np.matmul(ds, kb[: t + 1, g])",
     "dQ[b, t, hs] = np.matmul(ds, kb[: t + 1, g])"),
    ("bwd_dk_uses_dout", "dK[b, : t + 1, g] += scale * np.matmul(ds.T, qh)",
     "dK[b, : t + 1, g] += scale * np.matmul(ds.T, do)"),
    ("bwd_dv_transposed", "dV[b, : t + 1, g] += np.matmul(p.T, do)",
     "dV[b, : t + 1, g] += np.matmul(p.T, qh)"),
    ("boundary_off_by_one", "return float(srt[k - 1]), float(srt[k])",
     "return float(srt[k]), float(srt[k + 1]) if n > k + 1 else float(srt[k])"),
    ("boundary_ascending_sort", "srt = np.sort(s)[::-1]", "srt = np.sort(s)"),
    ("boundary_kth_twice", "return float(srt[k - 1]), float(srt[k])",
     "return float(srt[k - 1]), float(srt[k - 1])"),
    ("boundary_when_n_equals_k", "    if n <= k:\n        return None\n    srt",
     "    if n < k:\n        return None\n    srt"),
    ("boundary_distinct_values", "srt = np.sort(s)[::-1]", "srt = np.unique(s)[::-1]"),
    ("nsa_decode_window_without_self", "m_win[max(0, L - window): L] = True",
     "m_win[max(0, L - window): L - 1] = True"),
]


def _load_mutant(orig, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(orig) >= 1, f"pattern not found: {orig!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(orig, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,orig,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, orig, new):
    mod = _load_mutant(orig, new)
    caught_by = None
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception:          # AssertionError, or the mutant crashing on a pin's input
            caught_by = pin.__name__
            break
    assert caught_by, f"mutant {name} passes every pin"
