"""Cross-layer index reuse (F,S,S,S) through the GPU entry points against the oracle."""

import numpy as np
import pytest

import oracle.reference as orc
import sa_synth
import long_context_sparse_13_amd as sa
from tests.gpu_util import BF16_TOL, check_selection, dev, host, note

pytestmark = pytest.mark.gpu


def test_fsss_reuse_small():
    import torch
    T, k, W, Hq, D = 1200, 128, 64, 16, 128
    scale = 1 / np.sqrt(D)
    note(f"indexcache FSSS T={T} k={k} W={W}")
    x = sa_synth.indexer_inputs(701, 1, T, 4, 64, "bf16")
    layers = [sa_synth.attn_inputs(sa_synth.layer_seed(l), 1, T, Hq, 1, D, "bf16") for l in range(4)]
    sc = sa.sa_indexer_scores(dev(x["qi"], "bf16"), dev(x["ki"], "bf16"), dev(x["w"], "f32"))
    idx = sa.sa_topk_select(sc, k, T)
    outs = [host(sa.sa_sparse_attn_fwd(dev(l["q"], "bf16"), dev(l["k"], "bf16"),
                                       dev(l["v"], "bf16"), idx, W, scale)) for l in layers]
    rows = list(range(0, T, 11)) + [T - 1]
    ref, n_index = orc.indexcache_prefill(x["qi"], x["ki"], x["w"], layers, "FSSS", k, W, scale,
                                          rows)
    assert n_index == 1
    ig = host(idx)
    exact = []
    for t in rows:
        s = orc.indexer_scores_row(x["qi"], x["ki"], x["w"], 0, t)
        if check_selection(ig[0, t], orc.topk_select_row(s, k), s, k):
            exact.append(rows.index(t))
    for o, (O, _) in zip(outs, ref):
        err = np.abs(o[:, [rows[i] for i in exact]] - O[:, exact]).max()
        assert err <= BF16_TOL, err
