"""sa_indexer_scores against the oracle (GPU).  Integer-valued inputs with dyadic
weights make every score exact, so those cases must match bit for bit."""

import numpy as np
import pytest

import oracle.reference as orc
import sa_synth
import long_context_sparse_13_amd as sa
from tests.gpu_util import dev, host, note

pytestmark = pytest.mark.gpu


def _check(x, dtype, row_begin, row_end, ld, exact, rows=None):
    import torch
    qi, ki, w = x["qi"], x["ki"], x["w"]
    B, T, H, DI = qi.shape
    note(f"indexer B={B} T={T} H={H} DI={DI} {dtype} rows=[{row_begin},{row_end}) ld={ld}")
    R = row_end - row_begin
    sc = torch.full((B, R, ld), float("nan"), dtype=torch.float32, device="cuda")
    sa.sa_indexer_scores(dev(qi, dtype), dev(ki, dtype), dev(w, "f32"), row_begin, row_end, sc, ld)
    got = host(sc)
    rows = range(row_begin, row_end) if rows is None else rows
    for b in range(B):
        for t in rows:
            want = orc.indexer_scores_row(qi, ki, w, b, t)
            g = got[b, t - row_begin]
            if exact:
                assert np.array_equal(g[: t + 1].astype(np.float64), want), (b, t)
            else:
                err = np.abs(g[: t + 1] - want).max()
                assert err <= 1e-5 * max(1.0, np.abs(want).max()), (b, t, err)
            assert np.isnan(g[t + 1:]).all(), "entries s > t must stay untouched"


@pytest.mark.parametrize("H,DI", [(4, 64), (4, 32), (2, 128), (1, 64), (3, 40)])
def test_exact_integer_bf16(H, DI):
    x = sa_synth.integer_indexer_inputs(301, 2, 300, H, DI)
    _check(x, "bf16", 0, 300, 300, exact=True)


def test_exact_integer_f32_and_chunks():
    x = sa_synth.integer_indexer_inputs(302, 1, 520, 4, 32)
    _check(x, "f32", 0, 520, 520, exact=True)
    x = sa_synth.integer_indexer_inputs(303, 1, 1500, 4, 64)
    _check(x, "bf16", 1100, 1377, 1380, exact=True)


def test_random_bf16_and_f32():
    x = sa_synth.indexer_inputs(304, 1, 1200, 4, 64, "bf16")
    _check(x, "bf16", 0, 1200, 1200, exact=False, rows=list(range(0, 1200, 13)))
    x = sa_synth.indexer_inputs(305, 1, 2048, 4, 32, "f32")
    _check(x, "f32", 0, 2048, 2048, exact=False, rows=list(range(0, 2048, 31)))
