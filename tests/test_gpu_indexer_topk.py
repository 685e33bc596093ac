"""sa_indexer_topk (fused indexer + top-k) on the GPU.

The fused call must write exactly what sa_indexer_scores followed by sa_topk_select
write (bit for bit: both score through the same MFMA arithmetic), and agree with the
float64 oracle within the near-tie exemption.  Crafted inputs force the
other two selection paths (candidate set too large for the registers, candidate set
smaller than k) and check they stay exact."""

import numpy as np
import pytest

import oracle.reference as orc
import sa_synth
import long_context_sparse_13_amd as sa
from tests.gpu_util import check_selection, dev, host, note

pytestmark = pytest.mark.gpu


def _two_step(qi_d, ki_d, w_d, T, k, row_begin, row_end):
    sc = sa.sa_indexer_scores(qi_d, ki_d, w_d, row_begin, row_end)
    return host(sa.sa_topk_select(sc, k, T, row_begin, row_end))


def _fused(qi_d, ki_d, w_d, k, row_begin, row_end):
    import torch
    B, T, H, DI = qi_d.shape
    need = sa.sa_indexer_topk_workspace(B, T, H, DI, row_begin, row_end, k)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)  # garbage: the call must not depend on the workspace's contents
    idx = sa.sa_indexer_topk(qi_d, ki_d, w_d, k, row_begin, row_end, workspace=ws)
    n_recomputed = int(host(ws[:4]).view(np.uint32)[0])
    return host(idx), n_recomputed


def _case(x, k, row_begin=0, row_end=None, max_recomputed=None):
    qi, ki, w = x["qi"], x["ki"], x["w"]
    B, T, H, DI = qi.shape
    row_end = T if row_end is None else row_end
    note(f"indexer_topk B={B} T={T} H={H} DI={DI} k={k} rows=[{row_begin},{row_end})")
    qi_d, ki_d, w_d = dev(qi, "bf16"), dev(ki, "bf16"), dev(w, "f32")
    want = _two_step(qi_d, ki_d, w_d, T, k, row_begin, row_end)
    got, nrec = _fused(qi_d, ki_d, w_d, k, row_begin, row_end)
    bad = np.argwhere((got != want).any(axis=2))
    assert bad.shape[0] == 0, f"fused != two-step at (b, t) {bad[:5].tolist()}"
    if max_recomputed is not None:
        assert nrec <= max_recomputed, nrec
    return got, nrec


@pytest.mark.parametrize("H,DI,T,k", [(4, 64, 5000, 256), (4, 32, 2048, 256), (2, 128, 3000, 100),
                                      (1, 64, 2500, 512), (4, 128, 1500, 64)])
def test_matches_two_step(H, DI, T, k):
    x = sa_synth.indexer_inputs(601 + H + DI, 2, T, H, DI, "bf16")
    _case(x, k, max_recomputed=2)


def test_ragged_row_chunk_and_batch():
    x = sa_synth.indexer_inputs(611, 2, 4000, 4, 64, "bf16")
    _case(x, 300, 1000, 2345, max_recomputed=2)


def test_k_edges():
    x = sa_synth.indexer_inputs(612, 1, 600, 4, 64, "bf16")
    _case(x, 1)
    _case(x, 600)            # every row keeps all its positions
    _case(x, 1000)           # k > T
    x = sa_synth.indexer_inputs(613, 1, 12000, 4, 64, "bf16")
    _case(x, 2560, 11000, 12000, max_recomputed=8)
    # beyond ~3000 the candidate lists outgrow the registers: rows are selected by
    # passes over the lists, still exact and without recomputation
    _case(x, 4096, 11800, 12000, max_recomputed=2)


def test_integer_ties():
    # massive exact ties: the lower-position rule runs through the candidate lists
    x = sa_synth.integer_indexer_inputs(614, 1, 3000, 4, 64, lo=-1, hi=1)
    _case(x, 256)


def test_against_oracle():
    x = sa_synth.indexer_inputs(615, 1, 3000, 4, 64, "bf16")
    got, _ = _case(x, 256)
    qi = sa_synth.round_bf16(x["qi"])
    ki = sa_synth.round_bf16(x["ki"])
    rows = list(range(0, 300)) + list(range(300, 3000, 37)) + list(range(2990, 3000))
    exact = 0
    for t in rows:
        s = orc.indexer_scores_row(qi, ki, x["w"], 0, t)
        want = orc.topk_select_row(s, 256)
        exact += check_selection(got[0, t], want, s, 256)
    assert exact >= len(rows) - 3


def test_recompute_when_threshold_too_high():
    # the sampled positions (multiples of 4 for k = 256) below 400 score far above every
    # other position: the sample's threshold then admits only ~100 candidates (< k), so
    # every row t >= 396 is recomputed in full
    g = sa_synth.rng(616)
    T, H, DI, k = 3000, 4, 64, 256
    qi = np.ones((1, T, H, DI), np.float32)
    ki = g.integers(-1, 2, size=(1, T, DI)).astype(np.float32)
    ki[0, 0:400:4] = 3.0
    w = np.array([0.5, 0.25, 0.125, 1.0], np.float32)
    got, nrec = _case({"qi": qi, "ki": ki, "w": w}, k)
    assert nrec > 2000, nrec


def test_list_passes_when_candidates_overflow():
    # the sampled positions score 0 and the others >= 0: every position is a candidate,
    # more than the registers hold for rows t >= 4096 (selected by list passes, exact
    # ties at zero included); nothing is recomputed
    g = sa_synth.rng(617)
    T, H, DI, k = 8400, 4, 32, 256
    qi = np.ones((1, T, H, DI), np.float32)
    ki = g.integers(0, 4, size=(1, T, DI)).astype(np.float32)
    ki[0, ::4] = -1.0
    w = np.array([1.0, 0.5, 0.25, 0.125], np.float32)
    _case({"qi": qi, "ki": ki, "w": w}, k, 3900, 4300, max_recomputed=0)
    _case({"qi": qi, "ki": ki, "w": w}, 4000, 8100, 8400, max_recomputed=0)


def test_recompute_when_a_group_list_is_full():
    # the keys of chunks 0, 64 and 128 (positions [0, 256), [16384, 16640), [32768, 33024),
    # all scored by the same wavefront group and kept in one list of at most 256 entries)
    # score far above the rest: rows with two or three such chunks behind them have more
    # candidates in that list than it holds and are recomputed in full (more rows than
    # recompute slots); rows with only the first such chunk fit and are not
    g = sa_synth.rng(620)
    T, H, DI, k = 40000, 4, 32, 600
    qi = np.ones((1, T, H, DI), np.float32)
    ki = g.integers(-1, 2, size=(1, T, DI)).astype(np.float32)
    for c0 in (0, 16384, 32768):
        ki[0, c0:c0 + 256] = 3.0 + g.integers(0, 3, size=(256, DI))
    w = np.array([0.5, 0.25, 0.125, 1.0], np.float32)
    x = {"qi": qi, "ki": ki, "w": w}
    _, nrec = _case(x, k, 39000, 40000)
    assert nrec == 1000, nrec
    _, nrec = _case(x, k, 20000, 20300)
    assert nrec == 300, nrec
    _, nrec = _case(x, k, 10000, 10200, max_recomputed=0)


def test_64k_rows():
    # the 64K prefill sizes (k = 2048): the last rows of the longest chunk
    x = sa_synth.indexer_inputs(618, 1, 65536, 4, 64, "bf16")
    _case(x, 2048, 65536 - 48, 65536, max_recomputed=1)


def test_long_rows_sparser_sample():
    # rows of 150,000 keys: the sample is thinned to at most 4096 per row (wider margin)
    x = sa_synth.indexer_inputs(619, 1, 150000, 4, 64, "bf16")
    _case(x, 2048, 150000 - 16, 150000, max_recomputed=1)
    _case(x, 256, 150000 - 16, 150000, max_recomputed=1)
