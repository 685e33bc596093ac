"""sa_block_meanpool and sa_sparse_decode against the oracle (GPU)."""

import math

import numpy as np
import pytest

import oracle.reference as orc
import sa_synth
import long_context_sparse_13_amd as sa
from tests.gpu_util import BF16_TOL, TIE_REL, dev, host, note

pytestmark = pytest.mark.gpu


def _decode(seed, B, L, Hq, Hkv, D, block, top, W, lens=None, n_splits=0, reps=1):
    import torch
    note(f"decode seed={seed} B={B} L={L} Hq={Hq} Hkv={Hkv} D={D} block={block} top={top} W={W} "
         f"lens={None if lens is None else list(lens)[:6]} n_splits={n_splits}")
    x = sa_synth.decode_inputs(seed, B, L, Hq, Hkv, D, "bf16", lens=lens)
    scale = 1.0 / math.sqrt(D)
    q, kc, vc = dev(x["q"], "bf16"), dev(x["kcache"], "bf16"), dev(x["vcache"], "bf16")
    ln = dev(x["lens"], "i32")
    kbar = sa.sa_block_meanpool(kc, ln, block)
    need = sa.sa_sparse_decode_workspace(B, L, Hq, Hkv, D, block, top, W, n_splits)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for _ in range(reps):          # repeated calls reuse the workspace (counters self-reset)
        out, lse, sel = sa.sa_sparse_decode(q, kc, vc, kbar, ln, block, top, W, scale, n_splits,
                                            workspace=ws, return_lse=True, return_sel=True)
    kb_or = orc.block_meanpool(x["kcache"], x["lens"], block)
    kb_gpu = host(kbar)
    for b in range(B):
        nf = int(x["lens"][b]) // block
        if nf:
            assert np.abs(kb_gpu[b, :nf] - kb_or[b, :nf]).max() < 1e-5
    O, Lse, Sel = orc.sparse_decode(x["q"], x["kcache"], x["vcache"], x["lens"], block, top, W,
                                    scale, kbar=kb_or)
    sel_gpu = host(sel)
    ok = np.ones(B, bool)
    for b in range(B):
        for g in range(Hkv):
            if not np.array_equal(sel_gpu[b, g], Sel[b, g]):
                # allowed only within rounding distance of a tie (checked against scores)
                qg = x["q"][b, g * (Hq // Hkv):(g + 1) * (Hq // Hkv)].astype(np.float64)
                nf = int(x["lens"][b]) // block
                sc = (qg @ kb_or[b, :nf, g].T).sum(axis=0)
                a, bb = orc.topk_boundary(sc, top)
                assert a != bb and a - bb < TIE_REL * abs(a), (b, g, sel_gpu[b, g], Sel[b, g])
                ok[b] = False
    err = np.abs(host(out)[ok] - O[ok]).max()
    lerr = np.abs(host(lse)[ok] - Lse[ok]).max()
    assert err <= BF16_TOL, err
    assert lerr <= 2e-3, lerr
    # the merge counters (the workspace's last 256-aligned slice) are zero again
    cnt_bytes = ((4 * B * Hkv + 255) // 256) * 256
    assert int(ws[need - cnt_bytes:].sum()) == 0
    return host(out)


def test_small_varied_lengths():
    lens = [1000, 1024, 640, 63, 64, 130, 700, 1]
    _decode(601, 8, 1024, 16, 1, 128, 64, 4, 100, lens=lens)


def test_gqa_d64_blocks32():
    _decode(602, 3, 2000, 8, 2, 64, 32, 5, 70, lens=[2000, 1999, 517])


def test_split_count_invariance():
    a = _decode(603, 2, 4096, 16, 1, 128, 64, 16, 512, n_splits=1)
    b = _decode(603, 2, 4096, 16, 1, 128, 64, 16, 512, n_splits=7)
    c = _decode(603, 2, 4096, 16, 1, 128, 64, 16, 512, n_splits=0, reps=3)
    assert np.abs(a - b).max() <= 2e-2 and np.abs(a - c).max() <= 2e-2


def test_many_splits_mostly_empty():
    # 64 splits (the limit) over |U| <= 4 blocks + 128 window tokens: most split workgroups
    # get no tokens and publish an empty partial (max -inf, sum 0) that the merge must skip
    _decode(607, 2, 1000, 16, 1, 128, 64, 4, 128, lens=[1000, 333], n_splits=64, reps=2)


def test_splits_across_xcds():
    # 3 x 1 (sequence, KV head) pairs and 5 splits: a sequence's split workgroups land on
    # different XCDs, so the partials must travel through coherent memory
    _decode(606, 3, 3000, 16, 1, 128, 64, 8, 256, lens=[3000, 2500, 1777], n_splits=5, reps=3)


def test_many_top_blocks():
    # top_blocks above the 16 a scoring workgroup would keep by default; 64 is the maximum
    _decode(607, 2, 40000, 16, 1, 128, 64, 40, 300, lens=[40000, 20001])
    _decode(608, 1, 20000, 8, 1, 64, 16, 64, 64)


def test_window_zero_and_window_covers():
    _decode(604, 2, 800, 16, 1, 128, 64, 3, 0, lens=[800, 200])
    _decode(605, 2, 800, 16, 1, 128, 64, 3, 900, lens=[800, 333])


@pytest.mark.slow
def test_decode_workload_b32_128k():
    p = sa_synth.WORKLOADS[5].params
    _decode(1005, p["B"], p["L"], p["Hq"], p["Hkv"], p["D"], p["block"], p["top_blocks"],
            p["window"], reps=2)
