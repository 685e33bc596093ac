"""sa_sparse_attn_fwd against the float64 oracle (GPU)."""

import math

import numpy as np
import pytest

import oracle.reference as orc
import sa_synth
import long_context_sparse_13_amd as sa
from tests.gpu_util import BF16_TOL, F32_TOL, dev, host, note

pytestmark = pytest.mark.gpu


def _run(seed, B, T, Hq, Hkv, D, topk, W, dtype, scale=None, junk=False, rows=None, idx=None):
    note(f"sparse_attn seed={seed} B={B} T={T} Hq={Hq} Hkv={Hkv} D={D} topk={topk} W={W} {dtype}")
    x = sa_synth.attn_inputs(seed, B, T, Hq, Hkv, D, dtype)
    scale = scale if scale is not None else 1.0 / math.sqrt(D)
    if idx is None and topk > 0:
        idx = sa_synth.random_topk_idx(seed + 1, B, T, topk, junk=junk)
    q, k, v = dev(x["q"], dtype), dev(x["k"], dtype), dev(x["v"], dtype)
    di = dev(idx, "i32") if topk > 0 else None
    out, lse = sa.sa_sparse_attn_fwd(q, k, v, di, W, scale, return_lse=True)
    o_gpu, l_gpu = host(out), host(lse)
    rows = list(range(T)) if rows is None else rows
    ix = idx if topk > 0 else np.full((B, T, 1), -1, np.int32)
    O, L = orc.sparse_attn(x["q"], x["k"], x["v"], ix, W, scale, rows)
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    err = np.abs(o_gpu[:, rows] - O).max()
    lerr = np.abs(l_gpu[:, :, rows] - L).max()
    assert err <= tol, err
    assert lerr <= (2e-3 if dtype == "bf16" else 1e-4), lerr
    return err


@pytest.mark.parametrize("D", [64, 128])
def test_mfma_group16(D):
    _run(101, 1, 333, 16, 1, D, 48, 40, "bf16")


def test_mfma_gqa_padded_heads_batch():
    # G = 4 (12 padding head columns in the MFMA), two KV heads, batch 2, ragged window
    _run(102, 2, 257, 8, 2, 128, 33, 17, "bf16")


def test_mfma_window_only_and_topk_only():
    _run(103, 1, 300, 16, 1, 128, 0, 45, "bf16")
    _run(104, 1, 300, 16, 1, 128, 70, 0, "bf16")


def test_mfma_junk_indices_are_skipped():
    _run(105, 1, 200, 16, 1, 64, 96, 8, "bf16", junk=True)


def test_mfma_single_token_and_k_covers_all():
    _run(106, 1, 1, 16, 1, 128, 4, 1, "bf16")
    _run(107, 1, 90, 16, 1, 128, 128, 0, "bf16")   # topk >= T: full causal attention


def test_valu_fp32_workload1_shape():
    # the fp32 prefill workload: T=2048, 4 q heads on 1 KV head, D=64, k=256, W=64
    _run(1001, 1, 2048, 4, 1, 64, 256, 64, "f32", scale=1.0 / 8.0,
         rows=list(range(0, 2048, 7)) + [2047])


def test_valu_fp32_gqa_and_bf16_wide_group():
    _run(108, 2, 150, 6, 2, 128, 20, 9, "f32")
    _run(109, 1, 140, 32, 1, 64, 24, 16, "bf16")   # G = 32 > 16: VALU kernel


def test_lse_of_empty_set():
    # window 0 and only junk indices: nothing is attended -> out 0, lse -inf
    import torch
    note("sparse_attn empty selected set")
    x = sa_synth.attn_inputs(110, 1, 40, 16, 1, 64, "bf16")
    idx = np.full((1, 40, 8), -1, np.int32)
    out, lse = sa.sa_sparse_attn_fwd(dev(x["q"], "bf16"), dev(x["k"], "bf16"), dev(x["v"], "bf16"),
                                     dev(idx, "i32"), 0, 0.125, return_lse=True)
    assert torch.all(out.float() == 0)
    assert torch.all(torch.isinf(lse)) and torch.all(lse < 0)


def test_deterministic():
    import torch
    note("sparse_attn determinism x5")
    x = sa_synth.attn_inputs(111, 1, 500, 16, 1, 128, "bf16")
    idx = sa_synth.random_topk_idx(112, 1, 500, 64)
    args = [dev(x[n], "bf16") for n in ("q", "k", "v")] + [dev(idx, "i32")]
    ref = sa.sa_sparse_attn_fwd(*args, 32, 0.08)
    for _ in range(4):
        assert torch.equal(sa.sa_sparse_attn_fwd(*args, 32, 0.08), ref)
