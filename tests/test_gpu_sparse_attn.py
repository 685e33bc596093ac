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


def test_window_only_shared_tiles():
    """No index list: the sliding window through the shared-tile kernel (8 tokens of a
    workgroup share each K/V tile), against the oracle: long window, GQA with padded head
    columns and batch 2, a window longer than the sequence, window 1, ragged T."""
    _run(121, 1, 1000, 16, 1, 128, 0, 512, "bf16")
    _run(122, 2, 300, 8, 2, 64, 0, 45, "bf16")
    _run(123, 1, 77, 4, 1, 128, 0, 200, "bf16")
    _run(124, 1, 130, 16, 1, 64, 0, 1, "bf16")
    _run(125, 1, 517, 16, 1, 128, 0, 33, "bf16")


def test_window_only_row_ranges():
    """The shared-tile window over row ranges that start and end inside 8-token groups
    writes what the full call writes, bit for bit (tiles start at multiples of 32 keys
    whatever the range), and leaves the other rows untouched."""
    import torch
    B, T, Hq, Hkv, D, W = 2, 301, 16, 1, 64, 70
    note(f"window-only rows B={B} T={T} W={W}")
    x = sa_synth.attn_inputs(126, B, T, Hq, Hkv, D, "bf16")
    q, k, v = dev(x["q"], "bf16"), dev(x["k"], "bf16"), dev(x["v"], "bf16")
    full, lfull = sa.sa_sparse_attn_fwd(q, k, v, None, W, 0.125, return_lse=True)
    out = torch.full_like(q, 7.0)
    lse = torch.full((B, Hq, T), 7.0, dtype=torch.float32, device="cuda")
    sa.sa_sparse_attn_fwd_rows(q, k, v, None, W, 0.125, 43, 170, out, lse)
    assert bool((out[:, :43] == 7.0).all()) and bool((out[:, 170:] == 7.0).all())
    assert torch.equal(out[:, 43:170], full[:, 43:170])
    for r0, r1 in ((0, 43), (170, 299), (299, 301)):
        sa.sa_sparse_attn_fwd_rows(q, k, v, None, W, 0.125, r0, r1, out, lse)
    assert torch.equal(out, full) and torch.equal(lse, lfull)


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


@pytest.mark.parametrize("dtype,G", [("bf16", 16), ("bf16", 32), ("f32", 4)])
def test_row_ranges(dtype, G):
    """sa_sparse_attn_fwd_rows over ragged row ranges that cover [0, T) writes what the
    full call writes (bit for bit: same kernel, same per-row arithmetic), leaves every row
    outside its range untouched, and matches the oracle; an empty range writes nothing."""
    import torch
    B, T, Hkv, D, topk, W = 2, 301, 1, 64, 24, 16
    Hq = G * Hkv
    note(f"sparse_attn_fwd_rows B={B} T={T} Hq={Hq} D={D} {dtype}")
    x = sa_synth.attn_inputs(171, B, T, Hq, Hkv, D, dtype)
    idx = sa_synth.random_topk_idx(172, B, T, topk, junk=True)
    q, k, v = dev(x["q"], dtype), dev(x["k"], dtype), dev(x["v"], dtype)
    di = dev(idx, "i32")
    full, lfull = sa.sa_sparse_attn_fwd(q, k, v, di, W, 0.125, return_lse=True)
    out = torch.full_like(q, 7.0)
    lse = torch.full((B, Hq, T), 7.0, dtype=torch.float32, device="cuda")
    sa.sa_sparse_attn_fwd_rows(q, k, v, di, W, 0.125, 5, 5, out, lse)     # empty: no change
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())
    sa.sa_sparse_attn_fwd_rows(q, k, v, di, W, 0.125, 40, 177, out, lse)
    assert bool((out[:, :40] == 7.0).all()) and bool((out[:, 177:] == 7.0).all())
    assert bool((lse[:, :, :40] == 7.0).all()) and bool((lse[:, :, 177:] == 7.0).all())
    assert torch.equal(out[:, 40:177], full[:, 40:177])
    for r0, r1 in ((0, 40), (177, 300), (300, 301)):
        sa.sa_sparse_attn_fwd_rows(q, k, v, di, W, 0.125, r0, r1, out, lse)
    assert torch.equal(out, full) and torch.equal(lse, lfull)
    rows = [0, 39, 40, 176, 177, 299, 300]
    O, _ = orc.sparse_attn(x["q"], x["k"], x["v"], idx, W, 0.125, rows)
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    assert np.abs(host(out)[:, rows] - O).max() <= tol


@pytest.mark.slow
def test_mfma_offsets_beyond_32_bits():
    """T = 2^21 + 5 tokens with 16 query heads of dim 128: query, output and index offsets
    pass 2^32 elements (bytes for idx); sampled rows (early, middle, late, last) against the
    oracle's single-row form.  Inputs are drawn on the GPU (seeded), listed keys are distinct
    positions spread over [0, t - W - 1]."""
    import torch
    T, Hq, Hkv, D, topk, W = (1 << 21) + 5, 16, 1, 128, 64, 32
    note(f"sparse_attn T={T} Hq={Hq} D={D} topk={topk} W={W} (offsets past 2^32)")
    g = torch.Generator(device="cuda").manual_seed(181)
    q = torch.randn((1, T, Hq, D), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((1, T, Hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((1, T, Hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    t = torch.arange(T, device="cuda")[:, None]
    j = torch.arange(topk, device="cuda")[None, :]
    key = t - W - 1 - j * torch.clamp((t - W) // (topk + 1), min=1)
    idx = torch.where(key >= 0, key, -1).to(torch.int32)[None].contiguous()
    del t, j, key
    scale = D ** -0.5
    out, lse = sa.sa_sparse_attn_fwd(q, k, v, idx, W, scale, return_lse=True)
    assert (1 * T * Hq * D) > (1 << 32)
    kh, vh = host(k)[0], host(v)[0]
    for r in (0, 100, 70000, T // 2 + 3, T - 2, T - 1):
        o, l = orc.sparse_attn_row(host(q[0, r]), kh, vh, host(idx[0, r]), r, W, scale)
        assert np.abs(host(out[0, r]) - o).max() <= BF16_TOL, r
        assert np.abs(host(lse[0, :, r]) - l).max() <= 2e-3, r


@pytest.mark.slow
def test_mfma_row_offsets_beyond_4gb():
    """T = 2^21 + 3 tokens with 8 KV heads of dim 128: one KV head's rows span more than
    4 GB of bytes, so the kernel addresses rows with 64-bit offsets (below that it uses a
    uniform base plus a 32-bit offset).  Sampled rows of the first and last KV head
    against the oracle's single-row form on that head's keys and values.  Inputs are drawn
    on the GPU (seeded), listed keys are distinct positions spread over [0, t - W - 1]."""
    import torch
    T, Hq, Hkv, D, topk, W = (1 << 21) + 3, 8, 8, 128, 32, 32
    note(f"sparse_attn T={T} Hq={Hq} Hkv={Hkv} D={D} topk={topk} W={W} (row offsets past 4 GB)")
    assert T * Hkv * D * 2 >= (1 << 32)
    g = torch.Generator(device="cuda").manual_seed(183)
    q = torch.randn((1, T, Hq, D), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((1, T, Hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((1, T, Hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    t = torch.arange(T, device="cuda")[:, None]
    j = torch.arange(topk, device="cuda")[None, :]
    key = t - W - 1 - j * torch.clamp((t - W) // (topk + 1), min=1)
    idx = torch.where(key >= 0, key, -1).to(torch.int32)[None].contiguous()
    del t, j, key
    scale = D ** -0.5
    out, lse = sa.sa_sparse_attn_fwd(q, k, v, idx, W, scale, return_lse=True)
    for h in (0, Hkv - 1):  # query head h reads KV head h (one query head per group)
        kh, vh = host(k[0, :, h:h + 1]), host(v[0, :, h:h + 1])
        for r in ((0, 70001, T - 1) if h else (100, T // 2 + 1)):
            o, l = orc.sparse_attn_row(host(q[0, r, h:h + 1]), kh, vh, host(idx[0, r]), r, W, scale)
            assert np.abs(host(out[0, r, h]) - o[0]).max() <= BF16_TOL, (h, r)
            assert abs(float(host(lse[0, h, r])) - l[0]) <= 2e-3, (h, r)
        del kh, vh
