"""Helpers of the GPU parity tests: moving seeded host inputs to the device, comparing
selections with the near-tie exemption, and printing what names each case."""

from __future__ import annotations

import sys

import numpy as np

import oracle.reference as orc

BF16_TOL = 2e-2     # max abs error, bf16 storage
F32_TOL = 1e-4      # max abs error, float32
TIE_REL = 1e-5      # k-th / (k+1)-th relative gap below which a row is exempt


def note(msg: str):
    """Name the case before it runs on the GPU (flushed, so it survives a crash)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype == "f32":
        t = t.to(torch.float32)
    elif dtype == "i32":
        t = t.to(torch.int32)
    elif dtype == "fp8":  # E4M3 codes (uint8) viewed as float8_e4m3fn
        assert x.dtype == np.uint8
        t = t.view(torch.float8_e4m3fn)
    return t.cuda()


def host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def row_exempt(scores_row, k: int):
    """None if the row is not exempt (unique answer), else (hi, lo) bounds: every
    position with score > hi must be chosen, none with score < lo."""
    bd = orc.topk_boundary(scores_row, k)
    if bd is None:
        return None
    a, b = bd
    if a != b and (a - b) < TIE_REL * abs(a):
        return (a + TIE_REL * abs(a), b - TIE_REL * abs(b))
    return None


def check_selection(gpu_row, want_row, scores_row, k: int):
    """Bit-exact unless the row is exempt; then check validity.  Returns True if exact."""
    gpu_row = np.asarray(gpu_row)
    want_row = np.asarray(want_row)
    if np.array_equal(gpu_row, want_row):
        return True
    ex = row_exempt(scores_row, k)
    assert ex is not None, f"selection differs on a non-exempt row:\n gpu={gpu_row}\n want={want_row}"
    hi, lo = ex
    sel = gpu_row[gpu_row >= 0]
    assert sel.shape[0] == min(k, len(scores_row))
    assert np.unique(sel).shape[0] == sel.shape[0]
    assert (np.diff(sel) > 0).all()
    s = np.asarray(scores_row)
    must = np.flatnonzero(s > hi)
    assert np.isin(must, sel).all()
    assert (s[sel] >= lo).all()
    return False
