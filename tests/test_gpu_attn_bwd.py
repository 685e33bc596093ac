"""Sparse-attention backward on the GPU (sa_sparse_attn_bwd) against the float64 oracle
(oracle.reference.sparse_attn_bwd) on the same bf16 inputs and bf16 upstream gradient.

Tolerance: the kernel rounds P and dS to bf16 for the products that build dq, dk and dv
(relative 2^-9 per term) and uses the forward's bf16-rounded output in dout . out, with
float32 accumulation; each gradient tensor is held to max |err| <= 1e-2 * max |grad| of
that tensor (a bf16-level relative error on the largest entries)."""

import numpy as np
import pytest

import oracle.reference as orc
import sa_synth
import long_context_sparse_13_amd as sa
from tests.gpu_util import dev, host, note

pytestmark = pytest.mark.gpu

REL = 1e-2


def _run(x, idx, window, scale, seed):
    import torch
    B, T, Hq, D = x["q"].shape
    dout = sa_synth.round_bf16(sa_synth.rng(seed).standard_normal((B, T, Hq, D), dtype=np.float32))
    q, k, v = dev(x["q"], "bf16"), dev(x["k"], "bf16"), dev(x["v"], "bf16")
    idx_d = dev(idx, "i32") if idx is not None else None
    out, lse = sa.sa_sparse_attn_fwd(q, k, v, idx_d, window, scale, return_lse=True)
    dq, dk, dv = sa.sa_sparse_attn_bwd(q, k, v, idx_d, window, scale, out, lse, dev(dout, "bf16"))
    idx_o = idx if idx is not None else np.full((B, T, 1), -1, dtype=np.int32)
    want = orc.sparse_attn_bwd(x["q"], x["k"], x["v"], idx_o, window, scale, dout)
    for name, g, w in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        err = np.abs(host(g) - w).max()
        top = np.abs(w).max()
        print(f"  {name}: max err {err:.3e} of max |grad| {top:.3e} ({err / max(top, 1e-30):.2e})")
        assert err <= REL * max(top, 1e-6), (name, err, top)


@pytest.mark.parametrize("B,T,Hq,Hkv,D,k,W", [(2, 300, 4, 2, 64, 32, 16), (1, 700, 16, 1, 128, 64, 32),
                                              (1, 400, 8, 1, 128, 40, 0)])
def test_bwd_vs_oracle(B, T, Hq, Hkv, D, k, W):
    x = sa_synth.attn_inputs(901 + T, B, T, Hq, Hkv, D, "bf16")
    idx = sa_synth.random_topk_idx(902 + T, B, T, k, junk=True)
    note(f"sparse_attn_bwd B={B} T={T} Hq={Hq} Hkv={Hkv} D={D} k={k} W={W}")
    _run(x, idx, W, D ** -0.5, 903 + T)


def test_bwd_window_only():
    x = sa_synth.attn_inputs(911, 1, 500, 16, 1, 128, "bf16")
    note("sparse_attn_bwd window only T=500 W=128")
    _run(x, None, 128, 128 ** -0.5, 912)


def test_bwd_listed_keys_inside_window_count_once():
    # every listed key lies in the window (or is -1): the window alone decides the result
    T, k, W = 200, 16, 64
    x = sa_synth.attn_inputs(921, 1, T, 4, 1, 64, "bf16")
    idx = np.full((1, T, k), -1, dtype=np.int32)
    for t in range(T):
        idx[0, t, : min(k, t + 1)] = np.arange(t, max(-1, t - k), -1)[: min(k, t + 1)][::-1]
    note("sparse_attn_bwd listed keys inside the window")
    _run(x, idx, W, 0.125, 922)
