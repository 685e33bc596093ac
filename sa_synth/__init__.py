"""Seeded synthetic inputs shared by the tests, the bench and the oracle's callers.

This module draws random tensors and nothing else: it holds none of the
attention, indexer, selection or pooling arithmetic.  Both the HIP path (through
its Python binding) and the CPU oracle consume what it returns, so the two sides
always see bit-identical inputs.

Conventions
-----------
* RNG: ``numpy.random.Generator(PCG64(seed))``.  The five workloads use
  seed = 1000 + workload number.
* Normal draws are float32 ``standard_normal``.  Where a tensor is stored as
  bfloat16, the float32 draw is rounded to the nearest bfloat16 (ties to even)
  and returned *as float32 holding a bfloat16-exact value*, so that
  ``torch.from_numpy(x).to(torch.bfloat16)`` is exact and the oracle's float64
  upcast sees the very same number.
* Tensors are token-major and contiguous:
  ``Q[B,T,Hq,D]``, ``K,V[B,T,Hkv,D]``, ``qi[B,T,H_I,D_I]``, ``ki[B,T,D_I]``,
  ``cq,ck[B,T,H,3]``, decode ``q[B,Hq,D]``, caches ``[B,L,Hkv,D]``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "rng",
    "round_bf16",
    "encode_e4m3",
    "normal",
    "prefill_inputs",
    "indexer_inputs",
    "attn_inputs",
    "random_topk_idx",
    "graph_inputs",
    "decode_inputs",
    "integer_indexer_inputs",
    "WORKLOADS",
    "Workload",
]


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept in float32.

    Works on the bit pattern: add 0x7FFF plus the lowest kept bit, then clear the
    16 low bits.  Inputs must be finite (all draws here are).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((bits >> 16) & 1)
    out = ((bits + bias) & 0xFFFF0000).astype(np.uint32)
    return out.view(np.float32).reshape(x.shape)


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """The nearest 8-bit E4M3 code (OCP "fn" variant, ties to even) of each float32
    value, as uint8.  Values must lie within +-448 (every draw here does).  The rounding
    is torch's float32 -> float8_e4m3fn conversion."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.size and float(np.max(np.abs(x))) > 448.0:
        raise ValueError("E4M3 inputs must lie within +-448")
    t = torch.from_numpy(x).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().reshape(x.shape)


def normal(g: np.random.Generator, shape, dtype: str, std: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x = (x * np.float32(std)).astype(np.float32)
    if dtype == "bf16":
        x = round_bf16(x)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return x


def _normal_big(g: np.random.Generator, shape, dtype: str, chunk: int = 1 << 26) -> np.ndarray:
    """Same draws as ``normal`` (one stream, C order) but rounded chunk by chunk
    so that multi-GB caches do not need a second full-size temporary."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        g.standard_normal(size=e - s, dtype=np.float32, out=out[s:e])
        if dtype == "bf16":
            out[s:e] = round_bf16(out[s:e])
    return out.reshape(shape)


def indexer_inputs(seed: int, B: int, T: int, H_I: int, D_I: int, dtype: str, g=None):
    """qi[B,T,H_I,D_I], ki[B,T,D_I] ~ N(0,1) and per-head weights w[H_I] ~ U(0,1).

    ``dtype="fp8"``: the same float32 draws as "f32", returned as E4M3 codes (uint8)."""
    g = g if g is not None else rng(seed)
    if dtype == "fp8":
        qi = encode_e4m3(normal(g, (B, T, H_I, D_I), "f32"))
        ki = encode_e4m3(normal(g, (B, T, D_I), "f32"))
    else:
        qi = normal(g, (B, T, H_I, D_I), dtype)
        ki = normal(g, (B, T, D_I), dtype)
    w = g.uniform(0.0, 1.0, size=H_I).astype(np.float32)
    return {"qi": qi, "ki": ki, "w": w}


def attn_inputs(seed: int, B: int, T: int, Hq: int, Hkv: int, D: int, dtype: str, g=None):
    """Q[B,T,Hq,D], K,V[B,T,Hkv,D] ~ N(0,1)."""
    g = g if g is not None else rng(seed)
    q = normal(g, (B, T, Hq, D), dtype)
    k = normal(g, (B, T, Hkv, D), dtype)
    v = normal(g, (B, T, Hkv, D), dtype)
    return {"q": q, "k": k, "v": v}


def prefill_inputs(seed, B, T, Hq, Hkv, D, H_I, D_I, dtype):
    """Indexer tensors first, then attention tensors, from one stream."""
    g = rng(seed)
    out = indexer_inputs(seed, B, T, H_I, D_I, dtype, g=g)
    out.update(attn_inputs(seed, B, T, Hq, Hkv, D, dtype, g=g))
    return out


def random_topk_idx(seed: int, B: int, T: int, k: int, rows=None, junk: bool = False):
    """A random valid index list per row: min(k, t+1) distinct keys in [0, t],
    ascending, padded with -1.  With ``junk`` some padding slots instead hold
    out-of-range values (> t or < -1), which every consumer must skip."""
    g = rng(seed)
    rows = range(T) if rows is None else rows
    idx = np.full((B, T, k), -1, dtype=np.int32)
    for b in range(B):
        for t in rows:
            n = min(k, t + 1)
            if n == t + 1:
                sel = np.arange(t + 1, dtype=np.int32)
            else:
                sel = np.sort(g.choice(t + 1, size=n, replace=False)).astype(np.int32)
            idx[b, t, :n] = sel
            if junk and n < k:
                pad = k - n
                bad = g.integers(t + 1, t + 1 + 4 * k, size=pad, dtype=np.int64)
                bad[::3] = -7
                idx[b, t, n:] = np.clip(bad, -(2**31), 2**31 - 1).astype(np.int32)
    return idx


def graph_inputs(seed: int, B: int, T: int, H: int, D: int, dtype: str, bias_std: float = 0.1):
    """cq, ck[B,T,H,3] and V[B,T,H,D] ~ N(0,1) in ``dtype``; bias b[H] ~ N(0, bias_std^2) f32."""
    g = rng(seed)
    cq = normal(g, (B, T, H, 3), dtype)
    ck = normal(g, (B, T, H, 3), dtype)
    v = normal(g, (B, T, H, D), dtype)
    bias = (g.standard_normal(size=H, dtype=np.float32) * np.float32(bias_std)).astype(np.float32)
    return {"cq": cq, "ck": ck, "v": v, "bias": bias}


def decode_inputs(seed: int, B: int, L: int, Hq: int, Hkv: int, D: int, dtype: str, lens=None):
    """q[B,Hq,D], K/V caches [B,L,Hkv,D] ~ N(0,1); ``lens`` defaults to L for every sequence."""
    g = rng(seed)
    q = normal(g, (B, Hq, D), dtype)
    kc = _normal_big(g, (B, L, Hkv, D), dtype)
    vc = _normal_big(g, (B, L, Hkv, D), dtype)
    if lens is None:
        lens = np.full(B, L, dtype=np.int32)
    return {"q": q, "kcache": kc, "vcache": vc, "lens": np.asarray(lens, dtype=np.int32)}


def integer_indexer_inputs(seed: int, B: int, T: int, H_I: int, D_I: int, lo: int = -3, hi: int = 3):
    """Integer-valued qi, ki in [lo, hi] with dyadic weights (multiples of 1/8):
    every indexer score is then exact in float32 and float64 alike, and ties are
    plentiful."""
    g = rng(seed)
    qi = g.integers(lo, hi + 1, size=(B, T, H_I, D_I)).astype(np.float32)
    ki = g.integers(lo, hi + 1, size=(B, T, D_I)).astype(np.float32)
    w = (g.integers(1, 9, size=H_I) / 8.0).astype(np.float32)
    return {"qi": qi, "ki": ki, "w": w}


@dataclass(frozen=True)
class Workload:
    """One of the five synthetic workloads, with its sizes and parameters."""

    num: int
    name: str
    params: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return 1000 + self.num


WORKLOADS = {
    1: Workload(1, "topk-prefill-fp32-2k", dict(
        B=1, T=2048, Hq=4, Hkv=1, D=64, H_I=4, D_I=32, dtype="f32",
        topk=256, window=64, scale=1.0 / 8.0)),
    2: Workload(2, "graph-attn-bf16-16k", dict(
        B=1, T=16384, H=8, D=64, dtype="bf16", tau=1.0, local=32, n_pow2=14)),
    3: Workload(3, "dsa-prefill-bf16-64k", dict(
        B=1, T=65536, Hq=16, Hkv=1, D=128, H_I=4, D_I=64, dtype="bf16",
        topk=2048, window=128, scale=1.0 / math.sqrt(128.0))),
    4: Workload(4, "indexcache-FSSS-bf16-128k", dict(
        B=1, T=131072, Hq=16, Hkv=1, D=128, H_I=4, D_I=64, dtype="bf16",
        topk=2048, window=128, scale=1.0 / math.sqrt(128.0), pattern="FSSS")),
    5: Workload(5, "block-sparse-decode-bf16-b32-128k", dict(
        B=32, L=131072, Hq=16, Hkv=1, D=128, dtype="bf16",
        block=64, top_blocks=16, window=512, scale=1.0 / math.sqrt(128.0))),
}


def layer_seed(l: int) -> int:
    """Seed of the fresh Q/K/V of layer ``l`` in the layer-reuse workload."""
    return 1004 + 100 * (l + 1)
