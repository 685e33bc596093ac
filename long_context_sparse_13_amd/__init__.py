"""Python binding of libsa (causal sparse attention for MI355X / gfx950).

A thin ctypes layer over the C ABI declared in ``include/sa.h``: each ``sa_*`` function
here has the name of the C entry point it calls, checks that the tensors are CUDA (HIP)
tensors of the expected dtype, allocates the outputs with torch when they are not given,
and passes raw device pointers plus torch's current stream.  Every step of the
computation runs in the library's HIP kernels; there is no fallback: if ``libsa.so`` is
missing or fails to load, every call raises.

Build the library with ``python -m long_context_sparse_13_amd.build``.
"""

from __future__ import annotations

import ctypes
import os
import re

__all__ = [
    "SAError", "lib", "library_path", "declared_symbols",
    "sa_indexer_scores", "sa_topk_select", "sa_sparse_attn_fwd", "sa_sparse_attn_fwd_rows",
    "sa_graph_attn_fwd",
    "sa_block_meanpool", "sa_sparse_decode", "sa_sparse_decode_workspace",
    "sa_sparse_decode_auto_splits", "sa_sparse_decode_noalloc",
    "sa_sparse_decode_noalloc_max_scratch", "sa_version",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_HEADER = os.path.join(os.path.dirname(_HERE), "include", "sa.h")
SA_F32, SA_BF16, SA_FP8_E4M3 = 0, 1, 2

_c_void_p, _c_int, _c_int64, _c_float, _c_size_t = (
    ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t)

_SIGS = {
    "sa_indexer_scores": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int,
                                   _c_int, _c_int, _c_int, _c_void_p, _c_int64, _c_void_p]),
    "sa_topk_select": (_c_int, [_c_void_p, _c_int64, _c_int, _c_int, _c_int, _c_int, _c_int,
                                _c_void_p, _c_void_p]),
    "sa_indexer_topk": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int,
                                 _c_int, _c_int, _c_int, _c_int, _c_void_p, _c_void_p, _c_size_t,
                                 _c_void_p]),
    "sa_indexer_topk_workspace": (_c_size_t, [_c_int] * 7),
    "sa_sparse_attn_fwd": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int,
                                    _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _c_int,
                                    _c_void_p, _c_void_p, _c_void_p]),
    "sa_sparse_attn_fwd_rows": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int,
                                         _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                         _c_float, _c_int, _c_int, _c_int, _c_void_p, _c_void_p,
                                         _c_void_p]),
    "sa_sparse_attn_bwd": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int,
                                    _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _c_int,
                                    _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                    _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "sa_sparse_attn_bwd_workspace": (_c_size_t, [_c_int] * 7),
    "sa_graph_attn_fwd": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_float, _c_int,
                                   _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_void_p,
                                   _c_void_p, _c_void_p]),
    "sa_block_meanpool": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                   _c_int, _c_void_p, _c_void_p]),
    "sa_sparse_decode": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int,
                                  _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                  _c_float, _c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                  _c_size_t, _c_void_p]),
    "sa_sparse_decode_noalloc": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                          _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                          _c_int, _c_int, _c_float, _c_int, _c_void_p, _c_void_p,
                                          _c_void_p, _c_void_p]),
    "sa_sparse_decode_noalloc_max_scratch": (_c_size_t, []),
    "sa_sparse_decode_workspace": (_c_size_t, [_c_int] * 9),
    "sa_sparse_decode_auto_splits": (_c_int, [_c_int] * 6),
    "sa_cmp_attn_fwd": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int,
                                 _c_int, _c_int, _c_float, _c_int, _c_void_p, _c_void_p,
                                 _c_void_p, _c_size_t, _c_void_p]),
    "sa_cmp_attn_workspace": (_c_size_t, [_c_int] * 5),
    "sa_block_select": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                 _c_int, _c_int, _c_int, _c_int, _c_int, _c_void_p, _c_void_p,
                                 _c_size_t, _c_void_p]),
    "sa_block_select_workspace": (_c_size_t, [_c_int] * 7),
    "sa_block_meanpool_bf16": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int,
                                        _c_int, _c_int, _c_void_p, _c_void_p]),
    "sa_nsa_decode_branch": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int,
                                      _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                                      _c_int, _c_void_p, _c_void_p, _c_int, _c_void_p, _c_size_t,
                                      _c_void_p]),
    "sa_nsa_decode_branch_workspace": (_c_size_t, [_c_int] * 5),
    "sa_nsa_decode_cmp_win": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                       _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_int, _c_float, _c_int, _c_void_p, _c_void_p, _c_void_p,
                                       _c_void_p, _c_int, _c_int, _c_void_p, _c_size_t,
                                       _c_void_p]),
    "sa_nsa_decode_cmp_win_workspace": (_c_size_t, [_c_int] * 6),
    "sa_nsa_combine": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int,
                                _c_int, _c_int, _c_int, _c_void_p, _c_void_p]),
    "sa_status_str": (ctypes.c_char_p, [_c_int]),
    "sa_last_error": (ctypes.c_char_p, []),
    "sa_version": (_c_int, []),
}

_lib = None


class SAError(RuntimeError):
    """A libsa call returned an error status."""

    def __init__(self, fn: str, status: int, name: str, detail: str):
        super().__init__(f"{fn} failed: {name}: {detail}")
        self.status = status
        self.name = name
        self.detail = detail


def library_path() -> str:
    return os.environ.get("SA_LIBRARY", os.path.join(_HERE, "libsa.so"))


def lib() -> ctypes.CDLL:
    """Load libsa.so (once).  Raises if it is missing: there is no fallback path."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"libsa.so not found at {path}; build it with "
                               "`python -m long_context_sparse_13_amd.build`")
        L = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def declared_symbols() -> list[str]:
    """Names of the functions include/sa.h declares."""
    with open(_HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z0-9_]+)\s*\(", text)))


def sa_version() -> int:
    return lib().sa_version()


def _check(fn: str, rc: int):
    if rc != 0:
        L = lib()
        raise SAError(fn, rc, L.sa_status_str(rc).decode(), L.sa_last_error().decode())


# ------------------------------------------------------------------------ marshalling
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SA_BF16
    if t.dtype == torch.float32:
        return SA_F32
    if t.dtype == torch.float8_e4m3fn:
        return SA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16, float32 or float8_e4m3fn)")


def _dev(t, name: str, dtype=None):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _shape(t, name: str, *dims):
    """Raise ValueError unless t.shape matches dims (None matches any extent)."""
    if t is None:
        return
    if len(t.shape) != len(dims) or any(d is not None and int(e) != int(d)
                                        for e, d in zip(t.shape, dims)):
        want = "[" + ", ".join("*" if d is None else str(d) for d in dims) + "]"
        raise ValueError(f"{name} has shape {list(t.shape)}, expected {want}")


def _same_device(name: str, ref, *ts):
    for t in ts:
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name}: every tensor must be on {ref.device}, got {t.device}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


# ------------------------------------------------------------------------ entry points
def sa_indexer_scores(qi, ki, w, row_begin: int = 0, row_end: int | None = None,
                      scores=None, ld: int | None = None):
    """scores[b, r, s] = Σ_h w[h]·ReLU(qi[b,t,h]·ki[b,s]) for t = row_begin + r, s ≤ t.

    qi [B,T,H_I,D_I], ki [B,T,D_I] (bf16, f32 or float8_e4m3fn), w [H_I] f32.  Returns scores
    [B, row_end-row_begin, ld] f32 (entries s > t untouched / uninitialised)."""
    torch = _torch()
    _dev(qi, "qi"); _dev(ki, "ki", qi.dtype); _dev(w, "w", torch.float32)
    _shape(qi, "qi", None, None, None, None)
    B, T, H, DI = qi.shape
    _shape(ki, "ki", B, T, DI); _shape(w, "w", H)
    row_end = T if row_end is None else row_end
    ld = ld if ld is not None else ((row_end + 3) // 4) * 4
    R = row_end - row_begin
    if scores is None:
        scores = torch.empty((B, R, ld), dtype=torch.float32, device=qi.device)
    _dev(scores, "scores", torch.float32)
    _shape(scores, "scores", B, R, None)
    if ld > scores.shape[2]:
        raise ValueError(f"ld={ld} exceeds the scores row length {scores.shape[2]}")
    _same_device("sa_indexer_scores", qi, ki, w, scores)
    rc = lib().sa_indexer_scores(_p(qi), _p(ki), _p(w), B, T, H, DI, _dtype_code(qi), row_begin,
                                 row_end, _p(scores), ld, _stream(qi.device))
    _check("sa_indexer_scores", rc)
    return scores


def sa_topk_select(scores, k: int, T: int, row_begin: int = 0, row_end: int | None = None,
                   idx=None, ld: int | None = None):
    """idx[b, t, :k] for rows [row_begin, row_end): top-k positions, ascending, -1 padded.
    ``scores`` is [B, row_end-row_begin, ld] f32; ``idx`` is [B, T, k] int32."""
    torch = _torch()
    _dev(scores, "scores", torch.float32)
    _shape(scores, "scores", None, None, None)
    B, R, ld0 = scores.shape
    ld = ld0 if ld is None else ld
    row_end = row_begin + R if row_end is None else row_end
    if row_end - row_begin != R:
        raise ValueError(f"scores holds {R} rows but row_end - row_begin = {row_end - row_begin}")
    if ld > ld0:
        raise ValueError(f"ld={ld} exceeds the scores row length {ld0}")
    if idx is None:
        idx = torch.full((B, T, k), -1, dtype=torch.int32, device=scores.device)
    _dev(idx, "idx", torch.int32)
    _shape(idx, "idx", B, T, k)
    _same_device("sa_topk_select", scores, idx)
    rc = lib().sa_topk_select(_p(scores), ld, B, T, row_begin, row_end, k, _p(idx),
                              _stream(scores.device))
    _check("sa_topk_select", rc)
    return idx


def sa_indexer_topk_workspace(B, T, H_I, D_I, row_begin, row_end, k) -> int:
    return int(lib().sa_indexer_topk_workspace(B, T, H_I, D_I, row_begin, row_end, k))


def sa_indexer_topk(qi, ki, w, k: int, row_begin: int = 0, row_end: int | None = None,
                    idx=None, workspace=None):
    """Fused indexer + top-k: the idx rows [row_begin, row_end) that sa_indexer_scores
    followed by sa_topk_select would write, without the score matrix.  qi [B,T,H_I,D_I],
    ki [B,T,D_I] bf16, w [H_I] f32; ``idx`` [B,T,k] int32; ``workspace`` (uint8, no
    initialisation needed) is allocated when not given."""
    torch = _torch()
    _dev(qi, "qi"); _dev(ki, "ki", qi.dtype); _dev(w, "w", torch.float32)
    _shape(qi, "qi", None, None, None, None)
    B, T, H, DI = qi.shape
    _shape(ki, "ki", B, T, DI); _shape(w, "w", H)
    row_end = T if row_end is None else row_end
    need = sa_indexer_topk_workspace(B, T, H, DI, row_begin, row_end, k)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=qi.device)
    _dev(workspace, "workspace", torch.uint8)
    if idx is None:
        idx = torch.full((B, T, k), -1, dtype=torch.int32, device=qi.device)
    _dev(idx, "idx", torch.int32)
    _shape(idx, "idx", B, T, k)
    _same_device("sa_indexer_topk", qi, ki, w, idx, workspace)
    rc = lib().sa_indexer_topk(_p(qi), _p(ki), _p(w), B, T, H, DI, _dtype_code(qi), row_begin,
                               row_end, k, _p(idx), _p(workspace), workspace.numel(),
                               _stream(qi.device))
    _check("sa_indexer_topk", rc)
    return idx


def _attn_shapes(q, k, v, idx):
    """(B, T, Hq, D, Hkv, topk) of an attention call, after checking that k and v are
    [B,T,Hkv,D] with Hq a multiple of Hkv and idx (if any) is [B,T,topk] int32."""
    torch = _torch()
    _shape(q, "q", None, None, None, None)
    B, T, Hq, D = q.shape
    _shape(k, "k", B, T, None, D)
    Hkv = k.shape[2]
    _shape(v, "v", B, T, Hkv, D)
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    topk = 0
    if idx is not None:
        _dev(idx, "idx", torch.int32)
        _shape(idx, "idx", B, T, None)
        topk = idx.shape[-1]
    return B, T, Hq, D, Hkv, topk


def sa_sparse_attn_fwd(q, k, v, idx, window: int, scale: float, out=None, lse=None,
                       return_lse: bool = False):
    """O over S_t = idx[t] ∪ window; q [B,T,Hq,D], k/v [B,T,Hkv,D], idx [B,T,topk] int32
    (or None with topk = 0).  Returns out (and lse [B,Hq,T] f32 if asked)."""
    torch = _torch()
    _dev(q, "q"); _dev(k, "k", q.dtype); _dev(v, "v", q.dtype)
    B, T, Hq, D, Hkv, topk = _attn_shapes(q, k, v, idx)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    _shape(out, "out", B, T, Hq, D)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        _shape(lse, "lse", B, Hq, T)
    _same_device("sa_sparse_attn_fwd", q, k, v, idx, out, lse)
    rc = lib().sa_sparse_attn_fwd(_p(q), _p(k), _p(v), _p(idx), B, T, Hq, Hkv, D, topk, window,
                                  float(scale), _dtype_code(q), _p(out), _p(lse),
                                  _stream(q.device))
    _check("sa_sparse_attn_fwd", rc)
    return (out, lse) if return_lse else out


def sa_sparse_attn_fwd_rows(q, k, v, idx, window: int, scale: float, row_begin: int,
                            row_end: int, out, lse=None):
    """sa_sparse_attn_fwd for the query rows [row_begin, row_end) only, into the full-size
    out (and lse); other rows are not touched."""
    torch = _torch()
    _dev(q, "q"); _dev(k, "k", q.dtype); _dev(v, "v", q.dtype); _dev(out, "out", q.dtype)
    B, T, Hq, D, Hkv, topk = _attn_shapes(q, k, v, idx)
    _shape(out, "out", B, T, Hq, D)
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        _shape(lse, "lse", B, Hq, T)
    _same_device("sa_sparse_attn_fwd_rows", q, k, v, idx, out, lse)
    rc = lib().sa_sparse_attn_fwd_rows(_p(q), _p(k), _p(v), _p(idx), B, T, Hq, Hkv, D, topk,
                                       window, float(scale), _dtype_code(q), row_begin, row_end,
                                       _p(out), _p(lse), _stream(q.device))
    _check("sa_sparse_attn_fwd_rows", rc)
    return out


def sa_graph_attn_fwd(cq, ck, v, bias, tau: float, local: int, n_pow2: int, out=None,
                      return_lse: bool = False):
    """Fixed-graph distance attention; cq/ck [B,T,H,3], v [B,T,H,D] (same dtype), bias [H] f32."""
    torch = _torch()
    _dev(cq, "cq", v.dtype); _dev(ck, "ck", v.dtype); _dev(v, "v"); _dev(bias, "bias", torch.float32)
    _shape(v, "v", None, None, None, None)
    B, T, H, D = v.shape
    _shape(cq, "cq", B, T, H, 3); _shape(ck, "ck", B, T, H, 3); _shape(bias, "bias", H)
    if out is None:
        out = torch.empty_like(v)
    _dev(out, "out", v.dtype)
    _shape(out, "out", B, T, H, D)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=v.device) if return_lse else None
    _same_device("sa_graph_attn_fwd", v, cq, ck, bias, out)
    rc = lib().sa_graph_attn_fwd(_p(cq), _p(ck), _p(v), _p(bias), float(tau), B, T, H, D, local,
                                 n_pow2, _dtype_code(v), _p(out), _p(lse), _stream(v.device))
    _check("sa_graph_attn_fwd", rc)
    return (out, lse) if return_lse else out


def sa_block_meanpool(kcache, lens, block: int, kbar=None):
    """kbar [B, Lmax//block, Hkv, D] f32 of complete blocks (others untouched)."""
    torch = _torch()
    _dev(kcache, "kcache"); _dev(lens, "lens", torch.int32)
    _shape(kcache, "kcache", None, None, None, None)
    B, Lmax, Hkv, D = kcache.shape
    _shape(lens, "lens", B)
    if kbar is None:
        kbar = torch.zeros((B, Lmax // block, Hkv, D), dtype=torch.float32, device=kcache.device)
    _dev(kbar, "kbar", torch.float32)
    _shape(kbar, "kbar", B, Lmax // block, Hkv, D)
    _same_device("sa_block_meanpool", kcache, lens, kbar)
    rc = lib().sa_block_meanpool(_p(kcache), _p(lens), B, Lmax, Hkv, D, block,
                                 _dtype_code(kcache), _p(kbar), _stream(kcache.device))
    _check("sa_block_meanpool", rc)
    return kbar


def sa_sparse_decode_workspace(B, Lmax, Hq, Hkv, D, block, top_blocks, window, n_splits=0) -> int:
    return int(lib().sa_sparse_decode_workspace(B, Lmax, Hq, Hkv, D, block, top_blocks, window,
                                                n_splits))


def sa_sparse_decode_auto_splits(B, Lmax, Hkv, block, top_blocks, window) -> int:
    return int(lib().sa_sparse_decode_auto_splits(B, Lmax, Hkv, block, top_blocks, window))


def sa_sparse_decode(q, kcache, vcache, kbar, lens, block: int, top_blocks: int, window: int,
                     scale: float, n_splits: int = 0, workspace=None, out=None,
                     return_lse: bool = False, return_sel: bool = False):
    """One block-selected decode step.  q [B,Hq,D] bf16; caches [B,Lmax,Hkv,D] bf16;
    kbar from sa_block_meanpool; lens [B] int32.  ``workspace`` (uint8, zero-filled before
    its first use) is allocated when not given.  Returns out [, lse] [, sel]."""
    torch = _torch()
    _dev(q, "q"); _dev(kcache, "kcache", q.dtype); _dev(vcache, "vcache", q.dtype)
    _dev(kbar, "kbar", torch.float32); _dev(lens, "lens", torch.int32)
    _shape(q, "q", None, None, None)
    B, Hq, D = q.shape
    _shape(kcache, "kcache", B, None, None, D)
    _, Lmax, Hkv, _ = kcache.shape
    _shape(vcache, "vcache", B, Lmax, Hkv, D)
    _shape(kbar, "kbar", B, Lmax // block, Hkv, D)
    _shape(lens, "lens", B)
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    need = sa_sparse_decode_workspace(B, Lmax, Hq, Hkv, D, block, top_blocks, window, n_splits)
    if workspace is None:
        workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace", torch.uint8)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    _shape(out, "out", B, Hq, D)
    _same_device("sa_sparse_decode", q, kcache, vcache, kbar, lens, workspace, out)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if return_lse else None
    sel = (torch.empty((B, Hkv, top_blocks), dtype=torch.int32, device=q.device)
           if return_sel else None)
    rc = lib().sa_sparse_decode(_p(q), _p(kcache), _p(vcache), _p(kbar), _p(lens), B, Lmax, Hq,
                                Hkv, D, block, top_blocks, window, n_splits, float(scale),
                                _dtype_code(q), _p(out), _p(lse), _p(sel), _p(workspace),
                                workspace.numel(), _stream(q.device))
    _check("sa_sparse_decode", rc)
    res = [out]
    if return_lse:
        res.append(lse)
    if return_sel:
        res.append(sel)
    return res[0] if len(res) == 1 else tuple(res)


def sa_sparse_decode_noalloc_max_scratch() -> int:
    return int(lib().sa_sparse_decode_noalloc_max_scratch())


def sa_sparse_decode_noalloc(q, kcache, vcache, kbar, lens, block: int, top_blocks: int,
                             window: int, scale: float, n_splits: int = 0, out=None, lse=None,
                             sel=None, return_lse: bool = False, return_sel: bool = False):
    """sa_sparse_decode with the library's per-GPU scratch instead of a workspace: the C
    entry point allocates nothing (outputs are allocated here when not given).  Calls that
    overlap in time on one GPU race on the scratch."""
    torch = _torch()
    _dev(q, "q"); _dev(kcache, "kcache", q.dtype); _dev(vcache, "vcache", q.dtype)
    _dev(kbar, "kbar", torch.float32); _dev(lens, "lens", torch.int32)
    _shape(q, "q", None, None, None)
    B, Hq, D = q.shape
    _shape(kcache, "kcache", B, None, None, D)
    _, Lmax, Hkv, _ = kcache.shape
    _shape(vcache, "vcache", B, Lmax, Hkv, D)
    _shape(kbar, "kbar", B, Lmax // block, Hkv, D)
    _shape(lens, "lens", B)
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    _shape(out, "out", B, Hq, D)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        _shape(lse, "lse", B, Hq)
    if return_sel and sel is None:
        sel = torch.empty((B, Hkv, top_blocks), dtype=torch.int32, device=q.device)
    if sel is not None:
        _dev(sel, "sel", torch.int32)
        _shape(sel, "sel", B, Hkv, top_blocks)
    _same_device("sa_sparse_decode_noalloc", q, kcache, vcache, kbar, lens, out, lse, sel)
    rc = lib().sa_sparse_decode_noalloc(_p(q), _p(kcache), _p(vcache), _p(kbar), _p(lens), B,
                                        Lmax, Hq, Hkv, D, block, top_blocks, window, n_splits,
                                        float(scale), _dtype_code(q), _p(out), _p(lse), _p(sel),
                                        _stream(q.device))
    _check("sa_sparse_decode_noalloc", rc)
    res = [out]
    if return_lse:
        res.append(lse)
    if return_sel:
        res.append(sel)
    return res[0] if len(res) == 1 else tuple(res)


# ------------------------------------------------------------------------ NSA branches
def sa_cmp_attn_workspace(B, T, Hkv, D, block) -> int:
    return int(lib().sa_cmp_attn_workspace(B, T, Hkv, D, block))


def sa_cmp_attn_fwd(q, kbar, vbar, block: int, scale: float, out=None, lse=None,
                    workspace=None, want_lse: bool = False):
    """Compressed branch: q [B,T,Hq,D] bf16 over the complete-block means kbar, vbar
    [B,T/block,Hkv,D] f32.  Returns out (and lse [B,Hq,T] f32 when asked)."""
    torch = _torch()
    _dev(q, "q"); _dev(kbar, "kbar", torch.float32); _dev(vbar, "vbar", torch.float32)
    _shape(q, "q", None, None, None, None)
    B, T, Hq, D = q.shape
    _shape(kbar, "kbar", B, T // block, None, D)
    Hkv = kbar.shape[2]
    _shape(vbar, "vbar", B, T // block, Hkv, D)
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    _shape(out, "out", B, T, Hq, D)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        _shape(lse, "lse", B, Hq, T)
    if workspace is None:
        workspace = torch.empty(max(sa_cmp_attn_workspace(B, T, Hkv, D, block), 256),
                                dtype=torch.uint8, device=q.device)
    rc = lib().sa_cmp_attn_fwd(_p(q), _p(kbar), _p(vbar), B, T, Hq, Hkv, D, block, float(scale),
                               _dtype_code(q), _p(out), _p(lse), _p(workspace),
                               workspace.numel(), _stream(q.device))
    _check("sa_cmp_attn_fwd", rc)
    return (out, lse) if want_lse else out


def sa_block_select_workspace(B, T, Hkv, D, block, row_begin, row_end) -> int:
    return int(lib().sa_block_select_workspace(B, T, Hkv, D, block, row_begin, row_end))


def sa_block_select(q, kbar, block: int, top_blocks: int, row_begin: int = 0,
                    row_end: int | None = None, idx=None, workspace=None):
    """Top blocks per query row by sum_h q_h . kbar_j, written as token lists
    idx [B, T, top_blocks*block] int32 (rows [row_begin, row_end)), the chosen blocks
    j_0 < j_1 < ... interleaved: idx[b, t, e*top_blocks + i] = j_i*block + e, -1 where
    block i does not exist."""
    torch = _torch()
    _dev(q, "q"); _dev(kbar, "kbar", torch.float32)
    _shape(q, "q", None, None, None, None)
    B, T, Hq, D = q.shape
    _shape(kbar, "kbar", B, T // block, None, D)
    Hkv = kbar.shape[2]
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    row_end = T if row_end is None else row_end
    if idx is None:
        idx = torch.full((B, T, top_blocks * block), -1, dtype=torch.int32, device=q.device)
    _dev(idx, "idx", torch.int32)
    _shape(idx, "idx", B, T, top_blocks * block)
    if workspace is None:
        workspace = torch.empty(max(sa_block_select_workspace(B, T, Hkv, D, block, row_begin,
                                                              row_end), 256),
                                dtype=torch.uint8, device=q.device)
    rc = lib().sa_block_select(_p(q), _p(kbar), B, T, Hq, Hkv, D, block, top_blocks,
                               _dtype_code(q), row_begin, row_end, _p(idx), _p(workspace),
                               workspace.numel(), _stream(q.device))
    _check("sa_block_select", rc)
    return idx


def sa_nsa_combine(o_cmp, o_slc, o_win, gates, out=None):
    """out = g0*o_cmp + g1*o_slc + g2*o_win; gates [B,T,Hq,3] f32."""
    torch = _torch()
    _dev(o_cmp, "o_cmp"); _dev(o_slc, "o_slc", o_cmp.dtype); _dev(o_win, "o_win", o_cmp.dtype)
    _dev(gates, "gates", torch.float32)
    _shape(o_cmp, "o_cmp", None, None, None, None)
    B, T, Hq, D = o_cmp.shape
    _shape(o_slc, "o_slc", B, T, Hq, D); _shape(o_win, "o_win", B, T, Hq, D)
    _shape(gates, "gates", B, T, Hq, 3)
    if out is None:
        out = torch.empty_like(o_cmp)
    _dev(out, "out", o_cmp.dtype)
    _shape(out, "out", B, T, Hq, D)
    rc = lib().sa_nsa_combine(_p(o_cmp), _p(o_slc), _p(o_win), _p(gates), B, T, Hq, D,
                              _dtype_code(o_cmp), _p(out), _stream(o_cmp.device))
    _check("sa_nsa_combine", rc)
    return out


def sa_block_meanpool_bf16(kcache, lens, block: int, kbar=None):
    """Block means rounded to bf16: [B, Lmax//block, Hkv, D] (complete blocks only)."""
    torch = _torch()
    _dev(kcache, "kcache"); _dev(lens, "lens", torch.int32)
    _shape(kcache, "kcache", None, None, None, None)
    B, Lmax, Hkv, D = kcache.shape
    _shape(lens, "lens", B)
    if kbar is None:
        kbar = torch.zeros((B, Lmax // block, Hkv, D), dtype=torch.bfloat16, device=kcache.device)
    _dev(kbar, "kbar", torch.bfloat16)
    _shape(kbar, "kbar", B, Lmax // block, Hkv, D)
    _same_device("sa_block_meanpool_bf16", kcache, lens, kbar)
    rc = lib().sa_block_meanpool_bf16(_p(kcache), _p(lens), B, Lmax, Hkv, D, block,
                                      _dtype_code(kcache), _p(kbar), _stream(kcache.device))
    _check("sa_block_meanpool_bf16", rc)
    return kbar


def sa_nsa_decode_branch_workspace(B, Hq, Hkv, D, n_splits) -> int:
    return int(lib().sa_nsa_decode_branch_workspace(B, Hq, Hkv, D, n_splits))


def sa_nsa_decode_branch(q, keys, vals, lens, kind: int, block: int, window: int, scale: float,
                         out=None, lse=None, want_lse: bool = False, n_splits: int = 1,
                         workspace=None):
    """kind 0: q [B,Hq,D] over the window of the caches keys/vals [B,Lmax,Hkv,D];
    kind 1: over the complete blocks of the bf16 block means [B,Lmax/block,Hkv,D].
    n_splits > 1 needs a zero-filled workspace (allocated here, zeroed, when not given)."""
    torch = _torch()
    _dev(q, "q"); _dev(keys, "keys", q.dtype); _dev(vals, "vals", q.dtype)
    _dev(lens, "lens", torch.int32)
    _shape(q, "q", None, None, None)
    B, Hq, D = q.shape
    _shape(keys, "keys", B, None, None, D)
    _, Lrows, Hkv, _ = keys.shape
    _shape(vals, "vals", B, Lrows, Hkv, D)
    _shape(lens, "lens", B)
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    _shape(out, "out", B, Hq, D)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        _shape(lse, "lse", B, Hq)
    ws_bytes = 0
    if n_splits > 1:
        if workspace is None:
            workspace = torch.zeros(max(sa_nsa_decode_branch_workspace(B, Hq, Hkv, D, n_splits),
                                        256), dtype=torch.uint8, device=q.device)
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    rc = lib().sa_nsa_decode_branch(_p(q), _p(keys), _p(vals), _p(lens), B, Lrows, Hq, Hkv, D,
                                    kind, block, window, float(scale), _dtype_code(q), _p(out),
                                    _p(lse), n_splits, _p(workspace), ws_bytes, _stream(q.device))
    _check("sa_nsa_decode_branch", rc)
    return (out, lse) if want_lse else out


def sa_nsa_decode_cmp_win_workspace(B, Hq, Hkv, D, n_splits_cmp, n_splits_win) -> int:
    return int(lib().sa_nsa_decode_cmp_win_workspace(B, Hq, Hkv, D, n_splits_cmp, n_splits_win))


def sa_nsa_decode_cmp_win(q, kbar16, vbar16, kcache, vcache, lens, block: int, window: int,
                          scale: float, out_cmp=None, out_win=None, lse_cmp=None, lse_win=None,
                          want_lse: bool = False, n_splits_cmp: int = 1, n_splits_win: int = 1,
                          workspace=None):
    """The compressed (over the bf16 block means kbar16/vbar16 [B,Lmax/block,Hkv,D]) and the
    window (over the caches kcache/vcache [B,Lmax,Hkv,D]) branch of sa_nsa_decode_branch in
    one launch; returns (out_cmp, out_win), plus (lse_cmp, lse_win) with want_lse.  Split
    counts above 1 need a zero-filled workspace (allocated here, zeroed, when not given)."""
    torch = _torch()
    _dev(q, "q")
    for t, n in ((kbar16, "kbar16"), (vbar16, "vbar16"), (kcache, "kcache"), (vcache, "vcache")):
        _dev(t, n, q.dtype)
    _dev(lens, "lens", torch.int32)
    _shape(q, "q", None, None, None)
    B, Hq, D = q.shape
    _shape(kcache, "kcache", B, None, None, D)
    _, Lmax, Hkv, _ = kcache.shape
    _shape(vcache, "vcache", B, Lmax, Hkv, D)
    _shape(kbar16, "kbar16", B, Lmax // block, Hkv, D)
    _shape(vbar16, "vbar16", B, Lmax // block, Hkv, D)
    _shape(lens, "lens", B)
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    outs = []
    for o, n in ((out_cmp, "out_cmp"), (out_win, "out_win")):
        if o is None:
            o = torch.empty_like(q)
        _dev(o, n, q.dtype)
        _shape(o, n, B, Hq, D)
        outs.append(o)
    lses = []
    for l, n in ((lse_cmp, "lse_cmp"), (lse_win, "lse_win")):
        if want_lse and l is None:
            l = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
        if l is not None:
            _dev(l, n, torch.float32)
            _shape(l, n, B, Hq)
        lses.append(l)
    need = sa_nsa_decode_cmp_win_workspace(B, Hq, Hkv, D, n_splits_cmp, n_splits_win)
    ws_bytes = 0
    if need > 0:
        if workspace is None:
            workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    rc = lib().sa_nsa_decode_cmp_win(_p(q), _p(kbar16), _p(vbar16), _p(kcache), _p(vcache),
                                     _p(lens), B, Lmax, Hq, Hkv, D, block, window, float(scale),
                                     _dtype_code(q), _p(outs[0]), _p(lses[0]), _p(outs[1]),
                                     _p(lses[1]), n_splits_cmp, n_splits_win, _p(workspace),
                                     ws_bytes, _stream(q.device))
    _check("sa_nsa_decode_cmp_win", rc)
    return (outs[0], outs[1], lses[0], lses[1]) if want_lse else (outs[0], outs[1])


def sa_sparse_attn_bwd_workspace(B, T, Hkv, D, topk, window, rows=0) -> int:
    """Bytes of workspace for the partial-row backward over chunks of `rows` query rows
    (0: all T); 0 when the shapes are outside that path."""
    return int(lib().sa_sparse_attn_bwd_workspace(B, T, Hkv, D, topk, window, rows))


def sa_sparse_attn_bwd(q, k, v, idx, window: int, scale: float, out, lse, dout, dq=None,
                       dk=None, dv=None, workspace=None):
    """Gradients of sa_sparse_attn_fwd: returns (dq [B,T,Hq,D], dk, dv [B,T,Hkv,D]) float32.
    workspace: None (float atomics) or a device uint8 tensor (partial rows summed per key;
    its size sets the chunk of query rows, see sa_sparse_attn_bwd_workspace)."""
    torch = _torch()
    _dev(q, "q"); _dev(k, "k", q.dtype); _dev(v, "v", q.dtype)
    _dev(out, "out", q.dtype); _dev(dout, "dout", q.dtype); _dev(lse, "lse", torch.float32)
    B, T, Hq, D, Hkv, topk = _attn_shapes(q, k, v, idx)
    _shape(out, "out", B, T, Hq, D); _shape(dout, "dout", B, T, Hq, D)
    _shape(lse, "lse", B, Hq, T)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty((B, T, Hq, D), **f32) if dq is None else dq
    dk = torch.empty((B, T, Hkv, D), **f32) if dk is None else dk
    dv = torch.empty((B, T, Hkv, D), **f32) if dv is None else dv
    for t_, n_, shp in ((dq, "dq", (B, T, Hq, D)), (dk, "dk", (B, T, Hkv, D)),
                        (dv, "dv", (B, T, Hkv, D))):
        _dev(t_, n_, torch.float32)
        _shape(t_, n_, *shp)
    _same_device("sa_sparse_attn_bwd", q, k, v, idx, out, lse, dout, dq, dk, dv)
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    rc = lib().sa_sparse_attn_bwd(_p(q), _p(k), _p(v), _p(idx), B, T, Hq, Hkv, D, topk, window,
                                  float(scale), _dtype_code(q), _p(out), _p(lse), _p(dout),
                                  _p(dq), _p(dk), _p(dv), _p(workspace), ws_bytes,
                                  _stream(q.device))
    _check("sa_sparse_attn_bwd", rc)
    return dq, dk, dv
