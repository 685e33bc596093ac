"""The C ABI library: loads without a GPU, exports every symbol include/sa.h declares,
and rejects invalid arguments on the host before any GPU work (CPU only)."""

import ctypes
import subprocess

import pytest

import long_context_sparse_13_amd as sa


@pytest.fixture(scope="module")
def L():
    return sa.lib()


def test_every_declared_symbol_is_exported(L):
    names = sa.declared_symbols()
    assert {"sa_indexer_scores", "sa_topk_select", "sa_sparse_attn_fwd", "sa_graph_attn_fwd",
            "sa_sparse_decode", "sa_block_meanpool"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", sa.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported, set(names) - exported


def test_binding_names_match_header():
    for n in sa.declared_symbols():
        if n in ("sa_status_str", "sa_last_error"):
            continue
        assert hasattr(sa, n), n


def test_version_and_status_strings(L):
    assert L.sa_version() == 100
    assert L.sa_status_str(0) == b"SA_OK"
    assert L.sa_status_str(1) == b"SA_ERR_INVALID_ARG"
    assert L.sa_status_str(2) == b"SA_ERR_UNSUPPORTED"
    assert L.sa_status_str(3) == b"SA_ERR_WORKSPACE"
    assert L.sa_status_str(99) == b"SA_ERR_UNKNOWN"


# Fake device addresses: validation fails before any of them is dereferenced.
P = ctypes.c_void_p(1 << 20)
MIS = ctypes.c_void_p((1 << 20) + 4)


def _err(L):
    return L.sa_last_error().decode()


def test_indexer_topk_validation_and_workspace(L):
    f = L.sa_indexer_topk
    ws = L.sa_indexer_topk_workspace
    need = ws(1, 4096, 4, 64, 0, 4096, 256)
    assert need > 0
    assert ws(1, 4096, 4, 64, 0, 4097, 256) == 0                   # row_end > T
    assert ws(1, 4096, 4, 64, 0, 4096, 0) == 0                     # k
    # more rows or longer rows need more workspace
    assert ws(1, 8192, 4, 64, 0, 8192, 256) > need
    assert ws(2, 4096, 4, 64, 0, 4096, 256) > need
    # every case below fails validation, so nothing reaches the GPU
    args = (P, P, P, 1, 4096, 4, 64, 1, 0, 4096, 256, P)
    assert f(*args, None, need, None) == 3
    assert "workspace" in _err(L)
    assert f(*args, P, need - 1, None) == 3
    assert f(P, P, P, 1, 4096, 4, 64, 0, 0, 4096, 256, P, P, need, None) == 2   # f32: two-step path
    assert f(P, P, P, 1, 4096, 3, 64, 1, 0, 4096, 256, P, P, need, None) == 2   # H_I = 3
    assert f(P, P, P, 1, 4096, 4, 48, 1, 0, 4096, 256, P, P, need, None) == 2   # D_I = 48
    assert f(P, P, P, 1, 4096, 4, 64, 1, 0, 4096, 5000, P, P, need, None) == 1  # k too big
    assert f(P, P, P, 1, 4096, 4, 64, 1, 100, 100, 256, P, P, need, None) == 1  # empty rows
    assert f(P, P, None, 1, 4096, 4, 64, 1, 0, 4096, 256, P, P, need, None) == 1
    assert f(P, P, P, 1, 300000, 4, 64, 1, 0, 4096, 256, P, P, need, None) == 2  # T too long
    # E4M3 inputs (dtype 2) take the same MFMA configurations
    assert f(P, P, P, 1, 4096, 3, 64, 2, 0, 4096, 256, P, P, need, None) == 2   # H_I = 3
    assert f(P, P, P, 1, 4096, 4, 64, 2, 0, 4096, 5000, P, P, need, None) == 1  # k too big
    assert f(P, P, P, 1, 4096, 4, 64, 2, 0, 4096, 256, P, None, need, None) == 3
    assert f(P, P, P, 1, 4096, 4, 64, 3, 0, 4096, 256, P, P, need, None) == 1   # dtype


def test_e4m3_accepted_by_the_indexer_only(L):
    # every call fails validation before any launch
    g = L.sa_indexer_scores
    assert g(P, P, P, 1, 64, 3, 64, 2, 0, 64, P, 64, None) == 2    # E4M3 needs MFMA shapes
    assert g(P, P, P, 1, 64, 4, 48, 2, 0, 64, P, 64, None) == 2
    assert g(P, P, P, 1, 64, 4, 64, 2, 0, 64, P, 60, None) == 1    # ld < row_end
    assert "E4M3" in (g(P, P, P, 1, 64, 3, 64, 2, 0, 64, P, 64, None) and _err(L))
    assert L.sa_sparse_attn_fwd(P, P, P, P, 1, 8, 4, 1, 64, 4, 4, 0.1, 2, P, None, None) == 2
    assert "indexer" in _err(L)
    assert L.sa_graph_attn_fwd(P, P, P, P, 1.0, 1, 8, 2, 64, 4, 4, 2, P, None, None) == 2


def test_attn_validation(L):
    f = L.sa_sparse_attn_fwd
    assert f(None, P, P, P, 1, 8, 4, 1, 64, 4, 4, 0.1, 1, P, None, None) == 1
    assert "q is NULL" in _err(L)
    assert f(MIS, P, P, P, 1, 8, 4, 1, 64, 4, 4, 0.1, 1, P, None, None) == 1
    assert "aligned" in _err(L)
    assert f(P, P, P, P, 1, 8, 4, 3, 64, 4, 4, 0.1, 1, P, None, None) == 1      # Hq % Hkv
    assert f(P, P, P, P, 1, 8, 4, 1, 64, 0, 0, 0.1, 1, P, None, None) == 1      # empty selection
    assert f(P, P, P, None, 1, 8, 4, 1, 64, 4, 4, 0.1, 1, P, None, None) == 1   # idx NULL, topk>0
    assert f(P, P, P, P, 1, 8, 4, 1, 96, 4, 4, 0.1, 1, P, None, None) == 2      # D unsupported
    assert f(P, P, P, P, 1, 8, 4, 1, 64, 4, 4, 0.1, 7, P, None, None) == 1      # dtype
    assert f(P, P, P, P, 0, 8, 4, 1, 64, 4, 4, 0.1, 1, P, None, None) == 1      # B
    assert f(P, P, P, P, 1, 8, 128, 1, 64, 4, 4, 0.1, 1, P, None, None) == 2    # G*D too big


def test_attn_rows_validation(L):
    f = L.sa_sparse_attn_fwd_rows
    assert f(P, P, P, P, 1, 8, 4, 1, 64, 4, 4, 0.1, 1, -1, 4, P, None, None) == 1   # row_begin < 0
    assert f(P, P, P, P, 1, 8, 4, 1, 64, 4, 4, 0.1, 1, 5, 4, P, None, None) == 1    # begin > end
    assert f(P, P, P, P, 1, 8, 4, 1, 64, 4, 4, 0.1, 1, 0, 9, P, None, None) == 1    # end > T
    assert "row_begin" in _err(L)
    assert f(P, P, P, P, 1, 8, 4, 1, 96, 4, 4, 0.1, 1, 0, 8, P, None, None) == 2    # D
    assert f(P, P, P, None, 1, 8, 4, 1, 64, 4, 4, 0.1, 1, 0, 8, P, None, None) == 1  # idx NULL


def test_indexer_and_topk_validation(L):
    g = L.sa_indexer_scores
    assert g(P, P, P, 1, 16, 4, 64, 1, 0, 16, P, 15, None) == 1   # ld % 4
    assert g(P, P, P, 1, 16, 4, 64, 1, 0, 17, P, 20, None) == 1   # row_end > T
    assert g(P, P, P, 1, 16, 4, 64, 1, 8, 8, P, 16, None) == 1    # empty row range
    assert g(P, P, P, 1, 16, 4, 60, 1, 0, 16, P, 16, None) == 1   # D_I % 8
    assert g(P, P, P, 1, 16, 64, 128, 1, 0, 16, P, 16, None) == 2  # H_I*D_I too big
    assert g(P, P, None, 1, 16, 4, 64, 1, 0, 16, P, 16, None) == 1
    t = L.sa_topk_select
    assert t(P, 16, 1, 16, 0, 16, 0, P, None) == 1                # k
    assert t(P, 16, 1, 16, 0, 16, 5000, P, None) == 1             # k too big
    assert t(P, 8, 1, 16, 0, 16, 4, P, None) == 1                 # ld < row_end
    assert t(P, 18, 1, 16, 0, 16, 4, P, None) == 1                # ld % 4
    assert t(P, 300000, 1, 300000, 0, 300000, 4, P, None) == 2    # rows too long


def test_graph_meanpool_decode_validation(L):
    gr = L.sa_graph_attn_fwd
    assert gr(P, P, P, P, 1.0, 1, 8, 2, 64, 65, 4, 1, P, None, None) == 1   # local
    assert gr(P, P, P, P, 1.0, 1, 8, 2, 60, 4, 4, 1, P, None, None) == 1    # D % 8
    assert gr(P, P, P, None, 1.0, 1, 8, 2, 64, 4, 4, 1, P, None, None) == 1
    mp = L.sa_block_meanpool
    assert mp(P, P, 1, 256, 1, 128, 48, 1, P, None) == 1                     # block
    d = L.sa_sparse_decode
    args = [P, P, P, P, P, 2, 1024, 16, 1, 128, 64, 16, 512, 0, 0.1, 1, P, None, None]
    ws = L.sa_sparse_decode_workspace(2, 1024, 16, 1, 128, 64, 16, 512, 0)
    assert ws > 0
    assert d(*args, None, ws, None) == 3                                     # no workspace
    assert d(*args, P, ws - 1, None) == 3                                    # too small
    bad = list(args)
    bad[11] = 65                                                             # top_blocks
    assert d(*bad, P, ws, None) == 1
    bad = list(args)
    bad[15] = 0                                                              # f32 decode
    assert d(*bad, P, ws, None) == 2
    assert L.sa_sparse_decode_workspace(2, 1024, 16, 3, 128, 64, 16, 512, 0) == 0
    # the block means of one sequence must span less than 2 GiB: 2^18 blocks x 16 KV heads
    # x 128 dims x 4 bytes is 2 GiB exactly (no launch: the size check comes first)
    big = list(args)
    big[6], big[7], big[8], big[10] = 16 * 262144, 16, 16, 16
    assert d(*big, P, ws, None) == 2
    assert L.sa_sparse_decode_workspace(1, 16 * 262144, 16, 16, 128, 16, 16, 512, 0) == 0
    assert L.sa_sparse_decode_workspace(1, 16 * 262144, 16, 8, 128, 16, 16, 512, 0) > 0


def test_decode_auto_splits(L):
    # two 32-key tiles per wavefront of 4-wavefront splits: |U| = 16*64 + 512 = 1536 keys
    # -> 6 splits; a tiny U or a huge batch caps the splits
    assert L.sa_sparse_decode_auto_splits(32, 131072, 1, 64, 16, 512) == 6
    assert L.sa_sparse_decode_auto_splits(1, 64, 1, 64, 1, 0) == 1
    assert L.sa_sparse_decode_auto_splits(1, 131072, 1, 64, 64, 4096) == 32
    assert L.sa_sparse_decode_auto_splits(1024, 131072, 1, 64, 16, 512) == 1
    assert L.sa_sparse_decode_auto_splits(1024, 131072, 1, 64, 16, 512) == 1


def test_nsa_validation(L):
    # every call fails validation, so nothing reaches the GPU
    ws = L.sa_cmp_attn_workspace(1, 1024, 1, 128, 64)
    assert ws > 0 and L.sa_cmp_attn_workspace(1, 1024, 1, 128, 48) == 0
    c = L.sa_cmp_attn_fwd
    assert c(P, P, P, 1, 1024, 16, 1, 128, 64, 0.1, 0, P, None, P, ws, None) == 2   # f32
    assert c(P, P, P, 1, 1024, 16, 1, 96, 64, 0.1, 1, P, None, P, ws, None) == 2    # D
    assert c(P, P, P, 1, 1024, 16, 1, 128, 48, 0.1, 1, P, None, P, ws, None) == 1   # block
    assert c(P, P, P, 1, 1024, 16, 3, 128, 64, 0.1, 1, P, None, P, ws, None) == 1   # Hq % Hkv
    assert c(P, P, P, 1, 1024, 16, 1, 128, 64, 0.1, 1, P, None, None, ws, None) == 3
    assert c(P, P, P, 1, 1024, 16, 1, 128, 64, 0.1, 1, P, None, P, ws - 1, None) == 3
    assert c(P, P, P, 1, 1024, 32, 1, 128, 64, 0.1, 1, P, None, P, ws, None) == 2   # 32 heads/group
    s = L.sa_block_select
    w2 = L.sa_block_select_workspace(1, 1024, 1, 128, 64, 0, 1024)
    assert w2 > 0 and L.sa_block_select_workspace(1, 1024, 1, 128, 64, 0, 1025) == 0
    assert s(P, P, 1, 1024, 16, 1, 128, 64, 65, 1, 0, 1024, P, P, w2, None) == 1    # top_blocks
    assert s(P, P, 1, 1024, 16, 1, 128, 64, 16, 1, 5, 5, P, P, w2, None) == 1       # rows
    assert s(P, P, 1, 1024, 16, 1, 128, 64, 16, 2, 0, 1024, P, P, w2, None) == 2    # E4M3
    assert s(P, P, 1, 1024, 16, 1, 128, 64, 16, 1, 0, 1024, P, None, w2, None) == 3
    big = L.sa_block_select_workspace(1, 300000, 1, 128, 64, 0, 64)
    assert s(P, P, 1, 300000, 16, 1, 128, 64, 16, 1, 0, 64, P, P, big, None) == 2   # > 4096 blocks
    m = L.sa_nsa_combine
    assert m(P, P, P, P, 1, 64, 16, 128, 0, P, None) == 2                          # f32
    assert m(P, P, P, P, 1, 64, 16, 12, 1, P, None) == 1                           # D % 8
    assert m(P, P, None, P, 1, 64, 16, 128, 1, P, None) == 1
    d = L.sa_nsa_decode_branch
    assert d(P, P, P, P, 2, 1024, 16, 1, 128, 2, 64, 512, 0.1, 1, P, None, 1, None, 0, None) == 1   # kind
    assert d(P, P, P, P, 2, 1024, 16, 1, 128, 0, 64, -1, 0.1, 1, P, None, 1, None, 0, None) == 1    # window
    assert d(P, P, P, P, 2, 1024, 16, 1, 128, 0, 64, 512, 0.1, 0, P, None, 1, None, 0, None) == 2   # f32
    assert d(P, P, P, P, 2, 1024, 16, 1, 96, 0, 64, 512, 0.1, 1, P, None, 1, None, 0, None) == 2    # D
    assert d(P, P, P, None, 2, 1024, 16, 1, 128, 0, 64, 512, 0.1, 1, P, None, 1, None, 0, None) == 1
    assert d(P, P, P, P, 2, 1024, 16, 1, 128, 0, 64, 512, 0.1, 1, P, None, 0, None, 0, None) == 1   # splits
    assert d(P, P, P, P, 2, 1024, 16, 1, 128, 0, 64, 512, 0.1, 1, P, None, 65, None, 0, None) == 1
    wsd = L.sa_nsa_decode_branch_workspace(2, 16, 1, 128, 4)
    assert wsd > 0 and L.sa_nsa_decode_branch_workspace(2, 16, 1, 96, 4) == 0
    assert d(P, P, P, P, 2, 1024, 16, 1, 128, 0, 64, 512, 0.1, 1, P, None, 4, None, 0, None) == 3   # no workspace
    assert d(P, P, P, P, 2, 1024, 16, 1, 128, 0, 64, 512, 0.1, 1, P, None, 4, P, wsd - 1, None) == 3
    c = L.sa_nsa_decode_cmp_win
    cw = lambda Lmax=1024, D=128, block=64, window=512, dt=1, ns=(1, 1), ws=None, n=0, lens=P: c(
        P, P, P, P, P, lens, 2, Lmax, 16, 1, D, block, window, 0.1, dt, P, None, P, None, ns[0],
        ns[1], ws, n, None)
    assert cw(block=48) == 1                                                         # block
    assert cw(Lmax=32) == 1                                                          # no block
    assert cw(window=-1) == 1
    assert cw(dt=0) == 2                                                             # f32
    assert cw(D=96) == 2
    assert cw(lens=None) == 1
    assert cw(ns=(0, 1)) == 1 and cw(ns=(1, 65)) == 1                                # splits
    wcw = L.sa_nsa_decode_cmp_win_workspace(2, 16, 1, 128, 8, 4)
    assert wcw == wsd + L.sa_nsa_decode_branch_workspace(2, 16, 1, 128, 8)
    assert L.sa_nsa_decode_cmp_win_workspace(2, 16, 1, 128, 1, 1) == 0
    assert L.sa_nsa_decode_cmp_win_workspace(2, 16, 1, 96, 8, 4) == 0
    assert cw(ns=(8, 4)) == 3                                                        # no workspace
    assert cw(ns=(8, 4), ws=P, n=wcw - 1) == 3
    assert cw(ns=(8, 4), ws=MIS, n=wcw) == 1                                         # alignment
    mb = L.sa_block_meanpool_bf16
    assert mb(P, P, 1, 1024, 1, 128, 48, 1, P, None) == 1                              # block
    assert mb(P, P, 1, 1024, 1, 128, 64, 2, P, None) == 2                              # E4M3


def test_bwd_validation_and_workspace(L):
    # every call fails validation before any launch
    q = L.sa_sparse_attn_bwd_workspace
    w1, w2, wall = q(1, 4096, 1, 128, 64, 16, 1), q(1, 4096, 1, 128, 64, 16, 2), q(1, 4096, 1, 128, 64, 16, 0)
    assert 0 < w1 < w2 < wall and q(1, 4096, 1, 128, 64, 16, 4096) == wall
    assert w2 - w1 >= 80 * 4 * 128                      # one row: (topk + window) bf16 rows of 4*D bytes
    assert q(1, 4096, 1, 96, 64, 16, 0) == 0            # D
    assert q(1, 4096, 1, 128, 0, 0, 0) == 0             # empty selection
    assert q(1, (1 << 20) + 1, 1, 128, 64, 16, 1) == 0  # beyond the bucket histogram
    b = L.sa_sparse_attn_bwd
    args = lambda T=4096, Hq=16, D=128, dt=1, lse=P, ws=None, n=0: (
        P, P, P, P, 1, T, Hq, 1, D, 64, 16, 0.1, dt, P, lse, P, P, P, P, ws, n, None)
    assert b(*args(dt=0)) == 2                          # f32
    assert b(*args(D=96)) == 2
    assert b(*args(Hq=32)) == 2                         # 32 heads per group
    assert b(*args(lse=None)) == 1
    assert b(*args(ws=P, n=w1 - 1)) == 3                # smaller than one row
    assert "workspace" in _err(L)
    assert b(*args(ws=MIS, n=wall)) == 1                # alignment
    assert b(*args(T=(1 << 20) + 1, Hq=1, D=64, ws=P, n=1 << 40)) == 2


def test_decode_noalloc_validation(L):
    """The allocation-free decode refuses, on the host, sizes whose workspace exceeds its
    per-GPU scratch, and validates like sa_sparse_decode."""
    f = L.sa_sparse_decode_noalloc
    cap = L.sa_sparse_decode_noalloc_max_scratch()
    assert cap == 16 << 20
    assert L.sa_sparse_decode_workspace(4096, 131072, 16, 1, 128, 64, 16, 512, 64) > cap
    args = (P, P, P, P, P)
    assert f(*args, 4096, 131072, 16, 1, 128, 64, 16, 512, 64, 0.1, 1, P, None, None, None) == 2
    assert "scratch" in _err(L)
    assert f(*args, 2, 1024, 16, 1, 96, 64, 16, 512, 0, 0.1, 1, P, None, None, None) == 2   # D
    assert f(*args, 2, 1024, 16, 3, 128, 64, 16, 512, 0, 0.1, 1, P, None, None, None) == 1  # Hq % Hkv
    assert f(*args, 2, 1024, 16, 1, 128, 64, 0, 512, 0, 0.1, 1, P, None, None, None) == 1   # top_blocks
    assert f(*args, 2, 1024, 16, 1, 128, 64, 16, 512, 65, 0.1, 1, P, None, None, None) == 1  # splits
    assert f(P, P, P, P, P, 2, 1024, 16, 1, 128, 64, 16, 512, 0, 0.1, 0, P, None, None, None) == 2  # f32
    assert f(P, P, MIS, P, P, 2, 1024, 16, 1, 128, 64, 16, 512, 0, 0.1, 1, P, None, None, None) == 1
