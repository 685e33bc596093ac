"""NSA's branches on the GPU (prefill): the compressed branch (sa_cmp_attn_fwd), block
selection (sa_block_select), the selected and window branches (sa_sparse_attn_fwd on the
selected blocks' tokens / on the window) and the gated combine (sa_nsa_combine), against
the float64 oracle.  Outputs within the bf16 tolerance; selected block sets bit-exact
except rows whose top_blocks-th and next block scores are a near tie (relative 1e-5)."""

import numpy as np
import pytest

import oracle.reference as orc
import sa_synth
import long_context_sparse_13_amd as sa
from tests.gpu_util import BF16_TOL, TIE_REL, dev, host, note

pytestmark = pytest.mark.gpu

LSE_TOL = 2e-3


def _pool(x, T, block):
    import torch
    lens = torch.full((x["q"].shape[0],), T, dtype=torch.int32, device="cuda")
    k, v = dev(x["k"], "bf16"), dev(x["v"], "bf16")
    return sa.sa_block_meanpool(k, lens, block), sa.sa_block_meanpool(v, lens, block), k, v


def _oracle_pool(x, T, block):
    lens = np.full(x["q"].shape[0], T)
    return orc.block_meanpool(x["k"], lens, block), orc.block_meanpool(x["v"], lens, block)


@pytest.mark.parametrize("T,Hq,Hkv,D,block", [(700, 4, 2, 64, 16), (2000, 16, 1, 128, 64),
                                              (333, 8, 1, 128, 32)])
def test_cmp_attn_vs_oracle(T, Hq, Hkv, D, block):
    x = sa_synth.attn_inputs(801 + T, 2, T, Hq, Hkv, D, "bf16")
    note(f"cmp_attn B=2 T={T} Hq={Hq} Hkv={Hkv} D={D} block={block}")
    kbar, vbar, _, _ = _pool(x, T, block)
    out, lse = sa.sa_cmp_attn_fwd(dev(x["q"], "bf16"), kbar, vbar, block, D ** -0.5, want_lse=True)
    ok_, ov_ = _oracle_pool(x, T, block)
    rows = list(range(0, 3 * block)) + list(range(3 * block, T, 7)) + [T - 1]
    want, wl = orc.cmp_attn(x["q"], ok_, ov_, block, D ** -0.5, rows)
    got, gl = host(out), host(lse)
    for r, t in enumerate(rows):
        assert np.abs(got[:, t] - want[:, r]).max() < BF16_TOL, t
        if t + 1 < block:
            assert not got[:, t].any() and np.isneginf(gl[:, :, t]).all()
        else:
            assert np.abs(gl[:, :, t] - wl[:, :, r]).max() < LSE_TOL, t


def _check_blocks(gi, want_sel, q, kbar, block, top, rows):
    """Selected blocks per row: exact, or a near tie at the boundary of the selection."""
    n_exempt = 0
    for r, t in enumerate(rows):
        g = gi[t]
        gb = sorted(set(int(s) // block for s in g if s >= 0))
        wb = sorted(int(j) for j in want_sel[r] if j >= 0)
        toks = orc.block_tokens(np.array(wb + [-1] * (top - len(wb))), block)
        # the library lists the blocks interleaved: token e of the i-th block at e * top + i
        toks = toks.reshape(top, block).T.reshape(-1)
        if gb == wb:
            assert np.array_equal(g, toks), t
            continue
        nfull = (t + 1) // block
        sc = np.zeros(nfull)
        Hkv = kbar.shape[1]
        G = q.shape[1] // Hkv
        for gg in range(Hkv):
            sc += (q[t, gg * G:(gg + 1) * G].astype(np.float64) @ kbar[:nfull, gg].T).sum(axis=0)
        bd = orc.topk_boundary(sc, top)
        assert bd is not None and bd[0] != bd[1] and bd[0] - bd[1] < TIE_REL * abs(bd[0]), t
        n_exempt += 1
    return n_exempt


@pytest.mark.parametrize("T,Hq,Hkv,D,block,top", [(1500, 16, 1, 128, 64, 4), (1200, 4, 2, 64, 16, 16),
                                                  (700, 8, 1, 64, 32, 64), (900, 4, 1, 64, 16, 12)])
def test_block_select_vs_oracle(T, Hq, Hkv, D, block, top):
    x = sa_synth.attn_inputs(811 + T, 1, T, Hq, Hkv, D, "bf16")
    note(f"block_select T={T} Hq={Hq} Hkv={Hkv} D={D} block={block} top={top}")
    kbar, _, _, _ = _pool(x, T, block)
    idx = host(sa.sa_block_select(dev(x["q"], "bf16"), kbar, block, top))
    ok_, _ = _oracle_pool(x, T, block)
    rows = list(range(0, T, 3)) + [T - 1]
    want = orc.block_select_rows(x["q"], ok_, block, top, rows)
    ex = _check_blocks(idx[0], want[0], x["q"][0], ok_[0], block, top, rows)
    assert ex <= 3


def test_block_select_exact_ties():
    # every key row the same vector: all complete blocks score exactly alike, so each row
    # takes its lowest `top` blocks (12 of up to 56, a count that does not divide 64)
    T, block, top = 900, 16, 12
    x = sa_synth.attn_inputs(831, 1, T, 4, 1, 64, "bf16")
    x["k"][:] = x["k"][:, :1]
    note(f"block_select exact ties T={T} block={block} top={top}")
    kbar, _, _, _ = _pool(x, T, block)
    got = host(sa.sa_block_select(dev(x["q"], "bf16"), kbar, block, top))[0]
    for t in range(0, T, 7):
        nfull = (t + 1) // block
        take = min(top, nfull)
        want = np.full(top * block, -1, np.int64)
        for e in range(block):
            for i in range(take):
                want[e * top + i] = i * block + e
        assert (got[t] == want).all(), t


def test_block_select_row_range():
    T, block, top = 1000, 16, 8
    x = sa_synth.attn_inputs(821, 2, T, 4, 1, 64, "bf16")
    note(f"block_select rows [300, 777) B=2 T={T}")
    kbar, _, _, _ = _pool(x, T, block)
    import torch
    idx = torch.full((2, T, top * block), -7, dtype=torch.int32, device="cuda")
    sa.sa_block_select(dev(x["q"], "bf16"), kbar, block, top, 300, 777, idx=idx)
    got = host(idx)
    assert (got[:, :300] == -7).all() and (got[:, 777:] == -7).all()
    ok_, _ = _oracle_pool(x, T, block)
    rows = list(range(300, 777, 5))
    for b in range(2):
        want = orc.block_select_rows(x["q"], ok_, block, top, rows)
        _check_blocks(got[b], want[b], x["q"][b], ok_[b], block, top, rows)


def test_combine():
    import torch
    g = sa_synth.rng(831)
    B, T, Hq, D = 2, 50, 4, 64
    parts = [sa_synth.round_bf16(g.standard_normal((B, T, Hq, D), dtype=np.float32)) for _ in range(3)]
    gates = g.uniform(0, 1, size=(B, T, Hq, 3)).astype(np.float32)
    note("nsa_combine")
    out = host(sa.sa_nsa_combine(*[dev(p_, "bf16") for p_ in parts], dev(gates, "f32")))
    want = orc.nsa_combine(gates, *parts)
    # float32 arithmetic, one bf16 rounding of the result (relative 2^-9)
    assert (np.abs(out - want) <= 2.0 ** -8 * np.abs(want) + 1e-6).all()


def test_nsa_prefill_pipeline_vs_oracle():
    """The whole prefill: pooled K and V, the compressed branch, block selection, the
    selected and window branches through sa_sparse_attn_fwd, the gated combine."""
    import torch
    T, Hq, D, block, top, W = 1100, 16, 128, 64, 4, 128
    x = sa_synth.attn_inputs(841, 1, T, Hq, 1, D, "bf16")
    gates = sa_synth.rng(842).uniform(0, 1, size=(1, T, Hq, 3)).astype(np.float32)
    note(f"nsa prefill T={T} Hq={Hq} D={D} block={block} top={top} W={W}")
    scale = D ** -0.5
    kbar, vbar, k, v = _pool(x, T, block)
    q = dev(x["q"], "bf16")
    oc = sa.sa_cmp_attn_fwd(q, kbar, vbar, block, scale)
    idx = sa.sa_block_select(q, kbar, block, top)
    osl = sa.sa_sparse_attn_fwd(q, k, v, idx, 0, scale)
    ow = sa.sa_sparse_attn_fwd(q, k, v, None, W, scale)
    out = host(sa.sa_nsa_combine(oc, osl, ow, dev(gates, "f32")))
    rows = list(range(0, 200, 3)) + list(range(200, T, 17)) + [T - 1]
    want, _, sel = orc.nsa_prefill(x["q"], x["k"], x["v"], gates, block, top, W, scale, rows)
    gi = host(idx)[0]
    okb, _ = _oracle_pool(x, T, block)
    # every row's block set is exact or a near tie of its boundary block scores
    n_exempt = _check_blocks(gi, sel[0], x["q"][0], okb[0], block, top, rows)
    assert n_exempt <= 2
    for r, t in enumerate(rows):
        wb = sorted(int(j) for j in sel[0, r] if j >= 0)
        if sorted(set(int(s) // block for s in gi[t] if s >= 0)) != wb:
            continue  # an exempt near tie: the selected branch legitimately differs
        assert np.abs(out[0, t] - want[0, r]).max() < BF16_TOL, t


# ------------------------------------------------------------------------------ decode

def test_meanpool_bf16_is_rounded_float32_mean():
    import torch
    x = sa_synth.decode_inputs(851, 3, 500, 4, 2, 64, "bf16", lens=[500, 130, 63])
    note("block_meanpool_bf16")
    kc = dev(x["kcache"], "bf16")
    lens = dev(np.asarray(x["lens"], np.int32), "i32")
    f32 = sa.sa_block_meanpool(kc, lens, 32)
    b16 = sa.sa_block_meanpool_bf16(kc, lens, 32)
    for b, L in enumerate(x["lens"]):
        nfull = int(L) // 32
        assert torch.equal(b16[b, :nfull], f32[b, :nfull].to(torch.bfloat16))


@pytest.mark.parametrize("Hq,Hkv,D,block,top,W", [(16, 1, 128, 64, 4, 200), (8, 2, 64, 32, 8, 100)])
def test_nsa_decode_vs_oracle(Hq, Hkv, D, block, top, W):
    import torch
    lens_h = [1500, 999, 64, 1]
    x = sa_synth.decode_inputs(861 + D, 4, 1500, Hq, Hkv, D, "bf16", lens=lens_h)
    gates = sa_synth.rng(862).uniform(0, 1, size=(4, Hq, 3)).astype(np.float32)
    note(f"nsa decode B=4 Lmax=1500 Hq={Hq} Hkv={Hkv} D={D} block={block} top={top} W={W}")
    scale = D ** -0.5
    q, kc, vc = dev(x["q"], "bf16"), dev(x["kcache"], "bf16"), dev(x["vcache"], "bf16")
    lens = dev(np.asarray(lens_h, np.int32), "i32")
    kbar = sa.sa_block_meanpool(kc, lens, block)
    kb16 = sa.sa_block_meanpool_bf16(kc, lens, block)
    vb16 = sa.sa_block_meanpool_bf16(vc, lens, block)
    oc = sa.sa_nsa_decode_branch(q, kb16, vb16, lens, 1, block, W, scale)
    ow = sa.sa_nsa_decode_branch(q, kc, vc, lens, 0, block, W, scale)
    ws = torch.zeros(sa.sa_sparse_decode_workspace(4, 1500, Hq, Hkv, D, block, top, 0), dtype=torch.uint8,
                     device="cuda")
    osl = sa.sa_sparse_decode(q, kc, vc, kbar, lens, block, top, 0, scale, workspace=ws)
    out = sa.sa_nsa_combine(oc[:, None], osl[:, None], ow[:, None], dev(gates[:, None], "f32"))[:, 0]
    want, (wc, ws_, ww), sel = orc.nsa_decode(x["q"], x["kcache"], x["vcache"], np.asarray(lens_h),
                                              gates, block, top, W, scale)
    assert np.abs(host(oc) - wc).max() < BF16_TOL
    assert np.abs(host(ow) - ww).max() < BF16_TOL
    assert np.abs(host(osl) - ws_).max() < BF16_TOL
    assert np.abs(host(out) - want).max() < BF16_TOL
    assert not host(oc)[3].any()  # one token: no complete block


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 16, 1), (64, 8, 2)])
def test_nsa_decode_branch_splits(D, Hq, Hkv):
    """Both decode range branches with the range split over several workgroups (partials
    merged by log-sum-exp, the last split merging) against the oracle, lse included, on
    ragged lengths (the 1-token sequence has no complete block: out 0, lse -inf), twice on
    one workspace (the counters return to zero)."""
    import torch
    block, W = 32, 300
    lens_h = [1500, 999, 64, 1]
    x = sa_synth.decode_inputs(871 + D, 4, 1500, Hq, Hkv, D, "bf16", lens=lens_h)
    scale = D ** -0.5
    q, kc, vc = dev(x["q"], "bf16"), dev(x["kcache"], "bf16"), dev(x["vcache"], "bf16")
    lens = dev(np.asarray(lens_h, np.int32), "i32")
    kb16 = sa.sa_block_meanpool_bf16(kc, lens, block)
    vb16 = sa.sa_block_meanpool_bf16(vc, lens, block)
    gates = np.zeros((4, Hq, 3), np.float32)
    _, (wc, _, ww), _ = orc.nsa_decode(x["q"], x["kcache"], x["vcache"], np.asarray(lens_h),
                                       gates, block, 1, W, scale)
    for ns in (2, 5, 7, 64):  # 64 (the limit): most splits of the short ranges are empty
        ws = torch.zeros(sa.sa_nsa_decode_branch_workspace(4, Hq, Hkv, D, ns), dtype=torch.uint8,
                         device="cuda")
        for rep in range(2):
            note(f"nsa decode branches, {ns} splits, D={D} Hq={Hq} Hkv={Hkv}, call {rep}")
            oc, lc = sa.sa_nsa_decode_branch(q, kb16, vb16, lens, 1, block, W, scale, want_lse=True,
                                             n_splits=ns, workspace=ws)
            ow, lw = sa.sa_nsa_decode_branch(q, kc, vc, lens, 0, block, W, scale, want_lse=True,
                                             n_splits=ns, workspace=ws)
            o1, l1 = sa.sa_nsa_decode_branch(q, kb16, vb16, lens, 1, block, W, scale, want_lse=True)
            assert np.abs(host(oc) - wc).max() < BF16_TOL
            assert np.abs(host(ow) - ww).max() < BF16_TOL
            assert not host(oc)[3].any() and np.isneginf(host(lc)[3]).all()
            assert np.abs(host(lc)[:3] - host(l1)[:3]).max() < 1e-4
            # the per-(sequence, KV head) counters after the partials are back at zero
            part = (4 * Hkv * ns * (Hq // Hkv) * (D + 4) * 4 + 255) // 256 * 256
            assert not bool(ws[part: part + 4 * Hkv * 4].any())


@pytest.mark.parametrize("D,Hq,Hkv,ns_c,ns_w", [(128, 16, 1, 8, 1), (128, 16, 1, 1, 1),
                                                (64, 8, 2, 3, 5), (128, 4, 2, 64, 2)])
def test_nsa_decode_cmp_win_equals_branches(D, Hq, Hkv, ns_c, ns_w):
    """Both range branches in one launch equal the two separate branch calls bit for bit
    (outputs and lse), on ragged lengths, twice on one workspace (its counters return to
    zero), and against the oracle."""
    import torch
    block, W = 32, 300
    lens_h = [1500, 999, 64, 1]
    x = sa_synth.decode_inputs(881 + D, 4, 1500, Hq, Hkv, D, "bf16", lens=lens_h)
    scale = D ** -0.5
    q, kc, vc = dev(x["q"], "bf16"), dev(x["kcache"], "bf16"), dev(x["vcache"], "bf16")
    lens = dev(np.asarray(lens_h, np.int32), "i32")
    kb16 = sa.sa_block_meanpool_bf16(kc, lens, block)
    vb16 = sa.sa_block_meanpool_bf16(vc, lens, block)
    oc, lc = sa.sa_nsa_decode_branch(q, kb16, vb16, lens, 1, block, W, scale, want_lse=True,
                                     n_splits=ns_c)
    ow, lw = sa.sa_nsa_decode_branch(q, kc, vc, lens, 0, block, W, scale, want_lse=True,
                                     n_splits=ns_w)
    need = sa.sa_nsa_decode_cmp_win_workspace(4, Hq, Hkv, D, ns_c, ns_w)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    gates = np.zeros((4, Hq, 3), np.float32)
    _, (wc, _, ww), _ = orc.nsa_decode(x["q"], x["kcache"], x["vcache"], np.asarray(lens_h),
                                       gates, block, 1, W, scale)
    for rep in range(2):
        note(f"nsa decode cmp+win, splits {ns_c}/{ns_w}, D={D} Hq={Hq} Hkv={Hkv}, call {rep}")
        c, w_, lc2, lw2 = sa.sa_nsa_decode_cmp_win(q, kb16, vb16, kc, vc, lens, block, W, scale,
                                                   want_lse=True, n_splits_cmp=ns_c,
                                                   n_splits_win=ns_w, workspace=ws)
        assert torch.equal(c, oc) and torch.equal(w_, ow)
        assert torch.equal(lc2, lc) and torch.equal(lw2, lw)
        assert np.abs(host(c) - wc).max() < BF16_TOL
        assert np.abs(host(w_) - ww).max() < BF16_TOL
        # each side's per-(sequence, KV head) counters, after its partials, are back at zero
        a256 = lambda n: (n + 255) // 256 * 256
        base = 0
        for ns in (ns_c, ns_w):
            if ns > 1:
                part = a256(4 * Hkv * ns * (Hq // Hkv) * (D + 4) * 4)
                assert not bool(ws[base + part: base + part + 4 * Hkv * 4].any())
                base += part + a256(4 * Hkv * 4)
