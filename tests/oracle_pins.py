"""Pins of the float64 oracle against facts fixed by the pages and by mathematics.

Each ``pin_*`` function takes the oracle module (``oracle.reference``) and raises
``AssertionError`` when a pin fails.  ``test_oracle_pins.py`` runs them on the real
oracle; ``test_oracle_mutants.py`` runs them on deliberately broken copies of it and
requires every copy to fail at least one pin, which shows that the pins bite.

Pins used (none re-types the oracle's formula or re-calls its library routine the
same way):
* hand-worked fixtures in tests/golden/ (each cites the passage it follows);
* exact rational arithmetic (``fractions``) on integer-valued inputs;
* library special cases: torch's scaled_dot_product_attention in float64 on the CPU
  (full causal and banded masks, full attention for a decode query);
* brute force with pure-Python loops and ``math.exp`` on tiny inputs;
* closed forms (graph neighbour count, its sum 654,896 at T = 16,384) and invariants
  (softmax rows sum to one, permutation, bias and window invariances).
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

import sa_synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _sdpa64(q, k, v, mask=None, causal=False):
    """torch SDPA in float64 on the CPU.  q [H,Tq,D], k/v [H,Tk,D]; mask [Tq,Tk] bool."""
    import torch
    import torch.nn.functional as F
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64))[None]
    kt = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64))[None]
    vt = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64))[None]
    m = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask))
    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=causal,
                                         scale=1.0)
    return out[0].numpy()


def _lse64(logits, mask):
    import torch
    lg = torch.from_numpy(np.where(mask, logits, -np.inf))
    return torch.logsumexp(lg, dim=-1).numpy()


# ------------------------------------------------------------------------------ indexer

def pin_indexer_hand(orc):
    g = _golden("indexer_hand.json")
    qi = np.array(g["qi"], dtype=np.float32)
    ki = np.array(g["ki"], dtype=np.float32)
    w = np.array(g["w"], dtype=np.float32)
    for t, want in enumerate(g["scores"]):
        got = orc.indexer_scores_row(qi, ki, w, 0, t)
        assert got.shape == (t + 1,), got.shape
        assert np.array_equal(got, np.array(want)), (t, got, want)


def pin_indexer_exact_integers(orc):
    """Integer inputs and dyadic weights: every score is an exact rational; the
    float64 oracle must reproduce it exactly (brute force in Fractions)."""
    x = sa_synth.integer_indexer_inputs(11, 2, 9, 3, 5)
    qi, ki, w = x["qi"], x["ki"], x["w"]
    for b in range(2):
        for t in range(9):
            got = orc.indexer_scores_row(qi, ki, w, b, t)
            for s in range(t + 1):
                want = Fraction(0)
                for h in range(3):
                    dot = sum(Fraction(int(qi[b, t, h, d])) * Fraction(int(ki[b, s, d]))
                              for d in range(5))
                    want += Fraction(float(w[h])) * max(dot, Fraction(0))
                assert Fraction(float(got[s])) == want, (b, t, s, got[s], want)


def pin_indexer_odd_part(orc):
    """ReLU(x) - ReLU(-x) = x per head, so S(qi) - S(-qi) = Σ_h w_h qi_h·ki (checked
    with exact Fractions on integer inputs); S ≥ 0 everywhere since w ≥ 0."""
    x = sa_synth.integer_indexer_inputs(12, 1, 6, 2, 4)
    qi, ki, w = x["qi"], x["ki"], x["w"]
    for t in range(6):
        a = orc.indexer_scores_row(qi, ki, w, 0, t)
        bneg = orc.indexer_scores_row(-qi, ki, w, 0, t)
        assert (a >= 0).all()
        for s in range(t + 1):
            lin = sum(Fraction(float(w[h])) * sum(Fraction(int(qi[0, t, h, d])) * int(ki[0, s, d])
                                                  for d in range(4)) for h in range(2))
            assert Fraction(float(a[s])) - Fraction(float(bneg[s])) == lin


# ------------------------------------------------------------------------------ top-k

def _topk_brute(row, k):
    order = sorted(range(len(row)), key=lambda s: (-float(row[s]) + 0.0, s))
    sel = sorted(order[:k])
    return sel + [-1] * (k - len(sel))


def pin_topk_hand(orc):
    for c in _golden("topk_hand.json")["cases"]:
        got = orc.topk_select_row(np.array(c["row"], dtype=np.float64), c["k"])
        assert got.dtype == np.int32
        assert got.tolist() == c["idx"], (c, got)


def pin_topk_brute(orc):
    """Full stable sort by (score desc, position asc) on tiny rows with many ties."""
    g = sa_synth.rng(21)
    for _ in range(300):
        n = int(g.integers(1, 40))
        k = int(g.integers(1, 45))
        row = g.integers(0, 4, size=n).astype(np.float64) * 0.5
        if g.random() < 0.3:
            row = g.standard_normal(n)
        got = orc.topk_select_row(row, k).tolist()
        assert got == _topk_brute(row, k), (row, k, got)


def pin_topk_invariants(orc):
    g = sa_synth.rng(22)
    for _ in range(50):
        n = int(g.integers(50, 400))
        k = int(g.integers(1, 64))
        row = g.standard_normal(n)
        got = orc.topk_select_row(row, k)
        sel = got[got >= 0]
        assert sel.shape[0] == min(k, n)
        assert (np.diff(sel) > 0).all()
        uns = np.setdiff1d(np.arange(n), sel)
        if uns.size:
            assert row[sel].min() >= row[uns].max()


def _boundary_by_counting(row, k):
    """The k-th and (k+1)-th largest values by counting: the j-th largest value is the
    largest v in the row with #{s : row[s] >= v} >= j.  None when the row has <= k
    entries."""
    vals = [float(v) + 0.0 for v in row]
    if len(vals) <= k:
        return None

    def jth(j):
        return max(v for v in vals if sum(1 for u in vals if u >= v) >= j)

    return jth(k), jth(k + 1)


def pin_topk_boundary_hand(orc):
    """Hand-worked rows: the k-th and (k+1)-th largest scores (ties counted with their
    multiplicity), None when there is no (k+1)-th."""
    row = [3.0, 1.0, 3.0, 0.0, 2.0, 3.0, 0.0]
    for k, want in ((1, (3.0, 3.0)), (2, (3.0, 3.0)), (3, (3.0, 2.0)), (4, (2.0, 1.0)),
                    (5, (1.0, 0.0)), (6, (0.0, 0.0)), (7, None), (9, None)):
        got = orc.topk_boundary(np.array(row), k)
        assert (got is None) == (want is None), (k, got)
        if want is not None:
            assert tuple(got) == want, (k, got, want)
    assert orc.topk_boundary(np.array([5.0, 4.0]), 1) == (5.0, 4.0)        # n = k + 1
    assert orc.topk_boundary(np.array([4.0, 5.0]), 1) == (5.0, 4.0)
    assert orc.topk_boundary(np.array([2.5] * 6), 4) == (2.5, 2.5)           # all equal
    assert orc.topk_boundary(np.array([-1.0, -3.0, -2.0]), 2) == (-2.0, -3.0)
    assert orc.topk_boundary(np.array([1.0]), 1) is None                    # n = k
    bd = orc.topk_boundary(np.array([0.0, -0.0, 0.0, -1.0]), 3)             # -0 == +0
    assert bd[0] == 0.0 and bd[1] == -1.0


def pin_topk_boundary_counting_and_selection(orc):
    """Random and tie-heavy rows: the boundary equals the counting definition, and it
    brackets the selected set: a = min score of topk_select_row's set, b = max score of
    the rest (topk_select_row is pinned by brute force on its own)."""
    g = sa_synth.rng(23)
    for it in range(400):
        n = int(g.integers(1, 30))
        k = int(g.integers(1, 32))
        if it % 3 == 0:
            row = g.integers(-2, 3, size=n).astype(np.float64)
        elif it % 3 == 1:
            row = g.standard_normal(n)
        else:
            row = np.full(n, float(g.integers(-2, 3)))
        got = orc.topk_boundary(row, k)
        want = _boundary_by_counting(row.tolist(), k)
        assert (got is None) == (want is None), (row, k, got)
        if got is None:
            assert n <= k
            continue
        assert tuple(float(v) for v in got) == want, (row, k, got, want)
        sel = orc.topk_select_row(row, k)
        chosen = np.zeros(n, dtype=bool)
        chosen[sel[sel >= 0]] = True
        assert row[chosen].min() == got[0] and row[~chosen].max() == got[1], (row, k)


# ------------------------------------------------------------------------------ sparse attention

def pin_attn_hand(orc):
    g = _golden("attn_hand.json")
    q, k, v = (np.array(g[n], dtype=np.float64) for n in ("q", "k", "v"))
    for c in g["cases"]:
        idx = np.full((1, 3, 2), -1, dtype=np.int32)
        idx[0, 2] = c["idx_row2"]
        O, L = orc.sparse_attn(q, k, v, idx, c["window"], 1.0, rows=[c["row"]])
        assert abs(O[0, 0, 0, 0] - c["O"]) < 1e-12, (c, O[0, 0, 0, 0])
        assert abs(L[0, 0, 0] - c["LSE"]) < 1e-12, (c, L[0, 0, 0])


def _expand_gqa(x, G):
    return np.repeat(x, G, axis=0)    # [Hkv, T, D] -> [Hq, T, D]


def pin_attn_full_when_k_covers(orc):
    """k ≥ T (or W ≥ T) selects every earlier key: plain causal attention, checked
    against torch SDPA(is_causal=True) in float64 and torch.logsumexp, with GQA
    (Hq=4, Hkv=2)."""
    B, T, scale = 2, 37, 0.25
    x = sa_synth.attn_inputs(31, B, T, 4, 2, 16, "f32")
    q, k, v = x["q"], x["k"], x["v"]

    def listed(kk):
        ix = np.full((B, T, kk), -1, dtype=np.int32)
        for t in range(T):
            n = min(kk, t + 1)
            ix[:, t, :n] = np.arange(n, dtype=np.int32)
        return ix

    cases = ((listed(T), 0), (listed(T + 5), 3), (np.full((B, T, 1), -1, np.int32), T))
    causal = np.tril(np.ones((T, T), dtype=bool))
    for ix, W in cases:
        O, L = orc.sparse_attn(q, k, v, ix, W, scale)
        for b in range(B):
            qh = np.transpose(q[b], (1, 0, 2)).astype(np.float64) * scale
            kh = _expand_gqa(np.transpose(k[b], (1, 0, 2)), 2).astype(np.float64)
            vh = _expand_gqa(np.transpose(v[b], (1, 0, 2)), 2).astype(np.float64)
            want = _sdpa64(qh, kh, vh, causal=True)
            assert np.abs(O[b] - np.transpose(want, (1, 0, 2))).max() < 1e-12
            logits = np.matmul(qh, np.transpose(kh, (0, 2, 1)))
            assert np.abs(L[b] - _lse64(logits, causal[None])).max() < 1e-12


def pin_attn_window_only(orc):
    """No usable listed index (all -1, or junk outside [0, t]): the textbook
    sliding-window attention, checked against SDPA with a banded boolean mask."""
    T, W = 50, 7
    x = sa_synth.attn_inputs(32, 1, T, 2, 1, 8, "f32")
    q, k, v = x["q"], x["k"], x["v"]
    g = sa_synth.rng(5)
    junk = np.full((1, T, 4), -1, np.int32)
    for t in range(T):
        junk[0, t] = g.integers(t + 1, t + 100, size=4)
        junk[0, t, ::2] = -9
    ts = np.arange(T)
    band = (ts[None, :] <= ts[:, None]) & (ts[None, :] > ts[:, None] - W)
    want = _sdpa64(np.transpose(q[0], (1, 0, 2)) * 0.5,
                   _expand_gqa(np.transpose(k[0], (1, 0, 2)), 2),
                   _expand_gqa(np.transpose(v[0], (1, 0, 2)), 2), mask=band)
    for idx in (np.full((1, T, 4), -1, np.int32), junk):
        O, _ = orc.sparse_attn(q, k, v, idx, W, 0.5)
        assert np.abs(O[0] - np.transpose(want, (1, 0, 2))).max() < 1e-12


def pin_attn_brute_tiny(orc):
    """T ≤ 8: pure-Python loops with math.exp over the explicit selected set."""
    x = sa_synth.attn_inputs(33, 1, 8, 2, 1, 3, "f32")
    q, k, v = x["q"], x["k"], x["v"]
    idx = sa_synth.random_topk_idx(6, 1, 8, 2)
    W, scale = 2, 0.7
    O, L = orc.sparse_attn(q, k, v, idx, W, scale)
    for t in range(8):
        S = {int(s) for s in idx[0, t] if 0 <= s <= t} | set(range(max(0, t - W + 1), t + 1))
        for h in range(2):
            lg = {s: scale * sum(float(q[0, t, h, d]) * float(k[0, s, 0, d]) for d in range(3))
                  for s in S}
            mx = max(lg.values())
            wts = {s: math.exp(lg[s] - mx) for s in S}
            tot = sum(wts.values())
            for d in range(3):
                want = sum(wts[s] * float(v[0, s, 0, d]) for s in S) / tot
                assert abs(O[0, t, h, d] - want) < 1e-12
            assert abs(L[0, h, t] - (mx + math.log(tot))) < 1e-12


def pin_attn_rows_sum_to_one(orc):
    """With V ≡ 1 every output equals Σ_s p_s, which must be 1."""
    x = sa_synth.attn_inputs(34, 1, 300, 4, 1, 32, "f32")
    idx = sa_synth.random_topk_idx(7, 1, 300, 40)
    O, _ = orc.sparse_attn(x["q"], x["k"], np.ones_like(x["v"]), idx, 16, 0.2)
    assert np.abs(O - 1.0).max() <= 1e-12


def pin_attn_permutation_and_window_dedup(orc):
    """Permuting a row's listed indices changes nothing; listing only in-window
    positions gives the window-only result (each key counted once)."""
    x = sa_synth.attn_inputs(35, 1, 120, 2, 1, 16, "f32")
    q, k, v = x["q"], x["k"], x["v"]
    idx = sa_synth.random_topk_idx(8, 1, 120, 24)
    g = sa_synth.rng(9)
    perm = idx.copy()
    for t in range(120):
        perm[0, t] = perm[0, t, g.permutation(24)]
    a, _ = orc.sparse_attn(q, k, v, idx, 8, 0.25)
    b, _ = orc.sparse_attn(q, k, v, perm, 8, 0.25)
    assert np.array_equal(a, b)
    inwin = np.full((1, 120, 24), -1, np.int32)
    for t in range(120):
        ws = np.arange(max(0, t - 7), t + 1, dtype=np.int32)
        inwin[0, t, : ws.shape[0]] = ws[::-1]
    c, _ = orc.sparse_attn(q, k, v, inwin, 8, 0.25)
    d, _ = orc.sparse_attn(q, k, v, np.full((1, 120, 24), -1, np.int32), 8, 0.25)
    assert np.abs(c - d).max() < 1e-14


# ------------------------------------------------------------------------------ graph

def pin_graph_hand(orc):
    g = _golden("graph_hand.json")
    cq, ck, v = (np.array(g[n], dtype=np.float64) for n in ("cq", "ck", "v"))
    bias = np.array(g["bias"])
    for t, nb in enumerate(g["neighbours"]):
        assert orc.graph_neighbours(t, g["local"], g["n_pow2"]).tolist() == nb
    O, L = orc.graph_attn(cq, ck, v, bias, g["tau"], g["local"], g["n_pow2"])
    assert np.abs(O[0, :, 0, 0] - np.array(g["O"])).max() < 1e-12, O[0, :, 0, 0]
    assert np.abs(L[0, 0] - np.array(g["LSE"])).max() < 1e-12, L[0, 0]


def pin_graph_count_closed_form(orc):
    """|N(t)| = min(t,32)+1+#{j in [6,13]: 2^j ≤ t}, and Σ_{t<16384} |N(t)| = 654,896
    (= 540,144 local + 114,752 power-of-two; the closed-form sums are in the test)."""
    for t in range(0, 20000, 7):
        assert orc.graph_neighbours(t, 32, 14).shape[0] == orc.graph_neighbour_count(t, 32, 14)
        want = min(t, 32) + 1 + sum(1 for j in range(6, 14) if (1 << j) <= t)
        assert orc.graph_neighbour_count(t, 32, 14) == want
    T = 16384
    local_sum = sum(range(1, 34)) + (T - 33) * 33
    far_sum = sum(T - (1 << j) for j in range(6, 14))
    assert local_sum + far_sum == 654896
    assert sum(orc.graph_neighbour_count(t, 32, 14) for t in range(T)) == 654896
    assert orc.graph_offsets(32, 14).shape[0] == 41


def pin_graph_tau0_mean_and_bias(orc):
    """τ = 0: every neighbour weighs the same, O = plain mean of V over N(t).
    Adding a constant to the bias leaves O unchanged and shifts LSE by it."""
    x = sa_synth.graph_inputs(41, 1, 200, 3, 8, "f32")
    O, _ = orc.graph_attn(x["cq"], x["ck"], x["v"], x["bias"], 0.0, 4, 8)
    for t in range(200):
        nb = sorted({t - o for o in list(range(5)) + [1 << j for j in range(8)] if t - o >= 0})
        assert np.abs(O[0, t] - x["v"][0, nb].astype(np.float64).mean(axis=0)).max() < 1e-12
    a, la = orc.graph_attn(x["cq"], x["ck"], x["v"], x["bias"], 1.0, 4, 8)
    b, lb = orc.graph_attn(x["cq"], x["ck"], x["v"], x["bias"].astype(np.float64) + 3.0, 1.0, 4, 8)
    assert np.abs(a - b).max() < 1e-12
    assert np.abs((lb - la) - 3.0).max() < 1e-12


def pin_graph_brute_short(orc):
    """T ≤ local+1: N(t) = [0, t]; pure-Python distance softmax."""
    x = sa_synth.graph_inputs(42, 1, 10, 2, 3, "f32")
    tau = 0.8
    O, L = orc.graph_attn(x["cq"], x["ck"], x["v"], x["bias"], tau, 32, 14)
    for t in range(10):
        for h in range(2):
            lg = []
            for s in range(t + 1):
                d2 = sum((float(x["cq"][0, t, h, c]) - float(x["ck"][0, s, h, c])) ** 2 for c in range(3))
                lg.append(-tau * d2 + float(x["bias"][h]))
            mx = max(lg)
            wts = [math.exp(a - mx) for a in lg]
            for d in range(3):
                want = sum(wts[s] * float(x["v"][0, s, h, d]) for s in range(t + 1)) / sum(wts)
                assert abs(O[0, t, h, d] - want) < 1e-12
            assert abs(L[0, h, t] - (mx + math.log(sum(wts)))) < 1e-12


# ------------------------------------------------------------------------------ decode

def pin_decode_hand(orc):
    g = _golden("decode_hand.json")
    V = np.array(g["V"], dtype=np.float64).reshape(1, 4, 1, 1)
    for c in g["cases"]:
        K = np.array(c["K"], dtype=np.float64).reshape(1, 4, 1, 1)
        q = np.array([[[c["q"]]]])
        lens = np.array([4], np.int32)
        kbar = orc.block_meanpool(K, lens, g["block"])
        assert kbar[0, :, 0, 0].tolist() == c["kbar"]
        O, L, sel = orc.sparse_decode(q, K, V, lens, g["block"], g["top_blocks"], g["window"],
                                      g["scale"])
        assert sel[0, 0].tolist() == c["sel"], sel
        assert abs(O[0, 0, 0] - c["O"]) < 1e-12, (c, O)
        assert abs(L[0, 0] - c["LSE"]) < 1e-12, (c, L)


def pin_decode_pool_and_scores_brute(orc):
    """Block means and block scores by loops over raw cache rows (integer-valued cache:
    exact), and Σ_h q_h·kbar_j = mean over the block of (Σ_h q_h)·K_s."""
    g = sa_synth.rng(51)
    B, L, Hkv, D, G, blk = 2, 45, 2, 3, 2, 4
    K = g.integers(-3, 4, size=(B, L, Hkv, D)).astype(np.float64)
    q = g.integers(-2, 3, size=(B, Hkv * G, D)).astype(np.float64)
    lens = np.array([45, 17], np.int32)
    kbar = orc.block_meanpool(K, lens, blk)
    for b in range(B):
        nfull = lens[b] // blk
        assert np.isnan(kbar[b, nfull:]).all()
        for j in range(nfull):
            for hk in range(Hkv):
                for d in range(D):
                    want = Fraction(sum(int(K[b, blk * j + i, hk, d]) for i in range(blk)), blk)
                    assert Fraction(float(kbar[b, j, hk, d])) == want
    sel = orc.decode_select(q, kbar, lens, 3, blk)
    for b in range(B):
        nfull = int(lens[b]) // blk
        for hk in range(Hkv):
            sc = []
            for j in range(nfull):
                tot = Fraction(0)
                for i in range(blk):
                    for h in range(hk * G, hk * G + G):
                        tot += sum(Fraction(int(q[b, h, d])) * int(K[b, blk * j + i, hk, d])
                                   for d in range(D))
                sc.append(tot / blk)
            assert sel[b, hk].tolist() == _topk_brute(sc, 3), (b, hk, sel[b, hk], sc)


def pin_decode_full_when_all_blocks(orc):
    """L ≤ top_blocks·block: every block is chosen, so the step is full attention of
    the query over the whole cache (SDPA, float64, no mask)."""
    x = sa_synth.decode_inputs(52, 3, 200, 4, 2, 16, "f32", lens=[200, 131, 64])
    O, L, sel = orc.sparse_decode(x["q"], x["kcache"], x["vcache"], x["lens"], 16, 16, 8, 0.25)
    for b in range(3):
        n = int(x["lens"][b])
        assert (sel[b][sel[b] >= 0].shape[0]) == 2 * min(16, n // 16)
        for hk in range(2):
            qg = x["q"][b, 2 * hk: 2 * hk + 2][:, None, :] * 0.25
            kk = np.repeat(x["kcache"][b, :n, hk][None], 2, axis=0)
            vv = np.repeat(x["vcache"][b, :n, hk][None], 2, axis=0)
            want = _sdpa64(qg, kk, vv)[:, 0]
            assert np.abs(O[b, 2 * hk: 2 * hk + 2] - want).max() < 1e-12


def pin_decode_window_covers(orc):
    """window ≥ L: U is the whole cache whatever the blocks; and the mask of U is the
    chosen blocks' tokens before the window plus the window (checked by enumeration)."""
    x = sa_synth.decode_inputs(53, 1, 300, 2, 1, 8, "f32")
    a, _, _ = orc.sparse_decode(x["q"], x["kcache"], x["vcache"], x["lens"], 8, 2, 300, 0.3)
    want = _sdpa64(x["q"][0][:, None, :].astype(np.float64) * 0.3, np.repeat(x["kcache"][0, :, 0][None], 2, 0),
                   np.repeat(x["vcache"][0, :, 0][None], 2, 0))[:, 0]
    assert np.abs(a[0] - want).max() < 1e-12
    m = orc.decode_token_mask(np.array([3, 36, -1]), 300, 8, 20)
    expect = set(range(24, 32)) | set(range(280, 300))   # block 36 lies inside the window
    assert set(np.flatnonzero(m).tolist()) == expect


# ------------------------------------------------------------------------------ index reuse

def pin_indexcache(orc):
    """F,S,S,S: one indexer evaluation; each S layer is sparse attention over the F layer's
    selection.  The expected selection is brute force here: exact rational scores of
    integer indexer inputs (many ties) ranked by a full stable sort; each layer's output is
    float64 SDPA under the explicit mask (that selection united with the window).  The 3
    skipped evaluations are the '75%' of the IndexCache page (body paragraphs 2-4)."""
    T, k, W, scale = 40, 6, 3, 0.3
    x = sa_synth.integer_indexer_inputs(61, 1, T, 2, 4)
    qi, ki, w = x["qi"], x["ki"], x["w"]
    layers = [sa_synth.attn_inputs(62 + l, 1, T, 2, 1, 8, "f32") for l in range(4)]
    outs, n_index = orc.indexcache_prefill(qi, ki, w, layers, "FSSS", k, W, scale)
    assert n_index == 1
    sel = []
    for t in range(T):
        row = []
        for s in range(t + 1):
            sc = Fraction(0)
            for h in range(2):
                dot = sum(Fraction(int(qi[0, t, h, d])) * int(ki[0, s, d]) for d in range(4))
                sc += Fraction(float(w[h])) * max(dot, Fraction(0))
            row.append(sc)
        order = sorted(range(t + 1), key=lambda s_: (-row[s_], s_))
        sel.append(set(order[:k]))
    for lay, (O, L) in zip(layers, outs):
        for t in range(T):
            m = np.zeros(t + 1, dtype=bool)
            m[sorted(sel[t] | set(range(max(0, t - W + 1), t + 1)))] = True
            want = _mask_attend64(lay["q"][0, t], lay["k"][0, : t + 1, 0], lay["v"][0, : t + 1, 0],
                                  scale, m)
            assert np.abs(O[0, t] - want).max() < 1e-12, t


def pin_e4m3_closed_forms(orc):
    """Codes whose values the OCP E4M3 definition fixes directly: zeros of both signs, the
    smallest subnormal 2^-9, the largest subnormal 7*2^-9, the smallest normal 2^-6, 1,
    1.125, 2, the largest finite 448, 240 and 256 at the top of the exponent range, and
    the two NaN codes."""
    want = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
            0x39: 1.125, 0x40: 2.0, 0xC0: -2.0, 0x77: 240.0, 0x78: 256.0, 0x7E: 448.0,
            0xFE: -448.0, 0x81: -(2.0 ** -9)}
    codes = np.array(sorted(want), dtype=np.uint8)
    got = orc.decode_e4m3(codes)
    for c, g in zip(codes, got):
        assert g == want[int(c)], (hex(int(c)), g)
    z = orc.decode_e4m3(np.array([0x00, 0x80], dtype=np.uint8))
    assert z[0] == 0.0 and not math.copysign(1.0, z[0]) < 0
    assert z[1] == 0.0 and math.copysign(1.0, z[1]) < 0
    nan = orc.decode_e4m3(np.array([0x7F, 0xFF], dtype=np.uint8))
    assert np.isnan(nan).all()


def pin_e4m3_every_code_vs_torch(orc):
    """All 256 codes against torch's float8_e4m3fn -> float32 conversion (an independent
    implementation of the same format); also strictly increasing over 0x00..0x7E, and
    code c | 0x80 is the negative of code c."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    got = orc.decode_e4m3(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(got), ~fin)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))
    assert np.all(np.diff(got[:0x7F]) > 0)
    assert np.array_equal(got[0x80:0xFF], -got[:0x7F])


def pin_indexer_e4m3_exact(orc):
    """The 8-bit indexer: scores over decoded E4M3 inputs equal exact rational arithmetic
    on the same codes (each decoded by hand from sign, exponent and mantissa)."""
    g = sa_synth.rng(71)
    T, H, D = 7, 2, 5
    qc = g.integers(0, 256, size=(1, T, H, D)).astype(np.uint8)
    kc = g.integers(0, 256, size=(1, T, D)).astype(np.uint8)
    qc[(qc & 0x7F) == 0x7F] = 0x38   # no NaN inputs
    kc[(kc & 0x7F) == 0x7F] = 0x40
    w = np.array([0.75, 0.5], dtype=np.float32)

    def frac(c):
        c = int(c)
        e, m = (c >> 3) & 15, c & 7
        v = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        return -v if c >> 7 else v

    qd, kd = orc.decode_e4m3(qc), orc.decode_e4m3(kc)
    for t in range(T):
        row = orc.indexer_scores_row(qd, kd, w, 0, t)
        for s in range(t + 1):
            tot = Fraction(0)
            for h in range(H):
                dot = sum(frac(qc[0, t, h, d]) * frac(kc[0, s, d]) for d in range(D))
                tot += Fraction(float(w[h])) * max(dot, Fraction(0))
            assert abs(row[s] - float(tot)) <= 1e-12 * max(1.0, abs(float(tot))), (t, s)


# ------------------------------------------------------------------------------ backward

def pin_attn_bwd_vs_autograd(orc):
    """The gradients against torch autograd in float64 through a dense attention with the
    same boolean mask (masked logits set to -inf before softmax), two KV groups, listed
    indices that fall inside the window, -1 padding and out-of-range entries."""
    import torch
    B, T, Hq, Hkv, D, k, W = 1, 21, 4, 2, 8, 5, 3
    x = sa_synth.attn_inputs(91, B, T, Hq, Hkv, D, "f32")
    idx = sa_synth.random_topk_idx(92, B, T, k, junk=True)
    dout = sa_synth.rng(93).standard_normal((B, T, Hq, D))
    dQ, dK, dV = orc.sparse_attn_bwd(x["q"], x["k"], x["v"], idx, W, 0.3, dout)
    q = torch.tensor(x["q"], dtype=torch.float64, requires_grad=True)
    kk = torch.tensor(x["k"], dtype=torch.float64, requires_grad=True)
    vv = torch.tensor(x["v"], dtype=torch.float64, requires_grad=True)
    mask = np.zeros((T, T), dtype=bool)
    for t in range(T):
        for s_ in idx[0, t]:
            if 0 <= s_ <= t:
                mask[t, s_] = True
        mask[t, max(0, t - W + 1): t + 1] = True
    m = torch.from_numpy(mask)
    G = Hq // Hkv
    ke = kk[0].repeat_interleave(G, dim=1).transpose(0, 1)        # [Hq, T, D]
    ve = vv[0].repeat_interleave(G, dim=1).transpose(0, 1)
    qe = q[0].transpose(0, 1)
    lg = 0.3 * torch.matmul(qe, ke.transpose(1, 2))
    lg = lg.masked_fill(~m[None], float("-inf"))
    o = torch.matmul(torch.softmax(lg, dim=-1), ve).transpose(0, 1)[None]
    o.backward(torch.from_numpy(dout))
    assert np.abs(dQ - q.grad.numpy()).max() < 1e-12
    assert np.abs(dK - kk.grad.numpy()).max() < 1e-12
    assert np.abs(dV - vv.grad.numpy()).max() < 1e-12


def pin_attn_bwd_finite_differences(orc):
    """Central differences of <dout, O> through the forward oracle on a tiny case match
    every gradient entry (step 1e-5, error O(step^2))."""
    B, T, Hq, Hkv, D, k, W = 1, 7, 2, 1, 3, 3, 2
    x = sa_synth.attn_inputs(94, B, T, Hq, Hkv, D, "f32")
    q, kk, vv = (x[n].astype(np.float64) for n in ("q", "k", "v"))
    idx = sa_synth.random_topk_idx(95, B, T, k)
    dout = sa_synth.rng(96).standard_normal((B, T, Hq, D))
    dQ, dK, dV = orc.sparse_attn_bwd(q, kk, vv, idx, W, 0.7, dout)
    f = lambda a, b_, c: float(np.sum(orc.sparse_attn(a, b_, c, idx, W, 0.7)[0] * dout))
    eps = 1e-5
    for arr, grad, which in ((q, dQ, 0), (kk, dK, 1), (vv, dV, 2)):
        for pos in np.ndindex(arr.shape):
            a = [q.copy(), kk.copy(), vv.copy()]
            a[which][pos] += eps
            up = f(*a)
            a[which][pos] -= 2 * eps
            dn = f(*a)
            assert abs((up - dn) / (2 * eps) - grad[pos]) < 1e-7, (which, pos)


def pin_attn_row_form(orc):
    """The single-row form (explicit query row, key/value sequence, index row) equals the
    batched attention row by row, GQA with two groups, junk and in-window indices."""
    B, T, Hq, Hkv, D, k, W = 2, 37, 4, 2, 8, 5, 3
    x = sa_synth.attn_inputs(101, B, T, Hq, Hkv, D, "f32")
    idx = sa_synth.random_topk_idx(102, B, T, k, junk=True)
    O, L = orc.sparse_attn(x["q"], x["k"], x["v"], idx, W, 0.3)
    for b in range(B):
        for t in (0, 1, 4, 20, 36):
            o, l = orc.sparse_attn_row(x["q"][b, t], x["k"][b], x["v"][b], idx[b, t], t, W, 0.3)
            assert np.abs(o - O[b, t]).max() < 1e-12 and np.abs(l - L[b, :, t]).max() < 1e-12


def pin_attn_bwd_sampled_rows_and_keys(orc):
    """The sampled forms (dQ of chosen rows over S_t only; dK and dV of chosen keys summed
    over the rows that hold them) equal the full backward on a case with two sequences,
    two KV groups, listed keys inside the window, -1 padding and out-of-range entries."""
    B, T, Hq, Hkv, D, k, W = 2, 40, 4, 2, 8, 6, 4
    x = sa_synth.attn_inputs(97, B, T, Hq, Hkv, D, "f32")
    idx = sa_synth.random_topk_idx(98, B, T, k, junk=True)
    dout = sa_synth.rng(99).standard_normal((B, T, Hq, D))
    dQ, dK, dV = orc.sparse_attn_bwd(x["q"], x["k"], x["v"], idx, W, 0.4, dout)
    rows = [0, 1, 5, 17, 39]
    dq = orc.sparse_attn_bwd_rows(x["q"], x["k"], x["v"], idx, W, 0.4, dout, rows)
    assert np.abs(dq - dQ[:, rows]).max() < 1e-12
    for b in range(B):
        keys = [0, 3, 20, 38, 39]
        dk, dv = orc.sparse_attn_bwd_keys(x["q"], x["k"], x["v"], idx, W, 0.4, dout, b, keys)
        assert np.abs(dk - dK[b, keys]).max() < 1e-12
        assert np.abs(dv - dV[b, keys]).max() < 1e-12


# ------------------------------------------------------------------------------ NSA branches

def _mask_attend64(q, k, v, scale, mask):
    """[H,D] queries over [n,D] keys/values under a bool mask [n], via float64 SDPA."""
    H = q.shape[0]
    if not mask.any():
        return np.zeros((H, v.shape[1]))
    kk = np.repeat(np.asarray(k, np.float64)[mask][None], H, axis=0)
    vv = np.repeat(np.asarray(v, np.float64)[mask][None], H, axis=0)
    return _sdpa64(np.asarray(q, np.float64)[:, None, :] * scale, kk, vv)[:, 0]


def pin_cmp_attn_block1_is_causal_attention(orc):
    """block = 1: the block means are K and V themselves and every earlier token is a
    complete block, so the compressed branch is full causal attention (SDPA, causal)."""
    x = sa_synth.attn_inputs(81, 1, 37, 4, 2, 8, "f32")
    kbar = orc.block_meanpool(x["k"], np.array([37]), 1)
    vbar = orc.block_meanpool(x["v"], np.array([37]), 1)
    O, L = orc.cmp_attn(x["q"], kbar, vbar, 1, 0.3)
    for g in range(2):
        qg = np.transpose(x["q"][0, :, 2 * g: 2 * g + 2].astype(np.float64), (1, 0, 2)) * 0.3
        kg = np.repeat(x["k"][0, :, g][None], 2, axis=0)
        vg = np.repeat(x["v"][0, :, g][None], 2, axis=0)
        want = _sdpa64(qg, kg, vg, causal=True)
        assert np.abs(np.transpose(O[0, :, 2 * g: 2 * g + 2], (1, 0, 2)) - want).max() < 1e-12


def pin_cmp_attn_and_selection_brute(orc):
    """Tiny case by pure-Python loops: block means, the compressed softmax (math.exp) over
    the complete blocks at or before t, and the block ranking Σ_h q_h·kbar_j over both KV
    groups with ties to the lower block."""
    T, Hq, Hkv, D, blk = 23, 4, 2, 3, 4
    x = sa_synth.attn_inputs(82, 1, T, Hq, Hkv, D, "f32")
    q, k, v = (x[n].astype(np.float64) for n in ("q", "k", "v"))
    kbar = orc.block_meanpool(x["k"], np.array([T]), blk)
    vbar = orc.block_meanpool(x["v"], np.array([T]), blk)
    O, _ = orc.cmp_attn(x["q"], kbar, vbar, blk, 0.5)
    sel = orc.block_select_rows(x["q"], kbar, blk, 2)
    for t in range(T):
        nfull = (t + 1) // blk
        mean = lambda arr, j, g, d: sum(arr[0, j * blk + i, g, d] for i in range(blk)) / blk
        for h in range(Hq):
            g = h // (Hq // Hkv)
            if nfull == 0:
                assert not O[0, t, h].any()
                continue
            lg = [0.5 * sum(q[0, t, h, d] * mean(k, j, g, d) for d in range(D)) for j in range(nfull)]
            mx = max(lg)
            e = [math.exp(a - mx) for a in lg]
            for d in range(D):
                want = sum(e[j] * mean(v, j, g, d) for j in range(nfull)) / sum(e)
                assert abs(O[0, t, h, d] - want) < 1e-12
        sc = [sum(q[0, t, h, d] * mean(k, j, h // 2, d) for h in range(Hq) for d in range(D))
              for j in range(nfull)]
        order = sorted(range(nfull), key=lambda j: (-sc[j], j))[:2]
        want_sel = sorted(order) + [-1] * (2 - len(order))
        assert list(sel[0, t]) == want_sel, (t, list(sel[0, t]), want_sel)


def pin_nsa_prefill_branches_vs_sdpa(orc):
    """Each branch against SDPA with its own mask: with every complete block selected the
    selected branch attends to [0, (t+1)//block·block); the window branch to the last W
    tokens; block = 1 makes the compressed branch causal attention.  One-hot gates give the
    branches, random gates their weighted sum."""
    T, Hq, D, blk, W = 40, 2, 8, 1, 5
    x = sa_synth.attn_inputs(83, 1, T, Hq, 1, D, "f32")
    gates = sa_synth.rng(84).uniform(0, 1, size=(1, T, Hq, 3))
    O, (oc, osl, ow), sel = orc.nsa_prefill(x["q"], x["k"], x["v"], gates, blk, T, W, 0.4)
    k0, v0 = x["k"][0, :, 0], x["v"][0, :, 0]
    for t in range(T):
        q = x["q"][0, t]
        full = np.arange(T) <= t
        want_c = _mask_attend64(q, k0, v0, 0.4, full)                 # block = 1
        want_s = _mask_attend64(q, k0, v0, 0.4, np.arange(T) < (t + 1) // blk * blk)
        want_w = _mask_attend64(q, k0, v0, 0.4, (np.arange(T) <= t) & (np.arange(T) > t - W))
        assert np.abs(oc[0, t] - want_c).max() < 1e-12
        assert np.abs(osl[0, t] - want_s).max() < 1e-12
        assert np.abs(ow[0, t] - want_w).max() < 1e-12
        g = gates[0, t]
        want = g[:, 0:1] * want_c + g[:, 1:2] * want_s + g[:, 2:3] * want_w
        assert np.abs(O[0, t] - want).max() < 1e-12
    # block 4, two blocks chosen: the selected branch attends to exactly those tokens
    O2, (_, osl2, _), sel2 = orc.nsa_prefill(x["q"], x["k"], x["v"], gates, 4, 2, W, 0.4, rows=[33])
    m = np.zeros(T, dtype=bool)
    for j in sel2[0, 0]:
        m[j * 4: j * 4 + 4] = True
    assert m.sum() == 8 and not m[32:].any()
    assert np.abs(osl2[0, 0] - _mask_attend64(x["q"][0, 33], k0, v0, 0.4, m)).max() < 1e-12


def pin_nsa_decode_branches_vs_sdpa(orc):
    """Decode: the window branch over [L-W, L) and the selected branch over every token of
    the chosen blocks (window overlap kept: the branches are separate), each against SDPA;
    the compressed branch with block = 1 is full attention over the cache."""
    x = sa_synth.decode_inputs(85, 2, 90, 4, 2, 8, "f32", lens=[90, 37])
    gates = sa_synth.rng(86).uniform(0, 1, size=(2, 4, 3))
    O, (oc, osl, ow), sel = orc.nsa_decode(x["q"], x["kcache"], x["vcache"], x["lens"], gates,
                                           8, 3, 20, 0.3)
    O1, (oc1, _, _), _ = orc.nsa_decode(x["q"], x["kcache"], x["vcache"], x["lens"], gates,
                                        1, 3, 20, 0.3)
    for b in range(2):
        L = int(x["lens"][b])
        for g in range(2):
            q = x["q"][b, 2 * g: 2 * g + 2]
            kb, vb = x["kcache"][b, :L, g], x["vcache"][b, :L, g]
            m = np.zeros(L, dtype=bool)
            for j in sel[b, g]:
                if j >= 0:
                    m[j * 8: j * 8 + 8] = True
            assert m.sum() == 8 * min(3, L // 8)
            win = np.arange(L) >= L - 20
            ws = _mask_attend64(q, kb, vb, 0.3, m)
            ww = _mask_attend64(q, kb, vb, 0.3, win)
            wc1 = _mask_attend64(q, kb, vb, 0.3, np.ones(L, dtype=bool))
            hs = slice(2 * g, 2 * g + 2)
            assert np.abs(osl[b, hs] - ws).max() < 1e-12
            assert np.abs(ow[b, hs] - ww).max() < 1e-12
            assert np.abs(oc1[b, hs] - wc1).max() < 1e-12
            gg = gates[b, hs]
            want = gg[:, 0:1] * oc[b, hs] + gg[:, 1:2] * ws + gg[:, 2:3] * ww
            assert np.abs(O[b, hs] - want).max() < 1e-12


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
