"""Float64 CPU oracle of causal sparse attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg
may import this module.  It shares no code with the HIP library and imports nothing
from it.

Every function is the plain definition of what the method computes, written out in
float64 numpy, with no blocking, fusion or reordering beyond that definition.  The
attention functions evaluate *dense* causal attention over all earlier positions and
then apply the explicit selected-key mask (unselected logits are set to -inf before an
ordinary max-subtracted softmax), so selection and attention are checked separately.

Sources (web pages; the text is Spanish, cited by title and section):

* [IC] "IndexCache ... inferencia 82% más rápida" (larebelion.com, from VentureBeat),
  body paragraphs 2-4: a lightweight indexer scores every earlier token and the query
  attends only to the selected subset (DSA); F layers compute and cache the selected
  indices, S layers reuse those of the nearest preceding F layer.
* [HS2] "Xiaomi presenta HySparse2 ..." (diariobitcoin.com), sections "Dos niveles para
  compartir la caché" and "Más precisión con menos memoria": token-level (not block)
  selection, and the most recent tokens are forced into the selected set instead of a
  separate sliding-window branch (128 recent + up to 1,024 global).
* [SLM] "SpatialLM-Mini aceleró el entrenamiento con un contexto de 16K en 2,47 veces en
  una RTX 3050" (news.hamidun.com), section "Cómo eligen los tokens a quién escuchar":
  a fixed list of allowed positions — the token itself, near predecessors and positions
  at distances 1, 2, 4, 8, ... — never future ones; weights grow as the distance between
  learned 3-D query and key coordinates shrinks, adjusted by further learned parameters.
* [NSA] "Native Sparse Attention: Revolucionando el Procesamiento de Contexto Extenso ..."
  (ctol-es.com), sections "Puntos Clave" and "Análisis Profundo": coarse compression,
  blockwise fine-grained selection, sliding window; GQA group-centric loading with a
  shared KV fetch (one selection per KV head, shared by its query heads).
* [STAR] "NVIDIA AI Research presenta Star Attention ..." (7minutos.es), third body
  paragraph: partial attentions computed separately are combined with a distributed
  softmax.  The oracle has no split; its result is what any such combination must equal.

The pages give no formulas.  The concrete arithmetic of each workload (indexer score
Σ_h w_h·ReLU(qi_h[t]·ki[s]), window sizes, the power-of-two offsets, the distance logit
-τ‖c_q-c_k‖² + b_h, block size 64 and top-16 blocks) is the workload definition that
these pages' methods are instantiated with; each reading of an open point is marked
"Reading:" where it is used.

Pins: every function is checked by the CPU tests against closed forms, library special
cases, brute force on tiny inputs and hand-worked fixtures (tests/golden/); none of the
functions here is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------------------
# Indexer  [IC] body paragraphs 2-3 (the DSA indexer scores every earlier token)
# ----------------------------------------------------------------------------------------

def indexer_scores_row(qi, ki, w, b: int, t: int) -> np.ndarray:
    """Scores of query row ``t`` against keys s = 0..t (float64, length t+1).

    score(t, s) = Σ_h w[h] · max(0, qi[b,t,h,:] · ki[b,s,:])

    Reading: the indexer key ``ki`` is shared by the indexer heads, ``w`` is one
    constant per head shared by all rows, and there is no scale factor.
    """
    q = _f64(qi[b, t])                      # [H_I, D_I]
    k = _f64(ki[b, : t + 1])                # [t+1, D_I]
    dots = np.matmul(q, k.T)                # [H_I, t+1]: one dot product per head and key
    relu = np.maximum(dots, 0.0)
    return np.matmul(_f64(w), relu)         # Σ_h w_h · ReLU(.)


def decode_e4m3(codes) -> np.ndarray:
    """The value of each 8-bit E4M3 code (an array of uint8), in float64.

    Reading: the pages name no 8-bit format.  The indexer's 8-bit inputs are taken to
    be E4M3 codes as the OCP 8-bit floating point specification defines them (its "fn"
    variant): a sign bit, 4 exponent bits with bias 7 and 3 mantissa bits; exponent
    field 0 holds zero and the subnormals m/8 * 2^-6; there are no infinities, and the
    two codes with every exponent and mantissa bit set are NaN.  No scale factor comes
    with them: a positive factor shared by a whole row (a per-tensor or per-query scale)
    leaves that row's top-k unchanged, because ReLU commutes with it.  The 8-bit indexer
    is then ``indexer_scores_row`` over these values.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    negative = (c >> 7) == 1
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    magnitude = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = np.where(negative, -magnitude, magnitude)
    out[(e == 15) & ((c & 7) == 7)] = np.nan
    return out


def indexer_scores(qi, ki, w, rows=None):
    """All requested rows as a dict ``{(b, t): row}``; rows default to every (b, t)."""
    B, T = qi.shape[0], qi.shape[1]
    rows = range(T) if rows is None else rows
    return {(b, t): indexer_scores_row(qi, ki, w, b, t) for b in range(B) for t in rows}


# ----------------------------------------------------------------------------------------
# Top-k selection  [IC] paragraph 2 (select a small subset), [HS2] "Más precisión con
# menos memoria" (individual tokens, not blocks)
# ----------------------------------------------------------------------------------------

def topk_select_row(scores_row, k: int) -> np.ndarray:
    """The min(k, n) positions with the largest scores, ties to the lower position.

    Returned ascending and padded with -1 to length k (int32).  The order used is the
    total order (score descending, position ascending); -0.0 equals +0.0.
    Reading: every earlier position is a candidate, the window included (the window is
    added afterwards as a set union).
    """
    s = _f64(scores_row)
    n = s.shape[0]
    out = np.full(k, -1, dtype=np.int32)
    if k <= 0:
        return out
    if n <= k:
        out[:n] = np.arange(n, dtype=np.int32)
        return out
    kth = np.partition(s, n - k)[n - k]                 # the k-th largest value
    above = np.flatnonzero(s > kth)
    need = k - above.shape[0]
    ties = np.flatnonzero(s == kth)[:need]              # lowest positions among the ties
    sel = np.sort(np.concatenate([above, ties]))
    out[:] = sel.astype(np.int32)
    return out


def topk_select(scores: dict, k: int, B: int, T: int, rows=None) -> np.ndarray:
    """``idx[B, T, k]`` int32 for the requested rows (others stay -1)."""
    rows = range(T) if rows is None else rows
    idx = np.full((B, T, k), -1, dtype=np.int32)
    for b in range(B):
        for t in rows:
            idx[b, t] = topk_select_row(scores[(b, t)], k)
    return idx


def topk_boundary(scores_row, k: int):
    """(a, b): the k-th and (k+1)-th largest scores of a row with more than k entries,
    else None.  Used to decide which rows are within rounding distance of a tie."""
    s = _f64(scores_row)
    n = s.shape[0]
    if n <= k:
        return None
    srt = np.sort(s)[::-1]
    return float(srt[k - 1]), float(srt[k])


# ----------------------------------------------------------------------------------------
# Sparse attention over the selected set  [IC] paragraph 2, [HS2] "Dos niveles ..."
# (recent tokens forced into the set), [NSA] "Análisis Profundo" (shared KV per group)
# ----------------------------------------------------------------------------------------

def selected_mask_row(t: int, idx_row, window: int) -> np.ndarray:
    """Boolean mask over s = 0..t: s is attended iff s is a listed index in [0, t]
    or s lies in the window {t-window+1, ..., t}.  Each key counts once (a set)."""
    m = np.zeros(t + 1, dtype=bool)
    ids = np.asarray(idx_row, dtype=np.int64)
    ids = ids[(ids >= 0) & (ids <= t)]
    m[ids] = True
    if window > 0:
        m[max(0, t - window + 1): t + 1] = True
    return m


def _masked_softmax_attend(logits, mask, vals):
    """Dense logits [H, n] → masked softmax → (out [H, D], lse [H]).
    An empty mask gives out = 0 and lse = -inf."""
    H = logits.shape[0]
    if not mask.any():
        return np.zeros((H, vals.shape[-1])), np.full(H, NEG_INF)
    lg = np.where(mask[None, :], logits, NEG_INF)
    mx = lg.max(axis=1, keepdims=True)
    p = np.exp(lg - mx)                                  # exp(-inf) = 0 off the mask
    l = p.sum(axis=1, keepdims=True)
    out = np.matmul(p, vals) / l if vals.ndim == 2 else np.einsum("hs,hsd->hd", p, vals) / l
    lse = (mx + np.log(l))[:, 0]
    return out, lse


def sparse_attn(q, k, v, idx, window: int, scale: float, rows=None):
    """O[b,t,h,:] = Σ_{s∈S_t} softmax_s(scale·q[b,t,h]·k[b,s,g]) · v[b,s,g], g = h // (Hq/Hkv).

    S_t = {s ∈ idx[b,t] : 0 ≤ s ≤ t} ∪ {max(0, t-window+1), ..., t}.  Returns
    (O [B,R,Hq,D], LSE [B,Hq,R]) for the R requested rows (natural-log LSE).
    Reading: one selection per query row, shared by all heads of every KV group.
    """
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    rows = list(range(T)) if rows is None else list(rows)
    O = np.zeros((B, len(rows), Hq, D))
    LSE = np.zeros((B, Hq, len(rows)))
    for b in range(B):
        kb, vb = _f64(k[b]), _f64(v[b])
        for r, t in enumerate(rows):
            mask = selected_mask_row(t, idx[b, t], window)
            for g in range(Hkv):
                qh = _f64(q[b, t, g * G:(g + 1) * G])                 # [G, D]
                logits = scale * np.matmul(qh, kb[: t + 1, g].T)      # dense causal [G, t+1]
                o, lse = _masked_softmax_attend(logits, mask, vb[: t + 1, g])
                O[b, r, g * G:(g + 1) * G] = o
                LSE[b, g * G:(g + 1) * G, r] = lse
    return O, LSE


def sparse_attn_row(q_row, k_seq, v_seq, idx_row, t: int, window: int, scale: float):
    """One row of ``sparse_attn`` from explicit arrays: q_row [Hq, D] (the queries of row t),
    k_seq, v_seq [>= t+1, Hkv, D] (the sequence's keys and values), idx_row (its listed
    positions).  Returns (O [Hq, D], LSE [Hq]); the same dense masked softmax, for checks at
    sizes where whole query tensors do not fit the host."""
    Hq = q_row.shape[0]
    Hkv = k_seq.shape[1]
    G = Hq // Hkv
    mask = selected_mask_row(t, idx_row, window)
    O = np.zeros((Hq, q_row.shape[1]))
    LSE = np.zeros(Hq)
    for g in range(Hkv):
        qh = _f64(q_row[g * G:(g + 1) * G])
        logits = scale * np.matmul(qh, _f64(k_seq[: t + 1, g]).T)
        o, lse = _masked_softmax_attend(logits, mask, _f64(v_seq[: t + 1, g]))
        O[g * G:(g + 1) * G] = o
        LSE[g * G:(g + 1) * G] = lse
    return O, LSE


def sparse_attn_bwd(q, k, v, idx, window: int, scale: float, dout):
    """Gradients of ``sparse_attn`` with respect to q, k and v for the upstream gradient
    dout [B,T,Hq,D], on the same mask: with P[t,h,s] = softmax_s over S_t and
    dP[t,h,s] = dout[t,h] . v[s,g],

      dV[s,g] = Σ_t Σ_{h in g} P[t,h,s] dout[t,h]
      dS[t,h,s] = P[t,h,s] (dP[t,h,s] - Σ_{s'} P[t,h,s'] dP[t,h,s'])
      dQ[t,h] = scale Σ_s dS[t,h,s] k[s,g]
      dK[s,g] = scale Σ_t Σ_{h in g} dS[t,h,s] q[t,h]

    (the chain rule through the masked softmax; every unselected key has P = 0).
    Returns (dQ [B,T,Hq,D], dK [B,T,Hkv,D], dV [B,T,Hkv,D]) in float64.  [NSA] "Puntos
    Clave" reports the backward pass of sparse attention beside the forward."""
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    dQ = np.zeros((B, T, Hq, D))
    dK = np.zeros((B, T, Hkv, D))
    dV = np.zeros((B, T, Hkv, D))
    for b in range(B):
        kb, vb = _f64(k[b]), _f64(v[b])
        for t in range(T):
            mask = selected_mask_row(t, idx[b, t], window)
            if not mask.any():
                continue
            for g in range(Hkv):
                hs = slice(g * G, (g + 1) * G)
                qh = _f64(q[b, t, hs])                                   # [G, D]
                do = _f64(dout[b, t, hs])                                # [G, D]
                logits = scale * np.matmul(qh, kb[: t + 1, g].T)         # [G, t+1]
                lg = np.where(mask[None, :], logits, NEG_INF)
                p = np.exp(lg - lg.max(axis=1, keepdims=True))
                p = p / p.sum(axis=1, keepdims=True)                     # masked softmax
                dp = np.matmul(do, vb[: t + 1, g].T)                     # [G, t+1]
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dQ[b, t, hs] = scale * np.matmul(ds, kb[: t + 1, g])
                dK[b, : t + 1, g] += scale * np.matmul(ds.T, qh)
                dV[b, : t + 1, g] += np.matmul(p.T, do)
    return dQ, dK, dV


def _row_grads(q, k, v, idx, window: int, scale: float, dout, b: int, t: int, g: int, G: int):
    """The per-row pieces of ``sparse_attn_bwd`` for (b, t, KV group g), over the keys of
    S_t only: (keys [n], P [G, n], dS [G, n]); the softmax over S_t is the same as the
    masked dense one since every other key has P = 0."""
    keys = np.nonzero(selected_mask_row(t, idx[b, t], window))[0]
    hs = slice(g * G, (g + 1) * G)
    qh, do = _f64(q[b, t, hs]), _f64(dout[b, t, hs])
    logits = scale * np.matmul(qh, _f64(k[b, keys, g]).T)                  # [G, n]
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    dp = np.matmul(do, _f64(v[b, keys, g]).T)
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return keys, p, ds


def sparse_attn_bwd_rows(q, k, v, idx, window: int, scale: float, dout, rows):
    """dQ of ``sparse_attn_bwd`` for the requested rows only: [B, R, Hq, D] float64
    (dQ[t,h] = scale Σ_{s∈S_t} dS[t,h,s] k[s,g]); for sampled checks at sizes where the
    full gradient is out of reach."""
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    rows = list(rows)
    dQ = np.zeros((B, len(rows), Hq, D))
    for b in range(B):
        for r, t in enumerate(rows):
            for g in range(Hkv):
                keys, p, ds = _row_grads(q, k, v, idx, window, scale, dout, b, t, g, G)
                if keys.size:
                    dQ[b, r, g * G:(g + 1) * G] = scale * np.matmul(ds, _f64(k[b, keys, g]))
    return dQ


def sparse_attn_bwd_keys(q, k, v, idx, window: int, scale: float, dout, b: int, keys):
    """dK and dV of ``sparse_attn_bwd`` for the requested key positions of sequence b:
    ([R, Hkv, D], [R, Hkv, D]) float64, each summed over every row t whose S_t holds the
    key (the window rows t in [s, s + window) and the rows that list s with s <= t - window,
    each row once)."""
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    keys = list(keys)
    dK = np.zeros((len(keys), Hkv, D))
    dV = np.zeros((len(keys), Hkv, D))
    tt = np.arange(T)[:, None]
    for r, s in enumerate(keys):
        listed = np.nonzero(((idx[b] == s) & (s <= tt - window)).any(axis=1))[0]
        win = np.arange(s, min(T, s + window))
        for t in np.union1d(listed, win):
            for g in range(Hkv):
                ks, p, ds = _row_grads(q, k, v, idx, window, scale, dout, b, int(t), g, G)
                j = int(np.searchsorted(ks, s))
                hs = slice(g * G, (g + 1) * G)
                dK[r, g] += scale * np.matmul(ds[:, j], _f64(q[b, t, hs]))
                dV[r, g] += np.matmul(p[:, j], _f64(dout[b, t, hs]))
    return dK, dV


# ----------------------------------------------------------------------------------------
# Fixed-graph distance attention  [SLM] "Cómo eligen los tokens a quién escuchar"
# ----------------------------------------------------------------------------------------

def graph_offsets(local: int, n_pow2: int) -> np.ndarray:
    """The distinct backward offsets: 0 (the token itself), 1..local (near
    predecessors) and 2^j for j < n_pow2 (distances 1, 2, 4, 8, ...).  Sorted."""
    offs = set(range(0, local + 1)) | {1 << j for j in range(n_pow2)}
    return np.array(sorted(offs), dtype=np.int64)


def graph_neighbours(t: int, local: int, n_pow2: int) -> np.ndarray:
    """N(t) = {t - o : o in the offsets, o ≤ t}.  Reading: positions that would be
    negative are dropped (no future positions, no clamping to 0)."""
    o = graph_offsets(local, n_pow2)
    return np.sort(t - o[o <= t])


def graph_neighbour_count(t: int, local: int, n_pow2: int) -> int:
    """Closed form of |N(t)|: min(t, local) + 1 local ones (self included) plus the
    power-of-two offsets beyond ``local`` that still reach position ≥ 0."""
    far = sum(1 for j in range(n_pow2) if (1 << j) > local and (1 << j) <= t)
    return min(t, local) + 1 + far


def graph_attn(cq, ck, v, bias, tau: float, local: int, n_pow2: int, rows=None):
    """O[b,t,h,:] = Σ_{s∈N(t)} softmax_s(-tau·‖cq[b,t,h]-ck[b,s,h]‖² + bias[h]) · v[b,s,h,:].

    Dense over s ≤ t, then the fixed-graph mask.  Returns (O [B,R,H,D], LSE [B,H,R]).
    Reading: one coordinate triple per head for queries and keys; no dot-product term
    and no extra scale (the workload gives the whole logit).
    """
    B, T, H, D = v.shape
    rows = list(range(T)) if rows is None else list(rows)
    O = np.zeros((B, len(rows), H, D))
    LSE = np.zeros((B, H, len(rows)))
    bias = _f64(bias)
    for b in range(B):
        ckb, vb = _f64(ck[b]), _f64(v[b])
        for r, t in enumerate(rows):
            mask = np.zeros(t + 1, dtype=bool)
            mask[graph_neighbours(t, local, n_pow2)] = True
            cqt = _f64(cq[b, t])                                      # [H, 3]
            diff = cqt[None, :, :] - ckb[: t + 1]                     # [t+1, H, 3]
            dist2 = np.sum(diff * diff, axis=2).T                     # [H, t+1]
            logits = -tau * dist2 + bias[:, None]
            vals = np.transpose(vb[: t + 1], (1, 0, 2))               # [H, t+1, D]
            o, lse = _masked_softmax_attend(logits, mask, vals)
            O[b, r] = o
            LSE[b, :, r] = lse
    return O, LSE


# ----------------------------------------------------------------------------------------
# Block-selected decode  [NSA] "Puntos Clave" (coarse compression, blockwise selection,
# sliding window), [STAR] paragraph 3 (combine of partial attentions)
# ----------------------------------------------------------------------------------------

def block_meanpool(kcache, lens, block: int) -> np.ndarray:
    """kbar[b, j] = (1/block) Σ_{i<block} K[b, block·j + i] for complete blocks
    j < lens[b] // block; the other rows are NaN.  Shape [B, Lmax//block, Hkv, D]."""
    B, Lmax, Hkv, D = kcache.shape
    nb = Lmax // block
    kbar = np.full((B, nb, Hkv, D), np.nan)
    for b in range(B):
        nfull = int(lens[b]) // block
        if nfull:
            kb = _f64(kcache[b, : nfull * block]).reshape(nfull, block, Hkv, D)
            kbar[b, :nfull] = kb.mean(axis=1)
    return kbar


def decode_select(q, kbar, lens, top_blocks: int, block: int) -> np.ndarray:
    """sel[b, g, :]: the top ``top_blocks`` complete blocks of sequence b for KV head g by
    score_j = Σ_{h in group g} q[b,h,:] · kbar[b,j,g,:], ties to the lower j, ascending,
    padded with -1.  Reading: raw dot product (no scale, no softmax); every complete
    block is a candidate, including those the window also covers."""
    B, Hq, D = q.shape
    Hkv = kbar.shape[2]
    G = Hq // Hkv
    sel = np.full((B, Hkv, top_blocks), -1, dtype=np.int32)
    for b in range(B):
        nfull = int(lens[b]) // block
        for g in range(Hkv):
            qg = _f64(q[b, g * G:(g + 1) * G])                          # [G, D]
            scores = np.matmul(qg, kbar[b, :nfull, g].T).sum(axis=0)   # Σ_h q_h·kbar_j
            sel[b, g] = topk_select_row(scores, top_blocks)
    return sel


def decode_token_mask(sel_row, L: int, block: int, window: int) -> np.ndarray:
    """U over s = 0..L-1: tokens of the selected blocks before the window, united with
    the last ``window`` tokens [max(0, L-window), L).  Each token once."""
    m = np.zeros(L, dtype=bool)
    wstart = max(0, L - window)
    for j in np.asarray(sel_row):
        if j < 0:
            continue
        lo, hi = int(j) * block, min(int(j) * block + block, wstart)
        if hi > lo:
            m[lo:hi] = True
    m[wstart:L] = True
    return m


def sparse_decode(q, kcache, vcache, lens, block: int, top_blocks: int, window: int,
                  scale: float, kbar=None):
    """One decode step per sequence: dense attention of q[b,h] over the cache
    positions [0, lens[b]) under the mask U (selected blocks ∪ window).

    Returns (O [B,Hq,D], LSE [B,Hq], sel [B,Hkv,top_blocks])."""
    B, Hq, D = q.shape
    Hkv = kcache.shape[2]
    G = Hq // Hkv
    if kbar is None:
        kbar = block_meanpool(kcache, lens, block)
    sel = decode_select(q, kbar, lens, top_blocks, block)
    O = np.zeros((B, Hq, D))
    LSE = np.zeros((B, Hq))
    for b in range(B):
        L = int(lens[b])
        for g in range(Hkv):
            mask = decode_token_mask(sel[b, g], L, block, window)
            qg = _f64(q[b, g * G:(g + 1) * G])
            kb = _f64(kcache[b, :L, g])
            vb = _f64(vcache[b, :L, g])
            logits = scale * np.matmul(qg, kb.T)                        # dense [G, L]
            o, lse = _masked_softmax_attend(logits, mask, vb)
            O[b, g * G:(g + 1) * G] = o
            LSE[b, g * G:(g + 1) * G] = lse
    return O, LSE, sel


# ----------------------------------------------------------------------------------------
# NSA's three branches  [NSA] "Puntos Clave" (hierarchical sparsity: coarse token
# compression, fine-grained selection, sliding window) and "Análisis Profundo"
# (compression and selection combined; one KV fetch per GQA group)
# ----------------------------------------------------------------------------------------

def cmp_attn(q, kbar, vbar, block: int, scale: float, rows=None):
    """Compressed branch: O[b,t,h] = Σ_j softmax_j(scale·q[b,t,h]·kbar[b,j,g]) · vbar[b,j,g]
    over the complete blocks whose last token is at or before t, j < (t+1) // block.

    Returns (O [B,R,Hq,D], LSE [B,Hq,R]); a row with no complete block gets O = 0 and
    LSE = -inf.  Reading: the compressed keys and values are the block means of K and V
    (the decode path's pooling, ``block_meanpool``), and a block joins once it is complete.
    """
    B, T, Hq, D = q.shape
    Hkv = kbar.shape[2]
    G = Hq // Hkv
    rows = list(range(T)) if rows is None else list(rows)
    O = np.zeros((B, len(rows), Hq, D))
    LSE = np.zeros((B, Hq, len(rows)))
    for b in range(B):
        for r, t in enumerate(rows):
            nfull = (t + 1) // block
            for g in range(Hkv):
                qh = _f64(q[b, t, g * G:(g + 1) * G])
                kb = _f64(kbar[b, :nfull, g])
                logits = scale * np.matmul(qh, kb.T)                       # [G, nfull]
                o, lse = _masked_softmax_attend(logits, np.ones(nfull, dtype=bool),
                                                _f64(vbar[b, :nfull, g]))
                O[b, r, g * G:(g + 1) * G] = o
                LSE[b, g * G:(g + 1) * G, r] = lse
    return O, LSE


def block_select_rows(q, kbar, block: int, top_blocks: int, rows=None) -> np.ndarray:
    """sel[b, r, :]: for query row t = rows[r], the top ``top_blocks`` complete blocks
    (j < (t+1) // block) by score_j = Σ_h q[b,t,h] · kbar[b,j,g(h)] over every query head,
    ties to the lower j, ascending, padded with -1.  Reading: one selection per query row
    shared by all heads, as the token-level path shares its top-k (for one KV head this
    is the per-group rule of the decode path); raw dot products, no scale."""
    B, T, Hq, D = q.shape
    Hkv = kbar.shape[2]
    G = Hq // Hkv
    rows = list(range(T)) if rows is None else list(rows)
    sel = np.full((B, len(rows), top_blocks), -1, dtype=np.int32)
    for b in range(B):
        for r, t in enumerate(rows):
            nfull = (t + 1) // block
            scores = np.zeros(nfull)
            for g in range(Hkv):
                qg = _f64(q[b, t, g * G:(g + 1) * G])
                scores += np.matmul(qg, _f64(kbar[b, :nfull, g]).T).sum(axis=0)
            sel[b, r] = topk_select_row(scores, top_blocks)
    return sel


def block_tokens(sel_row, block: int) -> np.ndarray:
    """The token positions of the listed blocks (-1 entries skipped), ascending, padded
    with -1 to len(sel_row) * block entries."""
    out = np.full(len(sel_row) * block, -1, dtype=np.int32)
    toks = sorted(int(j) * block + i for j in np.asarray(sel_row) if j >= 0 for i in range(block))
    out[: len(toks)] = toks
    return out


def nsa_combine(gates, o_cmp, o_slc, o_win) -> np.ndarray:
    """O = g0·O_cmp + g1·O_slc + g2·O_win per (token, head); gates [..., Hq, 3].
    Reading: the page names the three branches but not how they are joined; NSA gates
    them, and the gates (learned from the query in NSA) are inputs here."""
    g = _f64(gates)
    return g[..., 0:1] * o_cmp + g[..., 1:2] * o_slc + g[..., 2:3] * o_win


def nsa_prefill(q, k, v, gates, block: int, top_blocks: int, window: int, scale: float,
                rows=None):
    """The three branches for every requested row, each its own softmax: compressed
    (``cmp_attn``), selected (the tokens of the row's ``block_select_rows`` blocks, all
    before or at t since the blocks are complete; no window), window (the last
    ``window`` tokens, self included); then ``nsa_combine``.
    Returns (O [B,R,Hq,D], (O_cmp, O_slc, O_win), sel [B,R,top_blocks])."""
    B, T, Hq, D = q.shape
    rows = list(range(T)) if rows is None else list(rows)
    lens = np.full(B, T)
    kbar = block_meanpool(k, lens, block)
    vbar = block_meanpool(v, lens, block)
    o_cmp, _ = cmp_attn(q, kbar, vbar, block, scale, rows)
    sel = block_select_rows(q, kbar, block, top_blocks, rows)
    idx = np.full((B, T, top_blocks * block), -1, dtype=np.int32)
    for b in range(B):
        for r, t in enumerate(rows):
            idx[b, t] = block_tokens(sel[b, r], block)
    o_slc, _ = sparse_attn(q, k, v, idx, 0, scale, rows)
    o_win, _ = sparse_attn(q, k, v, np.full((B, T, 1), -1, dtype=np.int32), window, scale, rows)
    g = np.stack([_f64(gates[:, t]) for t in rows], axis=1)
    return nsa_combine(g, o_cmp, o_slc, o_win), (o_cmp, o_slc, o_win), sel


def nsa_decode(q, kcache, vcache, lens, gates, block: int, top_blocks: int, window: int,
               scale: float, kbar=None, vbar=None):
    """One decode step per sequence with the three branches of the query at position
    lens[b]-1: compressed (every complete block j < lens[b] // block), selected (all tokens
    of the ``decode_select`` blocks of the query's KV group), window ([L-window, L)); each
    its own softmax, then ``nsa_combine`` with gates [B,Hq,3].
    Returns (O [B,Hq,D], (O_cmp, O_slc, O_win), sel [B,Hkv,top_blocks])."""
    B, Hq, D = q.shape
    Hkv = kcache.shape[2]
    G = Hq // Hkv
    if kbar is None:
        kbar = block_meanpool(kcache, lens, block)
    if vbar is None:
        vbar = block_meanpool(vcache, lens, block)
    sel = decode_select(q, kbar, lens, top_blocks, block)
    outs = [np.zeros((B, Hq, D)) for _ in range(3)]
    for b in range(B):
        L = int(lens[b])
        nfull = L // block
        for g in range(Hkv):
            qg = _f64(q[b, g * G:(g + 1) * G])
            hs = slice(g * G, (g + 1) * G)
            lc = scale * np.matmul(qg, _f64(kbar[b, :nfull, g]).T)
            outs[0][b, hs], _ = _masked_softmax_attend(lc, np.ones(nfull, dtype=bool),
                                                       _f64(vbar[b, :nfull, g]))
            kb, vb = _f64(kcache[b, :L, g]), _f64(vcache[b, :L, g])
            logits = scale * np.matmul(qg, kb.T)                              # dense [G, L]
            m_slc = np.zeros(L, dtype=bool)
            for j in sel[b, g]:
                if j >= 0:
                    m_slc[int(j) * block: int(j) * block + block] = True
            m_win = np.zeros(L, dtype=bool)
            m_win[max(0, L - window): L] = True
            outs[1][b, hs], _ = _masked_softmax_attend(logits, m_slc, vb)
            outs[2][b, hs], _ = _masked_softmax_attend(logits, m_win, vb)
    return nsa_combine(gates, *outs), tuple(outs), sel


# ----------------------------------------------------------------------------------------
# Cross-layer index reuse  [IC] paragraph 4 (F layers index and cache, S layers reuse)
# ----------------------------------------------------------------------------------------

def indexcache_prefill(qi, ki, w, layers, pattern: str, topk: int, window: int,
                       scale: float, rows=None):
    """Run the layer pattern (e.g. "FSSS"): an F layer computes indexer scores and the
    top-k indices and caches them; an S layer reuses the indices of the nearest
    preceding F layer.  ``layers`` is a list of dicts with q, k, v.  Returns the list of
    (O, LSE) per layer and the number of indexer evaluations made."""
    if not pattern or pattern[0] != "F":
        raise ValueError("the first layer must compute indices (F)")
    B, T = qi.shape[0], qi.shape[1]
    rows_l = list(range(T)) if rows is None else list(rows)
    idx = None
    n_index = 0
    outs = []
    for kind, lay in zip(pattern, layers):
        if kind == "F":
            sc = indexer_scores(qi, ki, w, rows_l)
            idx = topk_select(sc, topk, B, T, rows_l)
            n_index += 1
        outs.append(sparse_attn(lay["q"], lay["k"], lay["v"], idx, window, scale, rows_l))
    return outs, n_index
