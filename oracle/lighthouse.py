"""Pyramid-selection chunked prefill (Lighthouse attention, forward only).

"Lighthouse Attention" summary, Methodology:
  2A. a symmetric mean pyramid over Q, K and V with L levels and factor p;
      level 0 is full resolution and each level-l entry summarises p
      consecutive level-(l-1) entries;
  2B. a parameter-free score from the l2 norms of the projected Q and K of
      each entry; coarser levels inherit the max of the finer scores they
      cover; a top-K over all levels jointly picks the entries;
  2C. the chosen entries form a causally consistent dense subsequence,
      ordinary attention runs on it, and a scatter writes the outputs back to
      their original positions.

Readings (the summary leaves these open):
  * score of a level-0 entry = |q|^2 + |k|^2 (the squared l2 norm of (q, k);
    monotone in the norm, so the same ranking) - parity unpinned by the pages;
  * a coarse score is the max of its children's scores (pure inheritance);
  * selection is per block of ``q_block`` level-0 queries: the candidates are
    the entries whose span ends before the block starts; ranking is score
    descending, then level ascending, then index ascending; at most K are
    taken (all when fewer are visible);
  * each query of block b also attends, causally, to the block's own level-0
    keys, and a query's output is written to its own row;
  * symmetric queries (2A, 2C): a coarse query entry of level l >= 1 whose
    span lies in block b attends to the same selected entries and to the
    block's own level-l keys up to itself - the level-0 rule applied to level
    l - and its output goes back to its own slot of an output pyramid (the
    inverse of the gather).  How a model merges the levels of that pyramid is
    not the attention's to decide and is not modelled;
  * each stored coarse level is the exact mean of its level-0 rows rounded
    once to the workload element type.
"""
import numpy as np


from .numerics import round_store


def pyramid_levels(X, levels, factor, store="bf16"):
    """[X_1, ..., X_{L-1}] for X [N, d]: X_l[j] = mean of p entries of X_{l-1}.

    The p children's sums are added (the sum over the entry's p^l level-0
    rows) and divided once by p^l, so the mean of means carries no rounding
    of the unrounded intermediate levels; each level is rounded once for
    storage."""
    cur = np.asarray(X, np.float64)
    out = []
    width = 1
    for _ in range(1, levels):
        m = cur.shape[0] // factor
        cur = cur[: m * factor].reshape(m, factor, -1).sum(axis=1)
        width *= factor
        mean = cur / width
        out.append(round_store(mean, store) if store else mean)
    return out


def pyramid_scores(Q, K, levels, factor):
    """[s_0, s_1, ...]: s_0[i] = |q_i|^2 + |k_i|^2, s_l[j] = max of its p
    children in s_{l-1}."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    s = (Q * Q).sum(axis=1) + (K * K).sum(axis=1)
    out = [s]
    for _ in range(1, levels):
        m = s.shape[0] // factor
        s = s[: m * factor].reshape(m, factor).max(axis=1)
        out.append(s)
    return out


def level_offsets(N, levels, factor):
    """Offset of each level in the flat entry numbering (level 0 first)."""
    offs, o, m = [], 0, N
    for _ in range(levels):
        offs.append(o)
        o += m
        m //= factor
    return offs


def visible_entries(block, N, levels, factor, q_block):
    """(level, index) pairs whose span ends before position q_block*block."""
    start = q_block * block
    vis = []
    m = N
    for lvl in range(levels):
        span = factor ** lvl
        cnt = min(m, start // span)
        vis.extend((lvl, j) for j in range(cnt))
        m //= factor
    return vis


def block_select(scores, block, N, levels, factor, q_block, top_k):
    """Flat ids of the top-K visible entries for one query block, as a set
    sorted by (span end, level, index)."""
    start = q_block * block
    lv, ix, sc = [], [], []
    for lvl in range(levels):
        cnt = min(len(scores[lvl]), start // factor ** lvl)
        lv.append(np.full(cnt, lvl))
        ix.append(np.arange(cnt))
        sc.append(np.asarray(scores[lvl][:cnt], np.float64))
    lv, ix, sc = np.concatenate(lv), np.concatenate(ix), np.concatenate(sc)
    if lv.size == 0:
        return np.zeros(0, np.int64)
    order = np.lexsort((ix, lv, -sc))[:top_k]
    lv, ix = lv[order], ix[order]
    # canonical order of the chosen set: span end, then level, then index
    canon = np.lexsort((ix, lv, (ix + 1) * factor ** lv))
    offs = np.asarray(level_offsets(N, levels, factor))
    return (offs[lv[canon]] + ix[canon]).astype(np.int64)


def entry_rows(flat, X0, coarse, N, levels, factor):
    """Rows of level-0 X0 or of the coarse levels for flat entry ids."""
    offs = level_offsets(N, levels, factor)
    rows = []
    for f in np.asarray(flat).tolist():
        lvl = max(l for l in range(levels) if offs[l] <= f)
        j = f - offs[lvl]
        rows.append(np.asarray(X0[j] if lvl == 0 else coarse[lvl - 1][j], np.float64))
    return np.stack(rows) if rows else np.zeros((0, np.asarray(X0).shape[1]))


def prefill_block(Q, K, V, kc, vc, sel, block, q_block, levels, factor, scale=None):
    """Outputs [rows, d] of the queries of one block: each attends to the
    selected entries plus the block's own level-0 keys up to itself."""
    N, d = Q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    Ks = entry_rows(sel, K, kc, N, levels, factor)
    Vs = entry_rows(sel, V, vc, N, levels, factor)
    lo = q_block * block
    hi = min(N, lo + q_block)
    Qb = np.asarray(Q[lo:hi], np.float64)
    Kt = np.concatenate([Ks, np.asarray(K[lo:hi], np.float64)])
    Vt = np.concatenate([Vs, np.asarray(V[lo:hi], np.float64)])
    # row u sees every selected entry and the block's keys lo .. lo + u
    a = (Qb @ Kt.T) * scale
    rows = np.arange(hi - lo)[:, None]
    cols = np.arange(hi - lo)[None, :]
    a[:, len(Ks):] = np.where(cols <= rows, a[:, len(Ks):], -np.inf)
    w = np.exp(a - a.max(axis=1, keepdims=True))
    return (w / w.sum(axis=1, keepdims=True)) @ Vt


def prefill(Q, K, V, levels, factor, q_block, top_k, store="bf16", blocks=None):
    """Whole pipeline for one (sequence, head): pyramid, scores, per-block
    selection and attention.  Returns (out [N, d] with unvisited blocks as
    NaN, coarse K levels, coarse V levels, selections {block: flat ids})."""
    Q = np.asarray(Q, np.float64)
    N, d = Q.shape
    kc = pyramid_levels(K, levels, factor, store)
    vc = pyramid_levels(V, levels, factor, store)
    sc = pyramid_scores(Q, K, levels, factor)
    nb = (N + q_block - 1) // q_block
    blocks = range(nb) if blocks is None else blocks
    out = np.full((N, d), np.nan)
    sels = {}
    for b in blocks:
        sel = block_select(sc, b, N, levels, factor, q_block, top_k)
        sels[b] = sel
        lo = q_block * b
        out[lo:min(N, lo + q_block)] = prefill_block(Q, K, V, kc, vc, sel, b, q_block,
                                                     levels, factor)
    return out, kc, vc, sels


def coarse_block(QC, KC, VC, K, V, sel, block, q_block, levels, factor, scale=None):
    """Outputs of the coarse query entries of one block, one [n_l, d] array
    per level l = 1 .. L-1 (n_l = the block's level-0 length / p^l): entry j
    of level l in the block attends to the block's selected entries ``sel``
    (rows of level-0 K/V or of the coarse levels KC/VC) and to the block's own
    level-l keys up to and including itself.  QC, KC, VC: coarse levels 1 ..
    L-1 as lists of [N / p^l, d] arrays."""
    N, d = np.asarray(K).shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    Ks = entry_rows(sel, K, KC, N, levels, factor)
    Vs = entry_rows(sel, V, VC, N, levels, factor)
    lo0 = q_block * block
    hi0 = min(N, lo0 + q_block)
    outs = []
    for lvl in range(1, levels):
        span = factor ** lvl
        lo, hi = lo0 // span, hi0 // span
        Qb = np.asarray(QC[lvl - 1][lo:hi], np.float64)
        Kt = np.concatenate([Ks, np.asarray(KC[lvl - 1][lo:hi], np.float64)])
        Vt = np.concatenate([Vs, np.asarray(VC[lvl - 1][lo:hi], np.float64)])
        a = (Qb @ Kt.T) * scale
        rows = np.arange(hi - lo)[:, None]
        cols = np.arange(hi - lo)[None, :]
        a[:, len(Ks):] = np.where(cols <= rows, a[:, len(Ks):], -np.inf)
        w = np.exp(a - a.max(axis=1, keepdims=True))
        outs.append((w / w.sum(axis=1, keepdims=True)) @ Vt)
    return outs


def prefill_coarse(Q, K, V, levels, factor, q_block, top_k, store="bf16", blocks=None):
    """The coarse queries' outputs for one (sequence, head), scattered back to
    their slots: [O_1, ..., O_{L-1}] with O_l [N / p^l, d] (rows of blocks not
    visited are NaN), on the same pyramid and selections as ``prefill``."""
    Q = np.asarray(Q, np.float64)
    N, d = Q.shape
    qc = pyramid_levels(Q, levels, factor, store)
    kc = pyramid_levels(K, levels, factor, store)
    vc = pyramid_levels(V, levels, factor, store)
    sc = pyramid_scores(Q, K, levels, factor)
    nb = (N + q_block - 1) // q_block
    blocks = range(nb) if blocks is None else blocks
    outs = [np.full((N // factor ** l, d), np.nan) for l in range(1, levels)]
    for b in blocks:
        sel = block_select(sc, b, N, levels, factor, q_block, top_k)
        per = coarse_block(qc, kc, vc, K, V, sel, b, q_block, levels, factor)
        for lvl in range(1, levels):
            span = factor ** lvl
            lo = q_block * b // span
            outs[lvl - 1][lo:lo + per[lvl - 1].shape[0]] = per[lvl - 1]
    return outs
