"""Backward pass of the pyramid-selection prefill (Lighthouse attention).

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Lighthouse Attention" summary, Methodology 2B-2C: the top-K selection is
discrete and gets no gradient (no straight-through estimator, no auxiliary
loss); gradients pass only through the gather, the dense attention on the
gathered subsequence and the scatter back, and so reach Q, K and V (and the
projections behind them).  2A: every coarse entry is the mean of the p
entries below it, so the gradient of an entry at level l reaches each of the
p^l level-0 rows it covers divided by p^l.

Readings (the summary leaves these open; the forward readings of the
``lighthouse`` module stand):
  * only level-0 queries attend, so the coarse Q levels receive no gradient
    and dQ is the level-0 query gradient alone;
  * the rounding of a stored coarse level to the workload element type is
    taken as the identity for the gradient (the mean is differentiated);
  * an entry chosen by several blocks gets the sum of the blocks'
    contributions (the scatter adds).

The per-block gradient is the plain softmax-attention backward, written from
its definition: with a = scale q k^T (masked), P = softmax(a) row by row,
O = P V and the upstream gradient dO,
  dV = P^T dO,  dP = dO V^T,  dA_ij = P_ij (dP_ij - sum_k P_ik dP_ik),
  dQ = scale dA K,  dK = scale dA^T Q.
"""
import numpy as np

from .lighthouse import (block_select, entry_rows, level_offsets, pyramid_levels,
                         pyramid_scores)


def block_grads(Q, K, V, kc, vc, sel, block, q_block, levels, factor, dO, scale=None):
    """Gradients of one query block: (dQ rows, dK and dV of the selected
    entries in ``sel`` order, dK and dV of the block's own level-0 keys, and
    the probabilities P and score gradients dA [rows, len(sel) + rows])."""
    N, d = Q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    Ks = entry_rows(sel, K, kc, N, levels, factor)
    Vs = entry_rows(sel, V, vc, N, levels, factor)
    lo = q_block * block
    hi = min(N, lo + q_block)
    Qb = np.asarray(Q[lo:hi], np.float64)
    dOb = np.asarray(dO[lo:hi], np.float64)
    Kt = np.concatenate([Ks, np.asarray(K[lo:hi], np.float64)])
    Vt = np.concatenate([Vs, np.asarray(V[lo:hi], np.float64)])
    a = (Qb @ Kt.T) * scale
    rows = np.arange(hi - lo)[:, None]
    cols = np.arange(hi - lo)[None, :]
    a[:, len(Ks):] = np.where(cols <= rows, a[:, len(Ks):], -np.inf)
    w = np.exp(a - a.max(axis=1, keepdims=True))
    P = w / w.sum(axis=1, keepdims=True)
    dP = dOb @ Vt.T
    dA = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    dQb = scale * (dA @ Kt)
    dKt = scale * (dA.T @ Qb)
    dVt = P.T @ dOb
    n = len(Ks)
    return dQb, dKt[:n], dVt[:n], dKt[n:], dVt[n:], P, dA


def pyramid_backward(dflat, N, levels, factor):
    """Level-0 gradient [N, d] from gradients of the flat entries (level 0
    first, as ``level_offsets`` numbers them): each level-l entry's gradient
    goes to every level-0 row it covers, divided by p^l."""
    dflat = np.asarray(dflat, np.float64)
    offs = level_offsets(N, levels, factor)
    out = dflat[:N].copy()
    m = N
    for lvl in range(1, levels):
        m //= factor
        span = factor ** lvl
        g = dflat[offs[lvl]:offs[lvl] + m] / span
        out[: m * span] += np.repeat(g, span, axis=0)
    return out


def n_entries(N, levels, factor):
    """Number of flat entries over all levels."""
    return sum(N // factor ** lvl for lvl in range(levels))


def prefill_grads(Q, K, V, dO, levels, factor, q_block, top_k, store="bf16", sels=None,
                  scale=None):
    """Gradients (dQ, dK, dV) [N, d] of sum(O * dO) for one (sequence, head),
    O being the pyramid prefill's output.  ``sels``: {block: flat ids}, the
    selections to differentiate through (the forward's own when None)."""
    Q = np.asarray(Q, np.float64)
    N, d = Q.shape
    kc = pyramid_levels(K, levels, factor, store)
    vc = pyramid_levels(V, levels, factor, store)
    nb = (N + q_block - 1) // q_block
    if sels is None:
        sc = pyramid_scores(Q, K, levels, factor)
        sels = {b: block_select(sc, b, N, levels, factor, q_block, top_k) for b in range(nb)}
    E = n_entries(N, levels, factor)
    dQ = np.zeros((N, d))
    dKf = np.zeros((E, d))
    dVf = np.zeros((E, d))
    for b in range(nb):
        sel = np.asarray(sels[b], np.int64)
        dq, dks, dvs, dko, dvo, _, _ = block_grads(Q, K, V, kc, vc, sel, b, q_block, levels,
                                                   factor, dO, scale)
        lo = q_block * b
        hi = min(N, lo + q_block)
        dQ[lo:hi] = dq
        np.add.at(dKf, sel, dks)
        np.add.at(dVf, sel, dvs)
        dKf[lo:hi] += dko
        dVf[lo:hi] += dvo
    return dQ, pyramid_backward(dKf, N, levels, factor), pyramid_backward(dVf, N, levels, factor)
