"""Exact softmax attention restricted to a token set.

HGA summary, Core mechanism item 4 (and Contribution 2): once tokens are
chosen, the output is the ordinary softmax attention over exactly those
tokens' keys and values, with no synthetic values mixed in.  Lighthouse
summary 2C runs stock dense attention on the gathered subsequence.  The
definition written out: for query q and visible set T,

    a_j = q . k_j * scale,  pi_j = exp(a_j - max a) / sum_i exp(a_i - max a),
    o   = sum_{j in T} pi_j v_j,

with scale = 1/sqrt(d) (reading: standard scaled dot product).
"""
import numpy as np


def attend(q, K, V, scale=None):
    """o = softmax(K q * scale) V for one query q [d] over rows K, V [T, d]."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    a = (K @ q) * scale
    w = np.exp(a - a.max())
    return (w / w.sum()) @ V


def attend_heads(Q, K, V, scale=None):
    """Several query heads [G, d] against one shared key/value set."""
    return np.stack([attend(q, K, V, scale) for q in np.asarray(Q)])


def dense_causal(Q, K, V, scale=None):
    """Dense causal attention for queries at positions 0..N-1 (row i sees
    keys 0..i).  Used as the closed form that full selections reduce to."""
    Q = np.asarray(Q, np.float64)
    N = Q.shape[0]
    out = np.empty_like(Q)
    for i in range(N):
        out[i] = attend(Q[i], K[: i + 1], V[: i + 1], scale)
    return out
