"""Low-rank index, index logits and the top-p / top-k selector.

"Full Attention Strikes Back" summary (RTPurbo):
  * Methodology item 2: a projector to r (= 16) dims is applied to query and
    key features *before* RoPE; relevance is estimated in that subspace.
  * Methodology item 3: the dynamic top-p selector accumulates attention mass
    in the low-dim space until the cumulative threshold p (e.g. 0.9) is met;
    static top-k is the fixed-budget alternative it is compared with.
"Autonomia de Cabecas (AoH)" summary, Methodology item 4: under GQA, per-head
scores are aggregated to the KV group by their mean.

Readings (the pages are silent on these):
  * one projector per KV group, applied to both sides (P_q = P_k allowed);
  * logit l_j = qbar . k_idx_j / sqrt(r) (standard scaled dot product in r dims);
  * qbar = mean of the group's retrieval query heads' index queries, so one set
    per (sequence, KV group); the mean of the heads' logits equals the logit of
    the mean query;
  * order = logit descending, then position ascending (ties to the earlier
    token);
  * top-p: the smallest prefix of that order whose softmax mass is >= p; p >= 1
    takes every token; the prefix length is then raised to ``min_tokens`` and
    capped at n; top-k: prefix length min(k, n);
  * the index keys are stored in the workload element type (bf16 or fp32)
    and the index query in fp32, and selection is decided on those stored
    values.
"""
import numpy as np

from .numerics import round_store, round_fp32


def index_keys(k_pre, proj_k, store="bf16"):
    """k_idx[j] = P_k k_pre[j] (fp64), rounded once to the stored type.

    k_pre [..., n, d], proj_k [r, d] -> [..., n, r]."""
    k = np.asarray(k_pre, np.float64) @ np.asarray(proj_k, np.float64).T
    return round_store(k, store)


def index_query(q_pre_heads, proj_q):
    """Per-head index queries P_q q_pre (stored fp32): [G, d] -> [G, r]."""
    q = np.asarray(q_pre_heads, np.float64) @ np.asarray(proj_q, np.float64).T
    return round_fp32(q)


def index_logits(q_idx_heads, k_idx, r=None):
    """l_j = mean_h(q_idx[h]) . k_idx[j] / sqrt(r)   ([G, r], [n, r] -> [n])."""
    q_idx_heads = np.asarray(q_idx_heads, np.float64)
    r = q_idx_heads.shape[-1] if r is None else r
    qbar = q_idx_heads.mean(axis=0)
    return (np.asarray(k_idx, np.float64) @ qbar) / np.sqrt(r)


def order(logits):
    """Positions sorted by (logit desc, position asc): the ranking both
    selectors cut."""
    logits = np.asarray(logits, np.float64)
    pos = np.arange(logits.shape[0])
    return np.lexsort((pos, -logits))


def select_prefix(logits, m):
    """The first m tokens of the (logit desc, position asc) order, ascending."""
    return np.sort(order(logits)[:m]).astype(np.int64)


def _topp_count(logits, p):
    logits = np.asarray(logits, np.float64)
    n = logits.shape[0]
    if p >= 1.0:
        return n
    ranked = order(logits)
    w = np.exp(logits - logits.max())
    cs = np.cumsum(w[ranked] / w.sum())
    hit = np.nonzero(cs >= p)[0]
    return int(hit[0]) + 1 if hit.size else n


def select_topp(logits, p, min_tokens=0):
    """Top-p set (ascending positions) and its size m."""
    n = len(logits)
    m = min(n, max(_topp_count(logits, p), int(min_tokens)))
    return select_prefix(logits, m), m


def select_topk(logits, k):
    n = len(logits)
    m = min(int(k), n)
    return select_prefix(logits, m), m


def topp_margin(logits, p):
    """Mass distance of the top-p cut from p: min(cs_m - p, p - cs_{m-1}).

    Used to draw inputs whose cut cannot move under last-place rounding."""
    logits = np.asarray(logits, np.float64)
    ranked = order(logits)
    w = np.exp(logits - logits.max())
    cs = np.cumsum(w[ranked] / w.sum())
    m = _topp_count(logits, p)
    hi = cs[m - 1] - p
    lo = p - (cs[m - 2] if m >= 2 else 0.0)
    return float(min(hi, lo))


def cut_gap(logits, m):
    """Logit gap between the last selected and the first unselected token."""
    logits = np.asarray(logits, np.float64)
    if m >= len(logits) or m <= 0:
        return np.inf
    ranked = order(logits)
    return float(logits[ranked[m - 1]] - logits[ranked[m]])
