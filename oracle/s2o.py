"""Monotone-gain early stop over score-ordered candidates.

"S2O" summary, Methodology 2 and 3: candidate blocks are visited in
descending estimated importance; the marginal gain in attention mass that each
visited block adds is compared, relative to the mass accumulated so far, with a
threshold tau, and the computation ends once it falls below it.  A first
pass attends densely over a local window to initialise the online-softmax
state (m, l, acc); the second pass resumes that state over the candidates.

Readings (the page fixes none of these numbers for decode):
* candidates: the retrieval group's top-k tokens by index logit (the same
  selection as top-k), visited in (logit desc, position asc) order;
* first pass: the local rule's tokens (sinks + window) of the decode query;
  candidates that lie there are not visited again;
* blocks: consecutive runs of 64 visited candidates;
* rule, per query head: after a block, with S_block the block's sum of
  exp(score) and S_before the sum over everything attended before it,
  stop when S_block / S_before < tau; the block that triggers the stop is
  kept (its scores were computed to evaluate the rule);
* GQA heads share their group's candidates and order; each head stops on its
  own scores.
"""
import numpy as np

BLOCK = 64


def s2o_order(logits, candidates):
    """Candidates (positions) in (logit desc, position asc) order."""
    candidates = np.asarray(candidates, np.int64)
    lg = np.asarray(logits, np.float64)[candidates]
    return candidates[np.lexsort((candidates, -lg))]


def s2o_head(q, K, V, init, ordered, tau, block=BLOCK, scale=None, gains=None):
    """One query head: output [d] and the number of candidate blocks kept.

    init: positions of the first pass; ordered: the visit order of the
    candidates (those in init are skipped).  ``gains``: a list that receives
    each visited block's S_block / S_before (the quantity compared with tau),
    so that tests can keep clear of the threshold."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    init = np.asarray(init, np.int64)
    in_init = np.zeros(K.shape[0], bool)
    in_init[init] = True
    visit = np.asarray([j for j in ordered if not in_init[j]], np.int64)
    blocks = [visit[i:i + block] for i in range(0, len(visit), block)]
    kept = []
    # a common reference keeps the sums in range: the largest score of all
    ref = float(np.max(((K[np.r_[init, visit]] @ q) * scale))) if len(init) + len(visit) else 0.0
    S_before = np.sum(np.exp((K[init] @ q) * scale - ref)) if len(init) else 0.0
    nb = 0
    for blk in blocks:
        S_blk = np.sum(np.exp((K[blk] @ q) * scale - ref))
        kept.append(blk)
        nb += 1
        if gains is not None:
            gains.append(S_blk / S_before)
        if S_before > 0 and S_blk / S_before < tau:
            break
        S_before += S_blk
    T = np.concatenate([init] + kept) if kept else init
    a = (K[T] @ q) * scale
    w = np.exp(a - a.max())
    return (w / w.sum()) @ V[T], nb
