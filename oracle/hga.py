"""Hierarchical chunk/group routing (HGA) for decode and chunked prefill.

"Atencao Global Hierarquica (HGA)" summary, Core mechanism:
  1. the sequence is cut into fixed chunks (e.g. C = 64 tokens), each split
     into groups;
  2. level 1 routes the current query against compact chunk key summaries,
     level 2 routes against group summaries inside the chosen chunks; the
     current chunk, a number of initial sink chunks and recent local chunks
     are always visible;
  3. summaries are RoPE-aware and mixed: high-frequency RoPE pairs are rotated
     per token and then averaged, low-frequency pairs are averaged in raw key
     space and rotated at the chunk's representative position; they are built
     from the existing keys with no new weights;
  4. exact softmax attention then runs over the routed token set.

Readings (stated because the page gives no numbers for them):
  * pair i is high-frequency iff theta_i * (span - 1) > 1 rad, span = chunk size
    for chunk summaries and group size for group summaries;
  * representative position = the span's mean position (start + (span-1)/2);
  * routing score = qbar . summary / sqrt(d), qbar = mean of the KV group's
    post-RoPE query heads; ties go to the lower chunk / group index;
  * with t = n-1 and kappa = floor(t / C): sink chunks are [0, sink_chunks),
    local chunks are [kappa - local_chunks, kappa), the current chunk
    contributes tokens kappa*C .. t, candidates are the chunks in
    [sink_chunks, kappa - local_chunks); the top ``top_chunks`` candidates
    (all if fewer) are kept, and in each the top ``top_groups`` groups;
  * summaries are stored in the workload element type.
"""
import numpy as np

from .numerics import round_store
from .rope import rope_angles, rope_rotate


def high_freq_pairs(d, base, span):
    """Boolean mask over the d/2 pairs: theta_i * (span - 1) > 1."""
    i = np.arange(d // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / d)
    return theta * (span - 1) > 1.0


def chunk_summary(k_rows, start, base):
    """Mixed RoPE summary of consecutive pre-RoPE keys k_rows [span, d] that
    sit at positions start .. start + span - 1 (fp64, unrounded)."""
    k_rows = np.asarray(k_rows, np.float64)
    span, d = k_rows.shape
    pos = start + np.arange(span, dtype=np.float64)
    high = high_freq_pairs(d, base, span)
    # high pairs: rotate each token at its own position, then average
    rot_each = rope_rotate(k_rows, rope_angles(d, base, pos)).mean(axis=0)
    # low pairs: average the raw keys, rotate once at the mean position
    rep = start + (span - 1) / 2.0
    rot_mean = rope_rotate(k_rows.mean(axis=0), rope_angles(d, base, rep))
    h = d // 2
    hmask = np.concatenate([high, high])
    assert hmask.shape[0] == 2 * h
    return np.where(hmask, rot_each, rot_mean)


def _summaries(k_pre, span, base, store, count=None):
    k_pre = np.asarray(k_pre, np.float64)
    n = k_pre.shape[0]
    count = n // span if count is None else count
    out = np.stack([chunk_summary(k_pre[c * span:(c + 1) * span], c * span, base)
                    for c in range(count)]) if count else np.zeros((0, k_pre.shape[1]))
    return round_store(out, store) if store else out


def chunk_summaries(k_pre, chunk, base, store="bf16", count=None):
    """Summaries of every complete chunk of k_pre [n, d] -> [n // chunk, d]."""
    return _summaries(k_pre, chunk, base, store, count)


def group_summaries(k_pre, group, base, store="bf16", count=None):
    """Summaries of every complete group of k_pre [n, d] -> [n // group, d]."""
    return _summaries(k_pre, group, base, store, count)


def route_scores(qbar, summaries):
    qbar = np.asarray(qbar, np.float64)
    return (np.asarray(summaries, np.float64) @ qbar) / np.sqrt(qbar.shape[0])


def _top(scores, idx, k):
    """Top-k of idx by (score desc, index asc); returns chosen idx and the
    score gap at the cut (inf when every candidate is taken)."""
    scores = np.asarray(scores, np.float64)
    order = np.lexsort((idx, -scores))
    k = min(k, len(idx))
    gap = np.inf if k >= len(idx) else float(scores[order[k - 1]] - scores[order[k]])
    return np.asarray(idx)[order[:k]], gap


def route_token_list(q_heads, chunk_sum, group_sum, n, chunk=64, group=16,
                     top_chunks=16, top_groups=2, sink_chunks=4, local_chunks=8):
    """Visible token list of one KV group (ascending) plus routing details.

    q_heads [G, d] post-RoPE queries of the group, chunk_sum [>= kappa, d],
    group_sum [>= kappa * chunk / group, d]."""
    qbar = np.asarray(q_heads, np.float64).mean(axis=0)
    t = n - 1
    kappa = t // chunk
    gpc = chunk // group
    fixed = [c for c in range(kappa) if c < sink_chunks or c >= kappa - local_chunks]
    cand = np.arange(sink_chunks, max(sink_chunks, kappa - local_chunks))
    chosen_chunks, chunk_gap = np.zeros(0, np.int64), np.inf
    chosen_groups, group_gaps = [], []
    if cand.size:
        lam = route_scores(qbar, np.asarray(chunk_sum)[cand])
        chosen_chunks, chunk_gap = _top(lam, cand, top_chunks)
        for c in sorted(chosen_chunks.tolist()):
            gidx = np.arange(c * gpc, (c + 1) * gpc)
            mu = route_scores(qbar, np.asarray(group_sum)[gidx])
            gsel, ggap = _top(mu, gidx, top_groups)
            chosen_groups.extend(gsel.tolist())
            group_gaps.append(ggap)
    toks = [np.arange(c * chunk, (c + 1) * chunk) for c in fixed]
    toks.append(np.arange(kappa * chunk, t + 1))
    toks += [np.arange(gi * group, (gi + 1) * group) for gi in chosen_groups]
    tokens = np.unique(np.concatenate(toks)).astype(np.int64)
    info = dict(chunks=np.sort(chosen_chunks), groups=np.sort(np.asarray(chosen_groups, np.int64)),
                chunk_gap=chunk_gap, group_gaps=group_gaps, kappa=kappa)
    return tokens, info


# ------------------------------------------------------------ chunked prefill
# HGA summary, Core mechanism item 2: the current chunk routes against the
# summaries of earlier chunks; the page reports the routed prefill's speed-up,
# so routing also runs during (chunked) prefill.  Readings:
#   * a query block is one chunk (its C queries route together); its
#     chunk-level query is the mean of the block's post-RoPE query rows over
#     the KV group's heads (G x C rows, fewer in a last partial block);
#   * the block routes as the decode rule does at its last position t, so
#     kappa is the block itself, candidates are the complete chunks in
#     [sink_chunks, kappa - local_chunks), and sink and local chunks are
#     always visible;
#   * query i of the block sees that list (all of it lies before the block)
#     plus the block's own keys kappa*C .. i (causal).


def route_prefill_block(q_rows, chunk_sum, group_sum, block, n, chunk, group, top_chunks,
                        top_groups, sink_chunks, local_chunks):
    """Routed list (ascending positions before the block) of prefill query
    block ``block`` and the routing details.  q_rows: the block's query rows
    of the group's heads, [rows, d]."""
    t = min(n, (block + 1) * chunk) - 1
    toks, info = route_token_list(q_rows, chunk_sum, group_sum, t + 1, chunk, group,
                                  top_chunks, top_groups, sink_chunks, local_chunks)
    return toks[toks < block * chunk], info


def route_prefill_rows(q, K, V, lst, block, chunk, rows, scale=None):
    """Outputs [len(rows), d] of one query head for positions ``rows`` of
    block ``block``: each attends over the block's routed list ``lst`` and the
    block's keys block*chunk .. i.  q [n, d] of the head; K, V [n, d] of its
    KV group."""
    from .attention import attend
    out = np.empty((len(rows), np.asarray(q).shape[-1]))
    for r, i in enumerate(rows):
        T = np.concatenate([np.asarray(lst, np.int64), np.arange(block * chunk, i + 1)])
        out[r] = attend(q[i], K[T], V[T], scale)
    return out
