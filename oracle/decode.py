"""One sparse decode step, composed from the stage functions.

Per KV group g of sequence b the visible token set comes from the group's
label ("Full Attention Strikes Back" summary, Methodology item 1: retrieval
heads select dynamically in decode, local heads keep sinks plus a window; HGA
summary: routed heads use two-level routing), then every query head of the
group attends exactly over that set.  GQA heads share their group's set
(AoH summary, Methodology item 4: group-level aggregation by the mean).

Per-query-head mode (``per_head=True``): the RTPurbo summary speaks of
per-head selection; read literally, every query head picks its own set.  The
rule is the group rule applied to a group of one head: a retrieval head ranks
with its own index query, a routed head routes with its own query, and the
head attends over the keys and values of its KV group at those positions.
Local heads keep sinks plus a window either way.
"""
import numpy as np

from .attention import attend
from .hga import chunk_summaries, group_summaries, route_token_list
from .local import local_set
from .lowrank import index_keys, index_logits, index_query, select_topk, select_topp

LOCAL, RETRIEVAL, ROUTED = 0, 1, 2


def _group_kind(head_kind, g, G):
    kinds = set(int(k) for k in head_kind[g * G:(g + 1) * G])
    assert len(kinds) == 1, "labels must be uniform inside a GQA group"
    return kinds.pop()


def _visible(p, inp, b, g, kind, heads, k_idx, q_idx, chunk_sum, group_sum):
    """Visible set of the query heads ``heads`` (a slice of one KV group g of
    sequence b, all labelled ``kind``), aggregated over those heads."""
    n = p.n_ctx
    if kind == LOCAL:
        return local_set(n, p.sinks, p.window)
    if kind == RETRIEVAL:
        kk = (k_idx[b, g, :n] if k_idx is not None else
              index_keys(inp["k_pre"][b, g, :n], inp["proj"][g], p.dtype))
        qq = (q_idx[b, heads] if q_idx is not None else
              index_query(inp["q_pre"][b, heads], inp["proj"][g]))
        lg = index_logits(qq, kk, p.r)
        if p.top_k > 0:
            s, _ = select_topk(lg, p.top_k)
        else:
            s, _ = select_topp(lg, p.top_p, p.min_tokens)
        return s
    cs = (chunk_sum[b, g] if chunk_sum is not None else
          chunk_summaries(inp["k_pre"][b, g, :n], p.chunk, p.rope_base, p.dtype))
    gs = (group_sum[b, g] if group_sum is not None else
          group_summaries(inp["k_pre"][b, g, :n], p.group, p.rope_base, p.dtype))
    toks, _ = route_token_list(inp["q"][b, heads], cs, gs, n, p.chunk, p.group,
                               p.top_chunks, p.top_groups, p.sink_chunks, p.local_chunks)
    return toks


def decode_token_sets(p, inp, groups=None, k_idx=None, q_idx=None,
                      chunk_sum=None, group_sum=None):
    """Visible sets {(b, g): ascending token positions} for one step.

    ``p`` holds the workload parameters (attributes as in a DecodeConfig);
    ``inp`` the numpy inputs.  Index keys / queries and summaries are computed
    here from the pre-RoPE tensors unless given (exact-set tests pass lattice
    values straight in)."""
    B, Hq, Hkv = p.batch, p.n_q_heads, p.n_kv_heads
    G = Hq // Hkv
    kinds = np.asarray(inp["head_kind"])
    groups = [(b, g) for b in range(B) for g in range(Hkv)] if groups is None else groups
    return {(b, g): _visible(p, inp, b, g, _group_kind(kinds, g, G), slice(g * G, (g + 1) * G),
                             k_idx, q_idx, chunk_sum, group_sum)
            for b, g in groups}


def decode_token_sets_per_head(p, inp, heads=None, k_idx=None, q_idx=None,
                               chunk_sum=None, group_sum=None):
    """Per-query-head visible sets {(b, h): ascending token positions}: the
    group rule applied to each query head alone (its KV group g = h / G)."""
    B, Hq, Hkv = p.batch, p.n_q_heads, p.n_kv_heads
    G = Hq // Hkv
    kinds = np.asarray(inp["head_kind"])
    heads = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else heads
    return {(b, h): _visible(p, inp, b, h // G, int(kinds[h]), slice(h, h + 1),
                             k_idx, q_idx, chunk_sum, group_sum)
            for b, h in heads}


def decode_step(p, inp, groups=None, sets=None, per_head=False, **kw):
    """Outputs {(b, h): o [d]} for the query heads of the requested groups
    (per_head: of the requested (b, h) heads, each over its own set)."""
    G = p.n_q_heads // p.n_kv_heads
    out = {}
    if per_head:
        sets = decode_token_sets_per_head(p, inp, groups, **kw) if sets is None else sets
        for (b, h), T in sets.items():
            g = h // G
            out[(b, h)] = attend(inp["q"][b, h], inp["k_cache"][b, g][T], inp["v_cache"][b, g][T])
        return out
    sets = decode_token_sets(p, inp, groups, **kw) if sets is None else sets
    for (b, g), T in sets.items():
        K = inp["k_cache"][b, g][T]
        V = inp["v_cache"][b, g][T]
        for h in range(g * G, (g + 1) * G):
            out[(b, h)] = attend(inp["q"][b, h], K, V)
    return out
