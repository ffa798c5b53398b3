"""One sparse decode step, composed from the stage functions.

Per KV group g of sequence b the visible token set comes from the group's
label ("Full Attention Strikes Back" summary, Methodology item 1: retrieval
heads select dynamically in decode, local heads keep sinks plus a window; HGA
summary: routed heads use two-level routing), then every query head of the
group attends exactly over that set.  GQA heads share their group's set
(AoH summary, Methodology item 4: group-level aggregation by the mean).
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


def decode_token_sets(p, inp, groups=None, k_idx=None, q_idx=None,
                      chunk_sum=None, group_sum=None):
    """Visible sets {(b, g): ascending token positions} for one step.

    ``p`` holds the workload parameters (attributes as in a DecodeConfig);
    ``inp`` the numpy inputs.  Index keys / queries and summaries are computed
    here from the pre-RoPE tensors unless given (exact-set tests pass lattice
    values straight in)."""
    B, Hq, Hkv, n = p.batch, p.n_q_heads, p.n_kv_heads, p.n_ctx
    G = Hq // Hkv
    kinds = np.asarray(inp["head_kind"])
    groups = [(b, g) for b in range(B) for g in range(Hkv)] if groups is None else groups
    out = {}
    for b, g in groups:
        kind = _group_kind(kinds, g, G)
        if kind == LOCAL:
            out[(b, g)] = local_set(n, p.sinks, p.window)
        elif kind == RETRIEVAL:
            kk = (k_idx[b, g, :n] if k_idx is not None else
                  index_keys(inp["k_pre"][b, g, :n], inp["proj"][g], p.dtype))
            qq = (q_idx[b, g * G:(g + 1) * G] if q_idx is not None else
                  index_query(inp["q_pre"][b, g * G:(g + 1) * G], inp["proj"][g]))
            lg = index_logits(qq, kk, p.r)
            if p.top_k > 0:
                s, _ = select_topk(lg, p.top_k)
            else:
                s, _ = select_topp(lg, p.top_p, p.min_tokens)
            out[(b, g)] = s
        else:
            cs = (chunk_sum[b, g] if chunk_sum is not None else
                  chunk_summaries(inp["k_pre"][b, g, :n], p.chunk, p.rope_base, p.dtype))
            gs = (group_sum[b, g] if group_sum is not None else
                  group_summaries(inp["k_pre"][b, g, :n], p.group, p.rope_base, p.dtype))
            toks, _ = route_token_list(inp["q"][b, g * G:(g + 1) * G], cs, gs, n,
                                       p.chunk, p.group, p.top_chunks, p.top_groups,
                                       p.sink_chunks, p.local_chunks)
            out[(b, g)] = toks
    return out


def decode_step(p, inp, groups=None, sets=None, **kw):
    """Outputs {(b, h): o [d]} for the query heads of the requested groups."""
    G = p.n_q_heads // p.n_kv_heads
    sets = decode_token_sets(p, inp, groups, **kw) if sets is None else sets
    out = {}
    for (b, g), T in sets.items():
        K = inp["k_cache"][b, g][T]
        V = inp["v_cache"][b, g][T]
        for h in range(g * G, (g + 1) * G):
            out[(b, h)] = attend(inp["q"][b, h], K, V)
    return out
