"""Head-split prefill: each query head's visible keys follow from its label.

"Full Attention Strikes Back" summary (RTPurbo), Methodology item 1: during
prefill the local heads attend over attention sinks plus a sliding window,
while the retrieval heads keep the whole KV cache (dense causal attention);
the summary's Results attribute the long-context prefill speed-up to the
local heads' windows.  AoH summary, Methodology item 4: streaming heads keep
the first tokens plus a recent window.

Readings:
* the prefill query at position i of a local head sees exactly what a decode
  query would see with a cache of i + 1 keys: positions [0, s) and
  [i - w + 1, i], a union, clipped to [0, i];
* retrieval heads, and routed heads (whose chunk routing during prefill is a
  separate operation on the HGA page), attend densely and causally: [0, i];
* scale 1/sqrt(d), as for every other attention here.
GQA: query head h reads the keys and values of KV group h / G.
"""
import numpy as np

from .attention import attend
from .local import local_set

LOCAL = 0


def prefill_visible(i, kind, sinks, window):
    """Ascending key positions visible to the prefill query at position i."""
    if kind == LOCAL:
        return local_set(i + 1, sinks, window)
    return np.arange(i + 1)


def head_prefill_rows(Q, K, V, kind, sinks, window, rows, scale=None):
    """Outputs [len(rows), d] of one query head for the query positions
    ``rows``: Q [N, d] of the head, K, V [N, d] of its KV group."""
    out = np.empty((len(rows), np.asarray(Q).shape[-1]))
    for r, i in enumerate(rows):
        T = prefill_visible(int(i), kind, sinks, window)
        out[r] = attend(Q[i], K[T], V[T], scale)
    return out


def visible_pairs(N, kind, sinks, window):
    """Number of (query, key) pairs the head attends over in a prefill of N
    tokens (the unit of its arithmetic: 4 d flops per pair)."""
    if kind != LOCAL:
        return N * (N + 1) // 2
    total = 0
    for i in range(N):
        total += len(prefill_visible(i, kind, sinks, window))
    return total
