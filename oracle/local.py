"""Visible set of a local (streaming) head.

"Full Attention Strikes Back" summary, Methodology item 1: local heads use a
sliding window together with attention sinks.  AoH summary, Methodology item
4: streaming heads keep the first tokens (e.g. 128) and a recent window (e.g.
256).  Reading: the cache holds n keys including the current token, the
query sits at t = n - 1, sinks are positions [0, s), the window is the last w
positions including t, and overlap is a union.
"""
import numpy as np


def local_set(n, sinks, window):
    t = n - 1
    s = np.arange(min(sinks, n))
    w = np.arange(max(0, t - window + 1), n) if window > 0 else np.arange(0)
    return np.union1d(s, w).astype(np.int64)
