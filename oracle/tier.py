"""Tiered K/V storage of the routed decode: the cache policy and the row map.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Atencao Global Hierarquica (HGA)" summary, Memory architecture: the whole
token history of the K/V cache lives in host RAM (cold); a bounded LRU cache
in device memory keeps recently routed blocks (warm); the summaries and the
always-visible windows stay in device memory (hot).  Core mechanism item 4:
once routing has chosen its groups, the router brings their original
token-level K/V rows from host RAM into device memory, and attention runs
exactly over them.

Readings (the summary leaves these open):
  * the warm cache holds whole routing groups (`group` consecutive tokens);
    it has a fixed number of slots per (sequence, KV group);
  * hot rows: the sink chunks at their own positions, then a ring of the
    last local_chunks + 1 chunks (the local window and the current chunk),
    position p at hot row sink_rows + p mod ring;
  * each step, the groups the routed list needs that the warm cache already
    holds are hits (their last use becomes this step); each missing group
    takes a slot: empty slots first, then the least recently used slot that
    this step does not need (ties: lower slot index); missing groups are
    placed in ascending group order;
  * the list's positions are rewritten as rows of the device tier: hot rows
    for sinks, the local window and the current chunk, warm rows
    (hot_rows + slot * group + offset) for routed groups.
"""
import numpy as np


class WarmCache:
    """The warm tier of one (sequence, KV group): ``slots`` slots, each
    holding one routing group id (-1: empty) and the step it was last used."""

    def __init__(self, slots):
        self.group = [-1] * slots
        self.stamp = [0] * slots

    def step(self, needed, stamp):
        """Serve the sorted distinct group ids ``needed`` at step ``stamp``.
        Returns (hits, misses, {group: slot})."""
        held = {g: s for s, g in enumerate(self.group) if g >= 0}
        place = {}
        hits = 0
        for g in needed:
            if g in held:
                place[g] = held[g]
                hits += 1
        used = set(place.values())
        # candidates for the missing groups: empty slots first, then the
        # least recently used, ties to the lower slot index
        cand = sorted((s for s in range(len(self.group)) if s not in used),
                      key=lambda s: (self.group[s] >= 0, self.stamp[s], s))
        missing = [g for g in needed if g not in place]
        if len(missing) > len(cand):
            raise ValueError("more groups than warm slots")
        for g, s in zip(missing, cand):
            place[g] = s
            self.group[s] = g
        for s in place.values():
            self.stamp[s] = stamp
        return hits, len(missing), place


def split_positions(positions, n, chunk, group, sink_chunks, local_chunks):
    """(hot, routed) masks of a routed list's positions: sinks and the last
    local_chunks chunks plus the current chunk are hot, the rest routed."""
    p = np.asarray(positions, np.int64)
    kappa = (n - 1) // chunk
    hot = (p < sink_chunks * chunk) | (p >= (kappa - local_chunks) * chunk)
    return hot, ~hot


def tier_rows(positions, n, chunk, group, sink_chunks, local_chunks, place):
    """Rows of the device tier for a routed list's positions, the routed
    groups placed by ``place`` ({group: slot})."""
    p = np.asarray(positions, np.int64)
    sink_rows = sink_chunks * chunk
    ring = (local_chunks + 1) * chunk
    hot_rows = sink_rows + ring
    hot, routed = split_positions(p, n, chunk, group, sink_chunks, local_chunks)
    rows = np.empty_like(p)
    sink = p < sink_rows
    rows[sink] = p[sink]
    win = hot & ~sink
    rows[win] = sink_rows + p[win] % ring
    for i in np.nonzero(routed)[0]:
        g = int(p[i] // group)
        rows[i] = hot_rows + place[g] * group + p[i] % group
    return rows


def needed_groups(positions, n, chunk, group, sink_chunks, local_chunks):
    """Sorted distinct routing groups of a routed list's routed positions."""
    p = np.asarray(positions, np.int64)
    _, routed = split_positions(p, n, chunk, group, sink_chunks, local_chunks)
    return sorted(set((p[routed] // group).tolist()))
