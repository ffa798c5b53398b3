"""GPU parity of the tiered K/V store of the routed decode (cold host store,
warm LRU slots in device memory, hot sinks and window ring) against the
oracle's cache model, through the C ABI: over several decode steps whose
routing changes, every step's outputs from the device tier equal, bit for
bit, the decode over the whole cache in device memory, and the hits, misses,
slot tables and rewritten lists follow the oracle's LRU rule exactly."""
import numpy as np
import pytest
import torch

import oracle
import selection_sparse_attention_amd as sa
import workloads
from gpu_harness import DEV, DecodeRun, log

pytestmark = pytest.mark.gpu

SMALL = workloads.HGA_64K.with_(batch=2, n_q_heads=8, n_kv_heads=2, n_ctx=64 * 40 + 37,
                                top_chunks=4, top_groups=2, sink_chunks=2, local_chunks=3)


def _tier_steps(cfg, slots, steps, seed):
    n_cap = cfg.n_ctx + 40 * steps
    inp = workloads.decode_inputs(cfg.with_(n_ctx=n_cap), seed)
    run = DecodeRun(cfg.with_(n_ctx=n_cap), inp, n_cap=n_cap)
    B, Hq, Hkv, d = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    C, grp, sc, lc = cfg.chunk, cfg.group, cfg.sink_chunks, cfg.local_chunks
    sink_rows, ring = sc * C, (lc + 1) * C
    hot_rows = sink_rows + ring
    dev_rows = hot_rows + slots * grp
    dt = run.t["k_cache"].dtype
    cold_k = run.t["k_cache"].cpu().pin_memory()
    cold_v = run.t["v_cache"].cpu().pin_memory()
    dev_k = torch.zeros(B, Hkv, dev_rows, d, dtype=dt, device=DEV)
    dev_v = torch.zeros(B, Hkv, dev_rows, d, dtype=dt, device=DEV)
    slot_group = torch.full((B, Hkv, slots), -1, dtype=torch.int32, device=DEV)
    slot_stamp = torch.zeros(B, Hkv, slots, dtype=torch.int32, device=DEV)
    stats = torch.zeros(B, Hkv, 2, dtype=torch.int32, device=DEV)
    rows_t = torch.full((B, Hkv, dev_rows), -1, dtype=torch.int32, device=DEV)
    models = {(b, g): oracle.WarmCache(slots) for b in range(B) for g in range(Hkv)}
    gen = torch.Generator().manual_seed(seed)
    misses_total = hits_total = 0
    ws_dec = sa.Workspace(DEV)
    for s in range(steps):
        n = cfg.n_ctx + 37 * s
        run.params.n_ctx = n
        # a new decode query every step, so the routing moves
        run.t["q"].copy_((torch.randn(B, Hq, d, generator=gen) * 2.0).to(DEV, dt))
        run.summaries(0, n)
        run.select()
        torch.cuda.synchronize()
        pos = run.t["sel_idx"].cpu().numpy().copy()
        cnt = run.t["sel_count"].cpu().numpy().copy()
        run.decode()
        torch.cuda.synchronize()
        out_ref = run.t["out"].clone()
        # the caller's part of the hot tier: sinks and the ring of the last chunks
        kappa = (n - 1) // C
        win = torch.arange(max((kappa - lc) * C, sink_rows), n, device=DEV)
        for src, dst in ((run.t["k_cache"], dev_k), (run.t["v_cache"], dev_v)):
            dst[:, :, :sink_rows] = src[:, :, :sink_rows]
            dst[:, :, sink_rows + win % ring] = src[:, :, win]
        tier = sa.make_tier(cold_k=cold_k, cold_v=cold_v, dev_k=dev_k, dev_v=dev_v,
                            slot_group=slot_group, slot_stamp=slot_stamp, rows=rows_t, step=s + 1,
                            stats=stats)
        sa.tier_fetch(run.params, run.bufs(), tier)
        # decode over the device tier, from the lists as its rows
        pt = sa.params_from_config(cfg, n_cap=dev_rows)
        pt.n_ctx = dev_rows
        run.t["out"].fill_(float("nan"))
        sa.decode(pt, sa.make_buffers(q=run.t["q"], k_cache=dev_k, v_cache=dev_v,
                                      sel_idx=rows_t, sel_count=run.t["sel_count"],
                                      out=run.t["out"]), ws_dec)
        torch.cuda.synchronize()
        assert torch.equal(run.t["out"], out_ref), s
        rows = rows_t.cpu().numpy()
        st = stats.cpu().numpy()
        sg, ss = slot_group.cpu().numpy(), slot_stamp.cpu().numpy()
        for (b, g), m in models.items():
            p = pos[b, g, :cnt[b, g]]
            need = oracle.needed_groups(p, n, C, grp, sc, lc)
            hits, misses, place = m.step(need, s + 1)
            assert (st[b, g, 0], st[b, g, 1]) == (hits, misses), (s, b, g)
            assert np.array_equal(rows[b, g, :cnt[b, g]],
                                  oracle.tier_rows(p, n, C, grp, sc, lc, place)), (s, b, g)
            assert sg[b, g].tolist() == m.group and ss[b, g].tolist() == m.stamp, (s, b, g)
            hits_total += hits
            misses_total += misses
    log("tier steps", steps, "slots", slots, "hits", hits_total, "misses", misses_total)
    return hits_total, misses_total


def test_tier_decode_matches_whole_cache_and_lru_model():
    hits, misses = _tier_steps(SMALL, slots=12, steps=8, seed=3)
    assert hits > 0 and misses > 8 * 4       # reuse, and evictions past the first step


def test_tier_with_exactly_one_step_of_slots():
    """As many warm slots as one step routes: every group a step does not
    need again is evicted by the next."""
    _tier_steps(SMALL, slots=SMALL.top_chunks * SMALL.top_groups, steps=5, seed=4)


def test_tier_fp32_and_small_head_dim():
    _tier_steps(SMALL.with_(dtype="fp32", head_dim=64), slots=20, steps=4, seed=5)
