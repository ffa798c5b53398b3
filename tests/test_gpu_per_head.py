"""GPU parity of per-query-head selection - every query head selects its own
set against the index keys or summaries of its KV group - and of decode over
per-head sets, against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import DecodeRun, DEV, log, max_err, np64, np_inputs, to_dev

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-3
FP32_TOL = 1e-5


def _heads(cfg, kind):
    kinds = cfg.head_kind()
    return [h for h in range(cfg.n_q_heads) if kinds[h] == kind]


def _head_logits(cfg, k_idx, q_idx, b, h):
    return oracle.index_logits(q_idx[b, h:h + 1], k_idx[b, h // cfg.gqa, :cfg.n_ctx], cfg.r)


def _select_ref(cfg, lg):
    if cfg.top_k:
        return oracle.select_topk(lg, cfg.top_k)
    return oracle.select_topp(lg, cfg.top_p, cfg.min_tokens)


LATTICE_CASES = [
    # (config, k_amp, q_amp)
    (workloads.LLAMA_32K.with_(batch=2, n_ctx=5000, min_tokens=0, top_p=0.9), 24, 12),
    (workloads.LLAMA_32K.with_(batch=2, n_ctx=5000, top_p=1.0, top_k=300), 24, 12),
    (workloads.TINY.with_(n_q_heads=8, n_kv_heads=4, n_ret_q_heads=4, top_p=0.9), 24, 12),
    # 64 query heads of 8 KV groups (8 heads per group, the most per-head rows)
    (workloads.LLAMA_32K.with_(batch=1, n_ctx=3000, n_q_heads=64, n_kv_heads=8,
                               n_ret_q_heads=32), 24, 12),
    # the headline shapes: 64 rows of 32K, 32 rows of 128K
    (workloads.LLAMA_32K, 24, 12),
    (workloads.LLAMA_128K, 24, 12),
    (workloads.LLAMA_128K_TOPK, 24, 12),
]


@pytest.mark.parametrize("case", LATTICE_CASES,
                         ids=lambda c: f"{c[0].name}-{c[0].n_ctx}-h{c[0].n_q_heads}")
def test_per_head_lattice_sets_exact(case):
    cfg, ka, qa = case
    log("per-head select lattice", cfg.name, cfg.n_ctx, cfg.n_q_heads)
    ret = _heads(cfg, workloads.HEAD_RETRIEVAL)
    for s in range(64):
        inp = workloads.lattice_index_inputs(cfg, 300 + s, k_amp=ka, q_amp=qa)
        k, q = np64(inp["k_idx"]), np64(inp["q_idx"])
        if cfg.top_k or all(oracle.topp_margin(_head_logits(cfg, k, q, b, h), cfg.top_p) >= 1e-7
                            for b in range(cfg.batch) for h in ret):
            break
    else:
        pytest.fail("no robust lattice draw")
    run = DecodeRun(cfg, {}, n_cap=cfg.n_ctx, per_head=True)
    run.t["k_idx"].copy_(to_dev(inp["k_idx"], cfg.dtype))
    run.t["q_idx"].copy_(inp["q_idx"].to(DEV))
    run.select()
    torch.cuda.synchronize()
    idx, cnt = run.sets()
    for b in range(cfg.batch):
        for h in ret:
            ref, m = _select_ref(cfg, _head_logits(cfg, k, q, b, h))
            assert cnt[b, h] == m, (b, h, cnt[b, h], m)
            assert np.array_equal(idx[b, h, :m], ref), (b, h)
        for h in _heads(cfg, workloads.HEAD_LOCAL):        # rows nobody selects for
            assert cnt[b, h] == -1


ROUTE_SMALL = workloads.HGA_64K.with_(batch=2, n_q_heads=8, n_kv_heads=2, n_ctx=64 * 40 + 37)


@pytest.mark.parametrize("cfg", [ROUTE_SMALL, ROUTE_SMALL.with_(n_ctx=64 * 300 + 17, top_chunks=40,
                                                                top_groups=3)],
                         ids=lambda c: f"n{c.n_ctx}")
def test_per_head_route_lattice_exact(cfg):
    """Each routed query head routes with its own query over its KV group's
    lattice summaries."""
    lat = workloads.lattice_summary_inputs(cfg, 61, amp=16, q_amp=4)
    run = DecodeRun(cfg, {}, per_head=True)
    nc, ng = lat["chunk_sum"].shape[2], lat["group_sum"].shape[2]
    run.t["chunk_sum"][:, :, :nc] = to_dev(lat["chunk_sum"], cfg.dtype)
    run.t["group_sum"][:, :, :ng] = to_dev(lat["group_sum"], cfg.dtype)
    run.t["q"] = to_dev(lat["q"], cfg.dtype)
    run.select()
    torch.cuda.synchronize()
    idx, cnt = run.sets()
    q, cs, gs = np64(lat["q"]), np64(lat["chunk_sum"]), np64(lat["group_sum"])
    G = cfg.gqa
    differs = 0
    for b in range(cfg.batch):
        for h in range(cfg.n_q_heads):
            ref, _ = oracle.route_token_list(q[b, h:h + 1], cs[b, h // G], gs[b, h // G],
                                             cfg.n_ctx, cfg.chunk, cfg.group, cfg.top_chunks,
                                             cfg.top_groups, cfg.sink_chunks, cfg.local_chunks)
            assert cnt[b, h] == len(ref), (b, h, cnt[b, h], len(ref))
            assert np.array_equal(idx[b, h, :len(ref)], ref), (b, h)
            differs += not np.array_equal(idx[b, h, :cnt[b, h]], idx[b, (h // G) * G, :cnt[b, (h // G) * G]])
    assert differs > 0          # the heads of a group did route differently


@pytest.mark.parametrize("cfg", [
    workloads.TINY.with_(n_ctx=3000, n_q_heads=8, n_kv_heads=4, n_ret_q_heads=4),
    workloads.LLAMA_32K.with_(batch=2, n_ctx=4099),
    workloads.LLAMA_32K.with_(batch=2, n_ctx=4099, n_q_heads=16, n_kv_heads=2, n_ret_q_heads=8),
    workloads.LLAMA_32K.with_(batch=2, n_ctx=4099, n_q_heads=8, n_kv_heads=4, n_ret_q_heads=4),
    workloads.LLAMA_32K.with_(batch=1, n_ctx=150000, n_q_heads=8, n_kv_heads=2, n_ret_q_heads=4),
], ids=lambda c: f"{c.name}-{c.n_ctx}-{c.n_q_heads}-{c.n_kv_heads}")
def test_per_head_decode_over_given_lists(cfg):
    """The attention stage alone over random per-head lists (and sinks +
    window for local heads, each head on its own).  With bf16 caches the
    heads of a KV group are decoded together over the union of their sets,
    each masked to its own (GQA 4, 8 and 2 here, and a context of 150000
    whose union spans 74 slices of 2048 positions)."""
    log("per-head decode lists", cfg.name, cfg.n_ctx)
    inp = workloads.decode_inputs(cfg, 12)
    run = DecodeRun(cfg, inp, n_cap=cfg.n_ctx + 3, per_head=True)
    gen = torch.Generator().manual_seed(4)
    ret = set(_heads(cfg, workloads.HEAD_RETRIEVAL))
    sets = {}
    for b in range(cfg.batch):
        for h in range(cfg.n_q_heads):
            if h in ret:
                m = int(torch.randint(1, min(cfg.n_ctx, 20000) + 1, (1,), generator=gen))
                T = torch.sort(torch.randperm(cfg.n_ctx, generator=gen)[:m]).values
                run.t["sel_idx"][b, h, :m] = T.to(DEV, torch.int32)
                run.t["sel_count"][b, h] = m
                sets[(b, h)] = T.numpy()
            else:
                sets[(b, h)] = oracle.local_set(cfg.n_ctx, cfg.sinks, cfg.window)
    run.decode()
    torch.cuda.synchronize()
    out = np64(run.t["out"])
    ref = oracle.decode_step(cfg, np_inputs(inp), sets=sets, per_head=True)
    tol = FP32_TOL if cfg.dtype == "fp32" else BF16_TOL
    err = max(max_err(out[b, h], o) for (b, h), o in ref.items())
    log("max err", err)
    assert err <= tol


def _per_head_pipeline(cfg, seed, exact, sample_local=None):
    """Index -> per-head select -> decode on Gaussian inputs.  Every
    retrieval head's set is compared with the oracle's selection on the same
    stored index values (exactly, or - when ``exact`` is False - up to 4
    flipped tokens ranked within 4 of the cut); every checked head's output
    with the oracle's attention over the GPU's own set and over the oracle's
    own fp64 pipeline set."""
    inp = workloads.decode_inputs(cfg, seed)
    run = DecodeRun(cfg, inp, per_head=True)
    run.index()
    run.select()
    run.decode()
    torch.cuda.synchronize()
    idx, cnt = run.sets()
    out = np64(run.t["out"])
    k_gpu, q_gpu = np64(run.t["k_idx"]), np64(run.t["q_idx"])
    ni = np_inputs(inp)
    ret = _heads(cfg, workloads.HEAD_RETRIEVAL)
    loc = [(b, h) for b in range(cfg.batch) for h in _heads(cfg, workloads.HEAD_LOCAL)]
    if sample_local is not None and sample_local < len(loc):
        rng = np.random.default_rng(seed)
        loc = [loc[i] for i in sorted(rng.choice(len(loc), sample_local, replace=False))]
    heads = [(b, h) for b in range(cfg.batch) for h in ret] + loc
    osets = oracle.decode_token_sets_per_head(cfg, ni, heads=heads)
    tol = FP32_TOL if cfg.dtype == "fp32" else BF16_TOL
    worst = worst_own = 0.0
    flips = 0
    for (b, h), T in osets.items():
        own = T
        if h in ret:
            got = idx[b, h, :cnt[b, h]]
            assert cnt[b, h] >= 1 and np.all(np.diff(got) > 0), (b, h)
            lg = _head_logits(cfg, k_gpu, q_gpu, b, h)
            ref, m = _select_ref(cfg, lg)
            diff = np.setxor1d(got, ref)
            if exact:
                assert np.array_equal(got, ref), (b, h, len(got), len(ref))
            else:
                rank = np.empty(cfg.n_ctx, np.int64)
                rank[oracle.order(lg)] = np.arange(cfg.n_ctx)
                assert len(diff) <= 4 and np.all(np.abs(rank[diff] - m) <= 4), (b, h, len(diff))
            flips += len(diff)
            own = got
        o_e2e = oracle.decode_step(cfg, ni, sets={(b, h): T}, per_head=True)[(b, h)]
        o_own = oracle.decode_step(cfg, ni, sets={(b, h): own}, per_head=True)[(b, h)]
        worst = max(worst, max_err(out[b, h], o_e2e))
        worst_own = max(worst_own, max_err(out[b, h], o_own))
    log("per-head pipeline", cfg.name, cfg.n_ctx, "max err", worst, "on own sets", worst_own,
        "flips", flips)
    assert worst_own <= tol and worst <= tol


def _robust_seed(cfg, start, tries=40, gap=1e-4, margin=1e-6):
    """Seed whose oracle cut, for every retrieval head, has a logit gap >=
    gap and a mass margin >= margin."""
    ret = _heads(cfg, workloads.HEAD_RETRIEVAL)
    G = cfg.gqa
    for s in range(start, start + tries):
        ni = np_inputs(workloads.decode_inputs(cfg, s))
        ok = True
        for b in range(cfg.batch):
            for h in ret:
                g = h // G
                k = oracle.index_keys(ni["k_pre"][b, g, :cfg.n_ctx], ni["proj"][g], cfg.dtype)
                q = oracle.index_query(ni["q_pre"][b, h:h + 1], ni["proj"][g])
                lg = oracle.index_logits(q, k, cfg.r)
                _, m = _select_ref(cfg, lg)
                if not cfg.top_k and cfg.min_tokens < m < cfg.n_ctx and \
                        oracle.topp_margin(lg, cfg.top_p) < margin:
                    ok = False
                if oracle.cut_gap(lg, m) < gap:
                    ok = False
        if ok:
            return s
    raise AssertionError("no robust seed")


@pytest.mark.parametrize("cfg", [
    workloads.TINY.with_(n_q_heads=8, n_kv_heads=4, n_ret_q_heads=4),
    workloads.LLAMA_32K.with_(batch=2, n_ctx=5000),
    workloads.LLAMA_128K_TOPK.with_(batch=2, n_ctx=6000, top_k=500),
], ids=lambda c: f"{c.name}-{c.n_ctx}")
def test_per_head_pipeline_small(cfg):
    seed = _robust_seed(cfg, 0)
    log("per-head pipeline seed", seed)
    _per_head_pipeline(cfg, seed, exact=True)


def test_per_head_pipeline_32k_full_size():
    """The 32K decode layer with per-head sets: all 64 retrieval heads
    checked, 8 sampled local heads."""
    _per_head_pipeline(workloads.LLAMA_32K, 1, exact=False, sample_local=8)


def test_per_head_failed_head_poisons_only_itself():
    """A negative count for one head of a retrieval group (a selection that
    reported failure): that head's output is NaN, the other heads of its
    group (decoded over the group's union) stay exact."""
    cfg = workloads.LLAMA_32K.with_(batch=2, n_ctx=3001)
    inp = workloads.decode_inputs(cfg, 13)
    run = DecodeRun(cfg, inp, per_head=True)
    gen = torch.Generator().manual_seed(5)
    ret = _heads(cfg, workloads.HEAD_RETRIEVAL)
    sets = {}
    for b in range(cfg.batch):
        for h in ret:
            m = int(torch.randint(1, cfg.n_ctx + 1, (1,), generator=gen))
            T = torch.sort(torch.randperm(cfg.n_ctx, generator=gen)[:m]).values
            run.t["sel_idx"][b, h, :m] = T.to(DEV, torch.int32)
            run.t["sel_count"][b, h] = m
            sets[(b, h)] = T.numpy()
    bad = (1, ret[1])
    run.t["sel_count"][bad] = -1
    run.decode()
    torch.cuda.synchronize()
    out = np64(run.t["out"])
    assert np.isnan(out[bad]).all()
    del sets[bad]
    ref = oracle.decode_step(cfg, np_inputs(inp), sets=sets, per_head=True)
    err = max(max_err(out[b, h], ref[(b, h)]) for (b, h) in sets)
    assert err <= BF16_TOL
