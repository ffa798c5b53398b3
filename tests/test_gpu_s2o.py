"""GPU parity of the monotone-gain early stop (S2O) in decode: the top-k
candidates listed in index-score order, and the decode that visits them in
blocks after a dense first pass and stops on a block's marginal mass,
against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import selection_sparse_attention_amd as sa
import workloads
from gpu_harness import DecodeRun, DEV, log, max_err, np64, np_inputs, to_dev

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-3
MARGIN = 1e-3          # relative distance every visited block's gain keeps from tau


def _ret_groups(cfg):
    kinds = cfg.head_kind()
    return [g for g in range(cfg.n_kv_heads) if kinds[g * cfg.gqa] == workloads.HEAD_RETRIEVAL]


def _logits(cfg, k_idx, q_idx, b, g):
    G = cfg.gqa
    return oracle.index_logits(q_idx[b, g * G:(g + 1) * G], k_idx[b, g, :cfg.n_ctx], cfg.r)


def _select_by_score(run):
    sa.select(run.params, run.bufs(), sa.SEL_TOPK_BY_SCORE, run.ws_sel)


@pytest.mark.parametrize("case", [
    (workloads.LLAMA_32K.with_(batch=2, n_ctx=5000, top_p=1.0, top_k=300), 24, 12),
    (workloads.LLAMA_32K.with_(batch=2, n_ctx=5000, top_p=1.0, top_k=300), 2, 1),   # many ties
    (workloads.LLAMA_32K.with_(top_p=1.0, top_k=2048), 24, 12),
    (workloads.LLAMA_128K_TOPK.with_(top_k=8192), 24, 12),
    (workloads.TINY.with_(top_p=1.0, top_k=1), 8, 4),
], ids=lambda c: f"{c[0].n_ctx}-k{c[0].top_k}-a{c[1]}")
def test_topk_by_score_order_exact(case):
    """Lattice index values make every logit exact: the list must be the
    top-k set in (logit desc, position asc) order, element by element."""
    cfg, ka, qa = case
    log("top-k by score", cfg.n_ctx, cfg.top_k, ka)
    inp = workloads.lattice_index_inputs(cfg, 200, k_amp=ka, q_amp=qa)
    run = DecodeRun(cfg, {}, n_cap=cfg.n_ctx)
    run.t["k_idx"].copy_(to_dev(inp["k_idx"], cfg.dtype))
    run.t["q_idx"].copy_(inp["q_idx"].to(DEV))
    _select_by_score(run)
    torch.cuda.synchronize()
    idx, cnt = run.sets()
    k, q = np64(inp["k_idx"]), np64(inp["q_idx"])
    for b in range(cfg.batch):
        for g in _ret_groups(cfg):
            lg = _logits(cfg, k, q, b, g)
            cand, m = oracle.select_topk(lg, cfg.top_k)
            ref = oracle.s2o_order(lg, cand)
            assert cnt[b, g] == m
            assert np.array_equal(idx[b, g, :m], ref), (b, g)


def _s2o_reference(cfg, inp, idx, cnt, b, g, tau):
    """Oracle outputs of group (b, g)'s heads over the GPU's list (which the
    order test pins separately) and the smallest relative distance of a
    visited block's gain from tau.  ``inp``: the generator's tensors."""
    G = cfg.gqa
    init = oracle.local_set(cfg.n_ctx, cfg.sinks, cfg.window)
    order = idx[b, g, :cnt[b, g]]
    K, V = np64(inp["k_cache"][b, g]), np64(inp["v_cache"][b, g])
    outs, closest, blocks = {}, np.inf, []
    n_visit = len(np.setdiff1d(order, init))
    for h in range(g * G, (g + 1) * G):
        gains = []
        o, nb = oracle.s2o_head(np64(inp["q"][b, h]), K, V, init, order, tau, gains=gains)
        outs[(b, h)] = o
        blocks.append((nb, -(-n_visit // 64)))           # kept, visitable
        if tau > 0 and gains:
            closest = min(closest, float(np.min(np.abs(np.asarray(gains) - tau))) / tau)
    return outs, closest, blocks


def _local_reference(cfg, inp, groups):
    """Plain attention over sinks + window for the heads of ``groups``."""
    T = oracle.local_set(cfg.n_ctx, cfg.sinks, cfg.window)
    out = {}
    for b, g in groups:
        K, V = np64(inp["k_cache"][b, g])[T], np64(inp["v_cache"][b, g])[T]
        for h in range(g * cfg.gqa, (g + 1) * cfg.gqa):
            out[(b, h)] = oracle.attend(np64(inp["q"][b, h]), K, V)
    return out


def _s2o_run(cfg, seed, tau, device="cpu"):
    inp = workloads.decode_inputs(cfg, seed, device=device)
    run = DecodeRun(cfg, inp)
    run.params.s2o_tau = tau
    run.index()
    _select_by_score(run)
    run.decode()
    torch.cuda.synchronize()
    return inp, run


NEVER = 1e-20          # a tau no block's gain falls below here (0 turns the stop off)


@pytest.mark.parametrize("tau", [NEVER, 0.003, 0.02, 0.1, 10.0])
def test_s2o_decode_small(tau):
    """Every head of every group: retrieval heads against the oracle's early
    stop over the GPU's list, local heads against plain attention.  Seeds are
    drawn until no visited block's gain lies within 0.1 % of tau."""
    cfg = workloads.LLAMA_32K.with_(batch=2, n_ctx=5000, top_p=1.0, top_k=1024, window=256)
    for seed in range(30):
        inp, run = _s2o_run(cfg, seed, tau)
        idx, cnt = run.sets()
        ref, closest, blocks = {}, np.inf, []
        for b in range(cfg.batch):
            for g in _ret_groups(cfg):
                o, c, nb = _s2o_reference(cfg, inp, idx, cnt, b, g, tau)
                ref.update(o)
                closest = min(closest, c)
                blocks += nb
        if closest >= MARGIN:
            break
    else:
        pytest.fail("no seed keeps its gains clear of tau")
    out = np64(run.t["out"])
    ref.update(_local_reference(cfg, inp, [(b, g) for b in range(cfg.batch)
                                           for g in range(cfg.n_kv_heads)
                                           if g not in _ret_groups(cfg)]))
    err = max(max_err(out[b, h], o) for (b, h), o in ref.items())
    log("s2o tau", tau, "seed", seed, "blocks kept / visitable per head", blocks, "max err", err)
    assert err <= BF16_TOL
    stopped = sum(nb < total for nb, total in blocks)
    if tau == NEVER:
        assert stopped == 0
    elif tau >= 1.0:
        assert stopped == len(blocks)   # every head stops early (a block must outweigh
                                        # tau times all before it to go on)
    else:
        assert 0 < stopped           # the rule took effect somewhere


def test_s2o_never_stopping_is_attention_over_first_pass_and_candidates():
    """A tau that no gain falls below: every head attends over sinks +
    window and the whole top-k set."""
    cfg = workloads.LLAMA_32K.with_(batch=2, n_ctx=4099, top_p=1.0, top_k=777, window=100)
    inp, run = _s2o_run(cfg, 4, NEVER)
    idx, cnt = run.sets()
    ni = np_inputs(inp)
    out = np64(run.t["out"])
    init = oracle.local_set(cfg.n_ctx, cfg.sinks, cfg.window)
    worst = 0.0
    for b in range(cfg.batch):
        for g in _ret_groups(cfg):
            T = np.union1d(init, idx[b, g, :cnt[b, g]])
            ref = oracle.decode_step(cfg, ni, sets={(b, g): T})
            worst = max(worst, max(max_err(out[bb, h], o) for (bb, h), o in ref.items()))
    assert worst <= BF16_TOL


def test_s2o_decode_32k_full_size():
    """The 32K layer with top-k 2048 candidates by score and tau = 0.01: every
    retrieval group's heads against the oracle (gains kept clear of tau by
    the seed), four sampled local groups against plain attention."""
    cfg = workloads.LLAMA_32K.with_(top_p=1.0, top_k=2048)
    tau = 0.01
    for seed in range(10):
        inp, run = _s2o_run(cfg, seed, tau, device=DEV)
        idx, cnt = run.sets()
        ref, closest, blocks = {}, np.inf, []
        for b in range(cfg.batch):
            for g in _ret_groups(cfg):
                o, c, nb = _s2o_reference(cfg, inp, idx, cnt, b, g, tau)
                ref.update(o)
                closest = min(closest, c)
                blocks += nb
        if closest >= MARGIN:
            break
    else:
        pytest.fail("no seed keeps its gains clear of tau")
    out = np64(run.t["out"])
    loc = [(b, g) for b in range(cfg.batch) for g in range(cfg.n_kv_heads) if g not in _ret_groups(cfg)]
    rng = np.random.default_rng(seed)
    loc = [loc[i] for i in sorted(rng.choice(len(loc), 4, replace=False))]
    ref.update(_local_reference(cfg, inp, loc))
    err = max(max_err(out[b, h], o) for (b, h), o in ref.items())
    kept = [nb for nb, _ in blocks]
    log("s2o 32k seed", seed, "blocks kept: min", min(kept), "max", max(kept), "max err", err)
    assert err <= BF16_TOL
    assert any(nb < total for nb, total in blocks)
