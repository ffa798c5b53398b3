"""GPU parity of the decode path (index build -> select -> decode) against
the fp64 oracle, called through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import DecodeRun, log, max_err, np64, np_inputs, to_dev, DEV

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-3
FP32_TOL = 1e-5


def _ret_groups(cfg):
    G = cfg.gqa
    kinds = cfg.head_kind()
    return [g for g in range(cfg.n_kv_heads) if kinds[g * G] == workloads.HEAD_RETRIEVAL]


def _oracle_logits(cfg, k_idx, q_idx, b, g):
    G = cfg.gqa
    return oracle.index_logits(q_idx[b, g * G:(g + 1) * G], k_idx[b, g, :cfg.n_ctx], cfg.r)


def _robust_seed(cfg, make, accept, start=0, tries=64):
    """First seed whose oracle selection passes ``accept`` (inputs drawn so
    that the cut cannot move under last-place rounding)."""
    for s in range(start, start + tries):
        inp = make(s)
        if accept(inp):
            return s, inp
    raise AssertionError("no seed met the robustness criterion")


# ------------------------------------------------------------------ index
@pytest.mark.parametrize("cfg", [
    workloads.TINY,
    workloads.LLAMA_32K.with_(batch=2, n_ctx=3001),
])
def test_index_lowrank_matches_oracle(cfg):
    log("index", cfg.name, cfg.n_ctx)
    inp = workloads.decode_inputs(cfg, 7)
    run = DecodeRun(cfg, inp, n_cap=cfg.n_ctx + 37)
    run.index()
    torch.cuda.synchronize()
    k_gpu = np64(run.t["k_idx"])
    q_gpu = np64(run.t["q_idx"])
    ni = np_inputs(inp)
    G = cfg.gqa
    for b in range(cfg.batch):
        for g in _ret_groups(cfg):
            ref = oracle.index_keys(ni["k_pre"][b, g, :cfg.n_ctx], ni["proj"][g], cfg.dtype)
            got = k_gpu[b, g, :cfg.n_ctx]
            if cfg.dtype == "bf16":
                exact = ni["k_pre"][b, g, :cfg.n_ctx] @ ni["proj"][g].T
                # one bf16 ulp, plus the fp32 summation bound d * 2^-24 * sum|terms|
                # where cancellation leaves a value far below its terms
                ulp = np.maximum(oracle.bf16_ulp(exact), oracle.bf16_ulp(ref))
                acc = cfg.head_dim * 2.0 ** -24 * (np.abs(ni["k_pre"][b, g, :cfg.n_ctx])
                                                   @ np.abs(ni["proj"][g]).T)
                assert np.all(np.abs(got - ref) <= ulp * 1.0001 + acc)
                assert np.mean(got == ref) > 0.99
            else:
                np.testing.assert_allclose(got, ref, rtol=2e-6, atol=2e-6)
            qref = oracle.index_query(ni["q_pre"][b, g * G:(g + 1) * G], ni["proj"][g])
            np.testing.assert_allclose(q_gpu[b, g * G:(g + 1) * G], qref, rtol=2e-6, atol=2e-6)
            # untouched capacity rows stay zero
            assert np.all(k_gpu[b, g, cfg.n_ctx:] == 0)


# ------------------------------------------------------------------ selector, exact sets
LATTICE_CASES = [
    # (config, k_amp, q_amp, mode)
    (workloads.LLAMA_32K.with_(batch=2, n_ctx=5000, min_tokens=0, top_p=0.9), 8, 4, "topp"),
    (workloads.LLAMA_32K.with_(batch=2, n_ctx=5000, min_tokens=0, top_p=0.9), 24, 12, "topp"),
    (workloads.LLAMA_32K.with_(batch=2, n_ctx=5000, min_tokens=0, top_p=0.5), 64, 32, "topp"),
    (workloads.LLAMA_32K.with_(batch=2, n_ctx=5000, min_tokens=300, top_p=0.5), 64, 32, "topp"),
    (workloads.LLAMA_32K.with_(batch=1, n_ctx=777, top_p=0.95, min_tokens=64), 24, 12, "topp"),
    (workloads.LLAMA_32K.with_(batch=1, n_ctx=33000, top_p=0.95, min_tokens=64), 24, 12, "topp"),
    (workloads.TINY.with_(top_p=0.9), 24, 12, "topp"),
    (workloads.LLAMA_32K.with_(batch=2, n_ctx=5000, top_p=1.0, top_k=300), 24, 12, "topk"),
    (workloads.LLAMA_32K.with_(batch=2, n_ctx=5000, top_p=1.0, top_k=2048), 8, 4, "topk"),
    (workloads.LLAMA_32K.with_(batch=1, n_ctx=9000, top_p=1.0, top_k=1), 64, 32, "topk"),
    (workloads.TINY.with_(top_p=1.0, top_k=100), 8, 4, "topk"),
]


@pytest.mark.parametrize("case", LATTICE_CASES, ids=lambda c: f"{c[0].name}-{c[0].n_ctx}-{c[3]}-{c[1]}")
def test_select_lattice_sets_exact(case):
    cfg, ka, qa, mode = case
    log("select lattice", cfg.name, cfg.n_ctx, mode, ka, qa)

    def make(s):
        return workloads.lattice_index_inputs(cfg, 100 + s, k_amp=ka, q_amp=qa)

    def accept(inp):
        if mode != "topp":
            return True
        k, q = np64(inp["k_idx"]), np64(inp["q_idx"])
        for b in range(cfg.batch):
            for g in _ret_groups(cfg):
                if oracle.topp_margin(_oracle_logits(cfg, k, q, b, g), cfg.top_p) < 1e-7:
                    return False
        return True

    seed, inp = _robust_seed(cfg, make, accept)
    run = DecodeRun(cfg, {}, n_cap=cfg.n_ctx)
    run.t["k_idx"].copy_(to_dev(inp["k_idx"], cfg.dtype))
    run.t["q_idx"].copy_(inp["q_idx"].to(DEV))
    run.select()
    torch.cuda.synchronize()
    idx, cnt = run.sets()
    k, q = np64(inp["k_idx"]), np64(inp["q_idx"])
    for b in range(cfg.batch):
        for g in _ret_groups(cfg):
            lg = _oracle_logits(cfg, k, q, b, g)
            if mode == "topp":
                ref, m = oracle.select_topp(lg, cfg.top_p, cfg.min_tokens)
            else:
                ref, m = oracle.select_topk(lg, cfg.top_k)
            assert cnt[b, g] == m, (b, g, cnt[b, g], m)
            assert np.array_equal(idx[b, g, :m], ref), (b, g)


def test_select_strict_gap_variant():
    # lattice inputs redrawn until the cut falls between distinct logits, so
    # no tie-break decides the boundary (gap >= 1/512 > 1e-3)
    cfg = workloads.LLAMA_32K.with_(batch=1, n_ctx=4000, top_p=0.8, min_tokens=0)

    def make(s):
        return workloads.lattice_index_inputs(cfg, 500 + s, k_amp=24, q_amp=12)

    def accept(inp):
        k, q = np64(inp["k_idx"]), np64(inp["q_idx"])
        for g in _ret_groups(cfg):
            lg = _oracle_logits(cfg, k, q, 0, g)
            _, m = oracle.select_topp(lg, cfg.top_p)
            if oracle.cut_gap(lg, m) < 1e-3 or oracle.topp_margin(lg, cfg.top_p) < 1e-7:
                return False
        return True

    seed, inp = _robust_seed(cfg, make, accept, tries=400)
    log("strict gap seed", seed)
    run = DecodeRun(cfg, {}, n_cap=cfg.n_ctx)
    run.t["k_idx"].copy_(to_dev(inp["k_idx"], cfg.dtype))
    run.t["q_idx"].copy_(inp["q_idx"].to(DEV))
    run.select()
    idx, cnt = run.sets()
    k, q = np64(inp["k_idx"]), np64(inp["q_idx"])
    for g in _ret_groups(cfg):
        ref, m = oracle.select_topp(_oracle_logits(cfg, k, q, 0, g), cfg.top_p)
        assert cnt[0, g] == m and np.array_equal(idx[0, g, :m], ref)


# ------------------------------------------------------------------ decode over given lists
@pytest.mark.parametrize("cfg", [
    workloads.TINY.with_(n_ctx=3000),
    workloads.LLAMA_32K.with_(batch=2, n_ctx=4099),
    workloads.LLAMA_32K.with_(batch=1, n_ctx=700, n_q_heads=8, n_kv_heads=8, window=50),
])
def test_decode_over_given_lists(cfg):
    """The attention stage alone: random ascending lists (drawn by the
    generator side of the test) for the selecting groups, sinks+window for
    local ones."""
    log("decode lists", cfg.name, cfg.n_ctx)
    inp = workloads.decode_inputs(cfg, 11)
    run = DecodeRun(cfg, inp, n_cap=cfg.n_ctx + 5)
    gen = torch.Generator().manual_seed(3)
    sets = {}
    for b in range(cfg.batch):
        for g in range(cfg.n_kv_heads):
            if g in _ret_groups(cfg):
                m = int(torch.randint(1, cfg.n_ctx + 1, (1,), generator=gen))
                T = torch.sort(torch.randperm(cfg.n_ctx, generator=gen)[:m]).values
                run.t["sel_idx"][b, g, :m] = T.to(DEV, torch.int32)
                run.t["sel_count"][b, g] = m
                sets[(b, g)] = T.numpy()
            else:
                sets[(b, g)] = oracle.local_set(cfg.n_ctx, cfg.sinks, cfg.window)
    run.decode()
    out = np64(run.t["out"])
    ref = oracle.decode_step(cfg, np_inputs(inp), sets=sets)
    tol = FP32_TOL if cfg.dtype == "fp32" else BF16_TOL
    err = max(max_err(out[b, h], o) for (b, h), o in ref.items())
    log("max err", err)
    assert err <= tol


# ------------------------------------------------------------------ end to end
def _pipeline_check(cfg, seed, require_exact_sets, sample=None, alpha=1.0):
    inp = workloads.decode_inputs(cfg, seed, alpha=alpha)
    run = DecodeRun(cfg, inp)
    run.index()
    run.select()
    run.decode()
    torch.cuda.synchronize()
    idx, cnt = run.sets()
    out = np64(run.t["out"])
    ni = np_inputs(inp)
    groups = [(b, g) for b in range(cfg.batch) for g in range(cfg.n_kv_heads)]
    if sample is not None:
        rng = np.random.default_rng(seed)
        groups = [groups[i] for i in sorted(rng.choice(len(groups), sample, replace=False))]
    osets = oracle.decode_token_sets(cfg, ni, groups=groups)
    ret = set(_ret_groups(cfg))
    tol = FP32_TOL if cfg.dtype == "fp32" else BF16_TOL
    worst = 0.0
    for (b, g), T in osets.items():
        if g in ret:
            got = idx[b, g, :cnt[b, g]]
            assert np.all(np.diff(got) > 0)
            if require_exact_sets:
                assert np.array_equal(got, T), (b, g, len(got), len(T))
            else:
                # any disagreement sits at the cut: the oracle logits of the
                # tokens on one side only are within 2e-3 of the cut logit
                k = oracle.index_keys(ni["k_pre"][b, g, :cfg.n_ctx], ni["proj"][g], cfg.dtype)
                q = oracle.index_query(ni["q_pre"][b, g * cfg.gqa:(g + 1) * cfg.gqa], ni["proj"][g])
                lg = oracle.index_logits(q, k, cfg.r)
                cut = lg[T].min()
                diff = np.setxor1d(got, T)
                assert len(diff) <= max(8, len(T) // 1000), (b, g, len(diff))
                assert np.all(np.abs(lg[diff] - cut) <= 2e-3)
        ref = oracle.decode_step(cfg, ni, sets={(b, g): T})
        for (bb, h), o in ref.items():
            worst = max(worst, max_err(out[bb, h], o))
    log("pipeline", cfg.name, cfg.n_ctx, "max err", worst)
    assert worst <= tol


def _robust_pipeline_seed(cfg, start, tries=40, gap=1e-4, margin=1e-6):
    """Seed whose oracle cut, in every retrieval row, has a logit gap >= gap
    and a mass margin >= margin."""
    for s in range(start, start + tries):
        ni = np_inputs(workloads.decode_inputs(cfg, s))
        ok = True
        for b in range(cfg.batch):
            for g in _ret_groups(cfg):
                k = oracle.index_keys(ni["k_pre"][b, g, :cfg.n_ctx], ni["proj"][g], cfg.dtype)
                q = oracle.index_query(ni["q_pre"][b, g * cfg.gqa:(g + 1) * cfg.gqa], ni["proj"][g])
                lg = oracle.index_logits(q, k, cfg.r)
                if cfg.top_k:
                    s_, m = oracle.select_topk(lg, cfg.top_k)
                else:
                    s_, m = oracle.select_topp(lg, cfg.top_p, cfg.min_tokens)
                    if m < cfg.n_ctx and m > cfg.min_tokens and oracle.topp_margin(lg, cfg.top_p) < margin:
                        ok = False
                if oracle.cut_gap(lg, m) < gap:
                    ok = False
        if ok:
            return s
    raise AssertionError("no robust seed")


def test_pipeline_tiny_fp32():
    cfg = workloads.TINY
    seed = _robust_pipeline_seed(cfg, 0, gap=1e-4)
    log("tiny seed", seed)
    _pipeline_check(cfg, seed, require_exact_sets=True)


def test_pipeline_llama_small_bf16_topp():
    cfg = workloads.LLAMA_32K.with_(batch=2, n_ctx=5000)
    seed = _robust_pipeline_seed(cfg, 0)
    _pipeline_check(cfg, seed, require_exact_sets=True)


def test_pipeline_llama_small_bf16_topk():
    cfg = workloads.LLAMA_128K_TOPK.with_(batch=2, n_ctx=6000, top_k=500)
    seed = _robust_pipeline_seed(cfg, 0)
    _pipeline_check(cfg, seed, require_exact_sets=True)


@pytest.mark.parametrize("alpha", [0.5, 2.0])
def test_pipeline_entropy_variants(alpha):
    cfg = workloads.LLAMA_32K.with_(batch=1, n_ctx=4096)
    _pipeline_check(cfg, 21, require_exact_sets=False, alpha=alpha)


def test_pipeline_llama_32k_full_size_sampled():
    _pipeline_check(workloads.LLAMA_32K, 1, require_exact_sets=False, sample=6)


def test_pipeline_llama_128k_topk_full_size_sampled():
    _pipeline_check(workloads.LLAMA_128K_TOPK, 2, require_exact_sets=False, sample=4)


def test_pipeline_llama_128k_topp_full_size_sampled():
    """The 128K top-p step at full size: tens of thousands of selected tokens
    per group, so every work item spans many tiles."""
    _pipeline_check(workloads.LLAMA_128K, 3, require_exact_sets=False, sample=4)


# ------------------------------------------------------------------ edge cases
@pytest.mark.parametrize("cfg", [
    workloads.TINY.with_(n_ctx=1, needles_per_head=0),
    workloads.TINY.with_(n_ctx=2, needles_per_head=0, top_p=0.3),
    workloads.TINY.with_(n_ctx=100, window=1000),
    workloads.TINY.with_(n_ctx=100, sinks=0, window=1),
    workloads.TINY.with_(n_ctx=100, sinks=100, window=0),
    workloads.TINY.with_(n_ctx=1500, top_p=1.0),
    workloads.TINY.with_(n_ctx=1500, top_p=1.0, top_k=1500),
    workloads.TINY.with_(n_ctx=1500, top_p=1.0, top_k=1),
    workloads.LLAMA_32K.with_(batch=1, n_ctx=60, min_tokens=64),
    workloads.LLAMA_32K.with_(batch=1, n_ctx=1025, window=1),
])
def test_edge_cases(cfg):
    log("edge", cfg)
    _pipeline_check(cfg, 5, require_exact_sets=False)


def test_runs_are_bitwise_repeatable():
    cfg = workloads.LLAMA_32K.with_(batch=2, n_ctx=9000)
    inp = workloads.decode_inputs(cfg, 4)
    outs = []
    for _ in range(2):
        run = DecodeRun(cfg, inp)
        run.index(); run.select(); run.decode()
        torch.cuda.synchronize()
        outs.append((run.t["out"].clone(), run.t["sel_idx"].clone(), run.t["sel_count"].clone(),
                     run.t["k_idx"].clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_incremental_index_append_equals_full_build():
    cfg = workloads.LLAMA_32K.with_(batch=1, n_ctx=2000)
    inp = workloads.decode_inputs(cfg, 9)
    full = DecodeRun(cfg, inp)
    full.index()
    inc = DecodeRun(cfg, inp)
    inc.index(0, 1500)
    for t in range(1500, 2000, 97):
        inc.index(t, min(2000, t + 97))
    torch.cuda.synchronize()
    assert torch.equal(full.t["k_idx"], inc.t["k_idx"])


def test_workspace_reuse_across_calls():
    """The decode workspace's completion counters return to zero after every
    call: repeated calls on one workspace give identical, finite outputs, also
    after a smaller problem has used it."""
    cfg = workloads.LLAMA_32K.with_(batch=2, n_ctx=6000)
    inp = workloads.decode_inputs(cfg, 12)
    run = DecodeRun(cfg, inp)
    run.index(); run.select(); run.decode()
    first = run.t["out"].clone()
    assert torch.isfinite(first).all()
    small = DecodeRun(cfg.with_(n_ctx=1500), workloads.decode_inputs(cfg.with_(n_ctx=1500), 13))
    small.ws_dec = run.ws_dec
    small.index(); small.select(); small.decode()
    assert torch.isfinite(small.t["out"]).all()
    for _ in range(3):
        run.t["out"].fill_(float("nan"))
        run.decode()
        torch.cuda.synchronize()
        assert torch.equal(run.t["out"], first)


def test_select_workspace_reuse_changing_data_and_shape():
    """One selector workspace across calls whose data, context length (its
    tile count) and batch change: every call's sets equal the oracle's."""
    base = workloads.LLAMA_32K.with_(batch=2, n_ctx=5000, top_p=0.95, min_tokens=64)
    steps = [(base, 0), (base, 1), (base.with_(n_ctx=6100), 2), (base.with_(n_ctx=2100), 3),
             (base.with_(batch=1, n_ctx=6100), 4), (base, 5)]
    ws = None
    for cfg, s in steps:
        log("select reuse", cfg.batch, cfg.n_ctx, s)

        def accept(inp, cfg=cfg):
            k, q = np64(inp["k_idx"]), np64(inp["q_idx"])
            return all(oracle.topp_margin(_oracle_logits(cfg, k, q, b, g), cfg.top_p) >= 1e-7
                       for b in range(cfg.batch) for g in _ret_groups(cfg))

        _, inp = _robust_seed(cfg, lambda t, cfg=cfg: workloads.lattice_index_inputs(
            cfg, 500 + 10 * s + t, k_amp=24, q_amp=12), accept)
        run = DecodeRun(cfg, {}, n_cap=cfg.n_ctx)
        if ws is not None:
            run.ws_sel = ws
        ws = run.ws_sel
        run.t["k_idx"].copy_(to_dev(inp["k_idx"], cfg.dtype))
        run.t["q_idx"].copy_(inp["q_idx"].to(DEV))
        run.select()
        torch.cuda.synchronize()
        idx, cnt = run.sets()
        k, q = np64(inp["k_idx"]), np64(inp["q_idx"])
        for b in range(cfg.batch):
            for g in _ret_groups(cfg):
                ref, m = oracle.select_topp(_oracle_logits(cfg, k, q, b, g), cfg.top_p,
                                            cfg.min_tokens)
                assert cnt[b, g] == m, (s, b, g, cnt[b, g], m)
                assert np.array_equal(idx[b, g, :m], ref), (s, b, g)
