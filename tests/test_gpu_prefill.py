"""GPU parity of pyramid-selection prefill (pyramid build -> per-block joint
top-K -> chunked MFMA attention) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import lighthouse as LH
from gpu_harness import DEV, PrefillRun, log, max_err, np64

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-3
SMALL = workloads.PYRAMID_128K.with_(n_heads=2, n_ctx=2048, block_top_k=300)


def _np(inp):
    return {k: np64(v) for k, v in inp.items() if torch.is_tensor(v) and v.is_floating_point()}


def _oracle_head(cfg, ni, b, h):
    Q, K, V = ni["q"][b, h], ni["k"][b, h], ni["v"][b, h]
    kc = oracle.pyramid_levels(K, cfg.levels, cfg.factor, cfg.dtype)
    vc = oracle.pyramid_levels(V, cfg.levels, cfg.factor, cfg.dtype)
    qc = oracle.pyramid_levels(Q, cfg.levels, cfg.factor, cfg.dtype)
    sc = oracle.pyramid_scores(Q, K, cfg.levels, cfg.factor)
    return qc, kc, vc, sc


def _coarse(run, b, h, cfg, name):
    """Split a device coarse buffer into its levels."""
    x = np64(run.t[name][b, h])
    out, o, m = [], 0, cfg.n_ctx
    for _ in range(1, cfg.levels):
        m //= cfg.factor
        out.append(x[o:o + m])
        o += m
    return out


@pytest.mark.parametrize("cfg", [
    SMALL,
    SMALL.with_(levels=2, factor=2, n_ctx=1024 + 256),
    SMALL.with_(levels=4, factor=2, n_ctx=1024),
    SMALL.with_(levels=4, factor=3, n_ctx=27 * 40),           # spans of 27 rows: batches cross them
    SMALL.with_(levels=1, n_ctx=1000),                       # level 0 only: scores
    SMALL.with_(levels=2, factor=4, n_ctx=4096 + 64, batch=2),  # several runs per head, short last run
    SMALL.with_(head_dim=64, dtype="fp32", n_ctx=1024 + 16),
    SMALL.with_(head_dim=64, levels=5, factor=2, n_ctx=512),
], ids=lambda c: f"N{c.n_ctx}-L{c.levels}-p{c.factor}-d{c.head_dim}-{c.dtype}-B{c.batch}")
def test_pyramid_matches_oracle_exactly_on_lattice(cfg):
    """Lattice inputs: coarse means (accumulated exactly, rounded once) and
    squared-norm scores are exact on both sides."""
    inp = workloads.prefill_inputs(cfg, 1)
    run = PrefillRun(cfg, inp)
    run.pyramid()
    torch.cuda.synchronize()
    ni = _np(inp)
    for b in range(cfg.batch):
        for h in range(cfg.n_heads):
            qc, kc, vc, sc = _oracle_head(cfg, ni, b, h)
            for name, ref in (("pq", qc), ("pk", kc), ("pv", vc)):
                for lvl, (got, exp) in enumerate(zip(_coarse(run, b, h, cfg, name), ref)):
                    assert np.array_equal(got, exp), (name, lvl)
            got_s = np64(run.t["scores"][b, h])
            assert np.array_equal(got_s, np.concatenate(sc))


def test_pyramid_gaussian_within_one_ulp():
    cfg = SMALL
    g = torch.Generator().manual_seed(5)
    inp = {k: torch.randn(1, 2, cfg.n_ctx, 128, generator=g).to(torch.bfloat16).float()
           for k in ("q", "k", "v")}
    run = PrefillRun(cfg, inp)
    run.pyramid()
    torch.cuda.synchronize()
    ni = _np(inp)
    qc, kc, vc, sc = _oracle_head(cfg, ni, 0, 1)
    for name, ref in (("pk", kc), ("pv", vc)):
        for got, exp in zip(_coarse(run, 0, 1, cfg, name), ref):
            assert np.all(np.abs(got - exp) <= oracle.bf16_ulp(exp) * 1.0001)
    np.testing.assert_allclose(np64(run.t["scores"][0, 1]), np.concatenate(sc), rtol=2e-6)


SELECT_CASES = [
    SMALL,
    SMALL.with_(block_top_k=64),
    SMALL.with_(block_top_k=5000),                       # every visible entry
    SMALL.with_(n_ctx=2048 + 16 * 9, block_top_k=500),   # ragged last block
    SMALL.with_(levels=2, factor=2, n_ctx=1024, block_top_k=100),
    SMALL.with_(n_ctx=8192, block_top_k=300),           # intervals past the first: bound > 0
    SMALL.with_(n_ctx=8192, block_top_k=7000),          # no room for intervals: full passes
    SMALL.with_(levels=4, factor=3, n_ctx=27 * 200, q_block=54, block_top_k=700),
]


@pytest.mark.parametrize("cfg", SELECT_CASES,
                         ids=lambda c: f"N{c.n_ctx}-L{c.levels}-p{c.factor}-K{c.block_top_k}")
def test_block_select_exact_on_lattice(cfg):
    inp = workloads.prefill_inputs(cfg, 2)
    run = PrefillRun(cfg, inp)
    run.pyramid()
    run.select()
    torch.cuda.synchronize()
    idx = run.t["blk_idx"].cpu().numpy()
    cnt = run.t["blk_count"].cpu().numpy()
    ni = _np(inp)
    for b in range(cfg.batch):
        for h in range(cfg.n_heads):
            sc = oracle.pyramid_scores(ni["q"][b, h], ni["k"][b, h], cfg.levels, cfg.factor)
            for blk in range(run.nblk):
                ref = oracle.block_select(sc, blk, cfg.n_ctx, cfg.levels, cfg.factor,
                                          cfg.q_block, cfg.block_top_k)
                c = cnt[b, h, blk]
                assert c == len(ref), (h, blk, c, len(ref))
                got = idx[b, h, blk, :c]
                assert np.all(np.diff(got) > 0)            # ascending flat ids
                assert np.array_equal(np.sort(got), np.sort(ref)), (h, blk)


def _check_prefill(cfg, run, ni, blocks_of_head):
    out = np64(run.t["out"])
    idx = run.t["blk_idx"].cpu().numpy()
    cnt = run.t["blk_count"].cpu().numpy()
    worst = 0.0
    for (b, h), blocks in blocks_of_head.items():
        qc, kc, vc, sc = _oracle_head(cfg, ni, b, h)
        for blk in blocks:
            sel = oracle.block_select(sc, blk, cfg.n_ctx, cfg.levels, cfg.factor, cfg.q_block,
                                      cfg.block_top_k)
            got_sel = idx[b, h, blk, :cnt[b, h, blk]]
            assert np.array_equal(np.sort(got_sel), np.sort(sel)), (h, blk)
            ref = LH.prefill_block(ni["q"][b, h], ni["k"][b, h], ni["v"][b, h], kc, vc, sel, blk,
                                   cfg.q_block, cfg.levels, cfg.factor)
            lo = blk * cfg.q_block
            worst = max(worst, max_err(out[b, h, lo:lo + len(ref)], ref))
    log("prefill max err", worst)
    return worst


def test_prefill_end_to_end_small():
    cfg = SMALL.with_(n_ctx=2048 + 64)
    inp = workloads.prefill_inputs(cfg, 3)
    run = PrefillRun(cfg, inp)
    run.pyramid(); run.select(); run.prefill()
    torch.cuda.synchronize()
    ni = _np(inp)
    blocks = {(0, h): list(range(run.nblk)) for h in range(cfg.n_heads)}
    worst = _check_prefill(cfg, run, ni, blocks)
    assert worst <= BF16_TOL
    # the probabilities reach the PV product as a bf16 high part plus a bf16
    # remainder (~16 bits).  On these inputs that stays near 2e-5, where one
    # bf16 probability would reach 1.1e-2 and one fp16 probability 1.2e-3
    # (the same weights rounded in fp64, the rest exact)
    assert worst <= 2e-4


def _random_prefill_configs(count, seed):
    """Seeded pyramid prefill shapes: levels 1-5 with factor 2 or 4 (a span
    of the top level divides the 128-query block), a budget K from 1 to a
    full list, one or two sequences and heads, and contexts that end in a
    ragged block."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        p = int(rng.choice([2, 4]))
        L = int(rng.integers(1, (6 if p == 2 else 4) + 1))
        span = p ** (L - 1)
        n = span * int(rng.integers(max(1, 130 // span), 4096 // span + 1))
        out.append(SMALL.with_(batch=int(rng.integers(1, 3)), n_heads=int(rng.integers(1, 3)),
                               levels=L, factor=p, n_ctx=n,
                               block_top_k=int(rng.integers(1, 1500 if rng.random() < 0.8 else 8193))))
    return out


@pytest.mark.parametrize("cfg", _random_prefill_configs(12, 11),
                         ids=lambda c: f"N{c.n_ctx}-L{c.levels}-p{c.factor}-K{c.block_top_k}-B{c.batch}H{c.n_heads}")
def test_prefill_random_shapes(cfg):
    """Pyramid, block selection and attention on seeded random shapes: every
    block's set exact and every output within the bf16 tolerance."""
    log("prefill random", cfg.batch, cfg.n_heads, cfg.n_ctx, cfg.levels, cfg.factor, cfg.block_top_k)
    inp = workloads.prefill_inputs(cfg, 5)
    run = PrefillRun(cfg, inp)
    run.pyramid(); run.select(); run.prefill()
    torch.cuda.synchronize()
    blocks = {(b, h): list(range(run.nblk)) for b in range(cfg.batch) for h in range(cfg.n_heads)}
    assert _check_prefill(cfg, run, _np(inp), blocks) <= BF16_TOL


def test_prefill_largest_selection():
    """block_top_k at the largest list the attention kernel stages (8192): the
    late blocks see more entries than that, so their key sequence - the
    selection, the block's own keys and the tail the gathers ahead run past -
    fills the staging area exactly; the last block is ragged (64 queries)."""
    cfg = SMALL.with_(n_heads=1, n_ctx=8192 + 64, block_top_k=8192)
    inp = workloads.prefill_inputs(cfg, 9)
    run = PrefillRun(cfg, inp)
    run.pyramid(); run.select(); run.prefill()
    torch.cuda.synchronize()
    ni = _np(inp)
    cnt = run.t["blk_count"].cpu().numpy()
    assert cnt[0, 0, run.nblk - 1] == 8192                  # the list is full there
    blocks = [0, 1, 48, 49, 50, run.nblk - 2, run.nblk - 1]
    worst = _check_prefill(cfg, run, ni, {(0, 0): blocks})
    assert worst <= BF16_TOL


def test_prefill_over_given_selection():
    """The attention stage alone: blk_idx filled with random visible entries
    drawn by the test's generator, unsorted."""
    cfg = SMALL.with_(block_top_k=200)
    inp = workloads.prefill_inputs(cfg, 4)
    run = PrefillRun(cfg, inp)
    run.pyramid()
    torch.cuda.synchronize()
    gen = np.random.default_rng(8)
    sels = {}
    for blk in range(run.nblk):
        vis = oracle.visible_entries(blk, cfg.n_ctx, cfg.levels, cfg.factor, cfg.q_block)
        offs = LH.level_offsets(cfg.n_ctx, cfg.levels, cfg.factor)
        flat = np.array([offs[l] + j for l, j in vis], np.int64)
        m = int(gen.integers(0, min(len(flat), cfg.block_top_k) + 1))
        pick = gen.permutation(flat)[:m]
        sels[blk] = pick
        for h in range(cfg.n_heads):
            run.t["blk_idx"][0, h, blk, :m] = torch.tensor(pick, dtype=torch.int32)
            run.t["blk_count"][0, h, blk] = m
    run.prefill()
    torch.cuda.synchronize()
    out = np64(run.t["out"])
    ni = _np(inp)
    worst = 0.0
    for h in range(cfg.n_heads):
        _, kc, vc, _ = _oracle_head(cfg, ni, 0, h)
        for blk, sel in sels.items():
            ref = LH.prefill_block(ni["q"][0, h], ni["k"][0, h], ni["v"][0, h], kc, vc, sel, blk,
                                   cfg.q_block, cfg.levels, cfg.factor)
            lo = blk * cfg.q_block
            worst = max(worst, max_err(out[0, h, lo:lo + len(ref)], ref))
    log("given-selection max err", worst)
    assert worst <= BF16_TOL


def test_prefill_one_level_full_budget_is_dense_causal():
    cfg = SMALL.with_(levels=1, n_ctx=1024, block_top_k=1024)
    inp = workloads.prefill_inputs(cfg, 6)
    run = PrefillRun(cfg, inp)
    run.pyramid(); run.select(); run.prefill()
    torch.cuda.synchronize()
    ni = _np(inp)
    out = np64(run.t["out"])
    for h in range(cfg.n_heads):
        ref = oracle.dense_causal(ni["q"][0, h], ni["k"][0, h], ni["v"][0, h])
        assert max_err(out[0, h], ref) <= BF16_TOL


def test_prefill_full_size_sampled():
    """The 128K, 16-head workload at full size, inputs drawn on the GPU,
    against the oracle head by head: every head's scores; every block of
    heads 0 and 11 (selection sets and outputs); 64 seeded blocks of each of
    the other 14 heads."""
    cfg = workloads.PYRAMID_128K
    inp = workloads.prefill_inputs(cfg, 7, device=DEV)
    run = PrefillRun(cfg, inp)
    run.pyramid(); run.select(); run.prefill()
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    sub = cfg.with_(n_heads=1)
    worst = 0.0
    for h in range(cfg.n_heads):
        ni = {k: np64(inp[k][:, h:h + 1]) for k in ("q", "k", "v")}
        sc = oracle.pyramid_scores(ni["q"][0, 0], ni["k"][0, 0], cfg.levels, cfg.factor)
        assert np.array_equal(np64(run.t["scores"][0, h]), np.concatenate(sc)), h
        if h in (0, 11):
            blocks = list(range(run.nblk))
        else:
            blocks = sorted(set([0, run.nblk - 1] + rng.choice(run.nblk, 62, replace=False).tolist()))

        class One:                   # this head as a 1-head run
            t = {k: run.t[k][:, h:h + 1] for k in ("out", "blk_idx", "blk_count")}
        worst = max(worst, _check_prefill(sub, One, ni, {(0, 0): blocks}))
        log("prefill full size: head", h, "blocks", len(blocks))
    log("prefill full size max err", worst)
    assert worst <= BF16_TOL


def test_block_select_all_equal_scores():
    """Every score equal (zero queries and keys): every visible entry ties, so
    the later intervals hold more candidates than fit and their blocks take
    the full passes; the kept entries are the lowest flat ids."""
    cfg = SMALL.with_(n_ctx=8192, block_top_k=300)
    inp = workloads.prefill_inputs(cfg, 3)
    inp["q"] = torch.zeros_like(inp["q"])
    inp["k"] = torch.zeros_like(inp["k"])
    run = PrefillRun(cfg, inp)
    run.pyramid()
    run.select()
    torch.cuda.synchronize()
    idx = run.t["blk_idx"].cpu().numpy()
    cnt = run.t["blk_count"].cpu().numpy()
    ni = _np(inp)
    for h in range(cfg.n_heads):
        sc = oracle.pyramid_scores(ni["q"][0, h], ni["k"][0, h], cfg.levels, cfg.factor)
        for blk in range(run.nblk):
            ref = oracle.block_select(sc, blk, cfg.n_ctx, cfg.levels, cfg.factor, cfg.q_block,
                                      cfg.block_top_k)
            c = cnt[0, h, blk]
            assert c == len(ref), (h, blk, c, len(ref))
            assert np.array_equal(idx[0, h, blk, :c], np.sort(ref)), (h, blk)


def test_prefill_wide_score_range():
    """A few keys scaled x32 (still exact in bf16): their scores exceed the
    rest by thousands in the log2 domain, so the softmax reference must be the
    true maximum over the whole tile, or the weights overflow."""
    cfg = SMALL.with_(n_ctx=2048, block_top_k=300)
    inp = workloads.prefill_inputs(cfg, 5)
    g = torch.Generator().manual_seed(55)
    rows = torch.randperm(cfg.n_ctx, generator=g)[:24]
    inp["k"][:, :, rows] *= 32
    run = PrefillRun(cfg, inp)
    run.pyramid(); run.select(); run.prefill()
    torch.cuda.synchronize()
    assert torch.isfinite(run.t["out"]).all()
    ni = _np(inp)
    worst = _check_prefill(cfg, run, ni, {(0, h): range(run.nblk) for h in range(cfg.n_heads)})
    assert worst <= BF16_TOL
