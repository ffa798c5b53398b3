"""GPU parity of the coarse queries of the pyramid prefill (Lighthouse
summary, 2A and 2C: the symmetric pyramid's coarse query entries attend to
their block's selected entries and to their own level's entries of the block
up to themselves; each output returns to its own slot) against the fp64
oracle, through the C ABI."""
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


def _levels(x, cfg):
    """Split a [Nc, d] coarse buffer into its levels 1 .. L-1."""
    out, o, m = [], 0, cfg.n_ctx
    for _ in range(1, cfg.levels):
        m //= cfg.factor
        out.append(x[o:o + m])
        o += m
    return out


def _check(cfg, run, ni, blocks_of_head, sels=None):
    """Max error of the device's coarse outputs over the given blocks, the
    oracle fed the same stored pyramid rows and the device's lists (after
    checking those against the oracle's selection when ``sels`` is None)."""
    got = np64(run.t["out_pyr"])
    idx = run.t["blk_idx"].cpu().numpy()
    cnt = run.t["blk_count"].cpu().numpy()
    worst = 0.0
    for (b, h), blocks in blocks_of_head.items():
        qc = _levels(np64(run.t["pq"][b, h]), cfg)
        kc = _levels(np64(run.t["pk"][b, h]), cfg)
        vc = _levels(np64(run.t["pv"][b, h]), cfg)
        sc = oracle.pyramid_scores(ni["q"][b, h], ni["k"][b, h], cfg.levels, cfg.factor)
        out = _levels(got[b, h], cfg)
        for blk in blocks:
            sel = idx[b, h, blk, :cnt[b, h, blk]]
            if sels is None:
                ref_sel = oracle.block_select(sc, blk, cfg.n_ctx, cfg.levels, cfg.factor,
                                              cfg.q_block, cfg.block_top_k)
                assert np.array_equal(np.sort(sel), np.sort(ref_sel)), (h, blk)
            ref = oracle.coarse_block(qc, kc, vc, ni["k"][b, h], ni["v"][b, h], sel, blk,
                                      cfg.q_block, cfg.levels, cfg.factor)
            for lvl in range(1, cfg.levels):
                lo = blk * cfg.q_block // cfg.factor ** lvl
                r = ref[lvl - 1]
                worst = max(worst, max_err(out[lvl - 1][lo:lo + len(r)], r))
    return worst


def _np(inp):
    return {k: np64(v) for k, v in inp.items() if torch.is_tensor(v) and v.is_floating_point()}


CASES = [
    SMALL.with_(n_ctx=2048 + 64),                             # ragged last block
    SMALL.with_(levels=2, factor=2, n_ctx=1024 + 256, block_top_k=100),
    SMALL.with_(levels=4, factor=2, n_ctx=1024, block_top_k=700),
    SMALL.with_(levels=8, factor=2, n_ctx=1024, block_top_k=64),    # 127 coarse queries per block
    SMALL.with_(levels=2, factor=4, n_ctx=4096 + 64, batch=2),
]


@pytest.mark.parametrize("cfg", CASES,
                         ids=lambda c: f"N{c.n_ctx}-L{c.levels}-p{c.factor}-K{c.block_top_k}-B{c.batch}")
def test_coarse_queries_match_oracle(cfg):
    inp = workloads.prefill_inputs(cfg, 11)
    run = PrefillRun(cfg, inp)
    run.pyramid(); run.select(); run.coarse()
    torch.cuda.synchronize()
    ni = _np(inp)
    blocks = {(b, h): list(range(run.nblk)) for b in range(cfg.batch) for h in range(cfg.n_heads)}
    worst = _check(cfg, run, ni, blocks)
    log("coarse max err", cfg.levels, cfg.factor, worst)
    assert torch.isfinite(run.t["out_pyr"][:, :, :run.nc]).all()
    assert worst <= BF16_TOL
    # the same probability format as the level-0 queries (a bf16 high part
    # plus a bf16 remainder)
    assert worst <= 2e-4


def test_coarse_queries_over_given_selection_and_level0_unchanged():
    """The attention stage alone, over random unsorted visible entries; the
    level-0 outputs of the same lists are not touched by the coarse call."""
    cfg = SMALL.with_(block_top_k=200)
    inp = workloads.prefill_inputs(cfg, 12)
    run = PrefillRun(cfg, inp)
    run.pyramid()
    torch.cuda.synchronize()
    gen = np.random.default_rng(9)
    offs = LH.level_offsets(cfg.n_ctx, cfg.levels, cfg.factor)
    for blk in range(run.nblk):
        vis = oracle.visible_entries(blk, cfg.n_ctx, cfg.levels, cfg.factor, cfg.q_block)
        flat = np.array([offs[l] + j for l, j in vis], np.int64)
        m = int(gen.integers(0, min(len(flat), cfg.block_top_k) + 1))
        pick = gen.permutation(flat)[:m]
        for h in range(cfg.n_heads):
            run.t["blk_idx"][0, h, blk, :m] = torch.tensor(pick, dtype=torch.int32)
            run.t["blk_count"][0, h, blk] = m
    run.prefill()
    torch.cuda.synchronize()
    before = run.t["out"].clone()
    run.coarse()
    torch.cuda.synchronize()
    assert torch.equal(run.t["out"], before)
    worst = _check(cfg, run, _np(inp), {(0, h): range(run.nblk) for h in range(cfg.n_heads)},
                   sels="given")
    log("coarse given-selection max err", worst)
    assert worst <= BF16_TOL


def test_coarse_one_level_writes_nothing():
    cfg = SMALL.with_(levels=1, n_ctx=1024)
    run = PrefillRun(cfg, workloads.prefill_inputs(cfg, 13))
    run.pyramid(); run.select(); run.coarse()
    torch.cuda.synchronize()
    assert torch.isnan(run.t["out_pyr"]).all()


def test_coarse_full_size_sampled():
    """The 128K, 16-head workload at full size (inputs drawn on the GPU): all
    blocks of head 3, and 48 seeded blocks of heads 0 and 15."""
    cfg = workloads.PYRAMID_128K
    inp = workloads.prefill_inputs(cfg, 14, device=DEV)
    run = PrefillRun(cfg, inp)
    run.pyramid(); run.select(); run.coarse()
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    sub = cfg.with_(n_heads=1)
    worst = 0.0
    for h in (3, 0, 15):
        ni = {k: np64(inp[k][:, h:h + 1]) for k in ("q", "k", "v")}
        if h == 3:
            blocks = list(range(run.nblk))
        else:
            blocks = sorted(set([0, 1, run.nblk - 1] + rng.choice(run.nblk, 45, replace=False).tolist()))

        class One:                   # this head as a 1-head run
            t = {k: run.t[k][:, h:h + 1] for k in ("out_pyr", "blk_idx", "blk_count", "pq", "pk", "pv")}
        worst = max(worst, _check(sub, One, ni, {(0, 0): blocks}))
        log("coarse full size: head", h, "blocks", len(blocks))
    log("coarse full size max err", worst)
    assert worst <= BF16_TOL
