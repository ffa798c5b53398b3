"""GPU parity of hierarchical routing during chunked prefill (every query
block of one chunk routes with its mean query; the prefill kernel then adds
each query's causal part of the block) against the fp64 oracle, through the
C ABI."""
import numpy as np
import pytest
import torch

import oracle
import selection_sparse_attention_amd as sa
import workloads
from gpu_harness import DEV, log, max_err, np64, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-3


class RoutedPrefill:
    """Device buffers of one routed prefill and the calls that fill them."""

    def __init__(self, cfg):
        self.cfg = cfg
        B, Hq, Hkv, d, n = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_ctx
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        self.nblk = (n + cfg.chunk - 1) // cfg.chunk
        self.K = ((cfg.sink_chunks + cfg.local_chunks) * cfg.chunk
                  + cfg.top_chunks * cfg.top_groups * cfg.group)
        z = dict(device=DEV, dtype=dt)
        self.t = dict(q=torch.zeros(B, Hq, n, d, **z), k_pre=torch.zeros(B, Hkv, n, d, **z),
                      k_cache=torch.zeros(B, Hkv, n, d, **z), v_cache=torch.zeros(B, Hkv, n, d, **z),
                      chunk_sum=torch.zeros(B, Hkv, n // cfg.chunk, d, **z),
                      group_sum=torch.zeros(B, Hkv, n // cfg.group, d, **z))
        self.t["blk_idx"] = torch.full((B, Hkv, self.nblk, self.K), -1, dtype=torch.int32, device=DEV)
        self.t["blk_count"] = torch.full((B, Hkv, self.nblk), -1, dtype=torch.int32, device=DEV)
        self.t["out"] = torch.full((B, Hq, n, d), float("nan"), dtype=torch.float32, device=DEV)
        self.params = sa.make_params(
            batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, n_ctx=n, dtype=cfg.dtype,
            head_kind=[workloads.HEAD_ROUTED] * Hq, rope_base=cfg.rope_base, chunk=cfg.chunk,
            group=cfg.group, top_chunks=cfg.top_chunks, top_groups=cfg.top_groups,
            sink_chunks=cfg.sink_chunks, local_chunks=cfg.local_chunks, levels=1, factor=4,
            q_block=128, block_top_k=self.K)
        self.ws = sa.Workspace(DEV)
        self.ws_pf = sa.Workspace(DEV)

    def bufs(self):
        t = self.t
        return sa.make_buffers(q=t["q"], k_pre=t["k_pre"], k_cache=t["k_cache"],
                               v_cache=t["v_cache"], chunk_sum=t["chunk_sum"],
                               group_sum=t["group_sum"], blk_idx=t["blk_idx"],
                               blk_count=t["blk_count"], out=t["out"])

    def summaries(self):
        sa.index_build(self.params, self.bufs(), sa.IDX_CHUNK_SUMMARY, 0, self.cfg.n_ctx)

    def route(self):
        sa.select(self.params, self.bufs(), sa.SEL_ROUTE2_PREFILL, self.ws)

    def prefill(self):
        sa.prefill_chunked(self.params, self.bufs(), self.ws_pf)

    def lists(self):
        return self.t["blk_idx"].cpu().numpy(), self.t["blk_count"].cpu().numpy()


def _oracle_list(cfg, q, cs, gs, b, g, blk):
    G, C, n = cfg.gqa, cfg.chunk, cfg.n_ctx
    rows = np.arange(blk * C, min(n, (blk + 1) * C))
    qr = q[b, g * G:(g + 1) * G][:, rows].reshape(-1, q.shape[-1])
    return oracle.route_prefill_block(qr, cs[b, g], gs[b, g], blk, n, C, cfg.group,
                                      cfg.top_chunks, cfg.top_groups, cfg.sink_chunks,
                                      cfg.local_chunks)


SMALL = workloads.HGA_PREFILL_64K.with_(batch=2, n_q_heads=8, n_kv_heads=2, n_ctx=128 * 40,
                                        top_chunks=5, top_groups=2, sink_chunks=2,
                                        local_chunks=3)


@pytest.mark.parametrize("cfg", [
    SMALL,
    SMALL.with_(n_ctx=128 * 300, top_chunks=16),                 # many candidates
    SMALL.with_(n_ctx=128 * 6),                                  # no candidate block
    SMALL.with_(n_ctx=128 * 64, top_chunks=64, top_groups=4),    # every candidate kept
    SMALL.with_(head_dim=64, dtype="fp32", n_ctx=128 * 50),
], ids=lambda c: f"n{c.n_ctx}-d{c.head_dim}-{c.dtype}-t{c.top_chunks}")
@pytest.mark.parametrize("amp", [2, 16])
def test_route_prefill_lattice_exact(cfg, amp):
    """Lattice summaries and queries make every routing score exact on both
    sides (whole blocks: the mean over 4 x 128 rows is exact too); small
    amplitudes force ties, decided by the lower index."""
    log("route prefill lattice", cfg.n_ctx, cfg.head_dim, cfg.dtype, amp)
    lat = workloads.lattice_prefill_route_inputs(cfg, 50 + amp, amp=amp, q_amp=4)
    run = RoutedPrefill(cfg)
    for k in ("chunk_sum", "group_sum", "q"):
        run.t[k].copy_(to_dev(lat[k], cfg.dtype))
    run.route()
    torch.cuda.synchronize()
    idx, cnt = run.lists()
    q, cs, gs = np64(lat["q"]), np64(lat["chunk_sum"]), np64(lat["group_sum"])
    for b in range(cfg.batch):
        for g in range(cfg.n_kv_heads):
            for blk in range(run.nblk):
                ref, _ = _oracle_list(cfg, q, cs, gs, b, g, blk)
                assert cnt[b, g, blk] == len(ref), (b, g, blk, cnt[b, g, blk], len(ref))
                assert np.array_equal(idx[b, g, blk, :len(ref)], ref), (b, g, blk)


def _strict_gap_draw(cfg, seed0, tries=200):
    """Lattice draw whose last, partial block (its mean is over 4 x 45 rows,
    not exact in fp64) has every routing cut at least 1e-3 wide in every
    group; the whole blocks are exact on both sides anyway."""
    last = (cfg.n_ctx + 127) // 128 - 1
    for s in range(tries):
        lat = workloads.lattice_prefill_route_inputs(cfg, seed0 + s, amp=16, q_amp=4)
        q, cs, gs = np64(lat["q"]), np64(lat["chunk_sum"]), np64(lat["group_sum"])
        ok = True
        for b in range(cfg.batch):
            for g in range(cfg.n_kv_heads):
                _, info = _oracle_list(cfg, q, cs, gs, b, g, last)
                if info["chunk_gap"] < 1e-3 or (info["group_gaps"] and min(info["group_gaps"]) < 1e-3):
                    ok = False
        if ok:
            return s, lat, q, cs, gs
    pytest.fail("no strict-gap draw")


def test_route_prefill_ragged_strict_gap():
    cfg = SMALL.with_(n_ctx=128 * 37 + 45)
    s, lat, q, cs, gs = _strict_gap_draw(cfg, 900)
    log("strict gap draw", s)
    run = RoutedPrefill(cfg)
    for k in ("chunk_sum", "group_sum", "q"):
        run.t[k].copy_(to_dev(lat[k], cfg.dtype))
    run.route()
    torch.cuda.synchronize()
    idx, cnt = run.lists()
    for b in range(cfg.batch):
        for g in range(cfg.n_kv_heads):
            for blk in range(run.nblk):
                ref, _ = _oracle_list(cfg, q, cs, gs, b, g, blk)
                assert cnt[b, g, blk] == len(ref) and np.array_equal(idx[b, g, blk, :len(ref)], ref)


def _end_to_end(cfg, seed, blocks=None, rows_per_block=None, device="cpu"):
    """Summaries -> routing -> prefill on Gaussian inputs.  Lists: every
    checked block's list against the oracle's routing over the GPU's own
    summaries and queries, where every cut is at least GAP wide (at least 90 %
    of the checked blocks must be).  The kernel ranks by an fp32 sum of the
    block's <= 512 bf16 query rows, about 1e-6 relative error, and the scores
    here are about 0.05 in the oracle's units (mean query, 1/sqrt(d)), so a
    cut 1e-5 wide cannot be decided by rounding.  Outputs: the checked rows
    of every head against the oracle's attention over the GPU's list and the
    block's causal keys."""
    GAP = 1e-5
    inp = workloads.head_prefill_inputs(cfg.with_(n_ret_q_heads=cfg.n_q_heads), seed,
                                        device=device)
    run = RoutedPrefill(cfg)
    for k in ("q", "k_pre", "k_cache", "v_cache"):
        run.t[k].copy_(inp[k].to(run.t[k].dtype))
    del inp
    run.summaries()
    run.route()
    run.prefill()
    torch.cuda.synchronize()
    idx, cnt = run.lists()
    q = np64(run.t["q"])
    cs, gs = np64(run.t["chunk_sum"]), np64(run.t["group_sum"])
    G, C, n = cfg.gqa, cfg.chunk, cfg.n_ctx
    blocks = range(run.nblk) if blocks is None else blocks
    checked = exact = 0
    worst = 0.0
    for b in range(cfg.batch):
        for g in range(cfg.n_kv_heads):
            K = np64(run.t["k_cache"][b, g])
            V = np64(run.t["v_cache"][b, g])
            for blk in blocks:
                got = idx[b, g, blk, :cnt[b, g, blk]]
                assert cnt[b, g, blk] >= 0 and np.all(np.diff(got) > 0) and \
                    (len(got) == 0 or got[-1] < blk * C), (b, g, blk)
                ref, info = _oracle_list(cfg, q, cs, gs, b, g, blk)
                checked += 1
                if info["chunk_gap"] >= GAP and (not info["group_gaps"] or min(info["group_gaps"]) >= GAP):
                    assert np.array_equal(got, ref), (b, g, blk)
                    exact += 1
                rows = np.arange(blk * C, min(n, (blk + 1) * C))
                if rows_per_block is not None and len(rows) > rows_per_block:
                    rng = np.random.default_rng(blk)
                    rows = np.unique(np.r_[rows[0], rows[-1],
                                           rng.choice(rows, rows_per_block - 2, replace=False)])
                for h in range(g * G, (g + 1) * G):
                    ref_o = oracle.route_prefill_rows(q[b, h], K, V, got, blk, C, rows)
                    got_o = np64(run.t["out"][b, h][torch.as_tensor(rows, device=DEV)])
                    e = max_err(got_o, ref_o)
                    assert e <= TOL, (b, h, blk, e)
                    worst = max(worst, e)
    log("routed prefill", cfg.n_ctx, "blocks checked", checked, "exact", exact, "max err", worst)
    assert exact * 10 >= checked * 9


def test_routed_prefill_end_to_end_small():
    _end_to_end(SMALL.with_(batch=1, n_ctx=128 * 24 + 37), 3)


def test_routed_prefill_64k_full_size_sampled():
    """The 64K routed prefill at full size (32/8 heads, one sequence), inputs
    drawn on the GPU: 12 blocks of every KV group (the first, the last and
    seeded ones), 16 rows of each block for every query head."""
    cfg = workloads.HGA_PREFILL_64K
    nblk = cfg.n_ctx // cfg.chunk
    rng = np.random.default_rng(7)
    blocks = sorted(set([0, 5, 12, nblk - 1] + rng.choice(nblk, 8, replace=False).tolist()))
    _end_to_end(cfg, 5, blocks=blocks, rows_per_block=16, device=DEV)
