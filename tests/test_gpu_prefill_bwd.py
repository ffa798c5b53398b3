"""GPU parity of the pyramid prefill's backward pass (gradients of Q, K and
V through the gather, the attention and the scatter, the selection held
fixed) against the fp64 oracle, through the C ABI.

Tolerance.  The kernels feed P, dS and dO to the matrix cores rounded once
to bf16 (relative error <= 2^-9 each) and store each block's contribution to
a key as a bf16 partial row before the fp32 sum over blocks.  For every
gradient element the oracle's magnitude M - the same sums with every term
replaced by its absolute value, dP's terms included since dS = P (dP -
delta) carries dP's rounding - bounds the error by about 3 x 2^-9 M; the
tests allow 2^-6 M + 1e-6."""
import numpy as np
import pytest
import torch

import oracle
import selection_sparse_attention_amd as sa
import workloads
from oracle import lighthouse as LH
from gpu_harness import DEV, PrefillRun, log, np64

pytestmark = pytest.mark.gpu

SLACK = 2.0 ** -6
SMALL = workloads.PYRAMID_128K.with_(n_heads=2, n_ctx=2048 + 64, block_top_k=300)


class BwdRun(PrefillRun):
    """A pyramid prefill with the buffers of its backward pass."""

    def __init__(self, cfg, inp, dout):
        super().__init__(cfg, inp)
        B, H, N, d = cfg.batch, cfg.n_heads, cfg.n_ctx, cfg.head_dim
        self.t["lse"] = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=DEV)
        self.t["dout"] = dout.to(DEV, torch.float32)
        for k in ("dq", "dk", "dv"):
            self.t[k] = torch.full((B, H, N, d), float("nan"), dtype=torch.float32, device=DEV)
        self.ws_bw = sa.Workspace(DEV)

    def bufs(self):
        b = super().bufs()
        t = self.t
        for name, key in (("lse", "lse"), ("grad_out", "dout"), ("grad_q", "dq"),
                          ("grad_k", "dk"), ("grad_v", "dv")):
            setattr(b, name, t[key].data_ptr())
        return b

    def backward(self):
        sa.prefill_backward(self.params, self.bufs(), self.ws_bw)

    def forward_backward(self):
        self.pyramid(); self.select(); self.prefill(); self.backward()

    def sels(self, b, h):
        idx = self.t["blk_idx"][b, h].cpu().numpy()
        cnt = self.t["blk_count"][b, h].cpu().numpy()
        return {blk: idx[blk, :cnt[blk]].astype(np.int64) for blk in range(self.nblk)}


def _reference(cfg, run, b, h, blocks, flat_range=None):
    """Oracle gradients and magnitudes of head (b, h) from ``blocks``:
    dQ rows of those blocks, and the level-0 dK, dV with every contribution
    of those blocks (the full gradients when ``blocks`` is every block)."""
    N, L, p, qb = cfg.n_ctx, cfg.levels, cfg.factor, cfg.q_block
    Q, K, V = (np64(run.t[k][b, h]) for k in ("q", "k", "v"))
    dO = np64(run.t["dout"][b, h])
    kc = oracle.pyramid_levels(K, L, p, cfg.dtype)
    vc = oracle.pyramid_levels(V, L, p, cfg.dtype)
    sels = run.sels(b, h)
    E = oracle.n_entries(N, L, p)
    d = cfg.head_dim
    scale = 1.0 / np.sqrt(d)
    gQ, mQ = {}, {}
    gK, gV, mK, mV = (np.zeros((E, d)) for _ in range(4))
    for blk in blocks:
        sel = sels[blk]
        dq, dks, dvs, dko, dvo, P, dA = oracle.block_grads(Q, K, V, kc, vc, sel, blk, qb, L, p, dO)
        lo, hi = qb * blk, min(N, qb * blk + qb)
        Kt = np.concatenate([LH.entry_rows(sel, K, kc, N, L, p), K[lo:hi]])
        Vt = np.concatenate([LH.entry_rows(sel, V, vc, N, L, p), V[lo:hi]])
        A = np.abs(dO[lo:hi]) @ np.abs(Vt).T                 # sum_d |dO_d v_d|
        W = np.abs(dA) + P * A                               # |dS| and dP's rounding
        gQ[blk], mQ[blk] = dq, scale * (W @ np.abs(Kt))
        mk = scale * (W.T @ np.abs(Q[lo:hi]))
        mv = P.T @ np.abs(dO[lo:hi])
        n = len(sel)
        for g_, m_, vals, mags in ((gK, mK, np.concatenate([dks, dko]), mk),
                                   (gV, mV, np.concatenate([dvs, dvo]), mv)):
            np.add.at(g_, sel, vals[:n])
            np.add.at(m_, sel, mags[:n])
            g_[lo:hi] += vals[n:]
            m_[lo:hi] += mags[n:]
    return (gQ, mQ, oracle.pyramid_backward(gK, N, L, p), oracle.pyramid_backward(mK, N, L, p),
            oracle.pyramid_backward(gV, N, L, p), oracle.pyramid_backward(mV, N, L, p))


def _check(got, ref, mag, what):
    err = np.abs(got - ref)
    bound = SLACK * mag + 1e-6
    worst = float(np.max(err / bound)) if err.size else 0.0
    assert np.all(err <= bound), (what, float(err.max()), worst)
    return worst


def _check_head(cfg, run, b, h, blocks=None, rows=None):
    """Every block's dQ and all of dK, dV (or dQ of ``blocks`` and the
    level-0 rows ``rows`` of dK, dV, from contributions of ``blocks``)."""
    blocks = range(run.nblk) if blocks is None else blocks
    gQ, mQ, gK, mK, gV, mV = _reference(cfg, run, b, h, blocks)
    dq, dk, dv = (np64(run.t[k][b, h]) for k in ("dq", "dk", "dv"))
    qb = cfg.q_block
    worst = 0.0
    for blk in blocks:
        lo = qb * blk
        worst = max(worst, _check(dq[lo:lo + len(gQ[blk])], gQ[blk], mQ[blk], ("dq", blk)))
    sl = slice(None) if rows is None else rows
    worst = max(worst, _check(dk[sl], gK[sl], mK[sl], "dk"), _check(dv[sl], gV[sl], mV[sl], "dv"))
    return worst


@pytest.mark.parametrize("cfg", [
    SMALL,                                                        # ragged last block
    SMALL.with_(levels=2, factor=2, n_ctx=1024 + 256, block_top_k=100),
    SMALL.with_(levels=1, n_ctx=1000, block_top_k=128),           # token lists only
    SMALL.with_(levels=4, factor=2, n_ctx=1024, block_top_k=700),  # every visible entry early on
    SMALL.with_(batch=2, n_heads=1, n_ctx=4096, block_top_k=512),
], ids=lambda c: f"N{c.n_ctx}-L{c.levels}-p{c.factor}-K{c.block_top_k}-B{c.batch}")
def test_prefill_backward_matches_oracle(cfg):
    log("prefill backward", cfg.n_ctx, cfg.levels, cfg.factor, cfg.block_top_k, cfg.batch)
    inp = workloads.prefill_inputs(cfg, 11)
    run = BwdRun(cfg, inp, workloads.prefill_grad_inputs(cfg, 12))
    run.forward_backward()
    torch.cuda.synchronize()
    worst = 0.0
    for b in range(cfg.batch):
        for h in range(cfg.n_heads):
            worst = max(worst, _check_head(cfg, run, b, h))
    log("prefill backward worst error / bound", worst)


def test_prefill_backward_largest_list_and_determinism():
    """block_top_k = 8192 (the late blocks' lists are full), and a second
    backward call gives bit-identical gradients."""
    cfg = SMALL.with_(n_heads=1, n_ctx=8192 + 64, block_top_k=8192)
    inp = workloads.prefill_inputs(cfg, 13)
    run = BwdRun(cfg, inp, workloads.prefill_grad_inputs(cfg, 14))
    run.forward_backward()
    torch.cuda.synchronize()
    first = {k: run.t[k].clone() for k in ("dq", "dk", "dv")}
    run.backward()
    torch.cuda.synchronize()
    for k, v in first.items():
        assert torch.equal(v, run.t[k]), k
    worst = _check_head(cfg, run, 0, 0)
    log("largest list worst error / bound", worst)


def test_prefill_backward_zero_sum_invariants():
    """Each query's score gradients sum to zero and its weights to one: per
    head the key gradients sum to zero and the value gradients to sum(dO).
    Rounding leaves a residue near 2^-8 of the column's 2-norm (independent
    errors add like a random walk); a wrong or missing term leaves one of
    the order of the norm itself.  Bound: 2^-5 of the norm."""
    cfg = SMALL.with_(n_ctx=4096, n_heads=3)
    inp = workloads.prefill_inputs(cfg, 15)
    run = BwdRun(cfg, inp, workloads.prefill_grad_inputs(cfg, 16))
    run.forward_backward()
    torch.cuda.synchronize()
    dk, dv, dO = (np64(run.t[k]) for k in ("dk", "dv", "dout"))
    for h in range(cfg.n_heads):
        rk = np.abs(dk[0, h].sum(axis=0)) / np.linalg.norm(dk[0, h], axis=0)
        rv = np.abs(dv[0, h].sum(axis=0) - dO[0, h].sum(axis=0)) / np.linalg.norm(dv[0, h], axis=0)
        log("head", h, "zero-sum residue / norm: dk", rk.max(), "dv", rv.max())
        assert rk.max() <= 2.0 ** -5 and rv.max() <= 2.0 ** -5, h


def test_prefill_backward_broken_lists_give_nan_for_that_head_only():
    """Head 1's lists lose one entry in the middle of its run of choosing
    blocks (a gap the pyramid selection never makes): all of head 1's
    gradients are NaN, head 0's are unaffected."""
    cfg = SMALL.with_(n_ctx=2048)
    inp = workloads.prefill_inputs(cfg, 17)
    run = BwdRun(cfg, inp, workloads.prefill_grad_inputs(cfg, 18))
    run.pyramid(); run.select(); run.prefill()
    torch.cuda.synchronize()
    idx = run.t["blk_idx"][0, 1].cpu().numpy()
    cnt = run.t["blk_count"][0, 1].cpu().numpy()
    blk = run.nblk // 2
    assert cnt[blk] > 0 and cnt[blk - 1] > 0 and cnt[blk + 1] > 0
    both = np.intersect1d(np.intersect1d(idx[blk - 1, :cnt[blk - 1]], idx[blk, :cnt[blk]]),
                          idx[blk + 1, :cnt[blk + 1]])
    assert len(both) > 0
    keep = idx[blk, :cnt[blk]][idx[blk, :cnt[blk]] != both[0]]
    run.t["blk_idx"][0, 1, blk, :len(keep)] = torch.tensor(keep, dtype=torch.int32)
    run.t["blk_count"][0, 1, blk] = len(keep)
    run.backward()
    torch.cuda.synchronize()
    for k in ("dq", "dk", "dv"):
        assert torch.isnan(run.t[k][0, 1]).all(), k
        assert torch.isfinite(run.t[k][0, 0]).all(), k
    # head 0 against the oracle over its own (intact) lists
    _check_head(cfg, run, 0, 0, blocks=[0, 1, run.nblk - 1], rows=slice(0, 0))


def test_prefill_backward_full_size_sampled():
    """The 128K pyramid (16 heads, L = 3, p = 4, K = 4096) at full size,
    inputs drawn on the GPU: dQ of sampled blocks of every fourth head, and
    dK, dV of every row of the last three blocks - the positions whose keys
    and coarse ancestors only those blocks can choose, so their gradients
    are complete from three blocks of the oracle."""
    cfg = workloads.PYRAMID_128K
    inp = workloads.prefill_inputs(cfg, 7, device=DEV)
    run = BwdRun(cfg, inp, workloads.prefill_grad_inputs(cfg, 8, device=DEV))
    del inp
    run.forward_backward()
    torch.cuda.synchronize()
    nb = run.nblk
    rows = slice(cfg.q_block * (nb - 3), cfg.n_ctx)
    rng = np.random.default_rng(3)
    worst = 0.0
    for h in range(0, cfg.n_heads, 4):
        blocks = sorted(set([nb - 3, nb - 2, nb - 1] + rng.choice(nb - 3, 2, replace=False).tolist()))
        log("full-size backward head", h, "blocks", blocks)
        tail = [bb for bb in blocks if bb >= nb - 3]
        gQ, mQ, gK, mK, gV, mV = _reference(cfg, run, 0, h, blocks)
        dq, dk, dv = (np64(run.t[k][0, h]) for k in ("dq", "dk", "dv"))
        for blk in blocks:
            lo = cfg.q_block * blk
            worst = max(worst, _check(dq[lo:lo + cfg.q_block], gQ[blk], mQ[blk], ("dq", blk)))
        assert tail == [nb - 3, nb - 2, nb - 1]
        # the two early blocks add nothing to the tail rows' keys (they
        # cannot see them), so the reference for those rows is complete
        worst = max(worst, _check(dk[rows], gK[rows], mK[rows], "dk"),
                    _check(dv[rows], gV[rows], mV[rows], "dv"))
    for k in ("dq", "dk", "dv"):
        assert torch.isfinite(run.t[k]).all(), k
    log("full-size backward worst error / bound", worst)


def test_prefill_backward_lists_in_any_order():
    """The same selection with every list of head 1 shuffled: the backward
    sorts them itself.  dK and dV come out bit-identical (each key's partial
    row does not depend on its slot); dQ sums its keys in list order, so it
    only agrees to fp32 rounding."""
    cfg = SMALL.with_(n_ctx=2048)
    inp = workloads.prefill_inputs(cfg, 19)
    run = BwdRun(cfg, inp, workloads.prefill_grad_inputs(cfg, 20))
    run.forward_backward()
    torch.cuda.synchronize()
    ref = {k: run.t[k].clone() for k in ("dq", "dk", "dv")}
    gen = torch.Generator().manual_seed(21)
    cnt = run.t["blk_count"][0, 1].cpu()
    for blk in range(run.nblk):
        c = int(cnt[blk])
        if c > 1:
            perm = torch.randperm(c, generator=gen).to(DEV)
            run.t["blk_idx"][0, 1, blk, :c] = run.t["blk_idx"][0, 1, blk, :c][perm]
    run.backward()
    torch.cuda.synchronize()
    assert torch.equal(run.t["dk"], ref["dk"]) and torch.equal(run.t["dv"], ref["dv"])
    assert torch.equal(run.t["dq"][0, 0], ref["dq"][0, 0])
    scale = ref["dq"][0, 1].abs().max().item()
    assert (run.t["dq"][0, 1] - ref["dq"][0, 1]).abs().max().item() <= 1e-5 * scale
