"""GPU parity of the head-split prefill (local heads over sinks + sliding
window, retrieval heads dense causal) against the fp64 oracle, through the
C ABI."""
import numpy as np
import pytest
import torch

import oracle
import selection_sparse_attention_amd as sa
import workloads
from gpu_harness import DEV, log, max_err, np64, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-3          # bf16 inputs, fp32 accumulation

SMALL = workloads.LLAMA_32K.with_(batch=2, n_q_heads=8, n_kv_heads=2, n_ret_q_heads=4,
                                  n_ctx=1000, sinks=4, window=100, needles_per_head=0)


def _run(cfg, inp):
    B, Hq, n, d = cfg.batch, cfg.n_q_heads, cfg.n_ctx, cfg.head_dim
    t = {k: to_dev(inp[k], cfg.dtype) for k in ("q", "k_cache", "v_cache")}
    t["out"] = torch.full((B, Hq, n, d), float("nan"), dtype=torch.float32, device=DEV)
    p = sa.params_from_config(cfg, n_cap=inp["n_cap"])
    sa.prefill_heads(p, sa.make_buffers(q=t["q"], k_cache=t["k_cache"], v_cache=t["v_cache"],
                                        out=t["out"]))
    torch.cuda.synchronize()
    return t


def _check(cfg, inp, t, rows_of):
    """Compare the rows ``rows_of(b, h)`` of every head with the oracle."""
    kinds = cfg.head_kind()
    G = cfg.gqa
    worst = 0.0
    for b in range(cfg.batch):
        for h in range(cfg.n_q_heads):
            rows = rows_of(b, h)
            g = h // G
            K = np64(t["k_cache"][b, g, :cfg.n_ctx])
            V = np64(t["v_cache"][b, g, :cfg.n_ctx])
            ref = oracle.head_prefill_rows(np64(t["q"][b, h]), K, V, kinds[h], cfg.sinks,
                                           cfg.window, rows)
            got = np64(t["out"][b, h][torch.as_tensor(rows, device=DEV)])
            e = max_err(got, ref)
            assert e <= TOL, (b, h, e)
            worst = max(worst, e)
    log("head prefill", cfg.n_ctx, cfg.sinks, cfg.window, "max err", worst)
    return worst


@pytest.mark.parametrize("cfg", [
    SMALL,                                              # ragged last block (1000 = 7 x 128 + 104)
    SMALL.with_(sinks=4, window=300),
    SMALL.with_(sinks=300, window=0),                   # sinks only, past the first blocks
    SMALL.with_(sinks=0, window=1),                     # each query sees itself
    SMALL.with_(sinks=0, window=129),
    SMALL.with_(sinks=130, window=33),                  # sinks overlap windows of early blocks
    SMALL.with_(sinks=4, window=5000),                  # window >= n: dense causal
    SMALL.with_(n_ctx=1),
    SMALL.with_(n_ctx=129, sinks=1, window=1),
    SMALL.with_(n_q_heads=8, n_kv_heads=8, n_ret_q_heads=3, n_ctx=700),   # no GQA, mixed
    SMALL.with_(n_ret_q_heads=0, n_ctx=600),            # local heads only
    SMALL.with_(n_ret_q_heads=8, n_ctx=600),            # dense heads only
], ids=lambda c: f"n{c.n_ctx}-s{c.sinks}-w{c.window}-h{c.n_q_heads}r{c.n_ret_q_heads}")
def test_head_prefill_every_row(cfg):
    log("head prefill", cfg.n_ctx, cfg.sinks, cfg.window, cfg.n_q_heads, cfg.n_ret_q_heads)
    inp = workloads.head_prefill_inputs(cfg, 7, n_cap=cfg.n_ctx + 17)
    t = _run(cfg, inp)
    _check(cfg, inp, t, lambda b, h: np.arange(cfg.n_ctx))


def test_head_prefill_window_one_returns_values():
    # one visible key: the output is that key's value up to the rounding of
    # p / p (the weight is 2^(s - max) with the max taken once rounded)
    cfg = SMALL.with_(sinks=0, window=1, n_ret_q_heads=0, n_ctx=513)
    inp = workloads.head_prefill_inputs(cfg, 8)
    t = _run(cfg, inp)
    G = cfg.gqa
    for h in range(cfg.n_q_heads):
        v = t["v_cache"][:, h // G, :cfg.n_ctx].float()
        assert (t["out"][:, h] - v).abs().max().item() <= 1e-6 * max(1.0, v.abs().max().item())


def test_head_prefill_full_window_equals_dense_heads():
    # a local head whose window covers the whole prefill gives exactly what
    # a dense head computes
    cfg = SMALL.with_(n_ret_q_heads=4, sinks=0, window=1000)
    inp = workloads.head_prefill_inputs(cfg, 9)
    t_loc = _run(cfg, inp)
    t_den = _run(cfg.with_(n_ret_q_heads=8), inp)
    assert torch.equal(t_loc["out"], t_den["out"])


def test_head_prefill_32k_full_size_sampled():
    """The 32K layer at full size (8 dense heads, 24 local heads with 4
    sinks + 1024 window, one sequence), inputs drawn on the GPU; 24 query
    positions of every head against the oracle: the first and last rows,
    block and window boundaries and seeded random positions."""
    cfg = workloads.LLAMA_PREFILL_32K
    inp = workloads.head_prefill_inputs(cfg, 3, device=DEV)
    t = _run(cfg, inp)
    n = cfg.n_ctx
    rng = np.random.default_rng(5)
    fixed = [0, 1, 3, 4, 127, 128, 1023, 1024, 1027, 1028, 1151, n - 129, n - 128, n - 1]

    def rows_of(b, h):
        extra = rng.choice(n, 10, replace=False)
        return np.unique(np.r_[fixed, extra])

    _check(cfg, inp, t, rows_of)
    assert torch.isfinite(t["out"]).all()
