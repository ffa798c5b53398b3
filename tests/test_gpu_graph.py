"""A decode step (index append, selection, attention) and a prefill
(pyramid, block selection, attention) recorded into HIP graphs: every replay,
with the program's own eager work and synchronisations between replays, must
reproduce the eager result exactly (the kernels are deterministic, and the
library records only kernel launches)."""
import pytest
import torch

import selection_sparse_attention_amd as sa
import workloads
from gpu_harness import DEV, DecodeRun, PrefillRun

pytestmark = pytest.mark.gpu


def _snapshot(run, keys):
    return {k: run.t[k].clone() for k in keys}


def _same(a, b, groups=None):
    """Equal outputs; for the lists, only the selecting groups' counts and
    their first sel_count entries are defined (local groups are not listed)."""
    for k in a:
        if k in ("sel_idx", "sel_count"):
            cnt = a["sel_count"].cpu()
            for bb in range(cnt.shape[0]):
                for g in groups:
                    c = int(cnt[bb, g])
                    assert c == int(b["sel_count"][bb, g]), ("sel_count", bb, g)
                    assert torch.equal(a["sel_idx"][bb, g, :c], b["sel_idx"][bb, g, :c]), (k, bb, g)
        else:
            assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("cfg,per_head", [
    (workloads.LLAMA_32K.with_(batch=2, n_ctx=8192 + 77), False),
    (workloads.LLAMA_32K.with_(batch=2, n_ctx=4096, top_p=1.0, top_k=300), False),
    (workloads.HGA_64K.with_(batch=2, n_ctx=8192), False),
    (workloads.LLAMA_32K.with_(batch=2, n_ctx=4096, top_p=1.0, top_k=300, s2o_tau=0.01), False),
    (workloads.LLAMA_32K.with_(batch=2, n_ctx=8192 + 77), True),
    (workloads.LLAMA_32K.with_(batch=2, n_ctx=8192 + 77), "fused"),
], ids=["topp", "topk", "routed", "early-stop", "per-head", "fused-append"])
def test_decode_step_graph_replays_match_eager(cfg, per_head):
    """With "fused", the step's index append is done by the selection
    (SEL_APPEND); every replay also rewrites the index key and queries."""
    fused = per_head == "fused"
    per_head = per_head is True
    inp = workloads.decode_inputs(cfg, 21, device=DEV)
    run = DecodeRun(cfg, inp, per_head=per_head)
    n = cfg.n_ctx
    if cfg.routed:
        run.summaries(0, n)
    else:
        run.index(0, n)

    def step():
        if cfg.routed:
            t0 = (n // cfg.chunk) * cfg.chunk - 1 if n % cfg.chunk == 0 else n - 1
            run.summaries(max(0, t0), n)
        elif fused:
            mode = sa.SEL_TOPK if cfg.top_k > 0 else sa.SEL_TOPP
            sa.select(run.params, run.bufs(), mode | sa.SEL_APPEND, run.ws_sel)
        else:
            run.index(n - 1, n)
        if not fused:
            run.select()
        run.decode()

    keys = ["sel_idx", "sel_count", "out"] + (["k_idx", "q_idx"] if fused else [])
    kinds = cfg.head_kind()
    if per_head:
        groups = [h for h in range(cfg.n_q_heads) if kinds[h] != workloads.HEAD_LOCAL]
    else:
        groups = [g for g in range(cfg.n_kv_heads) if kinds[g * cfg.gqa] != workloads.HEAD_LOCAL]
    step()
    torch.cuda.synchronize()
    eager = _snapshot(run, keys)
    step()                                  # warm-up right before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    G = cfg.gqa
    for rep in range(4):
        for k in keys:                      # eager work between replays
            if k == "k_idx":                # the rows a step writes: token n - 1's
                for gg in groups:
                    run.t[k][:, gg, n - 1].fill_(-7)
            elif k == "q_idx":              # and the selecting groups' query heads'
                for gg in groups:
                    run.t[k][:, gg * G:(gg + 1) * G].fill_(-7)
            else:
                run.t[k].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(_snapshot(run, keys), eager, groups)
    step()                                  # and eager calls still agree afterwards
    torch.cuda.synchronize()
    _same(_snapshot(run, keys), eager, groups)


def test_prefill_graph_replays_match_eager():
    cfg = workloads.PYRAMID_128K.with_(n_heads=2, n_ctx=4096, block_top_k=700)
    inp = workloads.prefill_inputs(cfg, 22)
    run = PrefillRun(cfg, inp)

    def step():
        run.pyramid(); run.select(); run.prefill()

    keys = ["scores", "blk_idx", "blk_count", "out"]

    def same_prefill(a, b):
        for k in ("scores", "blk_count", "out"):
            assert torch.equal(a[k], b[k]), k
        cnt = a["blk_count"].cpu()                  # entries past the count are not defined
        for h in range(cnt.shape[1]):
            for blk in range(cnt.shape[2]):
                c = int(cnt[0, h, blk])
                assert torch.equal(a["blk_idx"][0, h, blk, :c], b["blk_idx"][0, h, blk, :c]), (h, blk)

    step()
    torch.cuda.synchronize()
    eager = _snapshot(run, keys)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for k in keys:
            run.t[k].fill_(-3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same_prefill(_snapshot(run, keys), eager)
