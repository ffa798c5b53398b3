"""The allocation-free decode entry point (static device scratch array)
against the workspace entry point, through the C ABI: two calls in a row, the
second on a smaller problem, each equal to sparse_attn_decode on the same
inputs and selections (same kernels, same plan: bitwise equal), and within
the bf16 tolerance of the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import selection_sparse_attention_amd as sa
import workloads
from gpu_harness import DecodeRun, log, max_err, np64, np_inputs

pytestmark = pytest.mark.gpu


def _one(cfg, seed):
    log("noalloc decode", cfg.name, cfg.batch, cfg.n_ctx, seed)
    inp = workloads.decode_inputs(cfg, seed)
    run = DecodeRun(cfg, inp)
    run.index()
    run.select()
    run.decode()
    torch.cuda.synchronize()
    ref_out = run.t["out"].clone()
    run.t["out"].fill_(float("nan"))
    sa.decode_noalloc(run.params, run.bufs())
    torch.cuda.synchronize()
    got = run.t["out"].clone()
    assert torch.equal(got, ref_out)
    idx, cnt = run.sets()
    ni = np_inputs(inp)
    G = cfg.gqa
    sets = {}
    for b in range(cfg.batch):
        for g in range(cfg.n_kv_heads):
            if cfg.head_kind()[g * G] == workloads.HEAD_RETRIEVAL:
                sets[(b, g)] = idx[b, g, :cnt[b, g]]
            else:
                sets[(b, g)] = oracle.local_set(cfg.n_ctx, cfg.sinks, cfg.window)
    ref = oracle.decode_step(cfg, ni, sets=sets)
    out = np64(got)
    err = max(max_err(out[b, h], o) for (b, h), o in ref.items())
    log("noalloc max err", err)
    assert err <= 2e-3


def test_decode_noalloc_matches_workspace_entry_point_twice():
    big = workloads.LLAMA_32K.with_(batch=4, n_ctx=9000)
    small = workloads.LLAMA_32K.with_(batch=2, n_ctx=3000, n_q_heads=16, n_kv_heads=4,
                                      n_ret_q_heads=4)
    _one(big, 31)
    _one(small, 32)
