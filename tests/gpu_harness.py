"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
on generator inputs, and turn tensors into fp64 numpy for the oracle."""
import sys

import numpy as np
import torch

import selection_sparse_attention_amd as sa
import workloads

DEV = "cuda:0"


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def tdt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_dev(x, dtype):
    return x.to(device=DEV, dtype=tdt(dtype)).contiguous()


class DecodeRun:
    """Device buffers of one decode step and the calls that fill them."""

    def __init__(self, cfg, inp, n_cap=None, per_head=False):
        self.cfg = cfg
        self.per_head = per_head
        B, Hq, Hkv, d, n = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_ctx
        cap = inp.get("n_cap", n) if n_cap is None else n_cap
        self.n_cap = cap
        dt = tdt(cfg.dtype)
        self.t = {}
        for k in ("q_pre", "q", "k_pre", "k_cache", "v_cache"):
            if k in inp:
                x = inp[k]
                if x.dim() == 4 and x.shape[2] < cap:        # token stride is n_cap
                    pad = torch.zeros(*x.shape[:2], cap - x.shape[2], x.shape[3], dtype=x.dtype)
                    x = torch.cat([x, pad.to(x.device)], dim=2)
                self.t[k] = to_dev(x, cfg.dtype)
        if "proj" in inp:
            self.t["proj"] = inp["proj"].to(DEV, torch.float32).contiguous()
        self.t["k_idx"] = torch.zeros(B, Hkv, cap, cfg.r, dtype=dt, device=DEV)
        self.t["q_idx"] = torch.zeros(B, Hq, cfg.r, dtype=torch.float32, device=DEV)
        ns = Hq if per_head else Hkv               # selection rows per sequence
        self.t["sel_idx"] = torch.full((B, ns, cap), -1, dtype=torch.int32, device=DEV)
        self.t["sel_count"] = torch.full((B, ns), -1, dtype=torch.int32, device=DEV)
        self.t["out"] = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
        if cfg.routed:
            self.t["chunk_sum"] = torch.zeros(B, Hkv, cap // cfg.chunk, d, dtype=dt, device=DEV)
            self.t["group_sum"] = torch.zeros(B, Hkv, cap // cfg.group, d, dtype=dt, device=DEV)
        self.params = sa.params_from_config(cfg, n_cap=cap)
        self.params.per_head_sets = int(per_head)
        self.ws_sel = sa.Workspace(DEV)
        self.ws_dec = sa.Workspace(DEV)

    def bufs(self):
        t = self.t
        return sa.make_buffers(
            q_pre=t.get("q_pre"), k_pre=t.get("k_pre"), q=t.get("q"), k_cache=t.get("k_cache"),
            v_cache=t.get("v_cache"), proj_q=t.get("proj"), proj_k=t.get("proj"),
            q_idx=t["q_idx"], k_idx=t["k_idx"], chunk_sum=t.get("chunk_sum"),
            group_sum=t.get("group_sum"), sel_idx=t["sel_idx"], sel_count=t["sel_count"],
            out=t["out"])

    def index(self, t0=0, t1=None):
        sa.index_build(self.params, self.bufs(), sa.IDX_LOWRANK, t0,
                       self.cfg.n_ctx if t1 is None else t1)

    def summaries(self, t0=0, t1=None):
        sa.index_build(self.params, self.bufs(), sa.IDX_CHUNK_SUMMARY, t0,
                       self.cfg.n_ctx if t1 is None else t1)

    def select(self):
        if self.cfg.routed:
            mode = sa.SEL_ROUTE2
        elif self.cfg.s2o_tau > 0:
            mode = sa.SEL_TOPK_BY_SCORE
        else:
            mode = sa.SEL_TOPK if self.cfg.top_k > 0 else sa.SEL_TOPP
        sa.select(self.params, self.bufs(), mode, self.ws_sel)

    def decode(self):
        sa.decode(self.params, self.bufs(), self.ws_dec)

    def sets(self):
        idx = self.t["sel_idx"].cpu().numpy()
        cnt = self.t["sel_count"].cpu().numpy()
        return idx, cnt


def max_err(got, ref):
    """max |got - ref|, +inf when either side holds a NaN or inf."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    if not (np.all(np.isfinite(got)) and np.all(np.isfinite(ref))):
        return float("inf")
    return float(np.max(np.abs(got - ref))) if got.size else 0.0


def np_inputs(inp):
    return {k: (np64(v) if torch.is_tensor(v) and v.is_floating_point() else
                (v.numpy() if torch.is_tensor(v) else v)) for k, v in inp.items()}


class PrefillRun:
    """Device buffers of one pyramid-selection prefill and the calls that
    fill them."""

    def __init__(self, cfg, inp):
        self.cfg = cfg
        B, H, N, d = cfg.batch, cfg.n_heads, cfg.n_ctx, cfg.head_dim
        dt = tdt(cfg.dtype)
        self.t = {k: to_dev(inp[k], cfg.dtype) for k in ("q", "k", "v")}
        nc, nt, m = 0, 0, N
        for lvl in range(cfg.levels):
            nt += m
            if lvl:
                nc += m
            m //= cfg.factor
        self.nc, self.nt = nc, nt
        self.nblk = (N + cfg.q_block - 1) // cfg.q_block
        for k in ("pq", "pk", "pv"):
            self.t[k] = torch.zeros(B, H, max(nc, 1), d, dtype=dt, device=DEV)
        self.t["scores"] = torch.zeros(B, H, nt, dtype=torch.float32, device=DEV)
        self.t["blk_idx"] = torch.full((B, H, self.nblk, cfg.block_top_k), -1, dtype=torch.int32,
                                       device=DEV)
        self.t["blk_count"] = torch.full((B, H, self.nblk), -1, dtype=torch.int32, device=DEV)
        self.t["out"] = torch.full((B, H, N, d), float("nan"), dtype=torch.float32, device=DEV)
        self.t["out_pyr"] = torch.full((B, H, max(nc, 1), d), float("nan"), dtype=torch.float32,
                                       device=DEV)
        self.params = sa.params_from_config(cfg)
        self.ws_sel = sa.Workspace(DEV)
        self.ws_pf = sa.Workspace(DEV)

    def bufs(self):
        t = self.t
        return sa.make_buffers(q=t["q"], k_cache=t["k"], v_cache=t["v"], pyr_q=t["pq"],
                               pyr_k=t["pk"], pyr_v=t["pv"], pyr_scores=t["scores"],
                               blk_idx=t["blk_idx"], blk_count=t["blk_count"], out=t["out"],
                               out_pyr=t["out_pyr"])

    def pyramid(self):
        sa.index_build(self.params, self.bufs(), sa.IDX_PYRAMID, 0, self.cfg.n_ctx)

    def select(self):
        sa.select(self.params, self.bufs(), sa.SEL_PYRAMID_TOPK, self.ws_sel)

    def prefill(self):
        sa.prefill_chunked(self.params, self.bufs(), self.ws_pf)

    def coarse(self):
        sa.prefill_coarse(self.params, self.bufs())
