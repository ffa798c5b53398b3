"""Seeded synthetic workloads for selection-based sparse attention.

This module only *draws inputs*: Gaussian or lattice-valued queries, keys,
values, projector matrices and head labels, with needle keys planted the way
the workload descriptions ask.  It holds none of the method's arithmetic (no
index scoring, no selection, no attention, no summaries, no pyramid), so the
oracle and the HIP path can both consume its outputs without sharing code.

The only transformation applied here is the rotary position embedding that a
model would already have applied to the cached keys and to the decode query
(half-split pairs, theta_i = base^(-2i/d), the same convention both sides are
told to use).  It is input synthesis: it produces the post-RoPE cache that the
decode kernels read.

Everything is generated with ``torch`` from an explicit seed so the same code
runs on the CPU (tests, oracle) and on the GPU (benchmark): the values differ
between devices (different counter-based engines) but each is reproducible.
Tensors are returned as float32 holding values exactly representable in the
workload dtype (bf16 or fp32).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

# Head labels (per query head).  Kept as plain ints so that this module and
# the C header agree by value only.
HEAD_LOCAL = 0
HEAD_RETRIEVAL = 1
HEAD_ROUTED = 2


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    """A decode workload: one query token per sequence attending to n keys."""
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_ctx: int
    dtype: str                      # "bf16" | "fp32"
    rope_base: float
    r: int = 16
    # retrieval / low-rank index
    n_ret_q_heads: int = 0          # query heads [0, n_ret_q_heads) are retrieval
    top_p: float = 1.0
    top_k: int = 0
    min_tokens: int = 0
    needles_per_head: int = 0
    # local heads
    sinks: int = 0
    window: int = 0
    # hierarchical routing (all heads routed when routed=True)
    routed: bool = False
    chunk: int = 64
    group: int = 16
    top_chunks: int = 16
    top_groups: int = 2
    sink_chunks: int = 4
    local_chunks: int = 8
    # monotone-gain early stop over the top-k candidates (0: off)
    s2o_tau: float = 0.0

    @property
    def gqa(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def head_kind(self) -> list:
        if self.routed:
            return [HEAD_ROUTED] * self.n_q_heads
        return [HEAD_RETRIEVAL if h < self.n_ret_q_heads else HEAD_LOCAL
                for h in range(self.n_q_heads)]

    def with_(self, **kw) -> "DecodeConfig":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    """A pyramid-selection prefill workload (multi-head, no GQA)."""
    name: str
    batch: int
    n_heads: int
    head_dim: int
    n_ctx: int
    dtype: str = "bf16"
    levels: int = 3
    factor: int = 4
    q_block: int = 128
    block_top_k: int = 4096
    heavy_frac: float = 0.01
    heavy_scale: float = 4.0
    lattice: float = 0.125
    clamp: float = 4.0

    def with_(self, **kw) -> "PrefillConfig":
        return dataclasses.replace(self, **kw)


# --- the five workloads -----------------------------------------------------
TINY = DecodeConfig(
    name="tiny_fp32_2k", batch=1, n_q_heads=4, n_kv_heads=4, head_dim=64,
    n_ctx=2048, dtype="fp32", rope_base=1e4, n_ret_q_heads=2, top_p=0.9,
    min_tokens=0, needles_per_head=8, sinks=4, window=128)

LLAMA_32K = DecodeConfig(
    name="llama3_8b_decode_32k", batch=8, n_q_heads=32, n_kv_heads=8,
    head_dim=128, n_ctx=32768, dtype="bf16", rope_base=5e5, n_ret_q_heads=8,
    top_p=0.95, min_tokens=64, needles_per_head=64, sinks=4, window=1024)

LLAMA_128K = LLAMA_32K.with_(name="llama3_8b_decode_128k", batch=4,
                             n_ctx=131072)
LLAMA_128K_TOPK = LLAMA_128K.with_(name="llama3_8b_decode_128k_topk",
                                   top_p=1.0, top_k=2048)

# the 32K layer with the early stop: its retrieval heads visit their top 2048
# candidates by index score after sinks + window, stopping at a gain of 1 %
LLAMA_32K_S2O = LLAMA_32K.with_(name="llama3_8b_decode_32k_s2o", top_p=1.0, top_k=2048,
                                s2o_tau=0.01)

HGA_64K = DecodeConfig(
    name="hga_route_decode_64k", batch=16, n_q_heads=32, n_kv_heads=8,
    head_dim=128, n_ctx=65536, dtype="bf16", rope_base=5e5, routed=True,
    needles_per_head=64, chunk=64, group=16, top_chunks=16, top_groups=2,
    sink_chunks=4, local_chunks=8)

# head-split prefill of the 32K decode layer's heads (one sequence): the 8
# retrieval heads attend densely, the 24 local heads over 4 sinks + 1024
LLAMA_PREFILL_32K = LLAMA_32K.with_(name="llama3_8b_head_split_prefill_32k", batch=1,
                                    needles_per_head=0)

# routed chunked prefill of the 64K routed layer's heads (one sequence): a
# query block is one chunk of 128 tokens (4 groups of 32), the routing
# budget as in the routed decode workload
HGA_PREFILL_64K = HGA_64K.with_(name="hga_route_prefill_64k", batch=1, chunk=128, group=32,
                                needles_per_head=0)

PYRAMID_128K = PrefillConfig(
    name="pyramid_prefill_128k", batch=1, n_heads=16, head_dim=128,
    n_ctx=131072)


def _gen(seed, device, *tags) -> torch.Generator:
    """A torch generator whose seed mixes the workload seed with slice tags."""
    s = int(seed) & 0xFFFFFFFF
    for t in tags:
        s = (s * 0x9E3779B1 + (int(t) & 0xFFFFFFFF) + 0x7F4A7C15) & 0xFFFFFFFFFFFF
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def _quant(x: torch.Tensor, dtype: str) -> torch.Tensor:
    """Round to the workload dtype and hand back float32 holding those values."""
    if dtype == "bf16":
        return x.to(torch.float32).to(torch.bfloat16).to(torch.float32)
    return x.to(torch.float32)


def rope_tables(d: int, base: float, pos: torch.Tensor):
    """cos/sin of pos*theta_i for the half-split pairs, in float64."""
    i = torch.arange(d // 2, dtype=torch.float64, device=pos.device)
    theta = torch.pow(torch.tensor(float(base), dtype=torch.float64,
                                   device=pos.device), -2.0 * i / d)
    ang = pos.to(torch.float64)[..., None] * theta
    return torch.cos(ang), torch.sin(ang)


def apply_rope(x: torch.Tensor, pos: torch.Tensor, base: float) -> torch.Tensor:
    """Rotate the (i, i + d/2) pairs of x[..., d] by pos*theta_i (float64)."""
    d = x.shape[-1]
    c, s = rope_tables(d, base, pos)
    x = x.to(torch.float64)
    a, b = x[..., : d // 2], x[..., d // 2:]
    return torch.cat([a * c - b * s, a * s + b * c], dim=-1)


def low_freq_dims(d: int) -> torch.Tensor:
    """Dims of the low-frequency pairs i in [d/4, d/2) and their partners."""
    lo = torch.arange(d // 4, d // 2)
    return torch.cat([lo, lo + d // 2])


def decode_inputs(cfg: DecodeConfig, seed: int, device="cpu", alpha: float = 1.0,
                  n_cap: Optional[int] = None) -> dict:
    """Draw one decode step's inputs.

    q_pre, k_pre, v ~ N(0,1); q_pre is scaled by ``alpha`` (entropy knob).
    For every head that selects (retrieval or routed), ``needles_per_head``
    cached keys at distinct uniform positions in [0, n-1) have their
    low-frequency dims replaced by 3x the head's pre-RoPE query on those dims.
    The cache holds post-RoPE keys (position j), the query is post-RoPE at
    position t = n - 1.  One projector P ~ N(0,1)/sqrt(d) per KV group is used
    for both the query and the key side of the low-rank index.
    """
    B, Hq, Hkv, d, n = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_ctx
    cap = n if n_cap is None else n_cap
    G = cfg.gqa
    f32 = dict(dtype=torch.float32, device=device)
    gq = _gen(seed, device, 1)
    q_pre = torch.randn(B, Hq, d, generator=gq, **f32) * alpha
    q_pre = _quant(q_pre, cfg.dtype)
    k_pre = torch.zeros(B, Hkv, cap, d, **f32)
    v = torch.zeros(B, Hkv, cap, d, **f32)
    kinds = cfg.head_kind()
    lf = low_freq_dims(d).to(device)
    needles = {}
    for b in range(B):
        for g in range(Hkv):
            gk = _gen(seed, device, 2, b, g)
            kk = torch.randn(n, d, generator=gk, **f32)
            vv = torch.randn(n, d, generator=gk, **f32)
            for hh in range(G):
                h = g * G + hh
                if kinds[h] == HEAD_LOCAL or cfg.needles_per_head == 0:
                    continue
                gn = _gen(seed, device, 3, b, h)
                perm = torch.randperm(n - 1, generator=gn, device=device)
                pos = perm[: min(cfg.needles_per_head, n - 1)]
                kk[pos[:, None], lf[None, :]] = 3.0 * q_pre[b, h, lf][None, :]
                needles[(b, h)] = pos.cpu()
            k_pre[b, g, :n] = _quant(kk, cfg.dtype)
            v[b, g, :n] = _quant(vv, cfg.dtype)
    gp = _gen(seed, device, 4)
    proj = torch.randn(Hkv, cfg.r, d, generator=gp, **f32) / math.sqrt(d)
    t = n - 1
    pos_k = torch.arange(cap, device=device)
    k_cache = _quant(apply_rope(k_pre, pos_k, cfg.rope_base), cfg.dtype)
    k_cache[:, :, n:] = 0
    q = _quant(apply_rope(q_pre, torch.full((1,), t, device=device)[0], cfg.rope_base), cfg.dtype)
    return dict(q_pre=q_pre, q=q, k_pre=k_pre, k_cache=k_cache, v_cache=v,
                proj=proj.contiguous(), head_kind=torch.tensor(kinds, dtype=torch.int8),
                needles=needles, n_cap=cap)


def redraw_query_dims(cfg: DecodeConfig, q_pre: torch.Tensor, seed: int, heads, round_: int,
                      alpha: float = 1.0):
    """Re-draw the dims of ``q_pre`` outside the low-frequency pairs (pairs
    i < d/4 and their partners) for the query heads ``heads`` [(b, h), ...],
    from generators tagged with ``round_``; the low-frequency dims, which the
    needle keys copy, are left as they are.  Returns new (q_pre, q), q being
    the post-RoPE query at t = n - 1, both rounded to the workload dtype."""
    d = cfg.head_dim
    dev = q_pre.device
    lf = set(low_freq_dims(d).tolist())
    hf = torch.tensor([i for i in range(d) if i not in lf], device=dev)
    q_pre = q_pre.clone()
    for b, h in heads:
        g = _gen(seed, dev, 5, b, h, round_)
        x = torch.randn(len(hf), generator=g, dtype=torch.float32, device=dev) * alpha
        q_pre[b, h, hf] = _quant(x, cfg.dtype)
    t = cfg.n_ctx - 1
    q = _quant(apply_rope(q_pre, torch.full((1,), t, device=dev)[0], cfg.rope_base), cfg.dtype)
    return q_pre, q


def lattice_index_inputs(cfg: DecodeConfig, seed: int, k_amp: int = 8,
                         q_amp: int = 4, device="cpu", n_cap: Optional[int] = None) -> dict:
    """Exact-arithmetic index inputs for set-exact selector tests.

    k_idx in (1/8)Z with |k| <= k_amp/8 and q_idx in (1/4)Z with
    |q| <= q_amp/4, written straight into the index buffers (no projection),
    so that every index logit is exactly representable in fp32 and fp64 and
    distinct logits differ by at least 1/512.
    """
    B, Hq, Hkv, n = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.n_ctx
    cap = n if n_cap is None else n_cap
    g = _gen(seed, device, 11)
    k_idx = torch.zeros(B, Hkv, cap, cfg.r, dtype=torch.float32, device=device)
    k_idx[:, :, :n] = torch.randint(-k_amp, k_amp + 1, (B, Hkv, n, cfg.r), generator=g,
                                    device=device).to(torch.float32) / 8.0
    q_idx = torch.randint(-q_amp, q_amp + 1, (B, Hq, cfg.r), generator=g,
                          device=device).to(torch.float32) / 4.0
    return dict(k_idx=k_idx, q_idx=q_idx, n_cap=cap,
                head_kind=torch.tensor(cfg.head_kind(), dtype=torch.int8))


def clustered_index_inputs(cfg: DecodeConfig, seed: int, spread: bool = True,
                           device="cpu") -> dict:
    """Exact-arithmetic index inputs whose logits crowd together.

    With ``spread``: every query head of a group has index-query component 0
    equal to 1, the group's first head also has component 1 equal to 1/4 (the
    others 0), and every index key has component 0 equal to 4 and component 1
    uniform in {0, 1/8, ..., 63/8}; all other components are 0.  For a group
    of G heads every logit is then 1 + k_1 / (16 G): 64 distinct values in
    the range [1, 1.125), each shared by about n/64 tokens.  Without
    ``spread`` every index key is zero, so every logit is 0 (one n-way tie).
    Values are exact in bf16 and fp32.
    """
    B, Hq, Hkv, n = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.n_ctx
    G = cfg.gqa
    g = _gen(seed, device, 13)
    k_idx = torch.zeros(B, Hkv, n, cfg.r, dtype=torch.float32, device=device)
    q_idx = torch.zeros(B, Hq, cfg.r, dtype=torch.float32, device=device)
    if spread:
        k_idx[..., 0] = 4.0
        k_idx[..., 1] = torch.randint(0, 64, (B, Hkv, n), generator=g,
                                      device=device).to(torch.float32) / 8.0
        q_idx[..., 0] = 1.0
        q_idx[:, ::G, 1] = 0.25
    return dict(k_idx=k_idx, q_idx=q_idx, n_cap=n,
                head_kind=torch.tensor(cfg.head_kind(), dtype=torch.int8))


def lattice_summary_inputs(cfg: DecodeConfig, seed: int, amp: int = 16,
                           q_amp: int = 8, device="cpu") -> dict:
    """Exact-arithmetic routing inputs: chunk/group summaries in (1/8)Z and a
    post-RoPE query in (1/8)Z, written straight into the summary buffers."""
    B, Hq, Hkv, d, n = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_ctx
    g = _gen(seed, device, 12)
    nc, ng = n // cfg.chunk, n // cfg.group
    cs = torch.randint(-amp, amp + 1, (B, Hkv, nc, d), generator=g, device=device).float() / 8
    gs = torch.randint(-amp, amp + 1, (B, Hkv, ng, d), generator=g, device=device).float() / 8
    q = torch.randint(-q_amp, q_amp + 1, (B, Hq, d), generator=g, device=device).float() / 8
    return dict(chunk_sum=cs, group_sum=gs, q=q)


def prefill_inputs(cfg: PrefillConfig, seed: int, device="cpu") -> dict:
    """Q, K, V ~ N(0,1) on a (lattice)Z grid clamped to +-clamp; a seeded
    ``heavy_frac`` of token positions is scaled by ``heavy_scale`` in Q, K and
    V of every head."""
    B, H, N, d = cfg.batch, cfg.n_heads, cfg.n_ctx, cfg.head_dim
    out = {}
    gh = _gen(seed, device, 21)
    n_heavy = int(round(cfg.heavy_frac * N))
    heavy = torch.randperm(N, generator=gh, device=device)[:n_heavy]
    scale = torch.ones(N, device=device)
    scale[heavy] = cfg.heavy_scale
    for i, name in enumerate(("q", "k", "v")):
        t = torch.empty(B, H, N, d, dtype=torch.float32, device=device)
        for b in range(B):
            for h in range(H):
                gg = _gen(seed, device, 22, i, b, h)
                x = torch.randn(N, d, generator=gg, dtype=torch.float32, device=device)
                x = torch.clamp(torch.round(x / cfg.lattice) * cfg.lattice, -cfg.clamp, cfg.clamp)
                t[b, h] = x * scale[:, None]
        out[name] = t
    out["heavy"] = heavy.cpu()
    return out


def prefill_grad_inputs(cfg: PrefillConfig, seed: int, device="cpu") -> torch.Tensor:
    """An upstream gradient dL/d(out) for a pyramid prefill: [B,H,N,d] fp32
    drawn N(0,1)."""
    g = _gen(seed, device, 23)
    return torch.randn(cfg.batch, cfg.n_heads, cfg.n_ctx, cfg.head_dim, generator=g,
                       dtype=torch.float32, device=device)


def head_prefill_inputs(cfg: DecodeConfig, seed: int, device="cpu",
                        n_cap: Optional[int] = None) -> dict:
    """Inputs of a head-split prefill over n = cfg.n_ctx tokens: q_pre
    [B,Hq,n,d] and k_pre, v [B,Hkv,n_cap,d] ~ N(0,1) rounded to the workload
    dtype (keys and values past n are zero), and the post-RoPE q and k at
    positions 0 .. n - 1 (rounded again)."""
    B, Hq, Hkv, d, n = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_ctx
    cap = n if n_cap is None else n_cap
    f32 = dict(dtype=torch.float32, device=device)
    q_pre = torch.empty(B, Hq, n, d, **f32)
    k_pre = torch.zeros(B, Hkv, cap, d, **f32)
    v = torch.zeros(B, Hkv, cap, d, **f32)
    for b in range(B):
        for h in range(Hq):
            q_pre[b, h] = _quant(torch.randn(n, d, generator=_gen(seed, device, 31, b, h), **f32),
                                 cfg.dtype)
        for g in range(Hkv):
            gk = _gen(seed, device, 32, b, g)
            k_pre[b, g, :n] = _quant(torch.randn(n, d, generator=gk, **f32), cfg.dtype)
            v[b, g, :n] = _quant(torch.randn(n, d, generator=gk, **f32), cfg.dtype)
    pos = torch.arange(n, device=device)
    q = _quant(apply_rope(q_pre, pos, cfg.rope_base), cfg.dtype)
    k = _quant(apply_rope(k_pre[:, :, :n], pos, cfg.rope_base), cfg.dtype)
    k_cache = torch.zeros_like(k_pre)
    k_cache[:, :, :n] = k
    return dict(q=q, k_pre=k_pre, k_cache=k_cache, v_cache=v, n_cap=cap,
                head_kind=torch.tensor(cfg.head_kind(), dtype=torch.int8))


def lattice_prefill_route_inputs(cfg: DecodeConfig, seed: int, amp: int = 16, q_amp: int = 4,
                                 device="cpu") -> dict:
    """Exact-arithmetic inputs for routing during prefill: chunk/group
    summaries in (1/8)Z with |x| <= amp/8 and prefill queries q [B,Hq,n,d] in
    (1/8)Z with |x| <= q_amp/8, written straight into the buffers."""
    B, Hq, Hkv, d, n = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_ctx
    g = _gen(seed, device, 14)
    nc, ng = n // cfg.chunk, n // cfg.group
    cs = torch.randint(-amp, amp + 1, (B, Hkv, nc, d), generator=g, device=device).float() / 8
    gs = torch.randint(-amp, amp + 1, (B, Hkv, ng, d), generator=g, device=device).float() / 8
    q = torch.randint(-q_amp, q_amp + 1, (B, Hq, n, d), generator=g, device=device).float() / 8
    return dict(chunk_sum=cs, group_sum=gs, q=q)


def to_device_dtype(x: torch.Tensor, dtype: str, device) -> torch.Tensor:
    """Cast generator output (float32 holding dtype-exact values) for a kernel."""
    t = torch.bfloat16 if dtype == "bf16" else torch.float32
    return x.to(device=device, dtype=t).contiguous()
