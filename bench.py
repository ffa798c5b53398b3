#!/usr/bin/env python3
"""Throughput of the sparse-attention hot path on one MI355X.

A decode "step" is one pass of the whole decode path over one batch: append
the step's row to the low-rank index (and project the step's index queries),
select every retrieval group's tokens (top-p or top-k), and run exact attention
for all heads (retrieval groups over their selected tokens, local groups over
sinks + window).  The routed workload swaps the index/select stages for chunk
summaries (the step's completed chunk) and two-level routing; the prefill
workload is the pyramid build, per-block selection and chunked attention.

Inputs are seeded and synthetic (see workloads/), generated on the GPU, and
rotated over several independent instances so that consecutive steps do not
hit the 256 MB Infinity Cache.  Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-decode tokens/s (B x heads x ctx) + achieved HBM GB/s vs peak, 32K/128K"
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3_8b_decode_32k",
                    choices=["llama3_8b_decode_32k", "llama3_8b_decode_128k",
                             "llama3_8b_decode_128k_topk", "hga_route_decode_64k",
                             "llama3_8b_decode_32k_s2o",
                             "hga_route_decode_64k_tiered",
                             "pyramid_prefill_128k", "pyramid_prefill_backward_128k",
                             "llama3_8b_head_split_prefill_32k", "hga_route_prefill_64k"])
    ap.add_argument("--per-head", action="store_true",
                    help="decode workloads: one set per query head (per_head_sets)")
    ap.add_argument("--instances", type=int, default=4,
                    help="independent input sets rotated across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other workloads (128K decode, routed decode, prefill)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--graph", action="store_true",
                    help="replay HIP graphs of the step instead of launching every call "
                         "(measured slower here: graph replay adds time between kernels)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain elementwise copy of known size (for scaling HBM "
                         "byte counters) and exit")
    return ap.parse_args()


def source_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "selection_sparse_attention_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_record(kernel, workload, sha):
    """Counter-derived HBM bytes per launch for this kernel and workload, if a
    profile of the current source exists."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(f"{kernel}:{workload}")
    if not rec or rec.get("source_sha") != sha:
        return None
    return rec.get("bytes_per_launch")


# ----------------------------------------------------------------- decode
class DecodeInstance:
    def __init__(self, cfg, seed, sa, torch, workloads, alpha=1.0, like=None, per_head=False,
                 ws=None):
        """One step's device buffers.  ``like``: copy another instance's
        inputs (same values at new addresses, so the Infinity Cache holds
        nothing of this one when the other has just run).  ``per_head``:
        every query head selects its own set.  ``ws``: the (selection,
        decode) workspaces, shared by instances run one after another on one
        stream as a model's layers would share them (own ones if None)."""
        B, Hq, Hkv, d, n = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_ctx
        self.cfg = cfg
        self.per_head = per_head
        ns = Hq if per_head else Hkv
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        if like is None:
            inp = workloads.decode_inputs(cfg, seed, device="cuda", alpha=alpha)
            self.t = {k: inp[k].to(dt).contiguous()
                      for k in ("q_pre", "q", "k_pre", "k_cache", "v_cache")}
            del inp["k_pre"], inp["k_cache"], inp["v_cache"]
            self.t["proj"] = inp["proj"].float().contiguous()
        else:
            self.t = {k: like.t[k].clone() for k in ("q_pre", "q", "k_pre", "k_cache", "v_cache",
                                                    "proj")}
        self.t["k_idx"] = torch.zeros(B, Hkv, n, cfg.r, dtype=dt, device="cuda")
        self.t["q_idx"] = torch.zeros(B, Hq, cfg.r, dtype=torch.float32, device="cuda")
        self.t["sel_idx"] = torch.zeros(B, ns, n, dtype=torch.int32, device="cuda")
        self.t["sel_count"] = torch.zeros(B, ns, dtype=torch.int32, device="cuda")
        self.t["out"] = torch.zeros(B, Hq, d, dtype=torch.float32, device="cuda")
        if cfg.routed:
            self.t["chunk_sum"] = torch.zeros(B, Hkv, n // cfg.chunk, d, dtype=dt, device="cuda")
            self.t["group_sum"] = torch.zeros(B, Hkv, n // cfg.group, d, dtype=dt, device="cuda")
        t = self.t
        self.params = sa.params_from_config(cfg)
        self.params.per_head_sets = int(per_head)
        self.bufs = sa.make_buffers(
            q_pre=t["q_pre"], k_pre=t["k_pre"], q=t["q"], k_cache=t["k_cache"],
            v_cache=t["v_cache"], proj_q=t["proj"], proj_k=t["proj"], q_idx=t["q_idx"],
            k_idx=t["k_idx"], chunk_sum=t.get("chunk_sum"), group_sum=t.get("group_sum"),
            sel_idx=t["sel_idx"], sel_count=t["sel_count"], out=t["out"])
        self.ws_sel, self.ws_dec = ws if ws is not None else (sa.Workspace("cuda"),
                                                              sa.Workspace("cuda"))
        self.sa = sa
        # prefill-time index over the whole history (not part of a step)
        if cfg.routed:
            sa.index_build(self.params, self.bufs, sa.IDX_CHUNK_SUMMARY, 0, n)
        else:
            sa.index_build(self.params, self.bufs, sa.IDX_LOWRANK, 0, n)
        self.sel_mode = (sa.SEL_ROUTE2 if cfg.routed else
                         (sa.SEL_TOPK_BY_SCORE if cfg.s2o_tau > 0 else
                          (sa.SEL_TOPK if cfg.top_k > 0 else sa.SEL_TOPP)))

    def index_and_select(self):
        sa, cfg = self.sa, self.cfg
        n = cfg.n_ctx
        if cfg.routed:
            # the step completes at most one chunk: rebuild the last one
            t0 = (n // cfg.chunk) * cfg.chunk - 1 if n % cfg.chunk == 0 else n - 1
            sa.index_build(self.params, self.bufs, sa.IDX_CHUNK_SUMMARY, max(0, t0), n)
            sa.select(self.params, self.bufs, self.sel_mode, self.ws_sel)
        elif cfg.dtype == "bf16":
            # the new token's index key and the step's index queries are
            # projected by the selection itself (the fused append)
            sa.select(self.params, self.bufs, self.sel_mode | sa.SEL_APPEND, self.ws_sel)
        else:
            sa.index_build(self.params, self.bufs, sa.IDX_LOWRANK, n - 1, n)
            sa.select(self.params, self.bufs, self.sel_mode, self.ws_sel)

    def decode(self):
        self.sa.decode(self.params, self.bufs, self.ws_dec)

    def counts(self, torch):
        """Selected counts per (b, KV group) as the step's bytes count them:
        with per-head sets, the size of the union of the group's heads' sets
        (the rows the group's heads read between them), plus the per-head
        counts (the list entries)."""
        cnt = self.t["sel_count"].cpu()
        if not self.per_head:
            return cnt.tolist(), None
        cfg = self.cfg
        G, n = cfg.gqa, cfg.n_ctx
        union = []
        for b in range(cfg.batch):
            row = []
            for g in range(cfg.n_kv_heads):
                seen = torch.zeros(n, dtype=torch.bool, device="cuda")
                for h in range(g * G, (g + 1) * G):
                    c = int(cnt[b, h])
                    if c > 0:
                        seen[self.t["sel_idx"][b, h, :c].long()] = True
                row.append(int(seen.sum()))
            union.append(row)
        return union, cnt.tolist()

    def capture(self, torch):
        """Record the step's two halves into HIP graphs (after a warm-up)."""
        self.g_sel, self.g_dec = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g_sel):
            self.index_and_select()
        with torch.cuda.graph(self.g_dec):
            self.decode()


def decode_bytes(cfg, counts, kinds, head_counts=None):
    """Algorithmic bytes of one decode step and of its attention kernel.
    ``counts``: visible tokens per (b, KV group) (with per-head sets, the
    union over the group's heads); ``head_counts``: per-head list lengths
    when the sets are per head."""
    e = 2 if cfg.dtype == "bf16" else 4
    B, Hq, Hkv, d, n, G = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_ctx, cfg.gqa
    kv = 0
    lists = 0
    for b in range(B):
        for g in range(Hkv):
            kind = kinds[g * G]
            if kind == 0:
                c = min(n, cfg.sinks + cfg.window)
            else:
                c = int(counts[b][g])
                if head_counts is None:
                    lists += 4 * c
                else:
                    lists += 4 * sum(int(head_counts[b][h]) for h in range(g * G, (g + 1) * G))
            kv += c * 2 * d * e
    qo = B * Hq * d * (e + 4)
    attn = kv + lists + qo
    n_ret = sum(1 for g in range(Hkv) if kinds[g * G] == 1)
    n_rt = sum(1 for g in range(Hkv) if kinds[g * G] == 2)
    index = B * n_ret * n * cfg.r * e                     # index scan
    if n_rt:
        index += B * n_rt * ((n // cfg.chunk) + 16 * (cfg.chunk // cfg.group)) * d * e
    step = attn + index + lists                          # lists are written once, read once
    return attn, step


DECODE_CONFIGS = {
    "llama3_8b_decode_32k": "LLAMA_32K",
    "llama3_8b_decode_128k": "LLAMA_128K",
    "llama3_8b_decode_128k_topk": "LLAMA_128K_TOPK",
    "hga_route_decode_64k": "HGA_64K",
    "llama3_8b_decode_32k_s2o": "LLAMA_32K_S2O",
}


MIN_TOUCHED_BYTES = 1 << 30     # rotated instances touch at least this much per round


def run_decode(args, torch, sa, workloads, workload=None, steps=None, warmup=None,
               instances=None, cpu=True, alpha=1.0, per_head=False):
    workload = workload or args.workload
    steps = steps or args.steps
    warmup = args.warmup if warmup is None else warmup
    instances = instances or args.instances
    cfg = getattr(workloads, DECODE_CONFIGS[workload])
    kinds = cfg.head_kind()
    log(f"[bench] generating {instances} instance(s) of {cfg.name} (alpha {alpha}"
        f"{', per-head sets' if per_head else ''})")
    # the instances stand for the layers of a model run one after another on
    # one stream: their inputs are distinct (cold), their workspaces are one
    # pair, as a layer loop reuses its scratch
    ws = (sa.Workspace("cuda"), sa.Workspace("cuda"))
    insts = [DecodeInstance(cfg, 1000 + i, sa, torch, workloads, alpha=alpha, per_head=per_head,
                            ws=ws)
             for i in range(instances)]
    # one step of each, then copies until a round of the rotation touches
    # >= 1 GiB (so no step finds its rows in the 256 MB Infinity Cache)
    for x in insts:
        x.index_and_select()
    torch.cuda.synchronize()
    per_step = 0
    for x in insts:
        c, hc = x.counts(torch)
        per_step += decode_bytes(cfg, c, kinds, hc)[1]
    per_step /= len(insts)
    want = max(len(insts), -(-MIN_TOUCHED_BYTES // int(per_step)))
    base = len(insts)
    while len(insts) < want:
        insts.append(DecodeInstance(cfg, 0, sa, torch, workloads, like=insts[len(insts) % base],
                                    ws=ws,
                                    per_head=per_head))
    if len(insts) > base:
        log(f"[bench] {len(insts) - base} copies added: {len(insts)} instances, "
            f"{len(insts) * per_step / 2**30:.2f} GiB touched per rotation")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        x = insts[i % len(insts)]
        x.index_and_select()
        x.decode()
    torch.cuda.synchronize()
    use_graph = args.graph
    if use_graph:
        # one graph for index append + selection and one for the attention call
        # per instance: the step is replayed with two launches, so the host
        # never starves the GPU between calls
        for x in insts:
            x.capture(torch)
        torch.cuda.synchronize()
    log(f"[bench] warmup done ({warmup} steps){' - replaying HIP graphs' if use_graph else ''}")
    # whole steps, events only around the timed region
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        x = insts[i % len(insts)]
        if use_graph:
            x.g_sel.replay()
            x.g_dec.replay()
        else:
            x.index_and_select()
            x.decode()
    end.record(stream)
    torch.cuda.synchronize()
    # the attention call alone, back to back over the rotated instances (its
    # selections are the ones the steps above left)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for i in range(steps):
        x = insts[i % len(insts)]
        if use_graph:
            x.g_dec.replay()
        else:
            x.decode()
    k1.record(stream)
    torch.cuda.synchronize()
    t_step = start.elapsed_time(end) / steps * 1e-3
    t_kernel = k0.elapsed_time(k1) / steps * 1e-3
    log(f"[bench] {cfg.name}: timed {steps} steps: {t_step * 1e6:.1f} us/step, "
        f"attention call {t_kernel * 1e6:.1f} us")
    # the spread: one event pair per step and per attention call, in a pass
    # of its own after the timed ones (the events add a little per step)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        x = insts[i % len(insts)]
        ev[i][0].record(stream)
        if use_graph:
            x.g_sel.replay()
        else:
            x.index_and_select()
        ev[i][1].record(stream)
        if use_graph:
            x.g_dec.replay()
        else:
            x.decode()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    per_step = [e[0].elapsed_time(e[2]) * 1e3 for e in ev]
    per_call = [e[1].elapsed_time(e[2]) * 1e3 for e in ev]
    # warm: the attention call of one instance repeated (its rows stay in the
    # 256 MB Infinity Cache as far as they fit)
    x = insts[0]
    call = x.g_dec.replay if use_graph else x.decode
    for _ in range(3):
        call()
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for _ in range(steps):
        call()
    w1.record(stream)
    torch.cuda.synchronize()
    t_warm = w0.elapsed_time(w1) / steps * 1e-3
    attn_b, step_b = 0, 0
    sel_frac = []
    for x in insts:
        c, hc = x.counts(torch)
        a, s_ = decode_bytes(cfg, c, kinds, hc)
        attn_b += a
        step_b += s_
        for b in range(cfg.batch):
            if hc is None:
                sel_frac += [c[b][g] / cfg.n_ctx for g in range(cfg.n_kv_heads)
                             if kinds[g * cfg.gqa] != 0]
            else:
                sel_frac += [hc[b][h] / cfg.n_ctx for h in range(cfg.n_q_heads) if kinds[h] != 0]
    attn_b /= len(insts)
    step_b /= len(insts)
    tokens = cfg.batch * cfg.n_q_heads * cfg.n_ctx
    kernel = "sparse_attn_decode (decode_mfma_kernel + decode_item_combine_kernel)"
    if per_head:
        kernel = ("sparse_attn_decode, per-head sets (head_union_mark_kernel + "
                  "head_union_compact_kernel + decode_mfma_kernel + decode_item_combine_kernel)")
    sha = source_sha(["decode.hip", "decode_mfma.hip", "common.hpp", "args.hpp"])
    achieved = attn_b / t_kernel / 1e9
    res = {
        "metric": METRIC, "value": tokens / t_step, "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": t_step * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "n_q_heads": cfg.n_q_heads,
                   "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim,
                   "n_ctx": cfg.n_ctx, "top_p": cfg.top_p if not cfg.top_k else None,
                   "top_k": cfg.top_k or None, "min_tokens": cfg.min_tokens,
                   "sinks": cfg.sinks, "window": cfg.window, "routed": cfg.routed,
                   "instances_rotated": len(insts), "alpha": alpha,
                   "per_head_sets": per_head, "s2o_tau": cfg.s2o_tau or None,
                   "touched_gib_per_rotation": len(insts) * step_b / 2**30,
                   "launch": "hip_graph" if args.graph else "eager"},
        "step_hbm_gbps": step_b / t_step / 1e9,
        "step_roofline": {"bound": "hbm", "achieved": step_b / t_step / 1e9,
                          "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                          "frac": step_b / t_step / 1e9 / PEAK_HBM_GBPS,
                          "bytes_per_step": step_b,
                          "note": "whole decode step (index append + selection + attention): "
                                  "the figure the 128K >= 70% target applies to"},
        "step_bytes": step_b,
        "selected_frac_mean": (sum(sel_frac) / len(sel_frac)) if sel_frac else None,
        "spread_us": {"step": percentiles(per_step), "attention_call": percentiles(per_call),
                      "attention_call_warm_mean": t_warm * 1e6,
                      "note": "one event pair per step in a separate pass; rotated instances "
                              "(cold in the 256 MB Infinity Cache); warm = one instance's call "
                              "repeated"},
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     # the counters were taken on the workload's own inputs (alpha 1)
                     "traffic": traffic_record(kernel, cfg.name, sha) if alpha == 1.0 else None,
                     "bytes_per_launch": attn_b, "launch_us": t_kernel * 1e6,
                     "source_sha": sha},
    }
    if cfg.s2o_tau > 0:
        # the early stop reads a data-dependent share of each group's
        # candidates (the kernel does not report how many): no byte count
        for k in ("roofline", "step_roofline", "step_hbm_gbps", "step_bytes"):
            res.pop(k, None)
        res["note"] = ("retrieval groups: top-k candidates in index-score order, early stop at "
                       f"tau {cfg.s2o_tau}; bytes read depend on the stop and are not reported")
    if cpu and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode(cfg, insts[0], args.cpu_seconds, torch)
    del insts
    torch.cuda.empty_cache()
    return res


def run_tier(args, torch, sa, workloads, steps=20, warmup=3):
    """The routed 64K decode step with the K/V history in pinned host memory
    (cold tier) and only the hot rows (sinks, a ring of the last chunks) and
    warm slots of routing groups in device memory; the device copy of the
    whole cache is freed.  Two regimes: 'warm' - the routing repeats, every
    routed group is already in a slot after the first step; 'cold' - the
    slot tables are emptied before every step, so every routed group comes
    over the host link."""
    cfg = workloads.HGA_64K
    log(f"[bench] generating {cfg.name} (tiered: history in host memory)")
    inst = DecodeInstance(cfg, 1000, sa, torch, workloads)
    B, Hkv, d, n = cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.n_ctx
    C, grp, sc, lc = cfg.chunk, cfg.group, cfg.sink_chunks, cfg.local_chunks
    slots = 4 * cfg.top_chunks * cfg.top_groups
    sink_rows, ring = sc * C, (lc + 1) * C
    dev_rows = sink_rows + ring + slots * grp
    dt = inst.t["k_cache"].dtype
    cold = {k: inst.t[k].cpu().pin_memory() for k in ("k_cache", "v_cache")}
    dev = {k: torch.zeros(B, Hkv, dev_rows, d, dtype=dt, device="cuda") for k in ("k", "v")}
    kappa = (n - 1) // C
    win = torch.arange(max((kappa - lc) * C, sink_rows), n, device="cuda")
    for src, dst in ((inst.t["k_cache"], dev["k"]), (inst.t["v_cache"], dev["v"])):
        dst[:, :, :sink_rows] = src[:, :, :sink_rows]
        dst[:, :, sink_rows + win % ring] = src[:, :, win]
    # the device no longer holds the history
    del inst.t["k_cache"], inst.t["v_cache"]
    torch.cuda.empty_cache()
    slot_group = torch.full((B, Hkv, slots), -1, dtype=torch.int32, device="cuda")
    slot_stamp = torch.zeros(B, Hkv, slots, dtype=torch.int32, device="cuda")
    stats = torch.zeros(B, Hkv, 2, dtype=torch.int32, device="cuda")
    rows = torch.zeros(B, Hkv, dev_rows, dtype=torch.int32, device="cuda")
    pt = sa.params_from_config(cfg, n_cap=dev_rows)
    pt.n_ctx = dev_rows
    bt = sa.make_buffers(q=inst.t["q"], k_cache=dev["k"], v_cache=dev["v"], sel_idx=rows,
                         sel_count=inst.t["sel_count"], out=inst.t["out"])
    ws = sa.Workspace("cuda")
    stream = torch.cuda.current_stream()
    counter = [0]

    def step(cold_regime, ev=None):
        inst.index_and_select()
        if cold_regime:
            slot_group.fill_(-1)
            slot_stamp.zero_()
        counter[0] += 1
        tier = sa.make_tier(cold_k=cold["k_cache"], cold_v=cold["v_cache"], dev_k=dev["k"],
                            dev_v=dev["v"], slot_group=slot_group, slot_stamp=slot_stamp, rows=rows,
                            step=counter[0], stats=stats)
        if ev:
            ev[0].record(stream)
        sa.tier_fetch(inst.params, inst.bufs, tier)
        if ev:
            ev[1].record(stream)
        sa.decode(pt, bt, ws)

    res = {}
    for regime in ("warm", "cold"):
        for _ in range(warmup):
            step(regime == "cold")
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for i in range(steps):
            step(regime == "cold", ev[i])
        end.record(stream)
        torch.cuda.synchronize()
        t_step = start.elapsed_time(end) / steps * 1e-3
        t_fetch = sum(a.elapsed_time(b) for a, b in ev) / steps * 1e-3
        st = stats.cpu()
        hits, misses = int(st[..., 0].sum()), int(st[..., 1].sum())
        fetched = misses * grp * d * (2 if cfg.dtype == "bf16" else 4) * 2
        res[regime] = {"ms_per_step": t_step * 1e3, "fetch_us": t_fetch * 1e6,
                       "hits_last_step": hits, "misses_last_step": misses,
                       "fetched_mb_per_step": fetched / 1e6,
                       "fetch_gbps": fetched / t_fetch / 1e9 if fetched else 0.0}
        log(f"[bench] {cfg.name} tiered, {regime}: {t_step * 1e6:.1f} us/step, fetch "
            f"{t_fetch * 1e6:.1f} us, {hits} hits / {misses} misses, "
            f"{fetched / 1e6:.1f} MB from host")
    dev_mb = sum(x.numel() * x.element_size() for x in dev.values()) / 1e6
    cold_mb = sum(x.numel() * x.element_size() for x in cold.values()) / 1e6
    out = {"value": B * cfg.n_q_heads * n / (res["warm"]["ms_per_step"] * 1e-3),
           "unit": "tokens/s (B x heads x ctx per step, warm regime)",
           "ms_per_step": res["warm"]["ms_per_step"],
           "config": {"workload": cfg.name + "_tiered", "batch": B, "n_ctx": n,
                      "warm_slots": slots, "device_kv_mb": dev_mb, "host_kv_mb": cold_mb},
           "regimes": res,
           "note": "history in pinned host memory (cold tier), read by the fetch kernel over the "
                   "host link; hot rows and warm slots in device memory; cold = every routed "
                   "group fetched each step"}
    del inst, cold, dev
    torch.cuda.empty_cache()
    return out


def percentiles(xs):
    """p10 / p50 / p90 of a list of times."""
    ys = sorted(xs)
    at = lambda q: ys[min(len(ys) - 1, int(round(q * (len(ys) - 1))))]
    return {"p10": at(0.1), "p50": at(0.5), "p90": at(0.9)}


def blas_threads():
    """Threads numpy's BLAS uses (the oracle's only parallel part)."""
    try:
        from threadpoolctl import threadpool_info
        return int(max((p.get("num_threads", 1) for p in threadpool_info()), default=1))
    except Exception:
        return 1


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline_decode(cfg, inst, budget_s, torch):
    """The fp64 oracle on whole (sequence, KV group) slices of the same step
    until ``budget_s`` of CPU time is spent; scaled to tokens/s.  A second,
    shorter sample runs with the BLAS pool held to one thread."""
    blas = blas_threads()
    done_heads, spent = _oracle_decode_sample(cfg, inst, budget_s, torch)
    one = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            d1, s1 = _oracle_decode_sample(cfg, inst, budget_s / 3, torch)
        one = d1 * cfg.n_ctx / s1
    except ImportError:
        pass
    return {"value": done_heads * cfg.n_ctx / spent, "unit": "tokens/s",
            "cores": int(blas), "kind": "oracle",
            "sample": f"{done_heads // cfg.gqa} whole (sequence, KV group) slices of the "
                      f"{cfg.name} step ({done_heads} query heads x {cfg.n_ctx} tokens), "
                      f"index + selection + attention, fp64 numpy, {spent:.1f} s",
            "value_1_thread": one,
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model()}


def _oracle_decode_sample(cfg, inst, budget_s, torch):
    import numpy as np
    import oracle
    G = cfg.gqa
    groups = [(b, g) for b in range(cfg.batch) for g in range(cfg.n_kv_heads)]
    t = inst.t
    done_heads, spent, i = 0, 0.0, 0
    while spent < budget_s or done_heads == 0:
        b, g = groups[(i * 7) % len(groups)]
        i += 1
        sl = {"q_pre": t["q_pre"][b:b + 1], "q": t["q"][b:b + 1],
              "k_pre": t["k_pre"][b:b + 1, g:g + 1], "k_cache": t["k_cache"][b:b + 1, g:g + 1],
              "v_cache": t["v_cache"][b:b + 1, g:g + 1], "proj": t["proj"][g:g + 1]}
        ni = {k: v.detach().to("cpu", torch.float64).numpy() for k, v in sl.items()}
        ni["q_pre"] = ni["q_pre"][:, g * G:(g + 1) * G]
        ni["q"] = ni["q"][:, g * G:(g + 1) * G]
        sub = cfg.with_(batch=1, n_kv_heads=1, n_q_heads=G,
                        n_ret_q_heads=G if cfg.head_kind()[g * G] == 1 else 0)
        ni["head_kind"] = np.array(sub.head_kind(), np.int8)
        t0 = time.perf_counter()
        oracle.decode_step(sub, ni)
        spent += time.perf_counter() - t0
        done_heads += G
    return done_heads, spent


def compact(r):
    keep = ("value", "unit", "ms_per_step", "step_hbm_gbps", "step_roofline",
            "selected_frac_mean", "config", "roofline", "step_tflops", "spread_us",
            "all_dense_ms", "speedup_vs_all_dense", "note", "forward_ms", "backward_ms")
    return {k: r[k] for k in keep if k in r}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path is "
              "data parallel across sequences and KV groups, so N GPUs run N independent "
              "copies with no exchange - run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads
    import selection_sparse_attention_amd as sa
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    if args.workload == "pyramid_prefill_128k":
        res = run_prefill(args, torch, sa, workloads)
    elif args.workload == "hga_route_decode_64k_tiered":
        res = run_tier(args, torch, sa, workloads, steps=min(args.steps, 20), warmup=3)
    elif args.workload == "pyramid_prefill_backward_128k":
        res = run_prefill(args, torch, sa, workloads, backward=True)
    elif args.workload == "llama3_8b_head_split_prefill_32k":
        res = run_prefill_heads(args, torch, sa, workloads)
    elif args.workload == "hga_route_prefill_64k":
        res = run_prefill_routed(args, torch, sa, workloads)
    else:
        res = run_decode(args, torch, sa, workloads, per_head=args.per_head)
    if not args.no_extras and args.workload == "llama3_8b_decode_32k":
        other = {}
        for w in ("llama3_8b_decode_128k_topk", "llama3_8b_decode_128k", "hga_route_decode_64k"):
            other[w] = compact(run_decode(args, torch, sa, workloads, workload=w, steps=20,
                                          warmup=3, instances=4, cpu=False))
        # the 32K step with the early stop over the top-2048 candidates
        other["llama3_8b_decode_32k_s2o"] = compact(run_decode(
            args, torch, sa, workloads, workload="llama3_8b_decode_32k_s2o", steps=20, warmup=3,
            instances=4, cpu=False))
        # the 32K step with one set per query head (no GQA sharing of sets)
        other["llama3_8b_decode_32k_per_head"] = compact(run_decode(
            args, torch, sa, workloads, workload="llama3_8b_decode_32k", steps=20, warmup=3,
            instances=4, cpu=False, per_head=True))
        # the 128K top-p step at other attention entropies (query norms x alpha)
        for a in (0.5, 2.0):
            other[f"llama3_8b_decode_128k_alpha{a:g}"] = compact(run_decode(
                args, torch, sa, workloads, workload="llama3_8b_decode_128k", steps=20, warmup=3,
                instances=4, cpu=False, alpha=a))
        other["hga_route_decode_64k_tiered"] = run_tier(args, torch, sa, workloads)
        other["pyramid_prefill_128k"] = compact(run_prefill(args, torch, sa, workloads, steps=5,
                                                            warmup=1, cpu=False))
        other["pyramid_prefill_backward_128k"] = compact(run_prefill(
            args, torch, sa, workloads, steps=3, warmup=1, cpu=False, backward=True))
        other["llama3_8b_head_split_prefill_32k"] = compact(run_prefill_heads(
            args, torch, sa, workloads, steps=5, warmup=1, cpu=False))
        other["hga_route_prefill_64k"] = compact(run_prefill_routed(
            args, torch, sa, workloads, steps=5, warmup=1, cpu=False))
        res["other_workloads"] = other
    print(json.dumps(res), flush=True)


def calibrate_copy(torch):
    """A 1 GiB bf16 negation (reads 1 GiB, writes 1 GiB) run five times: the
    ratio of a byte counter to these sizes scales the counter to bytes."""
    n = 1 << 29
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    for _ in range(5):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"kernel": "neg", "bytes_read": 2 * n, "bytes_written": 2 * n,
                      "launches": 5}), flush=True)


def prefill_flops(cfg, counts):
    """Algorithmic FLOP of the prefill attention: 4 d per (query, visible
    key) pair - QK^T and PV - with the causal block counted as a triangle."""
    pairs = 0
    N, qb = cfg.n_ctx, cfg.q_block
    for per_head in counts:
        for blk, c in enumerate(per_head):
            nq = min(qb, N - blk * qb)
            pairs += nq * int(c) + nq * (nq + 1) // 2
    return 4 * cfg.head_dim * pairs


def run_prefill(args, torch, sa, workloads, steps=None, warmup=None, cpu=True, backward=False):
    """The pyramid prefill step (pyramid, selection, attention); with
    ``backward`` a training step: the forward keeps each row's log-sum-exp
    and the backward pass follows with a synthetic upstream gradient."""
    cfg = workloads.PYRAMID_128K
    steps = steps or max(3, min(args.steps, 10))
    warmup = 1 if warmup is None else warmup
    B, H, N, d = cfg.batch, cfg.n_heads, cfg.n_ctx, cfg.head_dim
    log(f"[bench] generating {cfg.name}")
    inp = workloads.prefill_inputs(cfg, 2000, device="cuda")
    t = {k: inp[k].to(torch.bfloat16).contiguous() for k in ("q", "k", "v")}
    del inp
    nc, nt, m = 0, 0, N
    for lvl in range(cfg.levels):
        nt += m
        nc += m if lvl else 0
        m //= cfg.factor
    nblk = (N + cfg.q_block - 1) // cfg.q_block
    for k in ("pq", "pk", "pv"):
        t[k] = torch.zeros(B, H, max(nc, 1), d, dtype=torch.bfloat16, device="cuda")
    t["scores"] = torch.zeros(B, H, nt, dtype=torch.float32, device="cuda")
    t["blk_idx"] = torch.zeros(B, H, nblk, cfg.block_top_k, dtype=torch.int32, device="cuda")
    t["blk_count"] = torch.zeros(B, H, nblk, dtype=torch.int32, device="cuda")
    t["out"] = torch.zeros(B, H, N, d, dtype=torch.float32, device="cuda")
    grads = {}
    if backward:
        grads = dict(lse=torch.zeros(B, H, N, dtype=torch.float32, device="cuda"),
                     grad_out=workloads.prefill_grad_inputs(cfg, 2001, device="cuda"),
                     **{k: torch.zeros(B, H, N, d, dtype=torch.float32, device="cuda")
                        for k in ("grad_q", "grad_k", "grad_v")})
    p = sa.params_from_config(cfg)
    bufs = sa.make_buffers(q=t["q"], k_cache=t["k"], v_cache=t["v"], pyr_q=t["pq"],
                           pyr_k=t["pk"], pyr_v=t["pv"], pyr_scores=t["scores"],
                           blk_idx=t["blk_idx"], blk_count=t["blk_count"], out=t["out"], **grads)
    ws_s, ws_p, ws_b = sa.Workspace("cuda"), sa.Workspace("cuda"), sa.Workspace("cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        sa.index_build(p, bufs, sa.IDX_PYRAMID, 0, N)
        sa.select(p, bufs, sa.SEL_PYRAMID_TOPK, ws_s)
        if ev:
            ev[0].record(stream)
        sa.prefill_chunked(p, bufs, ws_p)
        if ev:
            ev[1].record(stream)
        if backward:
            sa.prefill_backward(p, bufs, ws_b)
            if ev:
                ev[2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        step(ev[i])
    end.record(stream)
    torch.cuda.synchronize()
    t_step = start.elapsed_time(end) / steps * 1e-3
    t_kernel = sum(e[0].elapsed_time(e[1]) for e in ev) / steps * 1e-3
    t_bwd = sum(e[1].elapsed_time(e[2]) for e in ev) / steps * 1e-3 if backward else 0.0
    counts = t["blk_count"].reshape(B * H, nblk).cpu().tolist()
    flops = prefill_flops(cfg, counts)
    log(f"[bench] {cfg.name}: {t_step * 1e3:.3f} ms/step, prefill kernel {t_kernel * 1e3:.3f} ms, "
        f"{flops / t_kernel / 1e12:.1f} TFLOP/s" +
        (f", backward {t_bwd * 1e3:.3f} ms ({2 * flops / t_bwd / 1e12:.1f} TFLOP/s)" if backward else ""))
    if backward:
        res = prefill_backward_result(args, cfg, t, steps, warmup, t_step, t_kernel, t_bwd, flops,
                                      cpu, torch)
        del t, grads, ws_b
        torch.cuda.empty_cache()
        return res
    sha = source_sha(["prefill.hip", "common.hpp", "args.hpp"])
    achieved = flops / t_kernel / 1e12
    res = {
        "metric": "pyramid-selection prefill tokens/s + achieved bf16 MFMA TFLOP/s vs peak",
        "value": B * H * N / t_step, "unit": "tokens/s (B x heads x N per step)",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": t_step * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "n_heads": H, "head_dim": d, "n_ctx": N,
                   "levels": cfg.levels, "factor": cfg.factor, "q_block": cfg.q_block,
                   "block_top_k": cfg.block_top_k},
        "step_tflops": flops / t_step / 1e12,
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel<false>", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic_record("prefill_kernel<false>", cfg.name, sha),
                     "flops_per_launch": flops, "launch_us": t_kernel * 1e6, "source_sha": sha},
    }
    if cpu and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(cfg, t, args.cpu_seconds, torch)
    del t
    torch.cuda.empty_cache()
    return res


def prefill_backward_result(args, cfg, t, steps, warmup, t_step, t_kernel, t_bwd, flops, cpu, torch):
    """The bench line of the pyramid prefill training step.  The backward's
    algorithmic work is 8 d FLOP per (query, visible key) pair - dV = P^T dO,
    dP = dO V^T, dQ = dS K, dK = dS^T Q - twice the forward's 4 d (the
    recomputed scores are not counted)."""
    B, H, N, d = cfg.batch, cfg.n_heads, cfg.n_ctx, cfg.head_dim
    bflops = 2 * flops
    achieved = bflops / t_bwd / 1e12
    sha = source_sha(["prefill_bwd.hip", "common.hpp", "args.hpp"])
    label = "sparse_attn_prefill_backward (all kernels of the call)"
    res = {
        "metric": "pyramid-selection prefill training step (forward + backward) tokens/s + "
                  "backward bf16 MFMA TFLOP/s vs peak",
        "value": B * H * N / t_step, "unit": "tokens/s (B x heads x N per step)",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": t_step * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name + "_forward_backward", "batch": B, "n_heads": H,
                   "head_dim": d, "n_ctx": N, "levels": cfg.levels, "factor": cfg.factor,
                   "q_block": cfg.q_block, "block_top_k": cfg.block_top_k},
        "forward_ms": t_kernel * 1e3, "backward_ms": t_bwd * 1e3,
        "roofline": {"bound": "mfma", "kernel": label, "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic_record(label, cfg.name, sha),
                     "flops_per_launch": bflops, "launch_us": t_bwd * 1e6, "source_sha": sha},
    }
    if cpu and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill_backward(cfg, t, args.cpu_seconds, torch)
    return res


def head_split_pairs(n, local, sinks, window):
    """(query, key) pairs one head attends over in a head-split prefill of n
    tokens: every i sees [0, i] (dense) or [0, min(s, i + 1)) and
    [max(0, i - w + 1), i] (local, a union)."""
    import numpy as np
    if not local:
        return n * (n + 1) // 2
    i = np.arange(n, dtype=np.int64)
    a = np.minimum(sinks, i + 1)
    lo = np.maximum(0, i - window + 1)
    w = (i + 1 - lo) if window > 0 else np.zeros_like(i)
    over = np.maximum(0, a - lo) if window > 0 else np.zeros_like(i)
    return int((a + w - over).sum())


def run_prefill_heads(args, torch, sa, workloads, steps=None, warmup=None, cpu=True):
    """Head-split prefill of the 32K decode layer's heads (one sequence):
    the retrieval heads dense causal, the local heads over sinks + window.
    Also times the same call with every head dense (the full-attention
    prefill this method replaces) for the speed-up."""
    cfg = workloads.LLAMA_PREFILL_32K
    steps = steps or max(3, min(args.steps, 10))
    warmup = 1 if warmup is None else warmup
    B, Hq, N, d = cfg.batch, cfg.n_q_heads, cfg.n_ctx, cfg.head_dim
    log(f"[bench] generating {cfg.name}")
    inp = workloads.head_prefill_inputs(cfg, 2100, device="cuda")
    t = {k: inp[k].to(torch.bfloat16).contiguous() for k in ("q", "k_cache", "v_cache")}
    del inp
    t["out"] = torch.zeros(B, Hq, N, d, dtype=torch.float32, device="cuda")
    bufs = sa.make_buffers(q=t["q"], k_cache=t["k_cache"], v_cache=t["v_cache"], out=t["out"])
    p = sa.params_from_config(cfg)
    p_dense = sa.params_from_config(cfg.with_(n_ret_q_heads=Hq))
    stream = torch.cuda.current_stream()

    def timed(params, n):
        for _ in range(warmup):
            sa.prefill_heads(params, bufs)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for a, b in ev:
            a.record(stream)
            sa.prefill_heads(params, bufs)
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / n * 1e-3

    t_kernel = timed(p, steps)
    t_dense = timed(p_dense, max(2, steps // 2))
    timed(p, 1)                                   # leave the head-split result in out
    kinds = cfg.head_kind()
    pairs = B * sum(head_split_pairs(N, k == workloads.HEAD_LOCAL, cfg.sinks, cfg.window)
                    for k in kinds)
    flops = 4 * d * pairs
    achieved = flops / t_kernel / 1e12
    log(f"[bench] {cfg.name}: prefill kernel {t_kernel * 1e3:.3f} ms, {achieved:.1f} TFLOP/s; "
        f"all heads dense {t_dense * 1e3:.3f} ms ({t_dense / t_kernel:.2f}x)")
    sha = source_sha(["prefill.hip", "common.hpp", "args.hpp"])
    res = {
        "metric": "head-split prefill tokens/s + achieved bf16 MFMA TFLOP/s vs peak",
        "value": B * Hq * N / t_kernel, "unit": "tokens/s (B x heads x N per call)",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": t_kernel * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "n_q_heads": Hq, "n_kv_heads": cfg.n_kv_heads,
                   "head_dim": d, "n_ctx": N, "dense_heads": Hq - kinds.count(workloads.HEAD_LOCAL),
                   "sinks": cfg.sinks, "window": cfg.window},
        "all_dense_ms": t_dense * 1e3, "speedup_vs_all_dense": t_dense / t_kernel,
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel<true>", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic_record("prefill_kernel<true>", cfg.name, sha),
                     "flops_per_launch": flops, "launch_us": t_kernel * 1e6, "source_sha": sha},
    }
    if cpu and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill_heads(cfg, t, args.cpu_seconds, torch)
    del t
    torch.cuda.empty_cache()
    return res


def run_prefill_routed(args, torch, sa, workloads, steps=None, warmup=None, cpu=True):
    """Routed chunked prefill of the 64K routed layer's heads (one
    sequence): chunk/group summaries of the whole prefix, every query block's
    routing, then attention over each block's list plus its causal keys."""
    cfg = workloads.HGA_PREFILL_64K
    steps = steps or max(3, min(args.steps, 10))
    warmup = 1 if warmup is None else warmup
    B, Hq, Hkv, N, d = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.n_ctx, cfg.head_dim
    C, G = cfg.chunk, cfg.gqa
    nblk = (N + C - 1) // C
    K = (cfg.sink_chunks + cfg.local_chunks) * C + cfg.top_chunks * cfg.top_groups * cfg.group
    log(f"[bench] generating {cfg.name}")
    inp = workloads.head_prefill_inputs(cfg.with_(n_ret_q_heads=Hq), 2200, device="cuda")
    t = {k: inp[k].to(torch.bfloat16).contiguous() for k in ("q", "k_pre", "k_cache", "v_cache")}
    del inp
    t["chunk_sum"] = torch.zeros(B, Hkv, N // C, d, dtype=torch.bfloat16, device="cuda")
    t["group_sum"] = torch.zeros(B, Hkv, N // cfg.group, d, dtype=torch.bfloat16, device="cuda")
    t["blk_idx"] = torch.zeros(B, Hkv, nblk, K, dtype=torch.int32, device="cuda")
    t["blk_count"] = torch.zeros(B, Hkv, nblk, dtype=torch.int32, device="cuda")
    t["out"] = torch.zeros(B, Hq, N, d, dtype=torch.float32, device="cuda")
    p = sa.make_params(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, n_ctx=N, dtype="bf16",
                       head_kind=[workloads.HEAD_ROUTED] * Hq, rope_base=cfg.rope_base, chunk=C,
                       group=cfg.group, top_chunks=cfg.top_chunks, top_groups=cfg.top_groups,
                       sink_chunks=cfg.sink_chunks, local_chunks=cfg.local_chunks, levels=1,
                       factor=4, q_block=C, block_top_k=K)
    bufs = sa.make_buffers(q=t["q"], k_pre=t["k_pre"], k_cache=t["k_cache"], v_cache=t["v_cache"],
                           chunk_sum=t["chunk_sum"], group_sum=t["group_sum"],
                           blk_idx=t["blk_idx"], blk_count=t["blk_count"], out=t["out"])
    ws_s, ws_p = sa.Workspace("cuda"), sa.Workspace("cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        sa.index_build(p, bufs, sa.IDX_CHUNK_SUMMARY, 0, N)
        sa.select(p, bufs, sa.SEL_ROUTE2_PREFILL, ws_s)
        if ev:
            ev[0].record(stream)
        sa.prefill_chunked(p, bufs, ws_p)
        if ev:
            ev[1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        step(ev[i])
    end.record(stream)
    torch.cuda.synchronize()
    t_step = start.elapsed_time(end) / steps * 1e-3
    t_kernel = sum(a.elapsed_time(b) for a, b in ev) / steps * 1e-3
    counts = t["blk_count"].cpu()
    pairs = 0
    for blk in range(nblk):
        nq = min(C, N - blk * C)
        pairs += G * (int(counts[:, :, blk].sum()) * nq + B * Hkv * nq * (nq + 1) // 2)
    flops = 4 * d * pairs
    achieved = flops / t_kernel / 1e12
    vis_frac = pairs / (B * Hq * N * (N + 1) / 2)
    log(f"[bench] {cfg.name}: {t_step * 1e3:.3f} ms/step, prefill kernel {t_kernel * 1e3:.3f} ms, "
        f"{achieved:.1f} TFLOP/s, {100 * vis_frac:.2f} % of the causal pairs")
    sha = source_sha(["prefill.hip", "common.hpp", "args.hpp"])
    res = {
        "metric": "routed chunked prefill tokens/s + achieved bf16 MFMA TFLOP/s vs peak",
        "value": B * Hq * N / t_step, "unit": "tokens/s (B x heads x N per step)",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": t_step * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv,
                   "head_dim": d, "n_ctx": N, "chunk": C, "group": cfg.group,
                   "top_chunks": cfg.top_chunks, "top_groups": cfg.top_groups,
                   "sink_chunks": cfg.sink_chunks, "local_chunks": cfg.local_chunks,
                   "visible_pair_frac": vis_frac},
        "step_tflops": flops / t_step / 1e12,
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel<false>", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic_record("prefill_kernel<false>", cfg.name, sha),
                     "flops_per_launch": flops, "launch_us": t_kernel * 1e6, "source_sha": sha},
    }
    if cpu and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill_routed(cfg, t, args.cpu_seconds, torch)
    del t
    torch.cuda.empty_cache()
    return res


def cpu_baseline_prefill_routed(cfg, t, budget_s, torch):
    """The fp64 oracle on whole query blocks of KV group 0 (routing over the
    GPU's summaries, then attention for the group's query heads), last blocks
    first, until ``budget_s`` is spent."""
    import numpy as np
    import oracle
    G, C, N = cfg.gqa, cfg.chunk, cfg.n_ctx
    q = t["q"][0, :G].to("cpu", torch.float64).numpy()
    K = t["k_cache"][0, 0].to("cpu", torch.float64).numpy()
    V = t["v_cache"][0, 0].to("cpu", torch.float64).numpy()
    cs = t["chunk_sum"][0, 0].to("cpu", torch.float64).numpy()
    gs = t["group_sum"][0, 0].to("cpu", torch.float64).numpy()
    nblk = (N + C - 1) // C
    t0 = time.perf_counter()
    done = 0
    while time.perf_counter() - t0 < budget_s or done == 0:
        blk = nblk - 1 - (done * 37) % nblk
        rows = np.arange(blk * C, min(N, (blk + 1) * C))
        lst, _ = oracle.route_prefill_block(q[:, rows].reshape(-1, q.shape[-1]), cs, gs, blk, N, C,
                                            cfg.group, cfg.top_chunks, cfg.top_groups,
                                            cfg.sink_chunks, cfg.local_chunks)
        for h in range(G):
            oracle.route_prefill_rows(q[h], K, V, lst, blk, C, rows)
        done += 1
    spent = time.perf_counter() - t0
    return {"value": done * C * G / spent, "unit": "tokens/s (B x heads x N)",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"{done} query blocks of KV group 0 ({G} query heads) of {cfg.name}: routing "
                      f"over the GPU's summaries and attention, fp64 numpy, {spent:.1f} s"}


def cpu_baseline_prefill_heads(cfg, t, budget_s, torch):
    """The fp64 oracle on query rows of the first dense head and the first
    local head, alternating, at positions spread over the sequence (a stride
    of 97 from the end), until ``budget_s`` is spent; the rate is scaled to
    the whole call's rows."""
    import numpy as np
    import oracle
    kinds = cfg.head_kind()
    hd = next(h for h, k in enumerate(kinds) if k != 0)      # a dense head
    hl = kinds.index(0)                                      # a local head
    G = cfg.gqa
    side = {h: (t["q"][0, h].to("cpu", torch.float64).numpy(),
                t["k_cache"][0, h // G, :cfg.n_ctx].to("cpu", torch.float64).numpy(),
                t["v_cache"][0, h // G, :cfg.n_ctx].to("cpu", torch.float64).numpy())
            for h in {hd, hl}}
    t0 = time.perf_counter()
    done = {hd: 0, hl: 0}
    spent_by = {hd: 0.0, hl: 0.0}
    k = 0
    while time.perf_counter() - t0 < budget_s or min(done.values()) == 0:
        h = hd if k % 2 == 0 else hl
        Q, K, V = side[h]
        i = cfg.n_ctx - 1 - (k // 2) * 97 % cfg.n_ctx
        s0 = time.perf_counter()
        oracle.head_prefill_rows(Q, K, V, kinds[h], cfg.sinks, cfg.window, np.array([i]))
        spent_by[h] += time.perf_counter() - s0
        done[h] += 1
        k += 1
    spent = time.perf_counter() - t0
    # seconds per row of each kind, weighted by the call's rows of each kind
    n_loc = kinds.count(0)
    per_row = (spent_by[hd] / done[hd]) * (len(kinds) - n_loc) + (spent_by[hl] / done[hl]) * n_loc
    return {"value": len(kinds) / per_row, "unit": "tokens/s (B x heads x N)",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"{done[hd]} query rows of dense head {hd} and {done[hl]} of local head "
                      f"{hl} of {cfg.name} (positions a stride of 97 apart from the end), fp64 "
                      f"numpy, {spent:.1f} s; per-row times weighted by the call's heads"}


def cpu_baseline_prefill(cfg, t, budget_s, torch):
    """The fp64 oracle on whole query blocks of head 0 (pyramid + scores once,
    then per block: selection and attention) until ``budget_s`` is spent."""
    import oracle
    from oracle import lighthouse as LH
    Q, K, V = (t[k][0, 0].to("cpu", torch.float64).numpy() for k in ("q", "k", "v"))
    t0 = time.perf_counter()
    kc = oracle.pyramid_levels(K, cfg.levels, cfg.factor, cfg.dtype)
    vc = oracle.pyramid_levels(V, cfg.levels, cfg.factor, cfg.dtype)
    sc = oracle.pyramid_scores(Q, K, cfg.levels, cfg.factor)
    nblk = cfg.n_ctx // cfg.q_block
    done = 0
    while time.perf_counter() - t0 < budget_s or done == 0:
        blk = nblk - 1 - (done * 37) % nblk
        sel = oracle.block_select(sc, blk, cfg.n_ctx, cfg.levels, cfg.factor, cfg.q_block,
                                  cfg.block_top_k)
        LH.prefill_block(Q, K, V, kc, vc, sel, blk, cfg.q_block, cfg.levels, cfg.factor)
        done += 1
    spent = time.perf_counter() - t0
    return {"value": done * cfg.q_block / spent, "unit": "tokens/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{done} query blocks of one head of {cfg.name} (pyramid and scores of "
                      f"the head once, then selection + attention per block), fp64 numpy, "
                      f"{spent:.1f} s"}


def cpu_baseline_prefill_backward(cfg, t, budget_s, torch):
    """The fp64 oracle's training step on whole query blocks of head 0
    (pyramid and scores once, then per block: selection, attention and its
    gradients) with a seeded upstream gradient, until ``budget_s`` is spent."""
    import numpy as np
    import oracle
    from oracle import lighthouse as LH
    Q, K, V = (t[k][0, 0].to("cpu", torch.float64).numpy() for k in ("q", "k", "v"))
    dO = np.random.default_rng(0).standard_normal(Q.shape)
    t0 = time.perf_counter()
    kc = oracle.pyramid_levels(K, cfg.levels, cfg.factor, cfg.dtype)
    vc = oracle.pyramid_levels(V, cfg.levels, cfg.factor, cfg.dtype)
    sc = oracle.pyramid_scores(Q, K, cfg.levels, cfg.factor)
    nblk = cfg.n_ctx // cfg.q_block
    done = 0
    while time.perf_counter() - t0 < budget_s or done == 0:
        blk = nblk - 1 - (done * 37) % nblk
        sel = oracle.block_select(sc, blk, cfg.n_ctx, cfg.levels, cfg.factor, cfg.q_block,
                                  cfg.block_top_k)
        LH.prefill_block(Q, K, V, kc, vc, sel, blk, cfg.q_block, cfg.levels, cfg.factor)
        oracle.block_grads(Q, K, V, kc, vc, sel, blk, cfg.q_block, cfg.levels, cfg.factor, dO)
        done += 1
    spent = time.perf_counter() - t0
    return {"value": done * cfg.q_block / spent, "unit": "tokens/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{done} query blocks of one head of {cfg.name} (pyramid and scores of "
                      f"the head once, then selection + attention + its gradients per block; "
                      f"the scatter of the gradients is not included), fp64 numpy, {spent:.1f} s"}


if __name__ == "__main__":
    main()
