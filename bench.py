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
                             "pyramid_prefill_128k"])
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
    def __init__(self, cfg, seed, sa, torch, workloads):
        B, Hq, Hkv, d, n = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_ctx
        self.cfg = cfg
        inp = workloads.decode_inputs(cfg, seed, device="cuda")
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        self.t = {k: inp[k].to(dt).contiguous() for k in ("q_pre", "q", "k_pre", "k_cache", "v_cache")}
        del inp["k_pre"], inp["k_cache"], inp["v_cache"]
        self.t["proj"] = inp["proj"].float().contiguous()
        self.t["k_idx"] = torch.zeros(B, Hkv, n, cfg.r, dtype=dt, device="cuda")
        self.t["q_idx"] = torch.zeros(B, Hq, cfg.r, dtype=torch.float32, device="cuda")
        self.t["sel_idx"] = torch.zeros(B, Hkv, n, dtype=torch.int32, device="cuda")
        self.t["sel_count"] = torch.zeros(B, Hkv, dtype=torch.int32, device="cuda")
        self.t["out"] = torch.zeros(B, Hq, d, dtype=torch.float32, device="cuda")
        if cfg.routed:
            self.t["chunk_sum"] = torch.zeros(B, Hkv, n // cfg.chunk, d, dtype=dt, device="cuda")
            self.t["group_sum"] = torch.zeros(B, Hkv, n // cfg.group, d, dtype=dt, device="cuda")
        t = self.t
        self.params = sa.params_from_config(cfg)
        self.bufs = sa.make_buffers(
            q_pre=t["q_pre"], k_pre=t["k_pre"], q=t["q"], k_cache=t["k_cache"],
            v_cache=t["v_cache"], proj_q=t["proj"], proj_k=t["proj"], q_idx=t["q_idx"],
            k_idx=t["k_idx"], chunk_sum=t.get("chunk_sum"), group_sum=t.get("group_sum"),
            sel_idx=t["sel_idx"], sel_count=t["sel_count"], out=t["out"])
        self.ws_sel = sa.Workspace("cuda")
        self.ws_dec = sa.Workspace("cuda")
        self.sa = sa
        # prefill-time index over the whole history (not part of a step)
        if cfg.routed:
            sa.index_build(self.params, self.bufs, sa.IDX_CHUNK_SUMMARY, 0, n)
        else:
            sa.index_build(self.params, self.bufs, sa.IDX_LOWRANK, 0, n)
        self.sel_mode = (sa.SEL_ROUTE2 if cfg.routed else
                         (sa.SEL_TOPK if cfg.top_k > 0 else sa.SEL_TOPP))

    def index_and_select(self):
        sa, cfg = self.sa, self.cfg
        n = cfg.n_ctx
        if cfg.routed:
            # the step completes at most one chunk: rebuild the last one
            t0 = (n // cfg.chunk) * cfg.chunk - 1 if n % cfg.chunk == 0 else n - 1
            sa.index_build(self.params, self.bufs, sa.IDX_CHUNK_SUMMARY, max(0, t0), n)
        else:
            sa.index_build(self.params, self.bufs, sa.IDX_LOWRANK, n - 1, n)
        sa.select(self.params, self.bufs, self.sel_mode, self.ws_sel)

    def decode(self):
        self.sa.decode(self.params, self.bufs, self.ws_dec)

    def capture(self, torch):
        """Record the step's two halves into HIP graphs (after a warm-up)."""
        self.g_sel, self.g_dec = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g_sel):
            self.index_and_select()
        with torch.cuda.graph(self.g_dec):
            self.decode()


def decode_bytes(cfg, counts, kinds):
    """Algorithmic bytes of one decode step and of its attention kernel."""
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
                lists += 4 * c
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
}


def run_decode(args, torch, sa, workloads, workload=None, steps=None, warmup=None,
               instances=None, cpu=True):
    workload = workload or args.workload
    steps = steps or args.steps
    warmup = args.warmup if warmup is None else warmup
    instances = instances or args.instances
    cfg = getattr(workloads, DECODE_CONFIGS[workload])
    log(f"[bench] generating {instances} instance(s) of {cfg.name}")
    insts = [DecodeInstance(cfg, 1000 + i, sa, torch, workloads) for i in range(instances)]
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
    kinds = cfg.head_kind()
    attn_b, step_b = 0, 0
    sel_frac = []
    for x in insts:
        c = x.t["sel_count"].cpu().tolist()
        a, s_ = decode_bytes(cfg, c, kinds)
        attn_b += a
        step_b += s_
        for b in range(cfg.batch):
            for g in range(cfg.n_kv_heads):
                if kinds[g * cfg.gqa] != 0:
                    sel_frac.append(c[b][g] / cfg.n_ctx)
    attn_b /= len(insts)
    step_b /= len(insts)
    tokens = cfg.batch * cfg.n_q_heads * cfg.n_ctx
    kernel = "sparse_attn_decode (decode_mfma_kernel + decode_item_combine_kernel)"
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
                   "instances_rotated": len(insts),
                   "launch": "hip_graph" if args.graph else "eager"},
        "step_hbm_gbps": step_b / t_step / 1e9,
        "step_bytes": step_b,
        "selected_frac_mean": (sum(sel_frac) / len(sel_frac)) if sel_frac else None,
        "spread_us": {"step": percentiles(per_step), "attention_call": percentiles(per_call),
                      "attention_call_warm_mean": t_warm * 1e6,
                      "note": "one event pair per step in a separate pass; rotated instances "
                              "(cold in the 256 MB Infinity Cache); warm = one instance's call "
                              "repeated"},
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": traffic_record(kernel, cfg.name, sha),
                     "bytes_per_launch": attn_b, "launch_us": t_kernel * 1e6,
                     "source_sha": sha},
    }
    if cpu and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode(cfg, insts[0], args.cpu_seconds, torch)
    del insts
    torch.cuda.empty_cache()
    return res


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
    keep = ("value", "unit", "ms_per_step", "step_hbm_gbps", "selected_frac_mean", "config",
            "roofline", "step_tflops")
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
    else:
        res = run_decode(args, torch, sa, workloads)
    if not args.no_extras and args.workload == "llama3_8b_decode_32k":
        other = {}
        for w in ("llama3_8b_decode_128k_topk", "llama3_8b_decode_128k", "hga_route_decode_64k"):
            other[w] = compact(run_decode(args, torch, sa, workloads, workload=w, steps=20,
                                          warmup=3, instances=2, cpu=False))
        other["pyramid_prefill_128k"] = compact(run_prefill(args, torch, sa, workloads, steps=5,
                                                            warmup=1, cpu=False))
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


def run_prefill(args, torch, sa, workloads, steps=None, warmup=None, cpu=True):
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
    p = sa.params_from_config(cfg)
    bufs = sa.make_buffers(q=t["q"], k_cache=t["k"], v_cache=t["v"], pyr_q=t["pq"],
                           pyr_k=t["pk"], pyr_v=t["pv"], pyr_scores=t["scores"],
                           blk_idx=t["blk_idx"], blk_count=t["blk_count"], out=t["out"])
    ws_s, ws_p = sa.Workspace("cuda"), sa.Workspace("cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        sa.index_build(p, bufs, sa.IDX_PYRAMID, 0, N)
        sa.select(p, bufs, sa.SEL_PYRAMID_TOPK, ws_s)
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
    counts = t["blk_count"].reshape(B * H, nblk).cpu().tolist()
    flops = prefill_flops(cfg, counts)
    log(f"[bench] {cfg.name}: {t_step * 1e3:.3f} ms/step, prefill kernel {t_kernel * 1e3:.3f} ms, "
        f"{flops / t_kernel / 1e12:.1f} TFLOP/s")
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
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic_record("prefill_kernel", cfg.name, sha),
                     "flops_per_launch": flops, "launch_us": t_kernel * 1e6, "source_sha": sha},
    }
    if cpu and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(cfg, t, args.cpu_seconds, torch)
    del t
    torch.cuda.empty_cache()
    return res


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


if __name__ == "__main__":
    main()
