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
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
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


def run_decode(args, torch, sa, workloads):
    cfg = {
        "llama3_8b_decode_32k": workloads.LLAMA_32K,
        "llama3_8b_decode_128k": workloads.LLAMA_128K,
        "llama3_8b_decode_128k_topk": workloads.LLAMA_128K_TOPK,
        "hga_route_decode_64k": workloads.HGA_64K,
    }[args.workload]
    log(f"[bench] generating {args.instances} instance(s) of {cfg.name}")
    insts = [DecodeInstance(cfg, 1000 + i, sa, torch, workloads) for i in range(args.instances)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        x = insts[i % len(insts)]
        x.index_and_select()
        x.decode()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        x = insts[i % len(insts)]
        x.index_and_select()
        ev[i][0].record(stream)
        x.decode()
        ev[i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    t_step = start.elapsed_time(end) / args.steps * 1e-3
    t_kernel = sum(a.elapsed_time(b) for a, b in ev) / args.steps * 1e-3
    log(f"[bench] timed {args.steps} steps: {t_step * 1e6:.1f} us/step, "
        f"attention kernel {t_kernel * 1e6:.1f} us")
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
    kernel = "decode_split_kernel"
    sha = source_sha(["decode.hip", "common.hpp", "args.hpp"])
    achieved = attn_b / t_kernel / 1e9
    res = {
        "metric": METRIC, "value": tokens / t_step, "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": t_step * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "n_q_heads": cfg.n_q_heads,
                   "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim,
                   "n_ctx": cfg.n_ctx, "top_p": cfg.top_p if not cfg.top_k else None,
                   "top_k": cfg.top_k or None, "min_tokens": cfg.min_tokens,
                   "sinks": cfg.sinks, "window": cfg.window, "routed": cfg.routed,
                   "instances_rotated": len(insts)},
        "step_hbm_gbps": step_b / t_step / 1e9,
        "step_bytes": step_b,
        "selected_frac_mean": (sum(sel_frac) / len(sel_frac)) if sel_frac else None,
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": traffic_record(kernel, cfg.name, sha),
                     "bytes_per_launch": attn_b, "launch_us": t_kernel * 1e6,
                     "source_sha": sha},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode(cfg, insts[0], args.cpu_seconds, torch)
    return res


def cpu_baseline_decode(cfg, inst, budget_s, torch):
    """The fp64 oracle on whole (sequence, KV group) slices of the same step
    until ``budget_s`` of CPU time is spent; scaled to tokens/s."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:
        blas = 1
    G = cfg.gqa
    groups = [(b, g) for b in range(cfg.batch) for g in range(cfg.n_kv_heads)]
    t = inst.t
    done_heads, spent, i = 0, 0.0, 0
    while (spent < budget_s or done_heads == 0) and i < 4 * len(groups):
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
    return {"value": done_heads * cfg.n_ctx / spent, "unit": "tokens/s",
            "cores": int(blas), "kind": "oracle",
            "sample": f"{done_heads // G} whole (sequence, KV group) slices of the "
                      f"{cfg.name} step ({done_heads} query heads x {cfg.n_ctx} tokens), "
                      f"index + selection + attention, fp64 numpy, {spent:.1f} s",
            "host_cpus": os.cpu_count()}


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
    if args.workload == "pyramid_prefill_128k":
        res = run_prefill(args, torch, sa, workloads)
    else:
        res = run_decode(args, torch, sa, workloads)
    print(json.dumps(res), flush=True)


def run_prefill(args, torch, sa, workloads):
    raise SystemExit("pyramid prefill benchmark is not wired yet")


if __name__ == "__main__":
    main()
