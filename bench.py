#!/usr/bin/env python3
"""Benchmark of one cascade-attention step on one MI355X.

A step is one cascade_attn_run() over one batch (prefix kernel + suffix kernel
+ merge for the cascade path). Default workload: the pages' worked example,
N=64 requests, a 4096-token shared prefix, 128-token suffixes, 1 query token
each, 32 query / 8 KV heads, head_dim 128, bf16, page size 16.

Inputs are resident in HBM before timing. To keep the 256 MB Infinity Cache
from serving the KV a step reads, the timed loop rotates over several
identical copies of Q and the KV cache (same plan), so each step reads data
the previous steps have not touched for >= 1 GiB of traffic.

Prints one JSON line (the driver's contract); extra fields carry the
per-kernel breakdown, the non-cascade GPU path and a warm-cache number.
"""

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA, TFLOP/s
KERNEL_SOURCES = ["attn_tile.hpp", "merge.hpp", "device_common.hpp", "run.hip"]


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "shared_prefix_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload, kernel):
    """HBM bytes per launch measured by rocprofv3 --pmc (FETCH_SIZE, WRITE_SIZE)
    for this kernel source; None when absent or taken on other source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    if not k:
        return None
    return k["hbm_bytes_per_launch"]


def time_steps(fn, steps, rotate):
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i % rotate)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def cpu_baseline(b, kv_bytes, budget_s=12.0, max_runs=5):
    """The fp64 oracle (test infrastructure) on this host, one BLAS thread."""
    import oracle
    from threadpoolctl import threadpool_limits
    kc, vc = b.k_cache.float().numpy(), b.v_cache.float().numpy()
    args = (b.q.float().numpy(), kc, vc, b.block_table.numpy(), b.query_start_loc.numpy(),
            b.seq_lens.numpy(), b.workload.page_size)
    times = []
    t_start = time.perf_counter()
    with threadpool_limits(1):
        while len(times) < max_runs and (time.perf_counter() - t_start) < budget_s:
            t0 = time.perf_counter()
            oracle.attention_full(*args)
            times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    return {"value": round(kv_bytes / t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"whole batch ({b.workload.num_reqs} requests), {len(times)} runs, median {t:.2f} s; "
                      f"fp64 numpy, 1 BLAS thread"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="worked_decode")
    ap.add_argument("--mode", default="auto", choices=["auto", "on", "off"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-noncascade", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    import shared_prefix_attention_amd as spa

    dev = torch.device("cuda:0")
    w = workloads.get(args.workload)
    b = workloads.make_batch(w)
    G = w.num_q_heads // w.num_kv_heads
    bpt = 2 * w.num_kv_heads * w.head_dim * 2

    def make_plan(mode):
        return spa.plan_batch(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                              k_cache=b.k_cache, block_table=b.block_table, query_start_loc=b.query_start_loc,
                              seq_lens=b.seq_lens, num_computed_tokens=b.num_computed, mode=mode)

    plan = make_plan(args.mode)
    info = plan.info
    T = b.total_q
    plen = info["common_prefix_len"] if info["use_cascade"] else 0
    kv_tokens = info["kv_tokens_cascade"] if info["use_cascade"] else info["kv_tokens_noncascade"]
    kv_bytes = kv_tokens * bpt
    touched = kv_bytes + b.q.numel() * 2
    rotate = int(min(64, max(2, math.ceil((1 << 30) / max(touched, 1)))))
    copies = []
    for _ in range(rotate):
        copies.append((b.q.to(dev), b.k_cache.to(dev), b.v_cache.to(dev)))
    bt, qsl, sl = b.block_table.to(dev), b.query_start_loc.to(dev), b.seq_lens.to(dev)
    out = torch.empty_like(copies[0][0])
    lse = torch.empty(T, w.num_q_heads, dtype=torch.float32, device=dev)

    def workspace_for(pl):
        return torch.empty(max(pl.workspace_bytes, 256), dtype=torch.uint8, device=dev)

    ws = workspace_for(plan)

    def step_with(pl, wsp):
        def f(i):
            q, k, v = copies[i]
            spa.cascade_attn_run(pl, q, k, v, bt, qsl, sl, out, lse, wsp)
        return f

    step = step_with(plan, ws)
    for i in range(args.warmup):
        step(i % rotate)
    ms = time_steps(step, args.steps, rotate)

    # per-kernel durations: HIP events around every launch, same stream
    spa.cascade_attn_profile_enable(True)
    ms_prof = time_steps(step, args.steps, rotate)
    spa.cascade_attn_profile_enable(False)
    prof = spa.cascade_attn_profile_read()
    kern = {}
    for kind, (tot_ms, cnt) in prof.items():
        if cnt:
            kern[kind] = {"avg_us": round(tot_ms * 1e3 / cnt, 3), "launches": int(cnt)}

    # algorithmic work per launch
    q_bytes = T * w.num_q_heads * w.head_dim * 2
    suffix_tokens = int(info["kv_tokens_cascade"] - plen) if info["use_cascade"] else int(info["kv_tokens_noncascade"])
    work = {
        "prefix": {"bytes": plen * bpt + q_bytes, "flops": 4.0 * T * w.num_q_heads * plen * w.head_dim},
        "suffix": {"bytes": suffix_tokens * bpt + q_bytes, "flops": None},
    }
    for kind in ("prefix", "suffix"):
        if kind in kern:
            sec = kern[kind]["avg_us"] * 1e-6
            kern[kind]["gbs"] = round(work[kind]["bytes"] / sec / 1e9, 1)
            kern[kind]["hbm_frac"] = round(work[kind]["bytes"] / sec / 1e9 / HBM_PEAK_GBS, 4)
            if work[kind]["flops"]:
                kern[kind]["tflops"] = round(work[kind]["flops"] / sec / 1e12, 2)
                kern[kind]["mfma_frac"] = round(work[kind]["flops"] / sec / 1e12 / BF16_PEAK_TFLOPS, 4)
    dom = max((k for k in ("prefix", "suffix") if k in kern), key=lambda k: kern[k]["avg_us"])
    traffic = load_traffic(args.workload, dom)
    roof = {"kernel": dom, "bound": "hbm", "achieved": kern[dom]["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": kern[dom]["hbm_frac"], "traffic": traffic}

    # warm-cache number (no rotation) and the GPU non-cascade path
    ms_warm = time_steps(step, args.steps, 1)
    extra = {}
    if not args.no_noncascade:
        plan_off = make_plan("off")
        ws_off = workspace_for(plan_off)
        step_off = step_with(plan_off, ws_off)
        for i in range(args.warmup):
            step_off(i % rotate)
        ms_off = time_steps(step_off, max(10, args.steps // 4), rotate)
        extra = {"noncascade_us_per_step": round(ms_off * 1e3, 3),
                 "speedup_vs_noncascade": round(ms_off / ms, 3)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(b, kv_bytes)

    gbs = kv_bytes / (ms * 1e-3) / 1e9
    line = {
        "metric": "cascade attn us/step + effective KV GB/s (N=64,P=4096,S=128), % of HBM roofline",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 3),
        "hbm_frac_step": round(gbs / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "num_reqs": w.num_reqs, "prefix": w.prefix,
                   "suffix": list(w.suffix), "q_len": list(w.q_len), "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "page_size": w.page_size,
                   "mode": args.mode, "use_cascade": info["use_cascade"], "common_prefix_len": plen,
                   "kv_bytes_per_step": kv_bytes, "rotating_copies": rotate},
        "roofline": roof,
        "kernels": kern,
        "profiled_us_per_step": round(ms_prof * 1e3, 3),
        "warm_us_per_step": round(ms_warm * 1e3, 3),
        "plan": {k: info[k] for k in ("prefix_splits", "prefix_row_tile", "suffix_chunks", "suffix_chunk_tokens",
                                       "suffix_kernel", "num_partial_slots", "workspace_bytes")},
        **extra,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
