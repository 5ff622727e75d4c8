#!/usr/bin/env python3
"""Benchmark of one cascade-attention step on one MI355X.

A step is one cascade_attn_run() over one batch: for the cascade path one
launch running the prefix and suffix work-groups plus one merge launch.
Default workload: the pages' worked example, N=64 requests, a 4096-token
shared prefix, 128-token suffixes, one query token each, 32 query / 8 KV
heads, head_dim 128, bf16, page size 16 (synthetic inputs).

Inputs are resident in HBM before timing. So that the 256 MB Infinity Cache
cannot serve the KV a step reads, the timed loop rotates over identical copies
of Q and the KV cache (same plan): each step reads data that >= 1 GiB of other
traffic has passed since its last use.

Prints one JSON line; extra fields carry the per-kernel breakdown, the GPU
non-cascade path, a warm-cache number and the oracle's CPU rate.

Other modes (measurement plumbing, used under rocprofv3):
  --traffic-probe       one device copy of known size, then --steps steps
                        (no timing; for `rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE`)
  --probe-separate      with --traffic-probe: the cascade phases as separate
                        launches (per-phase counters, e.g. the prefix's MFMA)
  --summarize-pmc F W   read the counter CSVs of those two runs and write the
                        HBM-traffic summary profiles/traffic_<workload>.json
  --decision-sweep      time the cascade and non-cascade paths over a grid of
                        batch shapes and print, per shape, AUTO's choice, both
                        times and the time AUTO loses against the faster path
"""

import argparse
import csv
import glob
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
# device code and the partition: what the traffic counters depend on
KERNEL_SOURCES = ["attn_tile.hpp", "merge.hpp", "device_common.hpp", "plan.cpp"]
COPY_BYTES = 512 << 20         # calibration copy for the traffic counters
KIND_KERNEL = {"cascade_phases": "cascade_phases_kernel", "attention": "attn_tile_kernel",
               "decode": "attn_tile_kernel", "merge": "merge_kernel"}


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "shared_prefix_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def load_traffic(workload, kind):
    """HBM bytes per launch of `kind` from the committed rocprofv3 summary,
    or None when absent or taken on other kernel source."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(KIND_KERNEL.get(kind, kind))
    return None if not k else k["hbm_bytes_per_launch"]


def time_steps(fn, steps, rotate):
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i % rotate)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def step_distribution(fn, steps, rotate):
    """Per-step GPU time (us) from events recorded around every run on the
    stream the runs use; returns p10 / median / p90."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record()
        fn(i % rotate)
        ev[i][1].record()
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    pick = lambda q: round(us[min(len(us) - 1, int(q * (len(us) - 1) + 0.5))], 3)
    return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads():
    """Threads the host gives this process: the affinity mask, capped by
    OMP_NUM_THREADS when that is set (the GPU machine sets it to its CPU share)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def cpu_baseline(b, kv_bytes, budget_s=12.0, max_runs=60):
    """The fp64 oracle (test infrastructure) on this host over the whole
    batch, repeated for about budget_s seconds per thread count: with every
    host thread given to numpy's BLAS, and with one. The oracle is the plain
    definition, untuned; it loops over requests and heads in Python, so
    extra BLAS threads help it little."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    w = b.workload
    if w.kv_dtype == "fp8":   # the oracle decodes the e4m3 codes itself
        kc = oracle.fp8_e4m3_decode(b.k_cache.numpy()) * w.k_scale
        vc = oracle.fp8_e4m3_decode(b.v_cache.numpy()) * w.v_scale
    else:
        kc, vc = b.k_cache.float().numpy(), b.v_cache.float().numpy()
    args = (b.q.float().numpy(), kc, vc, b.block_table.numpy(), b.query_start_loc.numpy(),
            b.seq_lens.numpy(), b.workload.page_size)

    def run(threads):
        times = []
        t_start = time.perf_counter()
        with threadpool_limits(threads):
            blas = [p.get("num_threads") for p in threadpool_info() if p.get("user_api") == "blas"]
            while len(times) < max_runs and (time.perf_counter() - t_start) < budget_s:
                t0 = time.perf_counter()
                oracle.attention_full(*args)
                times.append(time.perf_counter() - t0)
        return statistics.median(times), len(times), sum(times), (blas[0] if blas else None)

    n = host_threads()
    t_all, runs_all, tot_all, blas_all = run(n)
    t_one, runs_one, tot_one, _ = run(1)
    legs = {"all_threads": {"value": round(kv_bytes / t_all / 1e9, 4), "unit": "GB/s", "cores": n,
                            "sample": f"{runs_all} runs ({tot_all:.1f} s), median {t_all:.3f} s per batch, "
                                      f"{blas_all} BLAS threads"},
            "one_thread": {"value": round(kv_bytes / t_one / 1e9, 4), "unit": "GB/s", "cores": 1,
                           "sample": f"{runs_one} runs ({tot_one:.1f} s), median {t_one:.3f} s per batch"}}
    # the headline figure is the faster configuration; both are recorded
    best = "all_threads" if t_all <= t_one else "one_thread"
    t_best = min(t_all, t_one)
    return {"value": legs[best]["value"], "unit": "GB/s", "cores": legs[best]["cores"], "kind": "oracle",
            "sample": f"whole batch ({w.num_reqs} requests, every row), median {t_best:.3f} s per batch; fp64 "
                      f"numpy ({best.replace('_', ' ')}: the faster of {n} BLAS threads and 1)",
            "cpu_model": cpu_model(), "host_threads": n, **legs}


def summarize_pmc(fetch_dir, write_dir, workload, steps):
    """Traffic per launch = counter (KiB) x (bytes the calibration copy moves /
    what the same counter reads for it)."""
    def read(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            rows += [r for r in csv.DictReader(open(f)) if r["Counter_Name"] == counter]
        return rows
    out = {"workload": workload, "kernel_source_hash": kernel_source_hash(), "kernels": {},
           "command": f"rocprofv3 --pmc FETCH_SIZE -f csv -d {fetch_dir} -o p -- python3 -u bench.py --traffic-probe "
                      f"--workload {workload} --steps {steps}; the same with WRITE_SIZE into {write_dir}; then "
                      f"python3 bench.py --summarize-pmc {fetch_dir} {write_dir} --workload {workload} --steps {steps}"}
    for counter, d, key in (("FETCH_SIZE", fetch_dir, "fetch"), ("WRITE_SIZE", write_dir, "write")):
        rows = read(d, counter)
        copy = [float(r["Counter_Value"]) for r in rows if "copy" in r["Kernel_Name"].lower()]
        if not copy:
            raise SystemExit(f"no calibration copy dispatch in {d}")
        factor = COPY_BYTES / (max(copy) * 1024.0)
        out[f"{key}_factor"] = factor
        for kname in sorted(set(KIND_KERNEL.values())):
            vals = [float(r["Counter_Value"]) for r in rows if kname in r["Kernel_Name"]]
            if vals:
                k = out["kernels"].setdefault(kname, {})
                k[f"{key}_kib_raw"] = statistics.median(vals)
                k[f"{key}_bytes"] = statistics.median(vals) * 1024.0 * factor
    for k in out["kernels"].values():
        k["hbm_bytes_per_launch"] = k.get("fetch_bytes", 0.0) + k.get("write_bytes", 0.0)
    return out


# Batch shapes of the decision sweep: decode batches (one query token) over
# request counts, shared-prefix lengths and suffix lengths around the gates
# (256 tokens, 8 requests) and far from them, plus chunked-prefill batches
# (32 / 8 heads, head_dim 128, bf16); then decode batches with 64 / 8 heads,
# with head_dim 64, with fp8 e4m3 caches, and with two interleaved documents
# shared by the even and the odd requests after the prefix.
SWEEP_DECODE = [(n, p, s) for n in (2, 4, 8, 16, 64, 256) for p in (256, 1024, 4096, 16384) for s in (16, 512)]
SWEEP_PREFILL = [(n, p) for n in (8, 32, 128) for p in (256, 2048)]
SWEEP_WIDE = ([("h64", n, p, s) for n in (4, 16, 64, 256) for p in (1024, 8192) for s in (16, 512)] +
              [("d64", n, p, s) for n in (4, 16, 64) for p in (256, 4096) for s in (16, 512)] +
              [("fp8", n, p, s) for n in (4, 16, 64) for p in (1024, 4096) for s in (16, 512)] +
              [("docs", n, p, s) for n in (8, 32) for p in (256, 1024) for s in (16, 256)])


def sweep_workloads():
    """The decision sweep's batch shapes, as workloads (seed 7)."""
    import workloads
    W = workloads.Workload
    cases = [W(name=f"decode_n{n}_p{p}_s{sl}", num_reqs=n, prefix=p, suffix=(sl, sl), q_len=(1, 1),
               num_q_heads=32, num_kv_heads=8, head_dim=128, seed=7) for n, p, sl in SWEEP_DECODE]
    cases += [W(name=f"prefill_n{n}_p{p}", num_reqs=n, prefix=p, suffix=(64, 512), q_len=(1, 64),
                num_q_heads=32, num_kv_heads=8, head_dim=128, seed=7) for n, p in SWEEP_PREFILL]
    for fam, n, p, sl in SWEEP_WIDE:
        kw = dict(num_reqs=n, prefix=p, suffix=(sl, sl), q_len=(1, 1), num_q_heads=32, num_kv_heads=8,
                  head_dim=128, seed=7)
        if fam == "h64":
            kw["num_q_heads"] = 64
        elif fam == "d64":
            kw["head_dim"] = 64
        elif fam == "fp8":
            kw.update(kv_dtype="fp8", k_scale=0.125, v_scale=0.0625)
        else:
            kw["docs"] = ((tuple(range(0, n, 2)), 1024), (tuple(range(1, n, 2)), 2048))
        cases.append(W(name=f"{fam}_n{n}_p{p}_s{sl}", **kw))
    return cases


def decision_sweep(steps, warmup):
    """AUTO's use_cascade choice against both forced paths, per batch shape
    (GQA 32/8, head_dim 128, bf16, page 16; rotating input copies as in the
    main measurement; each path's time is the median of per-step events).
    Prints one JSON line per shape, with the planner's estimates, and a
    summary line."""
    import torch
    import workloads
    import shared_prefix_attention_amd as spa

    dev = torch.device("cuda:0")
    recs = []
    for w in sweep_workloads():
        b = workloads.make_batch(w)
        touched = b.k_cache.numel() * b.k_cache.element_size() * 2 + b.q.numel() * 2
        rotate = int(min(32, max(2, math.ceil((1 << 30) / max(touched, 1)))))
        copies = [(b.q.to(dev), b.k_cache.to(dev), b.v_cache.to(dev)) for _ in range(rotate)]
        bt, qsl, sl = b.block_table.to(dev), b.query_start_loc.to(dev), b.seq_lens.to(dev)
        out = torch.empty_like(copies[0][0])
        lse = torch.empty(b.total_q, w.num_q_heads, dtype=torch.float32, device=dev)
        times, infos, kern = {}, {}, {}
        for mode in ("auto", "on", "off"):
            pl = spa.plan_batch(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                                k_cache=b.k_cache, block_table=b.block_table, query_start_loc=b.query_start_loc,
                                seq_lens=b.seq_lens, num_computed_tokens=b.num_computed, mode=mode,
                                kv_dtype=w.kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
            ws = torch.zeros(max(pl.workspace_bytes, 256), dtype=torch.uint8, device=dev)

            def f(i, pl=pl, ws=ws):
                q, k, v = copies[i]
                spa.cascade_attn_run(pl, q, k, v, bt, qsl, sl, out, lse, ws)
            for i in range(warmup):
                f(i % rotate)
            times[mode] = step_distribution(f, steps, rotate)["p50"]   # median, robust to stray slow steps
            infos[mode] = pl.info
            if mode != "auto":
                spa.cascade_attn_profile_enable(4 * steps)
                time_steps(f, steps, rotate)
                kern[mode] = {k: round(t * 1e3 / c, 2) for k, (t, c) in spa.cascade_attn_profile_read().items() if c}
                spa.cascade_attn_profile_enable(0)
        casc = bool(infos["auto"]["use_cascade"])
        best = min(times["on"], times["off"])
        chosen = times["on"] if casc else times["off"]
        rec = {"case": w.name, "num_reqs": w.num_reqs, "prefix": w.prefix, "suffix": list(w.suffix),
               "q_len": list(w.q_len), "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
               "head_dim": w.head_dim, "kv_dtype": w.kv_dtype, "docs": len(w.docs),
               "levels": infos["on"]["shared_levels"],
               "gates_pass": infos["auto"]["gates_pass"], "auto_cascade": int(casc),
               "cascade_us": round(times["on"], 2), "noncascade_us": round(times["off"], 2),
               "auto_us": round(times["auto"], 2), "chosen_over_best": round(chosen / best, 3),
               "faster": "cascade" if times["on"] < times["off"] else "non-cascade",
               "est_cascade_us": round(infos["auto"]["est_us_cascade"], 1),
               "est_noncascade_us": round(infos["auto"]["est_us_noncascade"], 1),
               "noncascade_chunks": infos["off"]["suffix_chunks"], "prefix_splits": infos["on"]["prefix_splits"],
               "kernels_cascade_us": kern["on"], "kernels_noncascade_us": kern["off"]}
        recs.append(rec)
        print(json.dumps(rec), flush=True)
        del copies
        torch.cuda.empty_cache()
    right = sum(1 for r in recs if (r["auto_cascade"] == 1) == (r["faster"] == "cascade"))
    lost = [r["chosen_over_best"] for r in recs]
    print(json.dumps({"decision_sweep": len(recs), "auto_picked_faster": right,
                      "worst_chosen_over_best": max(lost),
                      "mean_chosen_over_best": round(sum(lost) / len(lost), 4),
                      "steps": steps, "warmup": warmup}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="worked_decode")
    ap.add_argument("--mode", default="auto", choices=["auto", "on", "off"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-noncascade", action="store_true")
    ap.add_argument("--no-phases", action="store_true")
    ap.add_argument("--no-warm", action="store_true", help="skip the warm-cache (no rotation) loop")
    ap.add_argument("--max-levels", type=int, default=0, help="shared levels of the cascade plan (0 = default)")
    ap.add_argument("--traffic-probe", action="store_true")
    ap.add_argument("--probe-separate", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--decision-sweep", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.decision_sweep:
        decision_sweep(args.steps, args.warmup)
        return
    if args.summarize_pmc:
        rec = summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload, args.steps)
        os.makedirs(os.path.dirname(traffic_path(args.workload)), exist_ok=True)
        with open(traffic_path(args.workload), "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return

    import torch
    import workloads
    import shared_prefix_attention_amd as spa

    dev = torch.device("cuda:0")
    w = workloads.get(args.workload)
    b = workloads.make_batch(w)
    bpt = 2 * w.num_kv_heads * w.head_dim * (1 if w.kv_dtype == "fp8" else 2)   # K+V bytes per token

    def make_plan(mode, **kw):
        return spa.plan_batch(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                              k_cache=b.k_cache, block_table=b.block_table, query_start_loc=b.query_start_loc,
                              seq_lens=b.seq_lens, num_computed_tokens=b.num_computed, mode=mode,
                              max_levels=args.max_levels, k_scale=w.k_scale, v_scale=w.v_scale, **kw)

    plan = make_plan(args.mode)
    info = plan.info
    T = b.total_q
    casc = bool(info["use_cascade"])
    plen = info["common_prefix_len"] if casc else 0
    kv_tokens = info["kv_tokens_cascade"] if casc else info["kv_tokens_noncascade"]
    kv_bytes = kv_tokens * bpt
    touched = kv_bytes + b.q.numel() * 2
    rotate = 1 if args.traffic_probe else int(min(64, max(2, math.ceil((1 << 30) / max(touched, 1)))))
    copies = [(b.q.to(dev), b.k_cache.to(dev), b.v_cache.to(dev)) for _ in range(rotate)]
    bt, qsl, sl = b.block_table.to(dev), b.query_start_loc.to(dev), b.seq_lens.to(dev)
    out = torch.empty_like(copies[0][0])
    lse = torch.empty(T, w.num_q_heads, dtype=torch.float32, device=dev)

    def workspace_for(pl):
        return torch.zeros(max(pl.workspace_bytes, 256), dtype=torch.uint8, device=dev)

    ws = workspace_for(plan)

    def step_with(pl, wsp):
        def f(i):
            q, k, v = copies[i]
            spa.cascade_attn_run(pl, q, k, v, bt, qsl, sl, out, lse, wsp)
        return f

    step = step_with(plan, ws)
    if args.traffic_probe and args.probe_separate and casc:
        plan = make_plan(args.mode, separate_phases=True)
        step = step_with(plan, workspace_for(plan))
    if args.traffic_probe:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        for i in range(args.steps):
            step(0)
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": args.workload, "steps": args.steps}))
        return

    for i in range(args.warmup):
        step(i % rotate)
    # The timed loop: K steps, nothing but the launches. Then the same K
    # steps again with a start / stop event pair on every kernel launch (from
    # a pool created before the loop, recorded on the launch's own stream):
    # the per-kernel durations of the roofline come from that pass. The
    # event records cost host time per launch, so that pass's wall time
    # (reported beside) is longer; the kernels' own durations are not.
    ms = time_steps(step, args.steps, rotate)
    spa.cascade_attn_profile_enable(4 * args.steps)
    ms_events = time_steps(step, args.steps, rotate)
    prof = spa.cascade_attn_profile_read()
    spa.cascade_attn_profile_enable(0)
    dist = step_distribution(step, args.steps, rotate)
    kern = {}
    for kind, (tot_ms, cnt) in prof.items():
        if cnt:
            kern[kind] = {"avg_us": round(tot_ms * 1e3 / cnt, 3), "launches": int(cnt)}

    # algorithmic work of one launch of each attention kernel: the KV
    # positions it must read (prefix once + each request's suffix) plus Q, and
    # its QK^T / PV flops
    q_bytes = T * w.num_q_heads * w.head_dim * 2
    qlen = (b.query_start_loc[1:] - b.query_start_loc[:-1]).tolist()
    seq = b.seq_lens.tolist()
    visible = sum(ql * (s - ql) + ql * (ql + 1) // 2 for ql, s in zip(qlen, seq))   # causal keys per query
    flops = 4.0 * w.num_q_heads * w.head_dim * visible
    attn_kind = "cascade_phases" if casc else ("decode" if info["suffix_kernel"] == 1 else "attention")
    work = {"bytes": kv_bytes + q_bytes, "flops": flops}
    if attn_kind in kern:
        sec = kern[attn_kind]["avg_us"] * 1e-6
        kern[attn_kind]["gbs"] = round(work["bytes"] / sec / 1e9, 1)
        kern[attn_kind]["hbm_frac"] = round(work["bytes"] / sec / 1e9 / HBM_PEAK_GBS, 4)
        kern[attn_kind]["tflops"] = round(work["flops"] / sec / 1e12, 2)
        kern[attn_kind]["mfma_frac"] = round(work["flops"] / sec / 1e12 / BF16_PEAK_TFLOPS, 4)
    traffic = load_traffic(args.workload, attn_kind)
    roof = {"kernel": attn_kind, "bound": "hbm", "achieved": kern[attn_kind]["gbs"], "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": kern[attn_kind]["hbm_frac"],
            "traffic": None if traffic is None else round(traffic)}

    # warm-cache number (no rotation) and the GPU non-cascade path
    ms_warm = None if args.no_warm else time_steps(step, args.steps, 1)
    extra = {}
    if not args.no_noncascade and casc:
        plan_off = make_plan("off")
        ws_off = workspace_for(plan_off)
        step_off = step_with(plan_off, ws_off)
        for i in range(args.warmup):
            step_off(i % rotate)
        ms_off = time_steps(step_off, max(10, args.steps // 4), rotate)
        extra = {"noncascade_us_per_step": round(ms_off * 1e3, 3),
                 "speedup_vs_noncascade": round(ms_off / ms, 3)}

    # each cascade phase on its own: the same work items as two launches, so
    # the prefix phase's MFMA rate and the suffix phase's HBM rate can be
    # read separately (the timed step above runs them as one launch)
    if not args.no_phases and casc:
        plan_sep = make_plan(args.mode, separate_phases=True)
        step_sep = step_with(plan_sep, workspace_for(plan_sep))
        for i in range(args.warmup):
            step_sep(i % rotate)
        spa.cascade_attn_profile_enable(4 * max(10, args.steps // 2))
        ms_sep = time_steps(step_sep, max(10, args.steps // 2), rotate)
        prof_sep = spa.cascade_attn_profile_read()
        spa.cascade_attn_profile_enable(0)
        # nested levels: each group's extra positions once, for its members' queries
        groups, deepest = spa.cascade_attn_plan_groups(plan_sep)
        qsl_l = b.query_start_loc.tolist()
        g_q = [0] * len(groups)
        for r, j in enumerate(deepest):
            while j >= 0:
                g_q[j] += qsl_l[r + 1] - qsl_l[r]
                j = groups[j][1]
        g_tokens = sum(ke - kb for _, _, kb, ke in groups)
        g_rows = sum(g_q)
        g_flops = sum(4.0 * q * w.num_q_heads * (ke - kb) * w.head_dim for q, (_, _, kb, ke) in zip(g_q, groups))
        suffix_visible = visible - plen * T - sum(q * (ke - kb) for q, (_, _, kb, ke) in zip(g_q, groups))
        ph_work = {"prefix": (plen * bpt + q_bytes, 4.0 * T * w.num_q_heads * plen * w.head_dim),
                   "level1": (g_tokens * bpt + g_rows * w.num_q_heads * w.head_dim * 2, g_flops),
                   "suffix": ((kv_tokens - plen - g_tokens) * bpt + q_bytes,
                              4.0 * w.num_q_heads * w.head_dim * suffix_visible)}
        phases = {"us_per_step": round(ms_sep * 1e3, 3)}
        for kind in ("prefix", "level1", "suffix", "merge"):
            tot_ms, cnt = prof_sep[kind]
            if not cnt:
                continue
            sec = tot_ms * 1e-3 / cnt
            rec = {"avg_us": round(sec * 1e6, 3)}
            if kind in ph_work:
                nbytes, nflops = ph_work[kind]
                rec.update({"bytes": int(nbytes), "gbs": round(nbytes / sec / 1e9, 1),
                            "hbm_frac": round(nbytes / sec / 1e9 / HBM_PEAK_GBS, 4),
                            "tflops": round(nflops / sec / 1e12, 2),
                            "mfma_frac": round(nflops / sec / 1e12 / BF16_PEAK_TFLOPS, 4)})
            phases[kind] = rec
        extra["separate_phases"] = phases

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(b, kv_bytes)

    gbs = kv_bytes / (ms * 1e-3) / 1e9
    props = torch.cuda.get_device_properties(dev)
    device = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
              "compute_units": props.multi_processor_count, "memory_gib": round(props.total_memory / 2**30, 1),
              "hip": torch.version.hip}
    line = {
        "metric": "cascade attn us/step + effective KV GB/s (N=64,P=4096,S=128), % of HBM roofline",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 3),
        "us_per_step_events": dist,
        "hbm_frac_step": round(gbs / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "device": device,
        "config": {"workload": args.workload, "num_reqs": w.num_reqs, "prefix": w.prefix,
                   "suffix": list(w.suffix), "q_len": list(w.q_len), "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "page_size": w.page_size,
                   "kv_dtype": w.kv_dtype,
                   "mode": args.mode, "use_cascade": int(casc), "common_prefix_len": plen,
                   "kv_bytes_per_step": kv_bytes, "rotating_copies": rotate},
        "roofline": roof,
        "kernels": kern,
        "us_per_step_with_kernel_events": round(ms_events * 1e3, 3),
        "warm_us_per_step": None if ms_warm is None else round(ms_warm * 1e3, 3),
        "plan": {k: info[k] for k in ("prefix_splits", "prefix_row_tile", "num_level1_groups", "level1_splits",
                                       "suffix_chunks", "suffix_chunk_tokens", "suffix_kernel", "num_partial_slots",
                                       "workspace_bytes")},
        **extra,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
