#!/usr/bin/env python3
"""Benchmark: ragged paged-KV attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload (the headline line): decode, batch 128 x q_len 1 x kv_len
1024, 8 qo / 1 kv heads, D 128, fp16, 64 contiguous pages per sequence (the
flashinfer issue #323 repro shape).  A step is one forward call (one launch of
the narrow-tile kernel, split pieces merged inside it) over the whole batch, with the plan built once
beforehand (as begin_forward is in the pages) and its build time reported
separately.  Eight copies of the KV cache are rotated so consecutive steps do
not hit in the 256 MB last-level cache.

value = KV GB/s = unique KV bytes of valid tokens / step time.
roofline = the decode kernel's (attn_narrow_kernel) algorithmic bytes per
launch (KV + Q + O + LSE + page table) / its average duration from HIP events
stamped by each dispatch on the launch stream, against 8 TB/s HBM.
cpu_baseline = the fp64 oracle on a bounded sample of the same batch.
prefill = a secondary measurement on the long-prompt part of the mixed
workload (4 causal prompts x 8192, 64 qo / 8 kv heads, bf16): TFLOP/s and
fraction of the 2.5 PFLOP/s dense bf16/fp16 MFMA peak.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0
METRIC = "attention TFLOP/s (prefill) + KV GB/s (decode), % roofline, 1 MI355X"


KERNEL_SRC = os.path.join(ROOT, "paged_kv_attention_ragged_amd", "csrc", "rpa_kernels.hip")
COUNTERS = os.path.join(ROOT, "profiles", "attn_narrow_kernel_decode_b128_kv1024_counters.txt")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    import hashlib
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def recorded_traffic():
    """HBM bytes per launch of the decode kernel on this workload, from the
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary in profiles/, or None when that
    summary is missing or was taken on a different kernel source."""
    try:
        kv = {}
        with open(COUNTERS) as f:
            for line in f:
                if ":" in line:
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256") != kernel_source_hash():
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def calibrate_copy():
    """A plain device-to-device copy of 256 MiB, three times: the reference the
    FETCH_SIZE / WRITE_SIZE counters are scaled against."""
    import torch
    n = 256 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copy calibration: 3 x %d bytes" % n)


def algorithmic(b, info):
    """Algorithmic work of one forward over batch b: visible-pair flops and bytes."""
    elt = 2
    D, H, Hk = b.head_dim, b.num_qo_heads, b.num_kv_heads
    flops = 4.0 * D * info["visible_pairs"]
    kv_bytes = float(info["kv_tokens"]) * Hk * D * 2 * elt  # unique: pages are private here
    q_bytes = float(b.total_q) * H * D * elt
    o_bytes = q_bytes
    lse_bytes = float(b.total_q) * H * 4
    pt_bytes = 4.0 * (len(b.kv_page_indices) + 2 * (b.batch + 1) + b.batch)
    return flops, kv_bytes, kv_bytes + q_bytes + o_bytes + lse_bytes + pt_bytes


def time_steps(plan, q, kvs, o, lse, steps, warmup):
    import torch
    for i in range(warmup):
        plan.run(q, kvs[i % len(kvs)], out=o, lse=lse, return_lse=True)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(st)
    for i in range(steps):
        plan.run(q, kvs[i % len(kvs)], out=o, lse=lse, return_lse=True)
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def kernel_times(plan, q, kvs, o, lse, steps):
    import torch
    import paged_kv_attention_ragged_amd as rpa
    torch.cuda.synchronize()
    rpa.prof_start()
    for i in range(steps):
        plan.run(q, kvs[i % len(kvs)], out=o, lse=lse, return_lse=True)
    torch.cuda.synchronize()
    return rpa.prof_stop()


def cpu_baseline(b, target_s=10.0):
    """The oracle (as is) on the first n sequences of the batch, with n sized
    from a short trial so the run takes about `target_s`; rate scaled to KV GB/s."""
    import oracle
    import workloads as W
    threads = len(os.sched_getaffinity(0))
    q_host = oracle._u16(b.q)
    kv_host = oracle._u16(b.kv_cache)

    def sample(n):
        sub = W.Batch(b.name, b.qo_indptr[:n + 1].copy(), b.kv_page_indptr[:n + 1].copy(),
                      b.kv_page_indices[:b.kv_page_indptr[n]].copy(), b.kv_last_page_len[:n].copy(),
                      None, None, b.num_qo_heads, b.num_kv_heads, b.head_dim, b.dtype)
        kw = sub.oracle_kwargs()
        kw["q"] = q_host[:b.qo_indptr[n]]
        kw["kv_cache"] = kv_host
        t0 = time.perf_counter()
        oracle.run(**kw, nthreads=threads)
        return sub, time.perf_counter() - t0

    n = min(b.batch, 2)
    sub, dt = sample(n)
    if n < b.batch:
        n = min(b.batch, max(n, int(n * target_s / max(dt, 1e-3))))
        sub, dt = sample(n)
    reps = 1
    while dt * reps < 0.3 * target_s and reps < 64:  # the whole batch is quick: repeat it
        _, t = sample(n)
        dt = (dt * reps + t) / (reps + 1)
        reps += 1
    kv_bytes = float(sub.kv_lens.sum()) * b.num_kv_heads * b.head_dim * 2 * 2
    return {"value": kv_bytes / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "first %d of %d sequences (%d query rows x %d heads, all their keys), mean of %d runs, "
                      "%.3f s each" % (n, b.batch, sub.total_q, b.num_qo_heads, reps, dt)}


def bench_decode(args):
    import torch
    import numpy as np
    import paged_kv_attention_ragged_amd as rpa
    import workloads as W
    b = W.decode_b128_kv1024(device="cuda")
    idx = torch.from_numpy(b.kv_page_indices).cuda()
    kvs = [b.kv_cache] + [torch.randn_like(b.kv_cache, dtype=torch.float32).to(b.kv_cache.dtype)
                          for _ in range(7)]
    t0 = time.perf_counter()
    plan = rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=b.num_qo_heads,
                    num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, dtype=b.dtype)
    plan_ms = (time.perf_counter() - t0) * 1e3
    plan.bind(idx, num_pages=b.num_pages)
    info = plan.info
    o = torch.empty_like(b.q)
    lse = torch.empty((b.total_q, b.num_qo_heads), dtype=torch.float32, device="cuda")
    ms, wall = time_steps(plan, b.q, kvs, o, lse, args.steps, args.warmup)
    kt = kernel_times(plan, b.q, kvs, o, lse, args.steps)
    flops, kv_bytes, alg_bytes = algorithmic(b, info)
    n_attn, ms_attn = kt["narrow"]  # every tile of a q_len = 1, G = 8 batch is narrow
    n_wide, _ = kt["wide"]
    assert n_wide == 0 and n_attn == args.steps
    attn_avg = ms_attn / max(n_attn, 1)
    achieved = alg_bytes / (attn_avg * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": kv_bytes / (ms * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": b.dtype, "data": "synthetic",
        "config": {"workload": "decode_b128_kv1024", "batch": b.batch, "q_len": 1, "kv_len": 1024,
                   "num_qo_heads": b.num_qo_heads, "num_kv_heads": b.num_kv_heads, "head_dim": b.head_dim,
                   "page_size": 16, "kv_cache_copies_rotated": len(kvs)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": recorded_traffic(),
                     "kernel": "attn_narrow_kernel", "avg_ms": attn_avg,
                     "algorithmic_bytes_per_launch": alg_bytes},
        "tflops": flops / (ms * 1e-3) / 1e12,
        "kernels": {"narrow_avg_ms": attn_avg, "launches_per_step": (n_attn + n_wide) / args.steps},
        "plan": {"host_ms": plan_ms, "tiles": info["num_tiles"], "split_groups": info["num_split_groups"],
                 "max_splits": info["max_splits"]},
        "wall_s_timed": wall,
    }
    plan.close()
    return res, b


def bench_prefill(args):
    """Long causal prompts: 4 x 8192, 64 qo / 8 kv heads, bf16."""
    import torch
    import paged_kv_attention_ragged_amd as rpa
    import workloads as W
    b = W.mixed_long_batch(part="prompts", device="cuda")
    idx = torch.from_numpy(b.kv_page_indices).cuda()
    plan = rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=b.num_qo_heads,
                    num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, dtype=b.dtype)
    plan.bind(idx, num_pages=b.num_pages)
    info = plan.info
    o = torch.empty_like(b.q)
    lse = torch.empty((b.total_q, b.num_qo_heads), dtype=torch.float32, device="cuda")
    steps = max(3, args.steps // 10)
    ms, _ = time_steps(plan, b.q, [b.kv_cache], o, lse, steps, 2)
    kt = kernel_times(plan, b.q, [b.kv_cache], o, lse, steps)
    flops, kv_bytes, alg_bytes = algorithmic(b, info)
    n_attn, ms_attn = kt["wide"]  # causal prompts: every tile is wide
    attn_avg = ms_attn / max(n_attn, 1)
    tf = flops / (attn_avg * 1e-3) / 1e12
    plan.close()
    return {"workload": "mixed_long_prompts_4x8192", "ms_per_step": ms, "tflops": flops / (ms * 1e-3) / 1e12,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / MFMA_PEAK_TFLOPS, "kernel": "attn_wide_kernel", "avg_ms": attn_avg,
                         "algorithmic_flops_per_launch": flops},
            "dtype": b.dtype, "tiles": info["num_tiles"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 256 MiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (see DESIGN.md for how it "
              "would shard); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import paged_kv_attention_ragged_amd as rpa
    rpa.load()
    if args.calibrate_copy:
        calibrate_copy()
    log("decode_b128_kv1024: %d warmup + %d timed steps" % (args.warmup, args.steps))
    res, b = bench_decode(args)
    if not args.no_prefill:
        log("long prefill 4x8192")
        res["prefill"] = bench_prefill(args)
    if not args.no_cpu_baseline:
        log("oracle baseline on host cores")
        res["cpu_baseline"] = cpu_baseline(b)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
