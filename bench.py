#!/usr/bin/env python3
"""Benchmark: ragged paged-KV attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline line: decode, batch 128 x q_len 1 x kv_len 1024, 8 qo / 1 kv heads, D
128, fp16, 64 contiguous pages per sequence (the flashinfer issue #323 repro
shape).  A step is one forward call (one launch of the narrow-tile kernel, split
pieces merged inside it) over the whole batch, with the plan built once
beforehand (as begin_forward is in the pages) and its build time reported
separately.  Eight copies of the KV cache are rotated so consecutive steps do
not hit in the 256 MB last-level cache; a cache-resident ("hot") time with one
copy is reported beside it.

value = KV GB/s = unique KV bytes of valid tokens / step time.
roofline = the decode kernel's algorithmic bytes per launch (KV + Q + O + LSE +
page table) / its average duration from HIP events stamped by each dispatch on
the launch stream, against 8 TB/s HBM; also against the HBM read rate measured
on this machine (floors.hbm_stream_gbs).  traffic = HBM bytes per launch from the
rocprofv3 FETCH_SIZE / WRITE_SIZE summary in profiles/, while it was taken on
the current kernel source.
floors = measured on this machine in this run: an empty launch, a plain HBM read
stream, the decode kernel's paged gather alone (its page table, no arithmetic;
on the headline plan's grid of 128 workgroups and on a split grid of 512), and
dense bf16 MFMA throughput.
prefill = the long prompts of the mixed workload (4 causal prompts x 8192, 64 qo /
8 kv heads, bf16) against the 2.5 PFLOP/s dense bf16 MFMA peak.
secondary = the pages' other workloads, each with median / mean per call, kernel
time and a roofline entry: ragged vs padded short prompts; the shared-prefix
suffix prefill and a decode step (direct and as a cascade); a long shared
prefix; the decode loop eager vs graph; the VALU decode kernel; the mixed long
batch's decode rows and whole batch; a batch-size sweep at 8192 total tokens.
cpu_baseline = the fp64 oracle on a bounded sample of the headline batch, plus a
labelled row sample of the mixed long batch.
"""
import argparse
import ctypes
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0
METRIC = "attention TFLOP/s (prefill) + KV GB/s (decode), % roofline, 1 MI355X"

KERNEL_SRC = os.path.join(ROOT, "paged_kv_attention_ragged_amd", "csrc", "rpa_kernels.hip")
COUNTERS = os.path.join(ROOT, "profiles", "attn_narrow_kernel_decode_b128_kv1024_counters.txt")
FLOORS_LIB = os.path.join(ROOT, "paged_kv_attention_ragged_amd", "librpa_floors.so")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    import hashlib
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def recorded_traffic():
    """HBM bytes per launch of the decode kernel on the headline workload, from the
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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


# ----------------------------------------------------------------------------------------------
# Algorithmic work and rooflines
# ----------------------------------------------------------------------------------------------

def algorithmic(b, info, unique_kv_tokens=None):
    """Algorithmic work of one forward over batch b: (flops, KV bytes, all bytes).
    Flops: 4 D per visible (query, key, qo head) pair.  Bytes: K/V of valid tokens,
    each physical slot once (unique_kv_tokens when pages are shared, else the sum of
    kv_len), + Q + O + LSE + page table."""
    elt = 2
    D, H, Hk = b.head_dim, b.num_qo_heads, b.num_kv_heads
    flops = 4.0 * D * info["visible_pairs"]
    tokens = float(info["kv_tokens"] if unique_kv_tokens is None else unique_kv_tokens)
    kv_bytes = tokens * Hk * D * 2 * elt
    q_bytes = float(b.total_q) * H * D * elt
    lse_bytes = float(b.total_q) * H * 4
    pt_bytes = 4.0 * (len(b.kv_page_indices) + 2 * (b.batch + 1) + b.batch)
    return flops, kv_bytes, kv_bytes + 2 * q_bytes + lse_bytes + pt_bytes


def roofline(flops, nbytes, ms, floors=None, bound=None, kernel=None):
    """Roofline entry of one launch (or call) of `ms` milliseconds doing `flops` and
    moving `nbytes` algorithmic bytes.  bound: 'hbm', 'mfma', or None for whichever
    ideal time is longer (a max-bound mixed call)."""
    t = ms * 1e-3
    if bound is None:
        bound = "mfma" if flops / (MFMA_PEAK_TFLOPS * 1e12) > nbytes / (HBM_PEAK_GBS * 1e9) else "hbm"
    if bound == "hbm":
        ach, peak, unit = nbytes / t / 1e9, HBM_PEAK_GBS, "GB/s"
        meas = floors.get("hbm_stream_gbs") if floors else None
    else:
        ach, peak, unit = flops / t / 1e12, MFMA_PEAK_TFLOPS, "TFLOP/s"
        meas = floors.get("mfma_tflops") if floors else None
    r = {"bound": bound, "achieved": ach, "peak": peak, "unit": unit, "frac": ach / peak,
         "measured_peak": meas, "frac_of_measured_peak": ach / meas if meas else None, "ms": ms}
    if kernel:
        r["kernel"] = kernel
    return r


def attach_measured_peaks(obj, floors):
    """Fill measured_peak / frac_of_measured_peak of every roofline entry in a result."""
    if isinstance(obj, list):
        for x in obj:
            attach_measured_peaks(x, floors)
    elif isinstance(obj, dict):
        if "bound" in obj and "achieved" in obj and "measured_peak" in obj:
            meas = floors.get("hbm_stream_gbs" if obj["bound"] == "hbm" else "mfma_tflops")
            obj["measured_peak"] = meas
            obj["frac_of_measured_peak"] = obj["achieved"] / meas if meas else None
        for v in obj.values():
            attach_measured_peaks(v, floors)


# ----------------------------------------------------------------------------------------------
# Timing helpers
# ----------------------------------------------------------------------------------------------

def bound_plan(b, narrow="mfma", kv_shared=False, **kw):
    """A plan for batch b bound to its page table (kw: further Plan arguments)."""
    import torch
    import paged_kv_attention_ragged_amd as rpa
    p = rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=b.num_qo_heads,
                 num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, dtype=b.dtype, causal=b.causal,
                 narrow_kernel=narrow, kv_shared=kv_shared, **kw)
    p.bind(torch.from_numpy(b.kv_page_indices).cuda(), num_pages=b.kv_cache.shape[0])
    return p


def per_call_ms(fn, steps, warmup):
    """Per-call times of fn() (GPU work on the current stream) from an event pair
    around each call, plus the mean over a loop bracketed by one event pair."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, c in ev:
        a.record()
        fn()
        c.record()
    torch.cuda.synchronize()
    calls = [a.elapsed_time(c) for a, c in ev]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return {"median_ms": float(np.median(calls)), "mean_ms": e0.elapsed_time(e1) / steps,
            "min_ms": float(np.min(calls))}


def kernel_ms(fn, steps):
    """Mean kernel time per call of fn() from the library's dispatch-stamped events:
    (total, per kind {'wide': ms, 'narrow': ms}, launches per call)."""
    import torch
    import paged_kv_attention_ragged_amd as rpa
    torch.cuda.synchronize()
    rpa.prof_start()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    kt = rpa.prof_stop()
    per = {k: (ms / steps if n else 0.0) for k, (n, ms) in kt.items()}
    return sum(per.values()), per, sum(n for n, _ in kt.values()) / steps


def measure(b, steps, warmup=3, rotate=1, unique_kv_tokens=None, floors=None, **plan_kw):
    """One workload: per-call and kernel times, algorithmic work and its roofline.
    rotate > 1 cycles through copies of the KV cache (misses in the last-level cache)."""
    import torch
    p = bound_plan(b, **plan_kw)
    q, kv0 = b.q.cuda(), b.kv_cache.cuda()
    kvs = [kv0] + [kv0.clone() for _ in range(rotate - 1)]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    it = iter(range(1 << 40))
    fn = lambda: p.run(q, kvs[next(it) % rotate], out=o, lse=lse, return_lse=True)
    t = per_call_ms(fn, steps, warmup)
    kms, per_kind, launches = kernel_ms(fn, steps)
    p.check()
    info = p.info
    p.close()
    flops, kv_bytes, nbytes = algorithmic(b, info, unique_kv_tokens)
    t.update({"kernel_ms": kms, "launches_per_call": launches, "tflops": flops / (t["mean_ms"] * 1e-3) / 1e12,
              "kv_gbs": kv_bytes / (t["mean_ms"] * 1e-3) / 1e9,
              "algorithmic": {"flops": flops, "kv_bytes": kv_bytes, "bytes": nbytes},
              "roofline": roofline(flops, nbytes, kms, floors)})
    if per_kind["wide"] and per_kind["narrow"]:
        t["kernel_ms_by_kind"] = per_kind
    return t


# ----------------------------------------------------------------------------------------------
# Floors measured on this machine
# ----------------------------------------------------------------------------------------------

def bench_floors(steps=20):
    """Empty launch, plain HBM read, the decode batch's paged gather alone with the
    page table of the decode kernel on two grids (the headline plan's 128 workgroups
    of 1024 keys, and a split grid of 128 x 4 pieces of 256 keys), and dense bf16
    MFMA throughput."""
    import torch
    import workloads as W
    lib = ctypes.CDLL(FLOORS_LIB)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.rpa_floor_empty.argtypes = [i32, P]
    lib.rpa_floor_stream.argtypes = [P, i64, P, i32, P]
    lib.rpa_floor_gather.argtypes = [P, P, i32, i32, i32, i32, i32, P, P]
    lib.rpa_floor_mfma.argtypes = [P, i32, i32, P]

    def ok(rc):
        if rc != 0:
            raise RuntimeError("floor kernel launch failed: hipError %d" % rc)

    st = lambda: torch.cuda.current_stream().cuda_stream
    out = {}
    # empty launch, the decode grid
    # (a per-call event pair around a short kernel also times the host's submission of
    # it; back-to-back calls of a kernel longer than that submission time the GPU alone)
    t = per_call_ms(lambda: ok(lib.rpa_floor_empty(512, st())), steps * 5, 5)
    out["empty_launch_per_call_us"] = t["median_ms"] * 1e3
    out["empty_launch_back_to_back_us"] = t["mean_ms"] * 1e3
    # plain read of 2 GiB (> the last-level cache), 4 workgroups per CU, each its own share
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.empty(1024 * 256, dtype=torch.int32, device="cuda")
    t = per_call_ms(lambda: ok(lib.rpa_floor_stream(buf.data_ptr(), nbytes, sink.data_ptr(), 1024, st())), steps, 3)
    out["hbm_stream_gbs"] = nbytes / (t["mean_ms"] * 1e-3) / 1e9
    del buf
    # the decode batch's gather: K and V of 128 x 1024 tokens, 8 rotated cache copies
    b = W.decode_b128_kv1024(device="cuda")
    kvs = [b.kv_cache] + [b.kv_cache.clone() for _ in range(7)]
    idx = torch.from_numpy(b.kv_page_indices).cuda()
    gsink = torch.empty(512 * 256, dtype=torch.int32, device="cuda")
    it = iter(range(1 << 40))
    gb = 128 * 1024 * 128 * 2 * 2.0
    # split grid: 512 workgroups of 256 keys (every CU busy)
    t = per_call_ms(lambda: ok(lib.rpa_floor_gather(kvs[next(it) % 8].data_ptr(), idx.data_ptr(), 128, 64, 4, 1, 1,
                                                    gsink.data_ptr(), st())), steps * 5, 5)
    out["decode_gather_us"] = t["mean_ms"] * 1e3
    out["decode_gather_per_call_us"] = t["median_ms"] * 1e3
    out["decode_gather_gbs"] = gb / (t["mean_ms"] * 1e-3) / 1e9
    # the headline plan's grid: 128 workgroups, one per sequence, each 4 runs of 256 keys
    t = per_call_ms(lambda: ok(lib.rpa_floor_gather(kvs[next(it) % 8].data_ptr(), idx.data_ptr(), 128, 64, 1, 4, 1,
                                                    gsink.data_ptr(), st())), steps * 5, 5)
    out["decode_gather_unsplit_us"] = t["mean_ms"] * 1e3
    out["decode_gather_unsplit_gbs"] = gb / (t["mean_ms"] * 1e-3) / 1e9
    del kvs, b
    # dense MFMA: 1024 workgroups x 4 waves x 4 chains x iters 32x32x16 bf16 products
    msink = torch.empty(1024 * 256, dtype=torch.float32, device="cuda")
    iters = 4096
    t = per_call_ms(lambda: ok(lib.rpa_floor_mfma(msink.data_ptr(), 1024, iters, st())), 10, 2)
    flops = 1024 * 4 * 4 * iters * 32768.0
    out["mfma_tflops"] = flops / (t["mean_ms"] * 1e-3) / 1e12
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------------------------
# Headline: decode 128 x 1024
# ----------------------------------------------------------------------------------------------

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


def bench_decode(args, floors):
    import torch
    import paged_kv_attention_ragged_amd as rpa
    import workloads as W
    b = W.decode_b128_kv1024(device="cuda")
    idx = torch.from_numpy(b.kv_page_indices).cuda()
    kvs = [b.kv_cache] + [torch.randn_like(b.kv_cache, dtype=torch.float32).to(b.kv_cache.dtype)
                          for _ in range(7)]
    t0 = time.perf_counter()
    plan = rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=b.num_qo_heads,
                    num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, dtype=b.dtype,
                    narrow_kernel=args.narrow_kernel)
    plan_ms = (time.perf_counter() - t0) * 1e3
    plan.bind(idx, num_pages=b.num_pages)
    info = plan.info
    o = torch.empty_like(b.q)
    lse = torch.empty((b.total_q, b.num_qo_heads), dtype=torch.float32, device="cuda")
    ms, wall = time_steps(plan, b.q, kvs, o, lse, args.steps, args.warmup)
    it = iter(range(1 << 40))
    fn = lambda: plan.run(b.q, kvs[next(it) % 8], out=o, lse=lse, return_lse=True)
    per_call = per_call_ms(fn, args.steps, 2)
    attn_avg, per_kind, launches = kernel_ms(fn, args.steps)
    assert per_kind["wide"] == 0 and launches == 1  # every tile of a q_len = 1, G = 8 batch is narrow
    hot = per_call_ms(lambda: plan.run(b.q, kvs[0], out=o, lse=lse, return_lse=True), args.steps, 2)
    plan.check()
    flops, kv_bytes, alg_bytes = algorithmic(b, info)
    achieved = alg_bytes / (attn_avg * 1e-3) / 1e9
    meas = floors.get("hbm_stream_gbs")
    res = {
        "metric": METRIC, "value": kv_bytes / (ms * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": b.dtype, "data": "synthetic",
        "config": {"workload": "decode_b128_kv1024", "batch": b.batch, "q_len": 1, "kv_len": 1024,
                   "num_qo_heads": b.num_qo_heads, "num_kv_heads": b.num_kv_heads, "head_dim": b.head_dim,
                   "page_size": 16, "kv_cache_copies_rotated": len(kvs)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": recorded_traffic(),
                     "kernel": "attn_narrow_kernel" if args.narrow_kernel == "mfma" else "attn_narrow_valu_kernel",
                     "avg_ms": attn_avg, "algorithmic_bytes_per_launch": alg_bytes,
                     "frac_per_step": alg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "measured_peak": meas, "frac_of_measured_peak": achieved / meas if meas else None},
        "tflops": flops / (ms * 1e-3) / 1e12,
        "per_call": {"median_ms": per_call["median_ms"], "mean_ms": per_call["mean_ms"],
                     "hot_median_ms": hot["median_ms"],
                     "hot_note": "one cache copy, resident in the last-level cache"},
        "plan": {"host_ms": plan_ms, "tiles": info["num_tiles"], "split_groups": info["num_split_groups"],
                 "max_splits": info["max_splits"]},
        "wall_s_timed": wall,
    }
    plan.close()
    return res, b


def walked_keys(b):
    """Keys the plan's tiles walk, summed over tiles (a host-only plan)."""
    import paged_kv_attention_ragged_amd as rpa
    p = rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=b.num_qo_heads,
                 num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, dtype=b.dtype, causal=b.causal)
    t = p.tiles()
    p.close()
    return float((t[:, 7].astype(np.int64) - t[:, 6]).sum())


def bench_prefill(args, floors):
    """Long causal prompts: 4 x 8192, 64 qo / 8 kv heads, bf16 (every tile wide)."""
    import workloads as W
    b = W.mixed_long_batch(part="prompts", device="cuda")
    r = measure(b, steps=max(3, args.steps // 10), warmup=2, floors=floors)
    rf = roofline(r["algorithmic"]["flops"], r["algorithmic"]["bytes"], r["kernel_ms"], floors, bound="mfma",
                  kernel="attn_wide_kernel")
    rf["algorithmic_flops_per_launch"] = r["algorithmic"]["flops"]
    # A/B: the same prompts with the causal tail skip switched off (tiles walk to kv_len
    # and mask); same results, so the time difference is what the skip saves
    if args.no_tail_skip_ab:
        return {"workload": "mixed_long_prompts_4x8192", "ms_per_step": r["mean_ms"], "median_ms": r["median_ms"],
                "tflops": r["tflops"], "roofline": rf, "dtype": b.dtype}
    log("long prompts without the tail skip")
    keys_on = walked_keys(b)
    os.environ["RPA_DISABLE_TAIL_SKIP"] = "1"
    try:
        ns = measure(b, steps=max(3, args.steps // 10), warmup=1, floors=floors)
        keys_off = walked_keys(b)
    finally:
        del os.environ["RPA_DISABLE_TAIL_SKIP"]
    ab = {"skip_kernel_ms": r["kernel_ms"], "no_skip_kernel_ms": ns["kernel_ms"],
          "no_skip_over_skip": ns["kernel_ms"] / r["kernel_ms"], "keys_walked_no_skip_over_skip": keys_off / keys_on}
    return {"workload": "mixed_long_prompts_4x8192", "ms_per_step": r["mean_ms"], "median_ms": r["median_ms"],
            "tflops": r["tflops"], "roofline": rf, "dtype": b.dtype, "tail_skip_ab": ab}


# ----------------------------------------------------------------------------------------------
# The other workloads
# ----------------------------------------------------------------------------------------------

def shared_unique_tokens(b):
    """Distinct physical token slots a shared-prefix batch reads: the shared full pages
    once, then each request's own tokens."""
    n_sh = len(b.extra["shared"]) if hasattr(b, "extra") else 0
    return int(n_sh * 16 + (np.asarray(b.kv_lens) - n_sh * 16).sum())


def bench_secondary(args, floors):
    import torch
    import paged_kv_attention_ragged_amd as rpa
    import workloads as W
    steps = max(5, args.steps // 10)
    out = {}

    def cascade(b, prefix):
        sh, pr = W.cascade_view(b, prefix=prefix, poison=False)
        pa, pb = bound_plan(sh), bound_plan(pr)
        q, kv = b.q.cuda(), sh.kv_cache.cuda()
        oa, ob = torch.empty_like(q), torch.empty_like(q)
        la = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
        lb = torch.empty_like(la)

        def step():
            pa.run(q, kv, out=oa, lse=la, return_lse=True)
            pb.run(q, kv, out=ob, lse=lb, return_lse=True)
            rpa.merge_states(oa, la, ob, lb, out=oa, lse_out=la)
        t = per_call_ms(step, steps, 3)
        pa.close()
        pb.close()
        return t

    # short ragged prompts (lengths U{1..200}) vs the same prompts padded to 200
    log("short prompts: ragged vs padded")
    sp, spp = W.short_prompt_prefill(), W.short_prompt_prefill(padded=True)
    r, p = measure(sp, steps, floors=floors), measure(spp, steps, floors=floors)
    out["short_prompts"] = {"ragged": r, "padded": p, "time_ratio": r["mean_ms"] / p["mean_ms"],
                            "kernel_time_ratio": r["kernel_ms"] / p["kernel_ms"],
                            "flops_ratio": r["algorithmic"]["flops"] / p["algorithmic"]["flops"],
                            "bytes_ratio": r["algorithmic"]["bytes"] / p["algorithmic"]["bytes"]}
    # shared prefix (256 requests x 200 shared + 30 own tokens), then one decode step
    log("shared prefix: direct vs cascade")
    b = W.shared_prefix_suffix()
    pre = measure(b, steps, unique_kv_tokens=shared_unique_tokens(b), floors=floors)
    pre["cascade_median_ms"] = cascade(b, 200)["median_ms"]
    d = W.decode_step(b, 1)
    d.extra = b.extra
    n_sh = len(b.extra["shared"])
    # the library's plan for it: the shared prefix declared, decode rows grouped over it
    dec = measure(d, steps, rotate=6, unique_kv_tokens=shared_unique_tokens(d), floors=floors, kv_shared=True,
                  shared_pages=n_sh)
    logical = float(d.kv_lens.sum()) * d.num_kv_heads * d.head_dim * 4
    dec["plan"] = "shared prefix declared (%d pages): decode rows grouped 4 per tile" % n_sh
    dec["logical_kv_bytes"] = logical
    dec["logical_kv_gbs"] = logical / (dec["kernel_ms"] * 1e-3) / 1e9
    direct = measure(d, steps, rotate=6, unique_kv_tokens=shared_unique_tokens(d), floors=floors, kv_shared=True)
    dec["direct"] = {"median_ms": direct["median_ms"], "kernel_ms": direct["kernel_ms"],
                     "roofline_frac": direct["roofline"]["frac"]}
    dec["cascade_median_ms"] = cascade(d, 200)["median_ms"]
    dec["direct_streamed_kv_median_ms"] = measure(d, steps, rotate=6, floors=floors)["median_ms"]
    dec["direct_valu_median_ms"] = measure(d, steps, rotate=6, floors=floors, narrow="valu",
                                           kv_shared=True)["median_ms"]
    out["shared_prefix"] = {"suffix_prefill": pre, "decode_step": dec}
    # a long shared prefix (4096 tokens) under the same 256 requests: one decode step
    log("long shared prefix decode: direct, grouped, cascade")
    lbase = W.shared_prefix_suffix(prefix=4096, decode_steps=1)
    lb = W.decode_step(lbase, 1)
    lb.extra = lbase.extra
    ld = measure(lb, steps, kv_shared=True, floors=floors)
    lg = measure(lb, steps, kv_shared=True, floors=floors, unique_kv_tokens=shared_unique_tokens(lb),
                 shared_pages=len(lbase.extra["shared"]))
    out["long_prefix_4096"] = {"decode_step_direct_median_ms": ld["median_ms"],
                               "decode_step_grouped_median_ms": lg["median_ms"],
                               "decode_step_grouped_roofline": lg["roofline"],
                               "decode_step_cascade_median_ms": cascade(lb, 4096)["median_ms"],
                               "logical_kv_gb": float(lb.kv_lens.sum()) * lb.num_kv_heads * lb.head_dim * 4 / 1e9}
    del lb, lbase
    log("decode loop: eager vs graph")
    out["decode_loop"] = bench_decode_loop()
    log("decode on the VALU kernel")
    db = W.decode_b128_kv1024(device="cuda")
    out["decode_b128_kv1024_valu_vs_mfma"] = {
        "valu": measure(db, steps, rotate=8, narrow="valu", floors=floors),
        "mfma_median_ms": measure(db, steps, rotate=8, floors=floors)["median_ms"]}
    del db
    log("mixed long batch: decode rows, whole batch")
    for part in ("decode", "all"):
        mb = W.mixed_long_batch(part=part, device="cuda")
        ent = measure(mb, steps, floors=floors)
        if part == "decode":
            ent["valu_median_ms"] = measure(mb, steps, narrow="valu", floors=floors)["median_ms"]
        out["mixed_long_" + part] = ent
        del mb
        torch.cuda.empty_cache()
    log("batch-size sweep at 8192 total tokens")
    out["sweep"] = bench_sweep(batches=(1, 8, 64, 256), steps=5, floors=floors, quiet=True)
    return out


def bench_decode_loop(steps=50):
    """The shared-prefix batch's decode loop (256 requests, one token per step after
    200 + 30 prompt tokens): per step, append the new token's K/V and attend.
    Eager: plan + bind + append + run per step.  Graph: the captured [upload,
    append, run] replayed after an in-place plan update.  Both synchronise every
    step, as a decode loop must; inputs of all steps are prepared beforehand."""
    import torch
    import paged_kv_attention_ragged_amd as rpa
    import workloads as W
    base = W.shared_prefix_suffix()
    n_req, H, Hk, D = base.batch, base.num_qo_heads, base.num_kv_heads, base.head_dim
    kv0 = base.kv_cache.cuda()
    ps = base.page_size
    prepared = []
    for st in range(1, steps + 1):
        d = W.decode_step(base, st)
        rows = []
        for s in range(n_req):
            pos = int(d.kv_lens[s]) - 1
            rows.append(base.kv_cache[d.kv_page_indices[d.kv_page_indptr[s] + pos // ps], :, pos % ps])
        prepared.append((d, torch.stack(rows).cuda(), d.q.cuda(),
                         [torch.from_numpy(a.astype(np.int32)).pin_memory()
                          for a in (d.kv_page_indptr, d.kv_page_indices, d.kv_last_page_len)]))
    cap = n_req * base.extra["pages_req"]
    q_buf = torch.empty(n_req, H, D, dtype=kv0.dtype, device="cuda")
    new_buf = torch.empty(n_req, 2, Hk, D, dtype=kv0.dtype, device="cuda")
    ip_buf = torch.zeros(n_req + 1, dtype=torch.int32, device="cuda")
    ix_buf = torch.zeros(cap, dtype=torch.int32, device="cuda")
    kl_buf = torch.zeros(n_req, dtype=torch.int32, device="cuda")
    ai_buf = torch.arange(n_req + 1, dtype=torch.int32, device="cuda")
    o_buf = torch.empty(n_req, H, D, dtype=kv0.dtype, device="cuda")
    l_buf = torch.empty(n_req, H, dtype=torch.float32, device="cuda")

    def load(i):
        d, new, q, (ip, ix, kl) = prepared[i]
        q_buf.copy_(q)
        new_buf.copy_(new)
        ip_buf.copy_(ip, non_blocking=True)
        ix_buf[:ix.numel()].copy_(ix, non_blocking=True)
        kl_buf.copy_(kl, non_blocking=True)
        return d

    # eager
    kv = kv0.clone()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        d = load(i)
        p = rpa.Plan(d.qo_indptr, d.kv_page_indptr, d.kv_last_page_len, num_qo_heads=H, num_kv_heads=Hk,
                     head_dim=D, dtype=d.dtype, kv_shared=True)
        p.bind(ix_buf, num_pages=kv.shape[0])
        rpa.append_kv(new_buf, kv, ai_buf, ip_buf, ix_buf, kl_buf)
        p.run(q_buf, kv, out=o_buf, lse=l_buf, return_lse=True)
        torch.cuda.synchronize()
        p.close()
    eager = (time.perf_counter() - t0) / steps * 1e3
    # graph
    kv = kv0.clone()
    d = load(0)
    plan = rpa.Plan(d.qo_indptr, d.kv_page_indptr, d.kv_last_page_len, num_qo_heads=H, num_kv_heads=Hk,
                    head_dim=D, dtype=d.dtype, kv_shared=True)
    plan.bind(ix_buf, num_pages=kv.shape[0])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.upload()
        rpa.append_kv(new_buf, kv, ai_buf, ip_buf, ix_buf, kl_buf)
        plan.run(q_buf, kv, out=o_buf, lse=l_buf, return_lse=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gpu_ms = []
    t0 = time.perf_counter()
    for i in range(steps):
        if i > 0:
            d = load(i)
            plan.update(d.qo_indptr, d.kv_page_indptr, d.kv_last_page_len)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        gpu_ms.append(e0.elapsed_time(e1))
    graph = (time.perf_counter() - t0) / steps * 1e3
    plan.check()
    plan.close()
    return {"steps": steps, "eager_step_ms": eager, "graph_step_ms": graph,
            "graph_replay_gpu_median_ms": float(np.median(gpu_ms))}


def bench_sweep(total_tokens=8192, batches=(1, 2, 4, 8, 16, 32, 64, 128, 256), steps=10, floors=None,
                quiet=False):
    """Batch-size sweep at constant total tokens (llama.cpp discussion #15958: batching
    prompts helps little unless they are very short): B causal prompts of
    total_tokens / B tokens each (32 qo / 8 kv heads, D 128, bf16), as one ragged
    call, against the same prompts run one call each."""
    import torch
    import workloads as W
    rows = []
    for B in batches:
        L = total_tokens // B
        b = W.make_batch("sweep_B%d" % B, [L] * B, [L] * B, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                         dtype="bf16", seed=4000 + B, permute=True, device="cuda")
        q, kv = b.q, b.kv_cache
        o = torch.empty_like(q)
        p = bound_plan(b)
        info = p.info
        one = W.Batch("one", np.array([0, L], np.int32), np.array([0, b.kv_page_indptr[1]], np.int32),
                      b.kv_page_indices[:b.kv_page_indptr[1]].copy(), b.kv_last_page_len[:1].copy(), q[:L], kv,
                      b.num_qo_heads, b.num_kv_heads, b.head_dim, b.dtype)
        p1 = bound_plan(one)
        # two interleaved rounds, the faster of each (the first timing of a run tends to
        # be slower: at B = 1 the two sides are the same call)
        bm, sm = [], []
        for _ in range(2):
            bm.append(per_call_ms(lambda: p.run(q, kv, out=o), steps, 5)["median_ms"])
            sm.append(per_call_ms(lambda: p1.run(q[:L], kv, out=o[:L]), steps, 5)["median_ms"])
        batched = {"median_ms": min(bm)}
        single = min(sm)
        kms = kernel_ms(lambda: p.run(q, kv, out=o), steps)[0]
        p.close()
        p1.close()
        flops, _, nbytes = algorithmic(b, info)
        r = {"sweep": "constant_total_tokens", "total_tokens": total_tokens, "batch": B, "prompt_len": L,
             "batched_median_ms": batched["median_ms"], "one_by_one_ms": single * B,
             "speedup": single * B / batched["median_ms"],
             "tflops_batched": flops / (batched["median_ms"] * 1e-3) / 1e12,
             "roofline": roofline(flops, nbytes, kms, floors)}
        if not quiet:
            print(json.dumps(r), flush=True)
        rows.append(r)
        del b, q, kv, o
        torch.cuda.empty_cache()
    return rows


# ----------------------------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on this machine's host cores
# ----------------------------------------------------------------------------------------------

def oracle_time(b, rows, threads, q_host, kv_host):
    import oracle
    kw = b.oracle_kwargs()
    kw["q"], kw["kv_cache"] = q_host, kv_host
    t0 = time.perf_counter()
    oracle.run(**kw, rows=rows, nthreads=threads)
    return time.perf_counter() - t0


def oracle_full(parts):
    """The oracle, once, over every row of the mixed long batch (C5), in parts that each
    fit a bounded run: part k is prompt k's 8192 rows (part 0 also the 256 decode rows),
    timed in chunks of 1024 rows with a line per chunk; the parts' seconds add up to the
    full timing.  Not part of the default run (about 29 minutes on 16 cores)."""
    import oracle
    import workloads as W
    b = W.mixed_long_batch()
    q_host, kv_host = oracle._u16(b.q), oracle._u16(b.kv_cache)
    threads = len(os.sched_getaffinity(0))
    model = next((l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name")), "?")
    for k in parts:
        a, e = int(b.qo_indptr[k]), int(b.qo_indptr[k + 1])
        rows = list(range(a, e)) + (list(range(int(b.qo_indptr[4]), b.total_q)) if k == 0 else [])
        total = 0.0
        for c in range(0, len(rows), 1024):
            chunk = rows[c:c + 1024]
            total += oracle_time(b, chunk, threads, q_host, kv_host)
            log("oracle part %d: rows %d..%d done, %.1f s so far" % (k, chunk[0], chunk[-1], total))
        flops = 4.0 * b.head_dim * b.num_qo_heads * visible_of_rows(b, rows)
        print(json.dumps({"oracle_full_part": k, "rows": len(rows), "seconds": total,
                          "fp64_gflops": flops / total / 1e9, "threads": threads, "cpu_model": model}), flush=True)


def visible_of_rows(b, rows):
    """Visible keys of each listed row (causal: its position + 1), summed."""
    seq = np.searchsorted(b.qo_indptr, np.asarray(rows), side="right") - 1
    kvl, ql = b.kv_lens[seq], b.q_lens[seq]
    pos = kvl - ql + (np.asarray(rows) - b.qo_indptr[seq])
    return int((pos + 1).sum()) if b.causal else int(kvl.sum())


def cpu_baseline(b, target_s=10.0):
    """The oracle (as is) on the first n sequences of the headline batch, n sized from
    a short trial so the run takes about `target_s`; rate in KV GB/s, with fp64
    GFLOP/s and rows/s; then a labelled row sample of the mixed long batch."""
    import oracle
    import workloads as W
    threads = len(os.sched_getaffinity(0))
    q_host, kv_host = oracle._u16(b.q), oracle._u16(b.kv_cache)

    def sample(n):
        sub = W.Batch(b.name, b.qo_indptr[:n + 1].copy(), b.kv_page_indptr[:n + 1].copy(),
                      b.kv_page_indices[:b.kv_page_indptr[n]].copy(), b.kv_last_page_len[:n].copy(),
                      None, None, b.num_qo_heads, b.num_kv_heads, b.head_dim, b.dtype)
        return sub, oracle_time(sub, None, threads, q_host[:b.qo_indptr[n]], kv_host)

    n = min(b.batch, 2)
    sub, dt = sample(n)
    if n < b.batch:
        n = min(b.batch, max(n, int(n * target_s / max(dt, 1e-3))))
        sub, dt = sample(n)
    reps = 1
    while dt * reps < target_s and reps < 200:  # the whole batch is quick: repeat it
        _, t = sample(n)
        dt = (dt * reps + t) / (reps + 1)
        reps += 1
    kv_bytes = float(sub.kv_lens.sum()) * b.num_kv_heads * b.head_dim * 2 * 2
    flops = 4.0 * b.head_dim * b.num_qo_heads * float(sub.kv_lens.sum())  # one row per sequence
    res = {"value": kv_bytes / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": "first %d of %d sequences of decode_b128_kv1024 (%d query rows x %d heads, all their keys), "
                     "mean of %d runs, %.3f s each" % (n, b.batch, sub.total_q, b.num_qo_heads, reps, dt),
           "fp64_gflops": flops / dt / 1e9, "rows_per_s": sub.total_q / dt, "seconds": dt, "cpu_model": cpu_model()}
    # the mixed long batch (4 prompts x 8192 + 256 decode rows, 64 qo heads): every 4th
    # decode row and the last 4 rows of each prompt, the rows that see the most keys
    log("oracle on a row sample of the mixed long batch")
    import torch
    m = W.mixed_long_batch(device="cuda")
    rows = [int(m.qo_indptr[s]) for s in range(4, m.batch, 4)]
    for s in range(4):
        e = int(m.qo_indptr[s + 1])
        rows += list(range(e - 4, e))
    rows = sorted(rows)
    mq, mkv = oracle._u16(m.q), oracle._u16(m.kv_cache)
    m.q, m.kv_cache = None, None  # host copies only from here
    torch.cuda.empty_cache()
    t = oracle_time(m, rows, threads, mq, mkv)
    fl = 4.0 * m.head_dim * m.num_qo_heads * visible_of_rows(m, rows)
    res["mixed_long_sample"] = {"rows": len(rows), "seconds": t, "rows_per_s": len(rows) / t,
                                "fp64_gflops": fl / t / 1e9,
                                "sample": "every 4th of the 256 decode rows and the last 4 rows of each of the "
                                          "4 prompts of mixed_long_batch, all 64 heads"}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-tail-skip-ab", action="store_true",
                    help="skip the long prompts' run without the causal tail skip (profiling runs)")
    ap.add_argument("--narrow-kernel", choices=("mfma", "valu"), default="mfma",
                    help="kernel for the headline decode tiles (default: the MFMA one)")
    ap.add_argument("--sweep", action="store_true",
                    help="only the full batch-size sweep at constant total tokens (one JSON line per batch size)")
    ap.add_argument("--oracle-full", type=str, default=None, metavar="PARTS",
                    help="only time the fp64 oracle over every row of the mixed long batch on the host "
                         "cores, for the listed parts (comma-separated of 0-3: prompt k, part 0 also the "
                         "decode rows; about 7 minutes each on 16 cores); one JSON line per part")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 256 MiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the path shards by "
              "sequence or kv head without communication); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.oracle_full is not None:
        oracle_full([int(x) for x in args.oracle_full.split(",")])
        return
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import paged_kv_attention_ragged_amd as rpa
    rpa.load()
    if args.sweep:
        bench_sweep()
        return
    if args.calibrate_copy:
        calibrate_copy()
    # The floors run last: right after their 2 GiB stream and dense MFMA burst the next
    # workload measured slower (the headline decode by 8% on one box).  Every roofline
    # entry gets the measured peaks once they are known.
    log("decode_b128_kv1024: %d warmup + %d timed steps" % (args.warmup, args.steps))
    res, b = bench_decode(args, {})
    if not args.no_prefill:
        log("long prefill 4x8192")
        res["prefill"] = bench_prefill(args, {})
    if not args.no_secondary:
        res["secondary"] = bench_secondary(args, {})
    log("floors: empty launch, HBM stream, decode gather, MFMA")
    floors = bench_floors()
    attach_measured_peaks(res, floors)
    res["floors"] = floors
    if not args.no_cpu_baseline:
        log("oracle baseline on host cores")
        res["cpu_baseline"] = cpu_baseline(b)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
