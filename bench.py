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
secondary = the pages' other workloads (ragged vs padded short prompts, the
shared-prefix suffix prefill and decode step directly and as a cascade, the
mixed long batch's decode rows and the whole batch).
"""
import argparse
import json
import os
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
    while dt * reps < target_s and reps < 200:  # the whole batch is quick: repeat it
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
                    num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, dtype=b.dtype,
                    narrow_kernel=args.narrow_kernel)
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
                     "kernel": "attn_narrow_kernel" if args.narrow_kernel == "mfma" else "attn_narrow_valu_kernel",
                     "avg_ms": attn_avg,
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


def time_fn(fn, steps, warmup):
    """Mean ms per call of fn() (GPU work on the current stream), by events around `steps` calls."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def bound_plan(b, narrow="mfma", kv_shared=False):
    import torch
    import paged_kv_attention_ragged_amd as rpa
    p = rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=b.num_qo_heads,
                 num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, dtype=b.dtype, causal=b.causal,
                 narrow_kernel=narrow, kv_shared=kv_shared)
    p.bind(torch.from_numpy(b.kv_page_indices).cuda(), num_pages=b.kv_cache.shape[0])
    return p


def bench_secondary(args):
    """The other workloads of the pages, one line each: ragged vs padded short
    prompts, the shared-prefix suffix prefill and a decode step (direct and as a
    cascade), and the mixed long batch's parts."""
    import torch
    import paged_kv_attention_ragged_amd as rpa
    import workloads as W
    steps = max(5, args.steps // 10)
    out = {}

    def direct(b, rotate=1, narrow="mfma", kv_shared=False):
        p = bound_plan(b, narrow, kv_shared)
        q, kv0 = b.q.cuda(), b.kv_cache.cuda()
        kvs = [kv0] + [kv0.clone() for _ in range(rotate - 1)]
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
        it = iter(range(1 << 30))
        ms = time_fn(lambda: p.run(q, kvs[next(it) % rotate], out=o, lse=lse, return_lse=True), steps, 3)
        info = p.info
        p.close()
        return ms, info

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
        ms = time_fn(step, steps, 3)
        pa.close()
        pb.close()
        return ms

    # short ragged prompts (lengths U{1..200}) vs the same prompts padded to 200
    log("short prompts: ragged vs padded")
    sp = W.short_prompt_prefill()
    spp = W.short_prompt_prefill(padded=True)
    ms_r, inf_r = direct(sp)
    ms_p, inf_p = direct(spp)
    out["short_prompts"] = {"ragged_ms": ms_r, "padded_ms": ms_p, "time_ratio": ms_r / ms_p,
                            "flops_ratio": inf_r["visible_pairs"] / inf_p["visible_pairs"],
                            "ragged_tflops": 4.0 * sp.head_dim * inf_r["visible_pairs"] / ms_r / 1e9}
    # shared prefix (256 requests x 200 shared + 30 own tokens), then one decode step
    log("shared prefix: direct vs cascade")
    b = W.shared_prefix_suffix()
    pre_direct, inf = direct(b)
    pre_cascade = cascade(b, 200)
    d = W.decode_step(b, 1)
    dec_direct, inf_d = direct(d, rotate=6, kv_shared=True)  # 12 pages shared by all requests
    dec_cascade = cascade(d, 200)
    logical = float(inf_d["kv_tokens"]) * d.num_kv_heads * d.head_dim * 4
    out["shared_prefix"] = {"suffix_prefill_direct_ms": pre_direct, "suffix_prefill_cascade_ms": pre_cascade,
                            "decode_step_direct_ms": dec_direct, "decode_step_cascade_ms": dec_cascade,
                            "decode_direct_logical_kv_gbs": logical / dec_direct / 1e6,
                            "suffix_prefill_tflops_direct": 4.0 * b.head_dim * inf["visible_pairs"] / pre_direct / 1e9}
    # a long shared prefix (4096 tokens) under the same 256 requests: one decode step
    log("long shared prefix decode: direct vs cascade")
    lb = W.decode_step(W.shared_prefix_suffix(prefix=4096, decode_steps=1), 1)
    ld_direct, inf_l = direct(lb, kv_shared=True)
    ld_cascade = cascade(lb, 4096)
    out["long_prefix_4096"] = {"decode_step_direct_ms": ld_direct, "decode_step_cascade_ms": ld_cascade,
                               "logical_kv_gb": float(inf_l["kv_tokens"]) * lb.num_kv_heads * lb.head_dim * 4 / 1e9}
    del lb
    # the decode loop: eager vs graph-captured steps
    log("decode loop: eager vs graph")
    out["decode_loop"] = bench_decode_loop()
    # decode tiles on the VALU kernel instead of MFMA (the pages' CUDA-core decode)
    log("decode on the VALU kernel")
    db = W.decode_b128_kv1024(device="cuda")
    v_ms, _ = direct(db, rotate=8, narrow="valu")
    m_ms, _ = direct(db, rotate=8)
    out["decode_b128_kv1024_valu_vs_mfma"] = {"valu_ms": v_ms, "mfma_ms": m_ms}
    del db
    out["shared_prefix"]["decode_step_valu_ms"] = direct(d, rotate=6, narrow="valu", kv_shared=True)[0]
    out["shared_prefix"]["decode_step_streamed_kv_ms"] = direct(d, rotate=6)[0]  # without the hint
    # mixed long batch: its decode rows alone and the whole batch in one call
    log("mixed long batch: decode rows, whole batch")
    for part in ("decode", "all"):
        mb = W.mixed_long_batch(part=part, device="cuda")
        ms, info = direct(mb)
        kvb = float(info["kv_tokens"]) * mb.num_kv_heads * mb.head_dim * 4
        ent = {"ms": ms, "tflops": 4.0 * mb.head_dim * info["visible_pairs"] / ms / 1e9}
        if part == "decode":
            ent["kv_gbs"] = kvb / ms / 1e6
            ent["hbm_frac"] = ent["kv_gbs"] / HBM_PEAK_GBS
            ent["valu_ms"] = direct(mb, narrow="valu")[0]
        out["mixed_long_" + part] = ent
        del mb
        torch.cuda.empty_cache()
    return out


def bench_decode_loop(steps=50):
    """The shared-prefix batch's decode loop (256 requests, one token per step after
    200 + 30 prompt tokens): per step, append the new token's K/V and attend.
    Eager: plan + bind + append + run per step.  Graph: the captured [upload,
    append, run] replayed after an in-place plan update.  Both synchronise every
    step, as a decode loop must; inputs of all steps are prepared beforehand."""
    import torch
    import numpy as np
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
    gpu_ms = 0.0
    t0 = time.perf_counter()
    for i in range(steps):
        if i > 0:
            d = load(i)
            plan.update(d.qo_indptr, d.kv_page_indptr, d.kv_last_page_len)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        gpu_ms += e0.elapsed_time(e1)
    graph = (time.perf_counter() - t0) / steps * 1e3
    plan.close()
    return {"steps": steps, "eager_step_ms": eager, "graph_step_ms": graph, "graph_replay_gpu_ms": gpu_ms / steps}


def bench_sweep(total_tokens=8192, batches=(1, 2, 4, 8, 16, 32, 64, 128, 256), steps=10):
    """Batch-size sweep at constant total tokens (llama.cpp discussion #15958: batching
    prompts helps little unless they are very short): B causal prompts of
    total_tokens / B tokens each (32 qo / 8 kv heads, D 128, bf16), as one ragged
    call, against the same prompts run one call each.  One JSON line per B."""
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
        batched = time_fn(lambda: p.run(q, kv, out=o), steps, 2)
        p.close()
        one = W.Batch("one", np.array([0, L], np.int32), np.array([0, b.kv_page_indptr[1]], np.int32),
                      b.kv_page_indices[:b.kv_page_indptr[1]].copy(), b.kv_last_page_len[:1].copy(), q[:L], kv,
                      b.num_qo_heads, b.num_kv_heads, b.head_dim, b.dtype)
        p1 = bound_plan(one)
        single = time_fn(lambda: p1.run(q[:L], kv, out=o[:L]), steps, 2)
        p1.close()
        r = {"sweep": "constant_total_tokens", "total_tokens": total_tokens, "batch": B, "prompt_len": L,
             "batched_ms": batched, "one_by_one_ms": single * B, "speedup": single * B / batched,
             "tflops_batched": 4.0 * b.head_dim * info["visible_pairs"] / batched / 1e9}
        print(json.dumps(r), flush=True)
        rows.append(r)
        del b, q, kv, o
        torch.cuda.empty_cache()
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the other workloads")
    ap.add_argument("--narrow-kernel", choices=("mfma", "valu"), default="mfma",
                    help="kernel for the headline decode tiles (default: the MFMA one)")
    ap.add_argument("--sweep", action="store_true",
                    help="only the batch-size sweep at constant total tokens (one JSON line per batch size)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 256 MiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the path shards by "
              "sequence or kv head without communication); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import paged_kv_attention_ragged_amd as rpa
    rpa.load()
    if args.sweep:
        bench_sweep()
        return
    if args.calibrate_copy:
        calibrate_copy()
    log("decode_b128_kv1024: %d warmup + %d timed steps" % (args.warmup, args.steps))
    res, b = bench_decode(args)
    if not args.no_prefill:
        log("long prefill 4x8192")
        res["prefill"] = bench_prefill(args)
    if not args.no_secondary:
        res["secondary"] = bench_secondary(args)
    if not args.no_cpu_baseline:
        log("oracle baseline on host cores")
        res["cpu_baseline"] = cpu_baseline(b)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
