"""Helpers for the GPU parity tests: run a batch through the library and
compare with the oracle.

Tolerance (per element, for fp16/bf16 inputs with fp32 accumulation):
    O:   |gpu - oracle| <= 2e-3 + 1e-2 * |oracle|
    LSE: |gpu - oracle| <= 1e-3 + 1e-4 * |oracle|
The O rule is the max-abs 2e-3 / max-rel 1e-2 target read as one combined
bound per element (bf16 output rounding alone reaches 2^-9 |o|, so a pure
2e-3 absolute bound is out of reach for |o| > 1).  LSE is fp32 arithmetic
from fp16/bf16 products accumulated in fp32, far inside its bound.
"""
import sys

import numpy as np
import torch

import paged_kv_attention_ragged_amd as rpa
import workloads as W

O_ATOL, O_RTOL = 2e-3, 1e-2
L_ATOL, L_RTOL = 1e-3, 1e-4


def say(msg):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print("[gpu] " + msg, flush=True)
    sys.stdout.flush()


def on_device(b: W.Batch, device="cuda"):
    q = b.q.to(device).contiguous()
    kv = b.kv_cache.to(device).contiguous()
    idx = torch.from_numpy(b.kv_page_indices.astype(np.int32)).to(device)
    return q, kv, idx


def run(b: W.Batch, max_kv_splits=0, num_cus=0, return_lse=True, sm_scale=None, dev=None, label="",
        narrow_kernel="mfma", kv_shared=False):
    """(O float64 [T,H,D], LSE float64 [T,H] or None, plan info) from the HIP path."""
    say("run %s %s splits=%d cus=%d T=%d narrow=%s kv_shared=%d" % (b.name, label, max_kv_splits, num_cus,
                                                                    b.total_q, narrow_kernel, kv_shared))
    q, kv, idx = dev if dev is not None else on_device(b)
    plan = rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=b.num_qo_heads,
                    num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, dtype=b.dtype, causal=b.causal,
                    sm_scale=sm_scale, max_kv_splits=max_kv_splits, num_cus=num_cus, narrow_kernel=narrow_kernel,
                    kv_shared=kv_shared)
    plan.bind(idx, num_pages=kv.shape[0])
    res = plan.run(q, kv, return_lse=return_lse)
    o, lse = res if return_lse else (res, None)
    torch.cuda.synchronize()
    plan.check()
    info = plan.info
    plan.close()
    o64 = o.double().cpu().numpy()
    l64 = lse.double().cpu().numpy() if lse is not None else None
    return o64, l64, info


def assert_close(o, lse, ro, rl, rows=None, what=""):
    if rows is not None:
        o, ro = o[rows], ro[rows]
        if lse is not None:
            lse, rl = lse[rows], rl[rows]
    assert np.isfinite(ro).all()
    assert np.isfinite(o).all(), "%s: non-finite GPU output" % what
    err = np.abs(o - ro)
    bound = O_ATOL + O_RTOL * np.abs(ro)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError("%s: %d of %d O elements out of tolerance; worst at %s: gpu %r oracle %r"
                             % (what, bad.sum(), bad.size, i, o[i], ro[i]))
    if lse is not None:
        lerr = np.abs(lse - rl)
        lb = L_ATOL + L_RTOL * np.abs(rl)
        lbad = lerr > lb
        if lbad.any():
            i = np.unravel_index(np.argmax(lerr - lb), lerr.shape)
            raise AssertionError("%s: %d LSE elements out of tolerance; worst at %s: gpu %r oracle %r"
                                 % (what, lbad.sum(), i, lse[i], rl[i]))
    return float(err.max()), float((err / np.maximum(np.abs(ro), 0.2)).max())
