"""fp64 CPU oracle for ragged attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  The product path never
imports this package, and this package imports nothing from the product.

The arithmetic lives in ``rpa_oracle.c`` (plain C, binary64); this module
builds it with gcc and marshals numpy arrays into it.  ``run`` returns
O[total_q, H_qo, D] and LSE[total_q, H_qo] as float64 arrays.

What is computed, and where it comes from:
  * page-table resolution (kv_page_indptr / kv_page_indices /
    kv_last_page_len, pages shaped [2, page_size, H_kv, D]):
    flashinfer issue #323, "How are prefill and decode kernels different?",
    the repro script's tensors;
  * ragged packing of queries by qo_indptr: the same repro's prefill wrapper;
  * causal mask with the queries at the last q_len positions: llama.cpp
    discussion #15958, "Pad for prefill stage?" (real tokens first, masked
    tails skipped);
  * grouped-query heads (qo head h reads kv head h // (H_qo // H_kv)):
    flashinfer issue #323 (64/8 qo heads over 8/8 kv heads);
  * softmax attention and its log-sum-exp, in natural log;
  * ``merge_states``: two attention states of the same query rows over
    disjoint key sets combined into the state over their union, with weights
    exp(LSE_x - max LSE) (the split-KV merge behind kv-parallelism in
    flashinfer issue #323, and the join of a cascade's shared-prefix and
    private halves in vLLM issue #227, "Question about efficient memory
    sharing").  Plain numpy in binary64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rpa_oracle.c")
_LIB = os.path.join(_HERE, "librpa_oracle.so")

ERRORS = {1: "E_ARG", 2: "E_INDPTR", 3: "E_LAST_PAGE_LEN", 4: "E_QLEN_GT_KVLEN",
          5: "E_PAGE_OOB", 6: "E_NOMEM"}

_lib = None


def build(force: bool = False, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle's C source with gcc into a shared library (next to the source)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                               "-shared", "-pthread", "-Wall", "-o", tmp, src, "-lm"])
        os.replace(tmp, out)
    return out


def load_library(path: str):
    """ctypes handle of a built oracle library, with its argument types set."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.rpa_oracle_run.argtypes = [i32, P, P, P, P, i64, i32, i32, i32, i32, i32, i32,
                                   ctypes.c_double, P, P, P, P, P, i64, i32]
    lib.rpa_oracle_run.restype = ctypes.c_int
    lib.rpa_oracle_decode.argtypes = [i32, i64, P, P]
    lib.rpa_oracle_decode.restype = None
    return lib


def _load():
    global _lib
    if _lib is None:
        _lib = load_library(build())
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _u16(a):
    """Raw 16-bit patterns of a torch fp16/bf16 tensor or a numpy uint16/float16 array."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return np.ascontiguousarray(a.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return np.ascontiguousarray(a)


def decode(raw, dtype: str) -> np.ndarray:
    """Exact binary64 value of every 16-bit pattern in `raw` ('f16' or 'bf16')."""
    raw = _u16(raw)
    out = np.empty(raw.shape, dtype=np.float64)
    _load().rpa_oracle_decode(0 if dtype == "f16" else 1, raw.size, _ptr(raw), _ptr(out))
    return out


def run(*, qo_indptr, kv_page_indptr, kv_page_indices, kv_last_page_len, q, kv_cache,
        num_qo_heads, num_kv_heads, head_dim, page_size=16, dtype="f16", causal=True,
        sm_scale=None, rows=None, nthreads=None, want_lse=True, lib=None):
    """Run the oracle.  Index arrays are host int32; q / kv_cache are fp16/bf16 torch
    tensors (any device; copied to host) or uint16 arrays of raw patterns.

    rows: optional list of token rows to compute; others are left NaN.
    Returns (O float64 [T, H, D], LSE float64 [T, H] or None).
    """
    lib = lib or _load()
    qo = _i32(qo_indptr)
    kp = _i32(kv_page_indptr)
    ki = _i32(kv_page_indices)
    kl = _i32(kv_last_page_len)
    qr = _u16(q)
    kv = _u16(kv_cache)
    batch = len(qo) - 1
    total_q = int(qo[-1])
    num_pages = kv.shape[0] if kv.ndim > 0 else 0
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(head_dim)
    o = np.full((total_q, num_qo_heads, head_dim), np.nan, dtype=np.float64)
    lse = np.full((total_q, num_qo_heads), np.nan, dtype=np.float64) if want_lse else None
    rows_a = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if nthreads is None:
        nthreads = len(os.sched_getaffinity(0))
    rc = lib.rpa_oracle_run(batch, _ptr(qo), _ptr(kp), _ptr(ki), _ptr(kl), num_pages,
                            num_qo_heads, num_kv_heads, head_dim, page_size,
                            0 if dtype == "f16" else 1, 1 if causal else 0, float(sm_scale),
                            _ptr(qr), _ptr(kv), _ptr(o), _ptr(lse), _ptr(rows_a),
                            0 if rows_a is None else len(rows_a), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the input: %s" % ERRORS.get(rc, rc))
    return o, lse


def merge_states(o_a, lse_a, o_b, lse_b):
    """(O, LSE) over the union of two disjoint key sets from the states over each:
    m = max(LSE_a, LSE_b), w_x = exp(LSE_x - m), O = (w_a O_a + w_b O_b) / (w_a + w_b),
    LSE = m + ln(w_a + w_b).  A state with LSE = -inf (no visible key) has weight 0
    and its O is not used (it may hold anything); with no visible key in either,
    O = 0 and LSE = -inf.  Inputs of any float type,
    O [..., D], LSE [...]; binary64 out."""
    o_a, o_b = np.asarray(o_a, np.float64), np.asarray(o_b, np.float64)
    lse_a, lse_b = np.asarray(lse_a, np.float64), np.asarray(lse_b, np.float64)
    m = np.maximum(lse_a, lse_b)
    none = np.isneginf(m)
    mu = np.where(none, 0.0, m)
    wa, wb = np.exp(lse_a - mu), np.exp(lse_b - mu)
    tot = wa + wb
    with np.errstate(invalid="ignore", divide="ignore"):
        ta = np.where((wa > 0)[..., None], wa[..., None] * o_a, 0.0)  # a weight-0 state's O is unused
        tb = np.where((wb > 0)[..., None], wb[..., None] * o_b, 0.0)
        o = (ta + tb) / tot[..., None]
        lse = mu + np.log(tot)
    o[none] = 0.0
    lse[none] = -np.inf
    return o, lse
