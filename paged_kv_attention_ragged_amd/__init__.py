"""Ragged batched attention over a paged KV cache on MI355X (gfx950).

A thin ctypes binding over librpa.so (include/rpa.h): it marshals arguments
and takes device memory and the current stream from PyTorch; every step of
the computation runs in the library's HIP kernels.  If the library is not
built, importing works but any call raises: there is no fallback path.

Lifecycle (mirrors begin_forward / forward / end_forward of the batch
prefill wrapper in flashinfer issue #323):

    plan = Plan(qo_indptr, kv_page_indptr, kv_last_page_len,
                num_qo_heads=64, num_kv_heads=8, head_dim=128, dtype=torch.bfloat16)
    plan.bind(kv_page_indices_gpu, num_pages=kv_cache.shape[0])   # upload schedule
    o, lse = plan.run(q, kv_cache, return_lse=True)                # repeatable
    plan.close()
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librpa.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "rpa.h")

STATUS = {0: "RPA_OK", 1: "RPA_E_ARG", 2: "RPA_E_SHAPE", 3: "RPA_E_INDPTR", 4: "RPA_E_LAST_PAGE_LEN",
          5: "RPA_E_QLEN_GT_KVLEN", 6: "RPA_E_WORKSPACE", 7: "RPA_E_UNSUPPORTED", 8: "RPA_E_HIP",
          9: "RPA_E_PAGE_OOB", 10: "RPA_E_V_RANGE"}
ERR_PAGE, ERR_V_RANGE = 1, 2  # bits of a plan's error word (rpa_plan_check)


class RPAError(RuntimeError):
    """A non-OK rpa_status; .status holds its name."""

    def __init__(self, status: int, message: str):
        self.status = STATUS.get(status, str(status))
        super().__init__("%s: %s" % (self.status, message))


class _Params(ctypes.Structure):
    _fields_ = [("num_qo_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("sm_scale", ctypes.c_float), ("max_kv_splits", ctypes.c_int32),
                ("num_cus", ctypes.c_int32), ("narrow_kernel", ctypes.c_int32), ("kv_shared", ctypes.c_int32)]


class _Info(ctypes.Structure):
    _fields_ = [("num_tiles", ctypes.c_int64), ("num_split_groups", ctypes.c_int64),
                ("max_splits", ctypes.c_int32), ("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32),
                ("tokens_per_tile", ctypes.c_int32), ("partial_rows", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_size_t), ("total_q", ctypes.c_int64),
                ("visible_pairs", ctypes.c_int64), ("kv_tokens", ctypes.c_int64)]


_lib = None


def load():
    """The ctypes handle of librpa.so; raises if the library has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("librpa.so is not built (python -m paged_kv_attention_ragged_amd.build); "
                               "there is no fallback implementation")
        lib = ctypes.CDLL(LIB_PATH)
        P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        st = ctypes.c_int
        sig = {
            "rpa_plan_create": (st, [ctypes.POINTER(_Params), i32, P, P, P, ctypes.POINTER(P)]),
            "rpa_plan_create_shared": (st, [ctypes.POINTER(_Params), i32, P, P, P, i32, ctypes.POINTER(P)]),
            "rpa_workspace_bytes": (st, [ctypes.POINTER(_Params), i32, i64, i64, ctypes.POINTER(ctypes.c_size_t)]),
            "rpa_plan_info": (st, [P, ctypes.POINTER(_Info)]),
            "rpa_plan_tiles": (st, [P, P, i64, ctypes.POINTER(i64)]),
            "rpa_plan_bind": (st, [P, P, i64, P, ctypes.c_size_t, P]),
            "rpa_run": (st, [P, P, P, P, P, P]),
            "rpa_run_noalloc": (st, [P, P, i64, P, P, P, P, P, P]),
            "rpa_plan_check": (st, [P, P, ctypes.POINTER(i32)]),
            "rpa_plan_destroy": (None, [P]),
            "rpa_validate_page_table": (st, [i32, P, P, i64]),
            "rpa_last_error": (ctypes.c_char_p, []),
            "rpa_version": (ctypes.c_char_p, []),
            "rpa_prof_start": (st, []),
            "rpa_prof_stop": (st, [P, P]),
            "rpa_merge_states": (st, [i64, i32, i32, i32, P, P, P, P, P, P, P]),
            "rpa_plan_update": (st, [P, P, P, P]),
            "rpa_plan_upload": (st, [P, P]),
            "rpa_append_kv": (st, [i32, i64, i32, i32, P, P, P, P, P, P, i64, P, P]),
            "rpa_trim_page_table": (st, [i32, P, P, P, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def declared_functions(header: str = HEADER):
    """Names of the functions include/rpa.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rpa_[a-z_]+)\s*\(", text)))


def _check(rc: int):
    if rc != 0:
        raise RPAError(rc, load().rpa_last_error().decode())


def _host_i32(a) -> np.ndarray:
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _dtype_code(dtype) -> int:
    if isinstance(dtype, str):
        return {"f16": 0, "fp16": 0, "float16": 0, "bf16": 1, "bfloat16": 1}[dtype]
    import torch
    return {torch.float16: 0, torch.bfloat16: 1}[dtype]


def _cuda_tensor(t, name, dtype=None, shape=None, min_numel=None):
    """Raise ValueError unless t is a contiguous CUDA tensor (of `dtype`, of `shape`, with
    at least `min_numel` elements): the C ABI takes raw device pointers and cannot check
    sizes, so a wrong tensor would become out-of-bounds device accesses."""
    import torch
    ok = (isinstance(t, torch.Tensor) and t.is_cuda and t.is_contiguous()
          and (dtype is None or t.dtype == dtype) and (shape is None or tuple(t.shape) == tuple(shape))
          and (min_numel is None or t.numel() >= min_numel))
    if not ok:
        want = "a contiguous CUDA tensor"
        if dtype is not None:
            want += " of %s" % dtype
        if shape is not None:
            want += " of shape %s" % (tuple(shape),)
        if min_numel is not None:
            want += " with at least %d elements" % min_numel
        got = ("%s %s on %s" % (t.dtype, tuple(t.shape), t.device)) if isinstance(t, torch.Tensor) else type(t).__name__
        raise ValueError("%s must be %s (got %s)" % (name, want, got))
    return t


def version() -> str:
    return load().rpa_version().decode()


def validate_page_table(kv_page_indptr, kv_page_indices, num_pages: int):
    """Host check that every page index is inside [0, num_pages)."""
    ip = _host_i32(kv_page_indptr)
    ix = _host_i32(kv_page_indices)
    _check(load().rpa_validate_page_table(len(ip) - 1, ip.ctypes.data, ix.ctypes.data if ix.size else None,
                                          int(num_pages)))


def _params(num_qo_heads, num_kv_heads, head_dim, page_size=16, dtype="f16", causal=True, sm_scale=None,
            max_kv_splits=0, num_cus=0, narrow_kernel="mfma", kv_shared=False) -> _Params:
    return _Params(num_qo_heads, num_kv_heads, head_dim, page_size, _dtype_code(dtype), 1 if causal else 0,
                   0.0 if sm_scale is None else float(sm_scale), max_kv_splits, num_cus,
                   {"mfma": 0, "valu": 1}[narrow_kernel], 1 if kv_shared else 0)


def workspace_bytes(batch: int, total_q: int, total_pages: int, **params) -> int:
    """Upper bound on the workspace of any plan for `batch` sequences with `total_q`
    query tokens and `total_pages` pages in all (keyword params as for Plan)."""
    p = _params(**params)
    out = ctypes.c_size_t()
    _check(load().rpa_workspace_bytes(ctypes.byref(p), int(batch), int(total_q), int(total_pages),
                                      ctypes.byref(out)))
    return int(out.value)


class Plan:
    """A schedule for one ragged batch (host page-table lengths), reusable across runs."""

    def __init__(self, qo_indptr, kv_page_indptr, kv_last_page_len, *, num_qo_heads: int, num_kv_heads: int,
                 head_dim: int, page_size: int = 16, dtype="f16", causal: bool = True,
                 sm_scale: Optional[float] = None, max_kv_splits: int = 0, num_cus: int = 0,
                 narrow_kernel: str = "mfma", kv_shared: bool = False, shared_pages: int = 0):
        """shared_pages > 0 declares that every sequence's first shared_pages page ids
        name the same pages (rpa_plan_create_shared): decode rows are then grouped
        so the shared prefix is read once per group."""
        lib = load()
        self._qo = _host_i32(qo_indptr)
        self._kp = _host_i32(kv_page_indptr)
        self._kl = _host_i32(kv_last_page_len)
        self.batch = len(self._qo) - 1
        self.params = _params(num_qo_heads, num_kv_heads, head_dim, page_size, dtype, causal, sm_scale,
                              max_kv_splits, num_cus, narrow_kernel, kv_shared)
        h = ctypes.c_void_p()
        p = lambda a: a.ctypes.data if a.size else None
        if shared_pages:
            _check(lib.rpa_plan_create_shared(ctypes.byref(self.params), self.batch, p(self._qo), p(self._kp),
                                              p(self._kl), int(shared_pages), ctypes.byref(h)))
        else:
            _check(lib.rpa_plan_create(ctypes.byref(self.params), self.batch, p(self._qo), p(self._kp),
                                       p(self._kl), ctypes.byref(h)))
        self.shared_pages = int(shared_pages)
        self._h = h
        self._keep = ()
        self.workspace = None

    # -- inspection --------------------------------------------------------------------------
    @property
    def info(self) -> dict:
        inf = _Info()
        _check(load().rpa_plan_info(self._h, ctypes.byref(inf)))
        return {k: getattr(inf, k) for k, _ in _Info._fields_}

    def tiles(self) -> np.ndarray:
        """Work items in launch order, int32 [n, 16] (fields documented in rpa.h)."""
        n = ctypes.c_int64()
        _check(load().rpa_plan_tiles(self._h, None, 0, ctypes.byref(n)))
        out = np.zeros((n.value, 16), dtype=np.int32)
        if n.value:
            _check(load().rpa_plan_tiles(self._h, out.ctypes.data, n.value, ctypes.byref(n)))
        return out

    # -- device side -------------------------------------------------------------------------
    def bind(self, kv_page_indices, num_pages: int, workspace=None, stream=None):
        """Upload the schedule into `workspace` (a uint8 CUDA tensor; allocated here
        with torch if None) and borrow `kv_page_indices` (int32 CUDA tensor)."""
        import torch
        _cuda_tensor(kv_page_indices, "kv_page_indices", torch.int32,
                     min_numel=int(self._kp[-1]) if self.batch > 0 else 0)
        need = self.info["workspace_bytes"]
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=kv_page_indices.device)
        _cuda_tensor(workspace, "workspace", torch.uint8)
        if stream is None:
            stream = torch.cuda.current_stream(kv_page_indices.device)
        _check(load().rpa_plan_bind(self._h, kv_page_indices.data_ptr() if kv_page_indices.numel() else None,
                                    int(num_pages), workspace.data_ptr(), workspace.numel(), stream.cuda_stream))
        self._keep = (kv_page_indices,)
        self.workspace = workspace
        self.num_pages = int(num_pages)
        return self

    def run(self, q, kv_cache, out=None, return_lse: bool = False, lse=None, stream=None):
        """O (and LSE if asked) for every query row: q [total_q, H_qo, D],
        kv_cache [num_pages, 2, 16, H_kv, D], both CUDA tensors of the plan's dtype."""
        import torch
        P = self.params
        dt = torch.float16 if P.dtype == 0 else torch.bfloat16
        T = int(self._qo[-1]) if self.batch > 0 else 0
        if q.dtype != dt or kv_cache.dtype != dt:
            raise ValueError("q and kv_cache must be %s" % dt)
        if tuple(q.shape) != (T, P.num_qo_heads, P.head_dim) or not q.is_contiguous() or not q.is_cuda:
            raise ValueError("q must be a contiguous CUDA tensor of shape %s" % ((T, P.num_qo_heads, P.head_dim),))
        if (kv_cache.dim() != 5 or tuple(kv_cache.shape[1:]) != (2, P.page_size, P.num_kv_heads, P.head_dim)
                or not kv_cache.is_contiguous() or not kv_cache.is_cuda or kv_cache.shape[0] != self.num_pages):
            raise ValueError("kv_cache must be a contiguous CUDA tensor [%d, 2, %d, %d, %d]"
                             % (self.num_pages, P.page_size, P.num_kv_heads, P.head_dim))
        if out is None:
            out = torch.empty_like(q)
        _cuda_tensor(out, "out", dt, tuple(q.shape))
        if return_lse and lse is None:
            lse = torch.empty((T, P.num_qo_heads), dtype=torch.float32, device=q.device)
        if lse is not None:
            _cuda_tensor(lse, "lse", torch.float32, (T, P.num_qo_heads))
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        _check(load().rpa_run(self._h, q.data_ptr(), kv_cache.data_ptr(), out.data_ptr(),
                              lse.data_ptr() if lse is not None else None, stream.cuda_stream))
        return (out, lse) if return_lse else out

    def run_noalloc(self, q, kv_cache, kv_page_indices, out, lse=None, err_flag=None, stream=None):
        """rpa_run_noalloc: the same computation without a bound workspace (the library's
        static device scratch holds the schedule and partials).  Every tensor is the
        caller's: q, kv_cache, kv_page_indices (int32), out, and optional lse (fp32)
        and err_flag (int32 [1], OR-ed with error bits)."""
        import torch
        P = self.params
        dt = torch.float16 if P.dtype == 0 else torch.bfloat16
        T = int(self._qo[-1]) if self.batch > 0 else 0
        _cuda_tensor(q, "q", dt, (T, P.num_qo_heads, P.head_dim))
        _cuda_tensor(kv_cache, "kv_cache", dt)
        if kv_cache.dim() != 5 or tuple(kv_cache.shape[1:]) != (2, P.page_size, P.num_kv_heads, P.head_dim):
            raise ValueError("kv_cache must be [num_pages, %d, %d, %d, %d]" % (2, P.page_size, P.num_kv_heads,
                                                                             P.head_dim))
        _cuda_tensor(kv_page_indices, "kv_page_indices", torch.int32,
                     min_numel=int(self._kp[-1]) if self.batch > 0 else 0)
        _cuda_tensor(out, "out", dt, tuple(q.shape))
        if lse is not None:
            _cuda_tensor(lse, "lse", torch.float32, (T, P.num_qo_heads))
        if err_flag is not None:
            _cuda_tensor(err_flag, "err_flag", torch.int32, min_numel=1)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        ptr = lambda t: t.data_ptr() if t is not None and t.numel() else None
        _check(load().rpa_run_noalloc(self._h, ptr(kv_page_indices), int(kv_cache.shape[0]), q.data_ptr(),
                                      kv_cache.data_ptr(), out.data_ptr(), ptr(lse), ptr(err_flag),
                                      stream.cuda_stream))
        return out

    def update(self, qo_indptr, kv_page_indptr, kv_last_page_len):
        """Re-plan in place for new lengths with the same launch shape (raises
        RPAError RPA_E_UNSUPPORTED otherwise); the device copy changes at upload()."""
        qo, kp, kl = _host_i32(qo_indptr), _host_i32(kv_page_indptr), _host_i32(kv_last_page_len)
        if len(qo) != self.batch + 1 or len(kp) != self.batch + 1 or len(kl) != self.batch:
            raise ValueError("update needs the plan's batch size (%d)" % self.batch)
        if self._keep and self.batch > 0 and self._keep[0].numel() < int(kp[-1]):
            raise ValueError("the bound kv_page_indices holds %d entries; the new lengths need %d: bind a "
                             "larger array" % (self._keep[0].numel(), int(kp[-1])))
        p = lambda a: a.ctypes.data if a.size else None
        _check(load().rpa_plan_update(self._h, p(qo), p(kp), p(kl)))
        self._qo, self._kp, self._kl = qo, kp, kl

    def upload(self, stream=None):
        """Enqueue the copy of the current schedule into the workspace (graph-capturable)."""
        import torch
        if stream is None:
            stream = torch.cuda.current_stream()
        _check(load().rpa_plan_upload(self._h, stream.cuda_stream))

    def check(self, stream=None, raise_on_error: bool = True) -> int:
        """Synchronise, read and clear the plan's error word (ERR_PAGE: an out-of-range
        page index; ERR_V_RANGE: bf16 V above the fp16 range).  Raises RPAError when a
        bit is set, unless raise_on_error is False; returns the bits."""
        import torch
        if stream is None:
            stream = torch.cuda.current_stream()
        flag = ctypes.c_int32()
        rc = load().rpa_plan_check(self._h, stream.cuda_stream, ctypes.byref(flag))
        if rc != 0 and (raise_on_error or flag.value == 0):
            _check(rc)
        return int(flag.value)

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            load().rpa_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def append_kv(new_kv, kv_cache, append_indptr, kv_page_indptr, kv_page_indices, kv_last_page_len,
              err_flag=None, stream=None):
    """Write new tokens' K/V (new_kv [n_new, 2, H_kv, D], the cache's dtype) into
    kv_cache [num_pages, 2, 16, H_kv, D] at the slots the page table (lengths after
    the append; int32 CUDA tensors) gives the last append_indptr[b+1] - append_indptr[b]
    tokens of each sequence.  err_flag: optional int32 CUDA tensor set to 1 for a
    token with no valid slot."""
    import torch
    n_new = new_kv.shape[0]
    Hk, D = kv_cache.shape[3], kv_cache.shape[4]
    _cuda_tensor(kv_cache, "kv_cache")
    if kv_cache.dim() != 5 or kv_cache.shape[1:3] != (2, 16):
        raise ValueError("kv_cache must be [num_pages, 2, 16, H_kv, D]")
    _cuda_tensor(new_kv, "new_kv", kv_cache.dtype, (n_new, 2, Hk, D))
    for name, t in (("append_indptr", append_indptr), ("kv_page_indptr", kv_page_indptr),
                    ("kv_page_indices", kv_page_indices), ("kv_last_page_len", kv_last_page_len)):
        _cuda_tensor(t, name, torch.int32)
    if kv_page_indptr.numel() != append_indptr.numel() or kv_last_page_len.numel() != append_indptr.numel() - 1:
        raise ValueError("append_indptr, kv_page_indptr ([batch + 1]) and kv_last_page_len ([batch]) disagree")
    if err_flag is not None:
        _cuda_tensor(err_flag, "err_flag", torch.int32, min_numel=1)
    if stream is None:
        stream = torch.cuda.current_stream(kv_cache.device)
    _check(load().rpa_append_kv(append_indptr.numel() - 1, n_new, Hk, D, append_indptr.data_ptr(),
                                kv_page_indptr.data_ptr(), kv_page_indices.data_ptr() if kv_page_indices.numel() else None,
                                kv_last_page_len.data_ptr(), new_kv.data_ptr(), kv_cache.data_ptr(), kv_cache.shape[0],
                                err_flag.data_ptr() if err_flag is not None else None, stream.cuda_stream))


def trim_page_table(kv_page_indptr, kv_page_indices, kv_last_page_len, new_kv_len):
    """Host page-table edit keeping each sequence's first new_kv_len[b] tokens:
    returns (kv_page_indptr, kv_page_indices, kv_last_page_len) as int32 numpy arrays."""
    ip, ix, kl, nl = (_host_i32(a) for a in (kv_page_indptr, kv_page_indices, kv_last_page_len, new_kv_len))
    batch = len(ip) - 1
    o_ip = np.zeros(batch + 1, np.int32)
    o_ix = np.zeros(max(len(ix), 1), np.int32)
    o_kl = np.zeros(max(batch, 1), np.int32)
    p = lambda a: a.ctypes.data if a.size else None
    _check(load().rpa_trim_page_table(batch, p(ip), p(ix), p(kl), p(nl), o_ip.ctypes.data, o_ix.ctypes.data,
                                      o_kl.ctypes.data))
    return o_ip, o_ix[:o_ip[-1]].copy(), o_kl[:batch].copy()


def merge_states(o_a, lse_a, o_b, lse_b, out=None, lse_out=None, stream=None):
    """Merge two attention states of the same rows over disjoint key sets:
    o_* [rows, H, D] (fp16 / bf16 CUDA tensors), lse_* [rows, H] fp32.  Returns
    (O, LSE); `out` / `lse_out` may be o_a / lse_a for an in-place merge."""
    import torch
    rows, H, D = o_a.shape
    for t in (o_a, o_b):
        if t.shape != o_a.shape or t.dtype != o_a.dtype or not t.is_cuda or not t.is_contiguous():
            raise ValueError("o_a and o_b must be contiguous CUDA tensors of one shape and dtype")
    for t in (lse_a, lse_b):
        if tuple(t.shape) != (rows, H) or t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("lse_a and lse_b must be contiguous fp32 CUDA tensors [rows, H]")
    if out is None:
        out = torch.empty_like(o_a)
    _cuda_tensor(out, "out", o_a.dtype, tuple(o_a.shape))
    if lse_out is None:
        lse_out = torch.empty_like(lse_a)
    _cuda_tensor(lse_out, "lse_out", torch.float32, (rows, H))
    if stream is None:
        stream = torch.cuda.current_stream(o_a.device)
    _check(load().rpa_merge_states(rows, H, D, _dtype_code(o_a.dtype), o_a.data_ptr(), lse_a.data_ptr(),
                                   o_b.data_ptr(), lse_b.data_ptr(), out.data_ptr(), lse_out.data_ptr(),
                                   stream.cuda_stream))
    return out, lse_out


def prof_start():
    _check(load().rpa_prof_start())


def prof_stop():
    """{'wide': (launches, ms), 'narrow': (launches, ms)} since prof_start(): the
    kernel of the wide tiles and the kernel of the narrow (decode-like) tiles."""
    counts = (ctypes.c_int64 * 2)()
    ms = (ctypes.c_double * 2)()
    _check(load().rpa_prof_stop(counts, ms))
    return {"wide": (counts[0], ms[0]), "narrow": (counts[1], ms[1])}
