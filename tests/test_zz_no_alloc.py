"""rpa_run_noalloc: the attention run for callers that cannot allocate device
memory, on the library's static device scratch.  Checked through the C ABI
against rpa_run with a bound workspace (same kernels, same schedule: the same
bits), and against the fp64 oracle, on two calls in a row, the second with a
smaller batch; then its error word and its size limit.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_ragged_amd as rpa
import workloads as W
from tests.gpu_util import assert_close, on_device, say


def plan_for(b, **kw):
    return rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=b.num_qo_heads,
                    num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, dtype=b.dtype, causal=b.causal, **kw)


def noalloc_call(plan, q, kv, idx, o, lse, flag):
    """rpa_run_noalloc through ctypes (the C ABI itself, no binding helper)."""
    lib = rpa.load()
    st = torch.cuda.current_stream().cuda_stream
    return lib.rpa_run_noalloc(plan._h, idx.data_ptr(), int(kv.shape[0]), q.data_ptr(), kv.data_ptr(),
                               o.data_ptr(), lse.data_ptr(), flag.data_ptr() if flag is not None else None, st)


@pytest.mark.gpu
def test_noalloc_equals_workspace_run_on_two_calls():
    big = W.decode_b128_kv1024(batch=64, kv_len=2000)   # split key ranges: partials, counters, merges
    small = W.tiny_ragged_prefill(poison=True, spare_pages=4)  # smaller, wide tiles after the fold
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    for b in (big, small):
        q, kv, idx = on_device(b)
        p = plan_for(b)
        info = p.info
        say("noalloc %s: %d tiles, %d split groups, %d workspace bytes"
            % (b.name, info["num_tiles"], info["num_split_groups"], info["workspace_bytes"]))
        assert b is small or info["num_split_groups"] > 0
        o = torch.full_like(q, float("nan"))
        lse = torch.full((b.total_q, b.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
        rc = noalloc_call(p, q, kv, idx, o, lse, flag)
        assert rc == 0, rpa.load().rpa_last_error()
        # the existing entry point: a bound workspace, rpa_run
        p.bind(idx, num_pages=kv.shape[0])
        o_ref, lse_ref = p.run(q, kv, return_lse=True)
        torch.cuda.synchronize()
        p.check()
        assert flag.item() == 0
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), b.name
        assert torch.equal(lse, lse_ref), b.name
        ro, rl = oracle.run(**b.oracle_kwargs())
        assert_close(o.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl, what="noalloc " + b.name)
        p.close()


@pytest.mark.gpu
def test_noalloc_raises_bits_in_the_callers_word():
    b = W.make_batch("oob", [3, 1], [100, 70], num_qo_heads=8, num_kv_heads=1, head_dim=64, dtype="f16", seed=38)
    q, kv, _ = on_device(b)
    bad = b.kv_page_indices.copy()
    bad[1] = b.num_pages  # one past the pool: read as zeros, flagged
    idx = torch.from_numpy(bad.astype(np.int32)).cuda()
    p = plan_for(b)
    o = torch.empty_like(q)
    lse = torch.empty((b.total_q, 8), dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("noalloc with a bad page index")
    assert noalloc_call(p, q, kv, idx, o, lse, flag) == 0
    torch.cuda.synchronize()
    assert flag.item() == rpa.ERR_PAGE
    # NULL error word: the bits are dropped, the output is the same
    o2 = torch.empty_like(q)
    assert noalloc_call(p, q, kv, idx, o2, lse, None) == 0
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    p.close()


def test_noalloc_refuses_plans_beyond_its_scratch():
    """Checked before any HIP call (no GPU needed): a plan whose workspace exceeds
    16 MiB is refused with RPA_E_WORKSPACE and a message naming both sizes."""
    W_ = W
    b = W_.Batch("big", np.array([0, 1, 2], np.int32), np.array([0, 60000, 120000], np.int32),
                 np.zeros(120000, np.int32), np.array([16, 16], np.int32), None, None, 64, 8, 128, "bf16")
    p = plan_for(b, num_cus=4096)  # split into many pieces: large partials
    need = p.info["workspace_bytes"]
    assert need > 16 << 20
    lib = rpa.load()
    rc = lib.rpa_run_noalloc(p._h, 256, 1, 256, 256, 256, None, None, None)
    assert rpa.STATUS[rc] == "RPA_E_WORKSPACE"
    msg = lib.rpa_last_error().decode()
    assert str(need) in msg and str(16 << 20) in msg
    p.close()
