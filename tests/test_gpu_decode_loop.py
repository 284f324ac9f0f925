"""GPU tests of the decode loop pieces: rpa_append_kv (new tokens' K/V into their
page slots, bit-exact) and a HIP-graph-captured decode step [plan upload, append,
attention] replayed for 50 steps with rpa_plan_update between replays (vLLM issue
#227's 50 generated tokens after a 200 + 30 token prompt; flashinfer issue #323's
plan-once / run-many lifecycle).  Every replay is checked against an eager run of
a freshly built plan (same schedule, same kernels: bitwise), and some against the
oracle."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_ragged_amd as rpa
import workloads as W
from tests.gpu_util import assert_close, say

pytestmark = pytest.mark.gpu


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).cuda()


def new_token_rows(base, d):
    """K/V the harness appended for decode batch d: [n_req, 2, H_kv, D], read from
    base.kv_cache (host) at each sequence's last position."""
    ps = d.page_size
    rows = []
    for s in range(d.batch):
        pos = int(d.kv_lens[s]) - 1
        pg = d.kv_page_indices[d.kv_page_indptr[s] + pos // ps]
        rows.append(base.kv_cache[pg, :, pos % ps])
    return torch.stack(rows).contiguous()


def test_append_kv_writes_the_slots_the_page_table_names():
    base = W.shared_prefix_suffix()
    kv = base.kv_cache.cuda()
    d = W.decode_step(base, 1)  # writes the new tokens into base.kv_cache (host)
    new = new_token_rows(base, d).cuda()
    say("append_kv %d tokens" % d.batch)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    rpa.append_kv(new, kv, i32(np.arange(d.batch + 1)), i32(d.kv_page_indptr), i32(d.kv_page_indices),
                  i32(d.kv_last_page_len), err_flag=flag)
    torch.cuda.synchronize()
    assert flag.item() == 0
    assert torch.equal(kv.cpu().view(torch.int16), base.kv_cache.view(torch.int16))
    # several tokens per sequence (a suffix of 3), and a bad page: flagged, not written
    g = torch.Generator("cpu").manual_seed(31)
    n = 3
    new3 = torch.randn(2 * n, 2, base.num_kv_heads, base.head_dim, generator=g).to(kv.dtype)
    npg = int(d.kv_page_indptr[1])  # pages per request (15 for 231 tokens)
    ix = d.kv_page_indices[:2 * npg].astype(np.int32)  # the first two requests' own page lists
    ip2 = np.array([0, npg, 2 * npg], np.int32)
    last = d.kv_last_page_len[:2].astype(np.int32)
    ref = kv.clone()
    rpa.append_kv(new3.cuda(), kv, i32([0, n, 2 * n]), i32(ip2), i32(ix), i32(last), err_flag=flag)
    torch.cuda.synchronize()
    for s in range(2):
        L = int((ip2[s + 1] - ip2[s] - 1) * 16 + last[s])
        for j in range(n):
            pos = L - n + j
            ref[int(ix[ip2[s] + pos // 16]), :, pos % 16] = new3[s * n + j].cuda()
    assert flag.item() == 0 and torch.equal(kv.view(torch.int16), ref.view(torch.int16))
    bad = ix.copy()
    bad[ip2[1] + (int((ip2[2] - ip2[1] - 1) * 16 + last[1]) - 1) // 16] = kv.shape[0]  # seq 1's last page
    before = kv.clone()
    rpa.append_kv(new3[:2].cuda(), kv, i32([0, 1, 2]), i32(ip2), i32(bad), i32(last), err_flag=flag)
    torch.cuda.synchronize()
    assert flag.item() == 1
    s0 = int((ip2[1] - 1) * 16 + last[0]) - 1
    before[int(ix[s0 // 16]), :, s0 % 16] = new3[0].cuda()  # seq 0's token lands; seq 1's does not
    assert torch.equal(kv.view(torch.int16), before.view(torch.int16))


def test_graph_captured_decode_loop_matches_eager_and_oracle():
    base = W.shared_prefix_suffix()
    n_req, H, Hk, D = base.batch, base.num_qo_heads, base.num_kv_heads, base.head_dim
    kv = base.kv_cache.cuda()
    cap = n_req * base.extra["pages_req"]
    # fixed device buffers the graph reads; refreshed by ordinary copies before each replay
    q_buf = torch.empty(n_req, H, D, dtype=kv.dtype, device="cuda")
    new_buf = torch.empty(n_req, 2, Hk, D, dtype=kv.dtype, device="cuda")
    ip_buf = torch.zeros(n_req + 1, dtype=torch.int32, device="cuda")
    ix_buf = torch.zeros(cap, dtype=torch.int32, device="cuda")
    kl_buf = torch.zeros(n_req, dtype=torch.int32, device="cuda")
    ai_buf = i32(np.arange(n_req + 1))
    o_buf = torch.empty(n_req, H, D, dtype=kv.dtype, device="cuda")
    l_buf = torch.empty(n_req, H, dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")

    def load_step(d):
        q_buf.copy_(d.q.cuda())
        new_buf.copy_(new_token_rows(base, d).cuda())
        ip_buf.copy_(i32(d.kv_page_indptr))
        ix_buf[:len(d.kv_page_indices)].copy_(i32(d.kv_page_indices))
        kl_buf.copy_(i32(d.kv_last_page_len))

    d = W.decode_step(base, 1)
    load_step(d)
    plan = rpa.Plan(d.qo_indptr, d.kv_page_indptr, d.kv_last_page_len, num_qo_heads=H, num_kv_heads=Hk,
                    head_dim=D, dtype=d.dtype)
    plan.bind(ix_buf, num_pages=kv.shape[0])
    torch.cuda.synchronize()
    say("capture decode step graph")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.upload()
        rpa.append_kv(new_buf, kv, ai_buf, ip_buf, ix_buf, kl_buf, err_flag=flag)
        plan.run(q_buf, kv, out=o_buf, lse=l_buf, return_lse=True)
    torch.cuda.synchronize()
    for step in range(1, 51):
        if step > 1:
            d = W.decode_step(base, step)
            load_step(d)
            plan.update(d.qo_indptr, d.kv_page_indptr, d.kv_last_page_len)
        say("replay step %d" % step)
        g.replay()
        torch.cuda.synchronize()
        assert flag.item() == 0
        # the plan's error word (bad pages, bf16 V range) survives the graph's upload
        # node and is read and cleared here, step by step
        assert plan.check() == 0
        o_g, l_g = o_buf.clone(), l_buf.clone()
        # eager: a new plan for the same lengths over the same (already appended) cache
        e = rpa.Plan(d.qo_indptr, d.kv_page_indptr, d.kv_last_page_len, num_qo_heads=H, num_kv_heads=Hk,
                     head_dim=D, dtype=d.dtype)
        e.bind(ix_buf, num_pages=kv.shape[0])
        o_e, l_e = e.run(q_buf, kv, return_lse=True)
        torch.cuda.synchronize()
        e.close()
        assert torch.equal(o_g.view(torch.int16), o_e.view(torch.int16)) and torch.equal(l_g, l_e), step
        if step in (1, 17, 50):
            say("oracle step %d" % step)
            ro, rl = oracle.run(**d.oracle_kwargs())
            assert_close(o_g.double().cpu().numpy(), l_g.double().cpu().numpy(), ro, rl,
                         what="graph decode step %d" % step)
    # the cache holds exactly what the harness appended
    assert torch.equal(kv.cpu().view(torch.int16), base.kv_cache.view(torch.int16))
    plan.close()
