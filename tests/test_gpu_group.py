"""GPU parity of shared-prefix plans (rpa_plan_create_shared): decode rows of
several requests grouped in one tile over the prefix they share (vLLM issue #227,
"Question about efficient memory sharing"), against the fp64 oracle, beside
ordinary tiles in the same launch, through update and graph replay, and on the
no-allocation path.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_ragged_amd as rpa
import workloads as W
from tests.gpu_util import assert_close, on_device, run, say

pytestmark = pytest.mark.gpu


def share_prefix(b: W.Batch, pages: int) -> W.Batch:
    """Point the first `pages` page-table entries of every sequence with at least that
    many pages at the first sequence's pages (a prefix stored once).  Layout only."""
    idx = b.kv_page_indices.copy()
    first = idx[b.kv_page_indptr[0]:b.kv_page_indptr[0] + pages].copy()
    for s in range(b.batch):
        a = int(b.kv_page_indptr[s])
        if int(b.kv_page_indptr[s + 1]) - a >= pages:
            idx[a:a + pages] = first
    return W.Batch(b.name + "_shared%d" % pages, b.qo_indptr, b.kv_page_indptr, idx, b.kv_last_page_len, b.q,
                   b.kv_cache, b.num_qo_heads, b.num_kv_heads, b.head_dim, b.dtype, b.causal)


def run_grouped(b, shared_pages, dev=None, **kw):
    say("grouped %s shared_pages=%d T=%d %s" % (b.name, shared_pages, b.total_q, kw))
    q, kv, idx = dev if dev is not None else on_device(b)
    plan = rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=b.num_qo_heads,
                    num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, dtype=b.dtype, causal=b.causal,
                    shared_pages=shared_pages, **kw)
    kinds = plan.tiles()[:, 12]
    plan.bind(idx, num_pages=kv.shape[0])
    o, lse = plan.run(q, kv, return_lse=True)
    torch.cuda.synchronize()
    plan.check()
    plan.close()
    return o.double().cpu().numpy(), lse.double().cpu().numpy(), kinds


def test_shared_prefix_decode_steps_grouped():
    """The shared-prefix workload's 50 decode steps (256 requests, 12 shared pages, 4
    query heads per kv head): every step as four-request group tiles, against the
    oracle on several steps and within tolerance of the ungrouped plan on all."""
    base = W.shared_prefix_suffix()
    kv = base.kv_cache.to("cuda")
    for step in range(1, 51):
        d = W.decode_step(base, step)
        pos = 229 + step
        pages = torch.from_numpy(d.kv_page_indices.reshape(base.batch, -1)[:, pos // 16].astype(np.int64))
        kv[pages.cuda(), :, pos % 16] = base.kv_cache[pages, :, pos % 16].cuda()
        dev = (d.q.cuda(), kv, torch.from_numpy(d.kv_page_indices).cuda())
        o, l, kinds = run_grouped(d, 12, dev=dev, kv_shared=True)
        assert (kinds == 2).all()
        o_direct, l_direct, _ = run(d, dev=dev, label="step %d direct" % step, kv_shared=True)
        assert_close(o, l, o_direct, l_direct, what="grouped vs direct step %d" % step)
        if step in (1, 2, 3, 17, 33, 50):
            ro, rl = oracle.run(**d.oracle_kwargs())
            assert_close(o, l, ro, rl, what="grouped decode step %d" % step)


@pytest.mark.parametrize("seed", range(6))
def test_random_grouped_batches_on_the_gpu(seed):
    """The CPU schedule executor's random shared-prefix mixes, run by the kernels: as
    planned and with forced splits, against the oracle on every row."""
    from tests.test_tile_interp import random_grouped_batch
    b, P = random_grouped_batch(seed)
    ro, rl = oracle.run(**b.oracle_kwargs())
    dev = on_device(b)
    for kw in ({}, {"num_cus": 4096}):
        o, l, kinds = run_grouped(b, P, dev=dev, **kw)
        assert_close(o, l, ro, rl, what="random grouped seed %d %s" % (seed, kw))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_grouped_page_slot_edges_on_the_gpu(dtype):
    """Group tiles with no private pages and with steps whose two 16-key blocks belong
    to different members (or to a member's empty padding page), against the oracle."""
    from tests.test_tile_interp import grouped_page_edges_batch
    b, P = grouped_page_edges_batch(dtype)
    ro, rl = oracle.run(**b.oracle_kwargs())
    o, l, kinds = run_grouped(b, P)
    assert (kinds == 2).any()
    assert_close(o, l, ro, rl, what="grouped page-slot edges %s" % dtype)


def test_long_shared_prefix_decode_step_grouped():
    """One decode step of 256 requests over a 4096-token shared prefix (256 shared
    pages; the benchmark's long-prefix leg): grouped tiles against the oracle on
    sampled rows, and within tolerance of the direct plan on every row."""
    base = W.shared_prefix_suffix(prefix=4096, decode_steps=1)
    d = W.decode_step(base, 1)
    n_sh = len(base.extra["shared"])
    assert n_sh == 256
    dev = on_device(d)
    o, l, kinds = run_grouped(d, n_sh, dev=dev, kv_shared=True)
    assert (kinds == 2).all()
    o_direct, l_direct, _ = run(d, dev=dev, label="long prefix direct", kv_shared=True)
    assert_close(o, l, o_direct, l_direct, what="long prefix grouped vs direct")
    rows = list(range(0, d.total_q, 7))
    ro, rl = oracle.run(**d.oracle_kwargs(), rows=rows)
    assert_close(o, l, ro, rl, rows=rows, what="long prefix grouped (sampled)")


@pytest.mark.parametrize("shape", [(32, 8, 128, "bf16", 12), (16, 2, 128, "f16", 5), (8, 4, 64, "bf16", 3),
                                   (8, 1, 64, "f16", 7)], ids=lambda s: "h%d_kv%d_d%d_%s_p%d" % s)
def test_grouped_rows_beside_ordinary_tiles(shape):
    """Decode rows over a shared prefix of P pages (odd P: a half-full last shared step)
    with varied own lengths, beside prompts (wide tiles), decode rows too short to see
    the whole prefix, and a decode row long enough to stay alone: one plan, one launch,
    against the oracle; NaN in every unowned slot."""
    H, Hk, D, dt, P = shape
    Ks = 16 * P
    q = [1, 1, 1, 37, 1, 1, 1, 1, 1, 1, 1, 5, 1, 1]
    kv = [Ks + 1, Ks + 40, Ks, Ks + 100, Ks - 9, Ks + 33, Ks + 31, Ks + 2000, Ks + 7, Ks + 64, Ks + 65,
          Ks + 50, Ks + 3, Ks + 90]
    b = share_prefix(W.make_batch("grp_mix", q, kv, num_qo_heads=H, num_kv_heads=Hk, head_dim=D, dtype=dt,
                                  seed=71, spare_pages=3, poison=True), P)
    ro, rl = oracle.run(**b.oracle_kwargs())
    for splits in (0, 1):
        o, l, kinds = run_grouped(b, P, max_kv_splits=splits)
        assert (kinds == 2).any() and ((kinds == 0) | (kinds == 1)).any()
        assert_close(o, l, ro, rl, what="grouped mix %s splits=%d" % (shape, splits))


def test_grouped_plan_is_deterministic_and_hint_neutral():
    b = share_prefix(W.make_batch("grp_det", [1] * 64, [16 * 12 + (7 * i) % 90 for i in range(64)],
                                  num_qo_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16", seed=72), 12)
    dev = on_device(b)
    o1, l1, k1 = run_grouped(b, 12, dev=dev)
    o2, l2, _ = run_grouped(b, 12, dev=dev)
    o3, l3, _ = run_grouped(b, 12, dev=dev, kv_shared=True)
    assert (k1 == 2).any()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


def test_grouped_decode_loop_graph_matches_eager():
    """[upload, run] captured once for a grouped plan, replayed after rpa_plan_update for
    each new step's lengths (the sequence table is part of the upload): bitwise equal
    to a freshly built grouped plan run eagerly."""
    base = W.shared_prefix_suffix(n_req=64)
    kv = base.kv_cache.cuda()
    n, H, Hk, D = base.batch, base.num_qo_heads, base.num_kv_heads, base.head_dim
    cap = n * base.extra["pages_req"]
    q_buf = torch.empty(n, H, D, dtype=kv.dtype, device="cuda")
    ix_buf = torch.zeros(cap, dtype=torch.int32, device="cuda")
    o_buf = torch.empty(n, H, D, dtype=kv.dtype, device="cuda")
    l_buf = torch.empty(n, H, dtype=torch.float32, device="cuda")
    d = W.decode_step(base, 1)
    kv.copy_(base.kv_cache.cuda())

    def load(d):
        q_buf.copy_(d.q.cuda())
        ix_buf[:len(d.kv_page_indices)].copy_(torch.from_numpy(d.kv_page_indices))
        kv.copy_(base.kv_cache.cuda())

    load(d)
    plan = rpa.Plan(d.qo_indptr, d.kv_page_indptr, d.kv_last_page_len, num_qo_heads=H, num_kv_heads=Hk,
                    head_dim=D, dtype=d.dtype, shared_pages=12)
    plan.bind(ix_buf, num_pages=kv.shape[0])
    torch.cuda.synchronize()
    say("capture grouped decode graph")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.upload()
        plan.run(q_buf, kv, out=o_buf, lse=l_buf, return_lse=True)
    torch.cuda.synchronize()
    for step in range(1, 21):
        if step > 1:
            d = W.decode_step(base, step)
            load(d)
            plan.update(d.qo_indptr, d.kv_page_indptr, d.kv_last_page_len)
        g.replay()
        torch.cuda.synchronize()
        assert plan.check() == 0
        e = rpa.Plan(d.qo_indptr, d.kv_page_indptr, d.kv_last_page_len, num_qo_heads=H, num_kv_heads=Hk,
                     head_dim=D, dtype=d.dtype, shared_pages=12)
        assert (e.tiles()[:, 12] == 2).all()
        e.bind(ix_buf, num_pages=kv.shape[0])
        o_e, l_e = e.run(q_buf, kv, return_lse=True)
        torch.cuda.synchronize()
        e.close()
        assert torch.equal(o_buf.view(torch.int16), o_e.view(torch.int16)) and torch.equal(l_buf, l_e), step
    ro, rl = oracle.run(**d.oracle_kwargs())
    assert_close(o_buf.double().cpu().numpy(), l_buf.double().cpu().numpy(), ro, rl, what="graph grouped step 20")
    plan.close()


def test_grouped_plan_on_the_noalloc_path():
    """rpa_run_noalloc copies the sequence table beside the tiles: same bits as rpa_run."""
    b = share_prefix(W.make_batch("grp_na", [1] * 24, [16 * 6 + 3 * i for i in range(24)], num_qo_heads=16,
                                  num_kv_heads=4, head_dim=128, dtype="f16", seed=73), 6)
    q, kv, idx = on_device(b)
    p = rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=16, num_kv_heads=4,
                 head_dim=128, dtype="f16", shared_pages=6)
    assert (p.tiles()[:, 12] == 2).any()
    o = torch.empty_like(q)
    lse = torch.empty((b.total_q, 16), dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("grouped noalloc")
    p.run_noalloc(q, kv, idx, o, lse=lse, err_flag=flag)
    p.bind(idx, num_pages=kv.shape[0])
    o2, l2 = p.run(q, kv, return_lse=True)
    torch.cuda.synchronize()
    assert flag.item() == 0
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)
    p.close()
