"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, on the
five workloads at full size and on smaller ragged cases, plus the bitwise
invariances the schedule guarantees (page placement, prefix sharing, padding,
decode row = prefill row, run-to-run determinism).
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_ragged_amd as rpa
import workloads as W
from tests.gpu_util import assert_close, on_device, run, say

pytestmark = pytest.mark.gpu


def ref(b, rows=None):
    return oracle.run(**b.oracle_kwargs(), rows=rows)


# ----------------------------------------------------------------------------------------------
# Small and mid-size ragged batches: every row compared.
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("poison", [False, True])
def test_tiny_ragged_prefill(poison):
    b = W.tiny_ragged_prefill(poison=poison, spare_pages=4 if poison else 0)
    ro, rl = ref(b)
    for splits in (1, 0):
        o, l, _ = run(b, max_kv_splits=splits)
        assert_close(o, l, ro, rl, what="tiny splits=%d" % splits)


SHAPES = [  # (H_qo, H_kv, D, dtype, causal)
    (8, 1, 128, "f16", True),
    (32, 8, 128, "bf16", True),
    (64, 8, 128, "bf16", True),
    (8, 8, 64, "f16", True),
    (12, 1, 128, "bf16", True),   # G = 12: 10 tokens x 12 heads per 128-row tile
    (16, 2, 64, "bf16", False),
    (4, 4, 128, "f16", False),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "h%d_kv%d_d%d_%s_%s" % (s[0], s[1], s[2], s[3],
                                                                                    "causal" if s[4] else "full"))
def test_ragged_shapes(shape):
    H, Hk, D, dt, causal = shape
    q_lens = [1, 17, 64, 3, 130, 0, 1]
    kv_lens = [1, 40, 300, 700, 130, 9, 333]
    b = W.make_batch("ragged", q_lens, kv_lens, num_qo_heads=H, num_kv_heads=Hk, head_dim=D, dtype=dt,
                     seed=31, spare_pages=5, poison=True, causal=causal)
    ro, rl = ref(b)
    for splits, cus in ((1, 0), (0, 0), (0, 4096)):
        o, l, info = run(b, max_kv_splits=splits, num_cus=cus)
        assert_close(o, l, ro, rl, what="%s splits=%d cus=%d" % (shape, splits, cus))
        if cus == 4096:
            assert info["num_split_groups"] > 0  # the split path really ran


@pytest.mark.parametrize("shape", [(8, 1, 128, "f16"), (8, 2, 128, "bf16"), (16, 1, 64, "bf16"), (8, 8, 128, "f16")],
                         ids=lambda s: "h%d_kv%d_d%d_%s" % s)
def test_narrow_tiles(shape):
    """Tiles of at most 16 rows take the decode path: multi-token causal rows (q_len * G
    <= 16), several key steps per wave, key ranges that end mid-step and mid-page."""
    H, Hk, D, dt = shape
    G = H // Hk
    tq = max(1, 16 // G)
    q_lens = [1, tq, 1, tq, 1]
    kv_lens = [1, 77, 1000, 2049, 5000]
    b = W.make_batch("narrow", q_lens, kv_lens, num_qo_heads=H, num_kv_heads=Hk, head_dim=D, dtype=dt, seed=39,
                     spare_pages=3, poison=True)
    ro, rl = ref(b)
    for splits, cus in ((1, 0), (0, 0), (0, 4096)):
        o, l, info = run(b, max_kv_splits=splits, num_cus=cus)
        assert_close(o, l, ro, rl, what="narrow %s splits=%d cus=%d" % (shape, splits, cus))


@pytest.mark.parametrize("head_dim,dtype,causal", [(128, "bf16", True), (128, "f16", False), (64, "bf16", True),
                                                    (64, "f16", False)])
def test_wide_tiles_at_unit_boundaries(head_dim, dtype, causal):
    """Wide tiles (3..40 tokens x 8 heads) whose key ranges end just before, on and
    just after a 32-key unit and a 16-key page, for 1 to 5 units per tile, over a
    cache whose unowned slots hold NaN (the slots past kv_len must read as zero V)."""
    lens = [3, 17, 31, 32, 33, 40, 63, 64, 65, 97, 128, 130, 160]
    b = W.make_batch("unitb", lens, lens, num_qo_heads=8, num_kv_heads=1, head_dim=head_dim, dtype=dtype,
                     seed=41, spare_pages=4, poison=True, causal=causal)
    ro, rl = ref(b)
    for splits in (1, 0):
        o, l, _ = run(b, max_kv_splits=splits)
        assert_close(o, l, ro, rl, what="unit boundaries D%d %s splits=%d" % (head_dim, dtype, splits))


def test_64k_token_sequences_sampled():
    """Long sequences: a decode row and a 256-token prefill chunk over 65536 cached
    tokens each (64 qo / 8 kv heads, bf16), and a 20000-token causal prompt; both
    kernels, splits and the 32-bit index arithmetic at this size."""
    say("generate 64k batch on cuda")
    b = W.make_batch("long64k", [1, 256, 20000], [65536, 65536, 20000], num_qo_heads=64, num_kv_heads=8,
                     head_dim=128, dtype="bf16", seed=51, device="cuda")
    dev = (b.q, b.kv_cache, torch.from_numpy(b.kv_page_indices).cuda())
    rows = [0, 1, 2, 100, 255, 256] + list(range(257, 257 + 20000, 997)) + [257 + 19999]
    ro, rl = ref(b, rows=rows)
    for cus in (0, 65536):  # as planned, and with the long key ranges split
        o, l, info = run(b, dev=dev, num_cus=cus)
        assert cus == 0 or info["num_split_groups"] > 0
        assert_close(o, l, ro, rl, rows=rows, what="64k sampled cus=%d" % cus)


def test_long_single_sequence_splits():
    b = W.make_batch("long1", [5], [4000], num_qo_heads=8, num_kv_heads=1, head_dim=128, dtype="bf16", seed=32)
    ro, rl = ref(b)
    o, l, info = run(b)
    assert info["max_splits"] > 1
    assert_close(o, l, ro, rl, what="long single")


def test_sm_scale_and_no_lse():
    b = W.make_batch("scale", [7, 1], [50, 90], num_qo_heads=8, num_kv_heads=2, head_dim=64, dtype="f16", seed=33)
    ro, rl = oracle.run(**b.oracle_kwargs(), sm_scale=0.05)
    o, l, _ = run(b, sm_scale=0.05)
    assert_close(o, l, ro, rl, what="sm_scale")
    o2, l2, _ = run(b, sm_scale=0.05, return_lse=False)
    assert l2 is None and np.array_equal(o, o2)


# ----------------------------------------------------------------------------------------------
# The five workloads at full size.
# ----------------------------------------------------------------------------------------------

def test_decode_b128_kv1024():
    b = W.decode_b128_kv1024()
    ro, rl = ref(b)
    for splits in (0, 1):
        o, l, info = run(b, max_kv_splits=splits)
        assert_close(o, l, ro, rl, what="decode splits=%d" % splits)
    assert info["num_tiles"] == 128


def test_short_prompt_prefill_and_padded_twin():
    """64 prompts of U{1..200} tokens and the same prompts padded to 200 (real tokens
    first): every real row of the padded run equals the ragged run's bit for bit, O
    and LSE.  The planner puts every row of both batches on the wide path (a
    sequence's path depends on its own length only, and the few rows of the shortest
    prompts join the wide launch), and tiles start at the same token offsets, so each
    row meets the same keys in the same units; the padded run's extra keys are masked
    (exactly zero weight) for real rows."""
    b = W.short_prompt_prefill()
    p = W.short_prompt_prefill(padded=True)
    for batch in (b, p):
        plan = rpa.Plan(batch.qo_indptr, batch.kv_page_indptr, batch.kv_last_page_len,
                        num_qo_heads=batch.num_qo_heads, num_kv_heads=batch.num_kv_heads, head_dim=128,
                        dtype="bf16", max_kv_splits=1)
        assert (plan.tiles()[:, 12] == 0).all(), "every tile wide"
        plan.close()
    ro, rl = ref(b)
    o, l, _ = run(b, max_kv_splits=1)
    assert_close(o, l, ro, rl, what="short prompts")
    po, pl, _ = run(p, max_kv_splits=1)
    pro, prl = ref(p)
    assert_close(po, pl, pro, prl, what="short prompts padded")
    for s in range(b.batch):
        L = int(b.q_lens[s])
        ra = slice(int(b.qo_indptr[s]), int(b.qo_indptr[s]) + L)
        rc = slice(int(p.qo_indptr[s]), int(p.qo_indptr[s]) + L)
        assert np.array_equal(o[ra], po[rc]), "sequence %d (length %d): O differs" % (s, L)
        assert np.array_equal(l[ra], pl[rc]), "sequence %d (length %d): LSE differs" % (s, L)


def test_shared_prefix_suffix_prefill_and_decode_steps():
    sh = W.shared_prefix_suffix()
    du = W.shared_prefix_suffix(duplicated=True)
    ro, rl = ref(sh)
    o, l, _ = run(sh)
    assert_close(o, l, ro, rl, what="shared prefix prefill")
    od, ld, _ = run(du)
    assert np.array_equal(o, od) and np.array_equal(l, ld), "shared and duplicated prefix differ"
    # 50 decode steps, appending one token per request per step
    dev_kv = sh.kv_cache.to("cuda")
    for step in range(1, 51):
        d = W.decode_step(sh, step)
        pos = 229 + step
        pages = torch.from_numpy(d.kv_page_indices.reshape(sh.batch, -1)[:, pos // 16].astype(np.int64))
        dev_kv[pages.cuda(), :, pos % 16] = sh.kv_cache[pages, :, pos % 16].cuda()
        dev = (d.q.cuda(), dev_kv, torch.from_numpy(d.kv_page_indices).cuda())
        o, l, _ = run(d, dev=dev, label="step %d" % step)
        if step in (1, 2, 17, 50):
            rro, rrl = ref(d)
            assert_close(o, l, rro, rrl, what="decode step %d" % step)
            # cacheable K/V loads (the hint for shared pages) give the same bits
            os_, ls_, _ = run(d, dev=dev, label="step %d kv_shared" % step, kv_shared=True)
            assert np.array_equal(o, os_) and np.array_equal(l, ls_), "kv_shared changed step %d" % step


@pytest.mark.parametrize("max_kv_splits", [0, 1])
def test_kv_shared_hint_is_bitwise_neutral(max_kv_splits):
    """The kv_shared caching hint switches narrow-tile K/V loads between
    non-temporal and cacheable; it must not change a bit of O or LSE, on the split
    (row-wise K through LDS off) and the unsplit (row-wise K through LDS) paths."""
    b = W.decode_b128_kv1024(batch=32, kv_len=777)
    dev = on_device(b)
    o0, l0, i0 = run(b, max_kv_splits=max_kv_splits, dev=dev, label="stream")
    o1, l1, i1 = run(b, max_kv_splits=max_kv_splits, dev=dev, label="cached", kv_shared=True)
    assert (i0["num_split_groups"] > 0) == (max_kv_splits == 0)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    ro, rl = ref(b)
    assert_close(o0, l0, ro, rl, what="decode 32 x 777")


def mixed_long_sample_rows(b):
    """All decode rows, plus the last 64 rows and a stride-61 sample of every prompt."""
    rows = []
    for s in range(b.batch):
        a, e = int(b.qo_indptr[s]), int(b.qo_indptr[s + 1])
        if e - a == 1:
            rows.append(a)
        else:
            rows.extend(range(a, e, 61))
            rows.extend(range(e - 64, e))
    return sorted(set(rows))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_mixed_launch_prompts_and_split_decode_rows(dtype):
    """Prompts and decode rows in one plan run in one launch with both kinds of tile
    interleaved; here the decode rows' key ranges are also split (few tiles), so the
    launch holds wide tiles, split narrow pieces and their in-kernel merges.  Checked
    against the oracle, and bitwise against the same plan with cacheable K/V loads."""
    q_lens = [150, 1, 40, 1, 3, 1]
    kv_lens = [150, 9000, 900, 7777, 2500, 16]  # decode rows: 17 MB of K/V, more than joins the wide launch
    b = W.make_batch("mixed_launch", q_lens, kv_lens, num_qo_heads=16, num_kv_heads=2, head_dim=128,
                     dtype=dtype, seed=77, spare_pages=5, poison=True)
    dev = on_device(b)
    o, l, info = run(b, dev=dev, label="mixed launch")
    assert info["num_split_groups"] > 0
    p = rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=16, num_kv_heads=2,
                 head_dim=128, dtype=dtype)
    kinds = p.tiles()[:, 12]
    p.close()
    assert (kinds == 0).any() and (kinds == 1).any() and (np.diff(kinds) < 0).any()  # interleaved
    ro, rl = ref(b)
    assert_close(o, l, ro, rl, what="mixed launch %s" % dtype)
    o2, l2, _ = run(b, dev=dev, label="mixed launch, kv_shared", kv_shared=True)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def test_mixed_long_batch_sampled():
    say("generate mixed_long_batch on cuda")
    b = W.mixed_long_batch(device="cuda")
    rows = mixed_long_sample_rows(b)
    o, l, info = run(b, dev=(b.q, b.kv_cache, torch.from_numpy(b.kv_page_indices).cuda()))
    say("oracle on %d sampled rows" % len(rows))
    ro, rl = ref(b, rows=rows)
    assert_close(o, l, ro, rl, rows=rows, what="mixed long (sampled)")


def test_long_prompts_alone_and_in_the_mixed_batch():
    """The mixed batch's 4 x 8192 prompts planned alone (the wide kernel by itself, as
    the benchmark's prefill leg runs them) against the oracle on sampled rows, and
    bitwise against the same rows of the whole batch's one mixed launch: a prompt's
    rows do not depend on what else the batch holds."""
    say("generate mixed_long_batch on cuda")
    b = W.mixed_long_batch(device="cuda")
    idx = torch.from_numpy(b.kv_page_indices).cuda()
    n = 4
    T = int(b.qo_indptr[n])
    sub = W.Batch("mixed_long_prompts_of_all", b.qo_indptr[:n + 1].copy(), b.kv_page_indptr[:n + 1].copy(),
                  b.kv_page_indices[:int(b.kv_page_indptr[n])].copy(), b.kv_last_page_len[:n].copy(),
                  b.q[:T], b.kv_cache, b.num_qo_heads, b.num_kv_heads, b.head_dim, b.dtype)
    o_all, l_all, info_all = run(b, dev=(b.q, b.kv_cache, idx), label="whole batch")
    o, l, info = run(sub, dev=(sub.q, sub.kv_cache, idx[:len(sub.kv_page_indices)]), label="prompts alone")
    assert info["num_split_groups"] == 0 and info_all["num_split_groups"] == 0
    assert np.array_equal(o, o_all[:T]) and np.array_equal(l, l_all[:T])
    rows = sorted(set(r for s in range(n) for r in list(range(int(sub.qo_indptr[s]), int(sub.qo_indptr[s + 1]), 509))
                      + list(range(int(sub.qo_indptr[s + 1]) - 16, int(sub.qo_indptr[s + 1])))))
    say("oracle on %d sampled prompt rows" % len(rows))
    ro, rl = ref(sub, rows=rows)
    assert_close(o, l, ro, rl, rows=rows, what="long prompts alone (sampled)")


def test_mixed_decode_rows_alone_and_in_the_mixed_batch():
    """The mixed batch's 256 decode rows (kv_len U[512, 8192]) planned alone (the narrow
    kernel by itself, as the benchmark's decode-rows leg runs them) against the oracle
    on sampled rows, and bitwise against the same rows of the whole batch's mixed
    launch, where the same tiles run beside the prompts' wide tiles."""
    say("generate mixed_long_batch on cuda")
    b = W.mixed_long_batch(device="cuda")
    idx = torch.from_numpy(b.kv_page_indices).cuda()
    n = 4
    T0, p0 = int(b.qo_indptr[n]), int(b.kv_page_indptr[n])
    sub = W.Batch("mixed_long_decode_of_all", (b.qo_indptr[n:] - T0).astype(np.int32),
                  (b.kv_page_indptr[n:] - p0).astype(np.int32), b.kv_page_indices[p0:].copy(),
                  b.kv_last_page_len[n:].copy(), b.q[T0:], b.kv_cache, b.num_qo_heads, b.num_kv_heads,
                  b.head_dim, b.dtype)
    o_all, l_all, _ = run(b, dev=(b.q, b.kv_cache, idx), label="whole batch")
    o, l, info = run(sub, dev=(sub.q, sub.kv_cache, idx[p0:]), label="decode rows alone")
    assert info["num_split_groups"] == 0
    assert np.array_equal(o, o_all[T0:]) and np.array_equal(l, l_all[T0:])
    rows = list(range(0, sub.total_q, 5))
    say("oracle on %d sampled decode rows" % len(rows))
    ro, rl = ref(sub, rows=rows)
    assert_close(o, l, ro, rl, rows=rows, what="mixed decode rows alone (sampled)")


@pytest.mark.parametrize("shape", [(1, 2, 64), (4, 1, 128), (16, 1, 64), (2, 3, 128)],
                         ids=lambda s: "g%d_hk%d_d%d" % s)
def test_random_ragged_batches_on_the_gpu(shape):
    """The CPU schedule executor's random ragged batches, run by the kernels with the
    same plans (as made, another machine size, forced splits) against the oracle on
    every row; unowned slots hold NaN."""
    from tests.test_tile_interp import random_ragged_batches
    for b, kws in random_ragged_batches(*shape):
        ro, rl = ref(b)
        dev = on_device(b)
        for kw in kws:
            o, l, _ = run(b, dev=dev, label=str(kw), **kw)
            assert_close(o, l, ro, rl, what="%s %s" % (b.name, kw))


@pytest.mark.parametrize("seed", range(12))
def test_random_configurations_on_the_gpu(seed):
    """The CPU schedule executor's random configurations (G 1..16, 1..8 kv heads, D 64 /
    128, fp16 / bf16, causal or not, sequences without queries, NaN in unowned slots),
    run by the kernels on the MFMA and VALU narrow paths, cacheable or streamed, as
    planned or split, against the oracle on every row."""
    from tests.test_tile_interp import random_config_batch
    b, kws = random_config_batch(seed)
    ro, rl = ref(b)
    dev = on_device(b)
    for kw in kws:
        o, l, _ = run(b, dev=dev, label=str(kw), **kw)
        assert_close(o, l, ro, rl, what="%s %s" % (b.name, kw))


@pytest.mark.parametrize("B", [1, 8, 64, 256])
def test_batch_size_sweep_shapes(B):
    """The batch-size sweep's batches (B causal prompts of 8192 / B tokens, 32 qo / 8 kv
    heads, bf16): the ragged call against the oracle on sampled rows, and its first
    prompt's rows bitwise equal to that prompt's own call (the sweep's one-call-each
    timing)."""
    L = 8192 // B
    b = W.make_batch("sweep_B%d" % B, [L] * B, [L] * B, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                     dtype="bf16", seed=4000 + B, device="cuda")
    idx = torch.from_numpy(b.kv_page_indices).cuda()
    o, l, _ = run(b, dev=(b.q, b.kv_cache, idx), label="batched")
    one = W.Batch("one", np.array([0, L], np.int32), np.array([0, b.kv_page_indptr[1]], np.int32),
                  b.kv_page_indices[:b.kv_page_indptr[1]].copy(), b.kv_last_page_len[:1].copy(), b.q[:L],
                  b.kv_cache, b.num_qo_heads, b.num_kv_heads, b.head_dim, b.dtype)
    o1, l1, _ = run(one, dev=(one.q, one.kv_cache, idx[:len(one.kv_page_indices)]), label="first prompt alone")
    assert np.array_equal(o1, o[:L]) and np.array_equal(l1, l[:L])
    step = max(1, b.total_q // 48)
    rows = sorted(set(list(range(0, b.total_q, step)) + [L - 1, b.total_q - 1]))
    ro, rl = ref(b, rows=rows)
    assert_close(o, l, ro, rl, rows=rows, what="sweep B=%d (sampled)" % B)


# ----------------------------------------------------------------------------------------------
# Bitwise invariances and error handling.
# ----------------------------------------------------------------------------------------------

def test_page_permutation_is_bitwise_invisible():
    b = W.make_batch("perm", [1, 40, 9], [700, 40, 300], num_qo_heads=16, num_kv_heads=2, head_dim=128,
                     dtype="bf16", seed=34, spare_pages=7)
    p = W.permute_pages(b, seed=35)
    o1, l1, _ = run(b)
    o2, l2, _ = run(p)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("case", [
    # (H_qo, H_kv, prefill q_len, same tile path for both calls?)
    (32, 1, 21, True),   # G = 32: a single decode token already fills a wide tile
    (8, 1, 2, True),     # 2 tokens x 8 heads = 16 rows: both calls take the narrow path
    (8, 2, 21, False),   # prefill tile wide, decode tile narrow
], ids=["wide_wide", "narrow_narrow", "wide_narrow"])
def test_decode_row_equals_prefill_row(case):
    """A prefill row at position p against a q_len = 1 call over the first p + 1
    tokens: bit-identical when both calls use the same tile path; otherwise within the
    allclose(atol=1e-3, rtol=1e-3) that flashinfer issue #323's repro asserts between
    its decode and prefill outputs (and each within the oracle tolerance)."""
    H, Hk, ql, same_path = case
    kvl = 337
    b = W.make_batch("pf", [ql], [kvl], num_qo_heads=H, num_kv_heads=Hk, head_dim=128, dtype="f16", seed=36)
    o, l, _ = run(b, max_kv_splits=1)
    ro, rl = ref(b)
    assert_close(o, l, ro, rl, what="prefill")
    for i in sorted({0, ql // 2, ql - 1}):
        pos = kvl - ql + i
        npg = W.pages_for(pos + 1)
        d = W.Batch("dec", np.array([0, 1], np.int32), np.array([0, npg], np.int32), b.kv_page_indices[:npg].copy(),
                    np.array([W.last_page_len_for(pos + 1)], np.int32), b.q[i:i + 1].clone(), b.kv_cache, H, Hk,
                    128, "f16")
        od, ld, _ = run(d, max_kv_splits=1, label="row %d" % i)
        if same_path:
            assert np.array_equal(od[0], o[i]) and np.array_equal(ld[0], l[i]), "row %d" % i
        else:
            np.testing.assert_allclose(od[0], o[i], atol=1e-3, rtol=1e-3)
            assert_close(od[:1], ld[:1], ro[i:i + 1], rl[i:i + 1], what="decode row %d" % i)


def test_runs_are_deterministic():
    b = W.make_batch("det", [1, 100, 7, 1], [2000, 100, 900, 64], num_qo_heads=32, num_kv_heads=8, head_dim=128,
                     dtype="bf16", seed=37)
    dev = on_device(b)
    o1, l1, info = run(b, dev=dev)
    assert info["num_split_groups"] > 0
    o2, l2, _ = run(b, dev=dev)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_out_of_range_page_index_is_flagged_not_read():
    import paged_kv_attention_ragged_amd as rpa
    b = W.make_batch("oob", [3, 1], [40, 20], num_qo_heads=8, num_kv_heads=1, head_dim=64, dtype="f16", seed=38)
    q, kv, idx = on_device(b)
    say("oob flag: page index %d with num_pages declared %d" % (int(b.kv_page_indices.max()), int(b.kv_page_indices.max())))
    plan = rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=8, num_kv_heads=1,
                    head_dim=64, dtype="f16")
    # declare fewer pages than the table references: the kernel must not read them
    plan.bind(idx, num_pages=int(b.kv_page_indices.max()))
    plan.num_pages = kv.shape[0]  # the binding checks kv_cache against its declared size
    plan.run(q, kv)
    plan.upload()  # a schedule re-upload (a graph replay's first node) keeps the error word
    with pytest.raises(rpa.RPAError) as e:
        plan.check()
    assert e.value.status == "RPA_E_PAGE_OOB"
    assert plan.check() == 0  # read and cleared
    plan.close()


@pytest.mark.parametrize("head_dim,dtype", [(64, "f16"), (128, "bf16")])
@pytest.mark.parametrize("splits", [1, 0])
def test_out_of_range_page_reads_as_zero(head_dim, dtype, splits):
    """The keys of a page whose index lies outside [0, num_pages) count as zero K and
    V (and the flag is raised): the output equals the oracle's over a cache in which
    that index names an all-zero page.  Sequence 0 takes the wide path (3 tokens x 8
    heads), sequence 1 the narrow one (1 token); a middle page of each is bad."""
    import paged_kv_attention_ragged_amd as rpa
    b = W.make_batch("oobz", [3, 1], [100, 70], num_qo_heads=8, num_kv_heads=1, head_dim=head_dim,
                     dtype=dtype, seed=39)
    n_pages = b.kv_cache.shape[0]
    bad_idx = b.kv_page_indices.copy()
    for s in range(2):
        bad_idx[int(b.kv_page_indptr[s]) + 2 - s] = n_pages  # one past the last page
    # oracle: the same indices over a cache with one more page, all zeros
    zero_page = torch.zeros((1,) + tuple(b.kv_cache.shape[1:]), dtype=b.kv_cache.dtype)
    kw = b.oracle_kwargs()
    kw.update(kv_page_indices=bad_idx, kv_cache=torch.cat([b.kv_cache, zero_page]))
    say("oob zero: D=%d %s splits=%d" % (head_dim, dtype, splits))
    ro, rl = oracle.run(**kw)
    q, kv, _ = on_device(b)
    plan = rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=8, num_kv_heads=1,
                    head_dim=head_dim, dtype=dtype, max_kv_splits=splits)
    plan.bind(torch.from_numpy(bad_idx.astype(np.int32)).cuda(), num_pages=n_pages)
    o, lse = plan.run(q, kv, return_lse=True)
    torch.cuda.synchronize()
    with pytest.raises(rpa.RPAError) as e:
        plan.check()
    assert e.value.status == "RPA_E_PAGE_OOB"
    plan.close()
    assert_close(o.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl, what="bad page as zeros")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_tail_skip_switch_changes_no_result(dtype, monkeypatch):
    """With RPA_DISABLE_TAIL_SKIP=1 the wide tiles of causal prompts walk to kv_len and
    mask the keys the skip would leave out (whole units masked for every row).  Masked
    keys add exact zeros, so without splits (the same pieces either way) the output is
    bitwise that of the skipping plan; with splits (other piece boundaries) it is held
    to the oracle."""
    b = W.make_batch("tailskip", [700, 300, 129, 1], [700, 450, 129, 600], num_qo_heads=8, num_kv_heads=1,
                     head_dim=128, dtype=dtype, seed=41)
    ro, rl = oracle.run(**b.oracle_kwargs())
    dev = on_device(b)
    o_on, l_on, _ = run(b, max_kv_splits=1, dev=dev, label="skip")
    monkeypatch.setenv("RPA_DISABLE_TAIL_SKIP", "1")
    o_off, l_off, _ = run(b, max_kv_splits=1, dev=dev, label="no skip")
    assert np.array_equal(o_on, o_off) and np.array_equal(l_on, l_off)
    o_sp, l_sp, info = run(b, num_cus=4096, dev=dev, label="no skip, split")
    assert info["num_split_groups"] > 0
    assert_close(o_sp, l_sp, ro, rl, what="no tail skip, split")
    assert_close(o_off, l_off, ro, rl, what="no tail skip")


def test_binding_checks_sizes_the_library_cannot():
    """Sizes the C ABI cannot see: a page-index array shorter than the plan's page
    table (at bind, and after an update that grows the table), a wrong-shaped LSE
    buffer, and a wrong-sized output on the allocation-free path are refused in the
    binding, before any launch."""
    b = W.tiny_ragged_prefill()
    q, kv, idx = on_device(b)
    plan = rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=8, num_kv_heads=1,
                    head_dim=64, dtype="f16")
    with pytest.raises(ValueError, match="kv_page_indices"):
        plan.bind(idx[:-1], num_pages=kv.shape[0])
    plan.bind(idx, num_pages=kv.shape[0])
    with pytest.raises(ValueError, match="lse"):
        plan.run(q, kv, lse=torch.empty((q.shape[0], 7), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError, match="out"):
        plan.run_noalloc(q, kv, idx, torch.empty((q.shape[0] - 1,) + tuple(q.shape[1:]), dtype=q.dtype,
                                                 device="cuda"))
    grown = b.kv_page_indptr.copy()
    grown[-1] += 1  # the last sequence one page longer: more entries than the bound array holds
    with pytest.raises(ValueError, match="bind a larger array"):
        plan.update(b.qo_indptr, grown, b.kv_last_page_len)
    o = plan.run(q, kv)  # the plan is unchanged and still runs
    torch.cuda.synchronize()
    plan.check()
    plan.close()
    assert torch.isfinite(o.float()).all()
