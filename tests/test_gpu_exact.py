"""GPU edge cases of the HIP path, through the C ABI:

  * exactness of the page-table indexing as a value: a key equal to 64 x its query
    (one-hot: every other key's weight underflows to 0) makes O equal that key's V
    bit for bit, on the wide path (prefill), the narrow path (decode rows) and the
    split path (pieces merged in the kernel);
  * large logits (|sm_scale q.k| far above the wide path's lazy-rescale threshold of
    8 in log2 units) against the fp64 oracle, on every path;
  * bf16 V outside the fp16 range of the P V product: flagged (RPA_E_V_RANGE), never
    silently wrong; in-range extremes are not flagged and match the oracle; the VALU
    decode kernel, which multiplies in fp32, takes any bf16 V;
  * run-to-run determinism of plans with many split groups (fused merges), 100 runs.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_ragged_amd as rpa
import workloads as W
from tests.gpu_util import assert_close, on_device, run, say

pytestmark = pytest.mark.gpu

# A power of two, so alpha * q is exact in fp16 and bf16.  With N(0,1) queries a
# row's own key scores alpha |q|^2 / sqrt(D) (about 8 alpha at D = 64) and another
# one-hot key alpha q.q' / sqrt(D), about N(0, alpha^2): the gap, roughly
# alpha (sqrt(D) - 3.5), is at least 98 (natural log) for the batches below, so
# every other key's weight is below 2^-141: nothing next to a V value of 2^-14 or
# more, even in fp32.
ALPHA = 64.0


def slot(b: W.Batch, s: int, t: int):
    """(page, slot) of token t of sequence s."""
    return int(b.kv_page_indices[b.kv_page_indptr[s] + t // 16]), t % 16


def fp16_exact_v(b: W.Batch):
    """V values of magnitude below 2^-14 (zeros included) become +-2^-14.  For bf16
    V such values would round toward zero in the fp16 P V product (an error under
    2^-24); and O[t] = V[t] bit for bit needs every V[t] element well above the
    weights of the other keys, which are tiny but not zero (they are in the oracle
    too): next to an exact 0 they would survive as a tiny value that bf16 can hold."""
    v = b.kv_cache[:, 1]
    tiny = v.abs() < 2.0 ** -14
    v[tiny] = torch.where(v[tiny] < 0, -(2.0 ** -14), 2.0 ** -14).to(v.dtype)


def bits(x):
    return x.view(torch.int16).numpy() if isinstance(x, torch.Tensor) else x


def gpu_o(b, **kw):
    """O and LSE as the kernel wrote them (int16 bit patterns of O)."""
    q, kv, idx = on_device(b)
    plan = rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=b.num_qo_heads,
                    num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, dtype=b.dtype, causal=b.causal, **kw)
    plan.bind(idx, num_pages=kv.shape[0])
    o, lse = plan.run(q, kv, return_lse=True)
    torch.cuda.synchronize()
    plan.check()
    info = plan.info
    kinds = plan.tiles()[:, 12]
    plan.close()
    return o.cpu(), lse.cpu(), info, kinds


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_one_hot_key_selects_its_value_on_the_wide_path(dtype, head_dim):
    """Prefill with one kv head per query head (so each query can own a key): key t of
    every sequence is 64 x query t, head by head.  Row t sees keys 0..t; its own key
    scores 64 |q|^2 / sqrt(D) (about 720 at D = 128), the others about N(0, 64^2),
    so every other weight is negligible and O[t] = V[t] exactly."""
    say("one-hot wide %s D%d" % (dtype, head_dim))
    b = W.make_batch("onehot_wide", [300, 130, 1], [300, 130, 1], num_qo_heads=8, num_kv_heads=8,
                     head_dim=head_dim, dtype=dtype, seed=61, spare_pages=3)
    fp16_exact_v(b)
    for s in range(b.batch):
        for t in range(int(b.q_lens[s])):
            pg, sl = slot(b, s, t)
            b.kv_cache[pg, 0, sl] = b.q[int(b.qo_indptr[s]) + t] * ALPHA
    for kw in (dict(max_kv_splits=1), dict(num_cus=4096)):  # direct, and split with in-kernel merges
        o, lse, info, kinds = gpu_o(b, **kw)
        assert (kinds == 0).all()
        assert kw.get("num_cus") is None or info["num_split_groups"] > 0
        for s in range(b.batch):
            for t in range(int(b.q_lens[s])):
                pg, sl = slot(b, s, t)
                r = int(b.qo_indptr[s]) + t
                assert np.array_equal(bits(o[r]), bits(b.kv_cache[pg, 1, sl])), (kw, s, t)
    ro, rl = oracle.run(**b.oracle_kwargs())
    assert_close(o.double().numpy(), lse.double().numpy(), ro, rl, what="one-hot wide")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("splits", [1, 0])
def test_one_hot_key_selects_its_value_on_the_narrow_path(dtype, splits):
    """Decode rows (8 query heads per kv head): for head g of row b, a key at a
    position of its own is 64 x that head's query, so O[b, g] is that key's V bit for
    bit, through the 4-wave combine and, split, the in-kernel merge."""
    say("one-hot narrow %s splits=%d" % (dtype, splits))
    B, L = 24, 1500
    b = W.make_batch("onehot_narrow", [1] * B, [L] * B, num_qo_heads=8, num_kv_heads=1, head_dim=128,
                     dtype=dtype, seed=62, spare_pages=2)
    fp16_exact_v(b)
    rng = np.random.default_rng(62)
    pos = np.stack([rng.choice(L, 8, replace=False) for _ in range(B)])
    for s in range(B):
        for g in range(8):
            pg, sl = slot(b, s, int(pos[s, g]))
            b.kv_cache[pg, 0, sl, 0] = b.q[s, g] * ALPHA
    o, lse, info, kinds = gpu_o(b, max_kv_splits=splits)
    assert (kinds == 1).all() and (splits == 1) == (info["num_split_groups"] == 0)
    for s in range(B):
        for g in range(8):
            pg, sl = slot(b, s, int(pos[s, g]))
            assert np.array_equal(bits(o[s, g]), bits(b.kv_cache[pg, 1, sl, 0])), (s, g)
    ro, rl = oracle.run(**b.oracle_kwargs())
    assert_close(o.double().numpy(), lse.double().numpy(), ro, rl, what="one-hot narrow")


def scaled_batch(name, q_lens, kv_lens, scale, seed, **kw):
    b = W.make_batch(name, q_lens, kv_lens, seed=seed, **kw)
    b.q.mul_(scale)
    b.kv_cache[:, 0].mul_(scale)
    return b


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_large_logits_match_the_oracle(dtype):
    """Q and K scaled by 4: scores sm_scale q.k have standard deviation 16 (23 in log2
    units), so the running maximum moves by far more than the wide path's lazy
    threshold (8) many times per row, and most weights underflow.  Prompts (wide
    tiles), decode rows (narrow), with and without split key ranges, against the
    oracle."""
    say("large logits %s" % dtype)
    b = scaled_batch("large_logits", [200, 37, 1, 1, 5], [200, 900, 3000, 64, 700], 4.0, 63,
                     num_qo_heads=16, num_kv_heads=2, head_dim=128, dtype=dtype, spare_pages=3, poison=True)
    ro, rl = oracle.run(**b.oracle_kwargs())
    assert np.abs(rl).max() > 40  # the logits are large indeed
    for splits, cus in ((1, 0), (0, 0), (0, 4096)):
        o, l, info = run(b, max_kv_splits=splits, num_cus=cus)
        assert_close(o, l, ro, rl, what="large logits splits=%d cus=%d" % (splits, cus))
    # a sharper softmax still: sm_scale 1 (8 x the default at D = 64)
    b2 = scaled_batch("large_logits_scale1", [64, 1], [64, 500], 1.0, 64, num_qo_heads=8, num_kv_heads=1,
                      head_dim=64, dtype=dtype)
    ro2, rl2 = oracle.run(**b2.oracle_kwargs(), sm_scale=1.0)
    o2, l2, _ = run(b2, sm_scale=1.0)
    assert_close(o2, l2, ro2, rl2, what="sm_scale 1")


def planted_v(value, seed):
    """bf16 batch (a prompt on the wide path, decode rows on the narrow path) with
    `value` planted in V of one visible key of each sequence, head 0."""
    b = W.make_batch("vrange", [40, 1, 1], [40, 500, 3000], num_qo_heads=16, num_kv_heads=2, head_dim=128,
                     dtype="bf16", seed=seed, spare_pages=2)
    for s, t in ((0, 7), (1, 123), (2, 2999)):
        pg, sl = slot(b, s, t)
        b.kv_cache[pg, 1, sl, 0, 5] = value
    return b


@pytest.mark.parametrize("kernel", ["mfma", "valu"])
def test_bf16_v_above_the_fp16_range_is_flagged(kernel):
    """bf16 V of magnitude above 65504 would saturate in the fp16 P V product: the MFMA
    paths (wide and narrow tiles) raise RPA_E_V_RANGE instead of returning a silently
    wrong O; the VALU decode kernel multiplies in fp32 and matches the oracle."""
    b = planted_v(-1.0e5, 65)
    ro, rl = oracle.run(**b.oracle_kwargs())
    for splits in (1, 0):
        say("V range flag kernel=%s splits=%d" % (kernel, splits))
        q, kv, idx = on_device(b)
        plan = rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=16, num_kv_heads=2,
                        head_dim=128, dtype="bf16", max_kv_splits=splits, narrow_kernel=kernel)
        plan.bind(idx, num_pages=kv.shape[0])
        o, lse = plan.run(q, kv, return_lse=True)
        torch.cuda.synchronize()
        if kernel == "mfma":
            with pytest.raises(rpa.RPAError) as e:
                plan.check()
            assert e.value.status == "RPA_E_V_RANGE"
            assert plan.check() == 0  # read and cleared
        else:
            # the prompt still runs on the wide kernel: only the decode rows are exact here
            flags = plan.check(raise_on_error=False)
            assert flags == rpa.ERR_V_RANGE
            rows = [int(b.qo_indptr[1]), int(b.qo_indptr[2])]
            assert_close(o.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl, rows=rows,
                         what="VALU decode rows with large V")
        plan.close()


def test_bf16_v_extremes_inside_the_fp16_range_are_exact():
    """65280 (the largest bf16 below 65504) and values beyond 65504 in slots no
    sequence owns raise nothing, and O matches the oracle."""
    b = planted_v(65280.0, 66)
    # beyond every sequence's kv_len: read by no row (zeroed before conversion)
    for s in range(b.batch):
        L = int(b.kv_lens[s])
        if L % 16:
            pg, sl = slot(b, s, L)  # first unowned slot of the last page
            b.kv_cache[pg, 1, sl] = 3.0e38
    ro, rl = oracle.run(**b.oracle_kwargs())
    for splits in (1, 0):
        o, l, _ = run(b, max_kv_splits=splits)  # run() calls plan.check(): raises on any flag
        assert_close(o, l, ro, rl, what="V extremes splits=%d" % splits)


@pytest.mark.parametrize("case", ["decode_b64_kv1024", "mixed_split"])
def test_split_merges_are_deterministic_over_100_runs(case):
    """Plans with many split groups, whose pieces finish in varying order and are
    merged by whichever piece comes last, give the same bits every run (the merge
    combines pieces in a fixed order).  Stops at the first differing run."""
    if case == "decode_b64_kv1024":
        b, kw = W.decode_b128_kv1024(batch=64), {}  # 4 pieces per sequence: 64 split groups
    else:
        b = W.make_batch("mixed_split", [150, 1, 40, 1, 3], [150, 4000, 900, 2500, 2500], num_qo_heads=16,
                         num_kv_heads=2, head_dim=128, dtype="bf16", seed=67)
        kw = dict(num_cus=4096)
    q, kv, idx = on_device(b)
    plan = rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=b.num_qo_heads,
                    num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, dtype=b.dtype, **kw)
    plan.bind(idx, num_pages=kv.shape[0])
    groups = plan.info["num_split_groups"]
    assert groups >= 10
    say("determinism %s: %d split groups, 100 runs" % (case, groups))
    o0, l0 = plan.run(q, kv, return_lse=True)
    o0, l0 = o0.clone(), l0.clone()
    o, l = torch.empty_like(o0), torch.empty_like(l0)
    for i in range(100):
        plan.run(q, kv, out=o, lse=l, return_lse=True)
        assert torch.equal(o.view(torch.int16), o0.view(torch.int16)) and torch.equal(l, l0), "run %d" % i
    plan.check()
    plan.close()
    ro, rl = oracle.run(**b.oracle_kwargs())
    assert_close(o0.double().cpu().numpy(), l0.double().cpu().numpy(), ro, rl, what=case)
