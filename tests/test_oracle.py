"""Pins of the fp64 oracle against things other than itself.

Each check ties the oracle to something it does not share code with: a
library routine (numpy's and torch's 16-bit decoders, torch's fp64
scaled-dot-product attention with an explicit mask), a closed form, or an
invariant of the definition (page placement, padding, prefix sharing, GQA
expansion, decode = prefill).  test_oracle_mutations.py then plants
plausible mistakes in a copy of the oracle and checks that these pins catch
every one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def sdpa_reference(b: W.Batch, sm_scale=None):
    """O and LSE from torch's fp64 CPU scaled_dot_product_attention (a library
    routine) on contiguous per-sequence K/V, with an explicit boolean mask that
    puts the queries at the last q_len positions."""
    H, Hk, D = b.num_qo_heads, b.num_kv_heads, b.head_dim
    G = H // Hk
    scale = 1.0 / math.sqrt(D) if sm_scale is None else sm_scale
    O = np.full((b.total_q, H, D), np.nan)
    L = np.full((b.total_q, H), np.nan)
    for s in range(b.batch):
        ql, kl = int(b.q_lens[s]), int(b.kv_lens[s])
        if ql == 0:
            continue
        k, v = W.contiguous_kv(b, s)
        k = k.double().repeat_interleave(G, dim=1).transpose(0, 1)  # [H, L, D]
        v = v.double().repeat_interleave(G, dim=1).transpose(0, 1)
        q = b.q[b.qo_indptr[s]:b.qo_indptr[s + 1]].double().transpose(0, 1)  # [H, ql, D]
        i = torch.arange(ql)[:, None]
        j = torch.arange(kl)[None, :]
        mask = (j <= kl - ql + i) if b.causal else torch.ones(ql, kl, dtype=torch.bool)
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
        scores = torch.where(mask, scale * (q @ k.transpose(1, 2)), torch.tensor(-math.inf, dtype=torch.float64))
        O[b.qo_indptr[s]:b.qo_indptr[s + 1]] = o.transpose(0, 1).numpy()
        L[b.qo_indptr[s]:b.qo_indptr[s + 1]] = torch.logsumexp(scores, dim=-1).transpose(0, 1).numpy()
    return O, L


def small_cases():
    """Tiny ragged batches: several GQA ratios, head dims, dtypes, causal and not."""
    yield W.tiny_ragged_prefill()
    yield W.tiny_ragged_prefill(poison=True, spare_pages=4)
    yield W.make_batch("gqa4_bf16", [5, 1, 16, 9], [5, 33, 40, 9], num_qo_heads=8, num_kv_heads=2,
                       head_dim=32, dtype="bf16", seed=7, spare_pages=3, poison=True)
    yield W.make_batch("mha_f16", [3, 7, 0, 2], [16, 7, 4, 31], num_qo_heads=3, num_kv_heads=3,
                       head_dim=16, dtype="f16", seed=8, spare_pages=1)
    yield W.make_batch("full_attn", [4, 1, 6], [10, 17, 6], num_qo_heads=4, num_kv_heads=1,
                       head_dim=8, dtype="bf16", seed=9, causal=False)
    # non-causal with more queries than keys (a cascade's shared-prefix segment)
    yield W.make_batch("full_attn_q_gt_kv", [21, 2, 5], [5, 17, 1], num_qo_heads=4, num_kv_heads=2,
                       head_dim=16, dtype="f16", seed=10, causal=False, spare_pages=2, poison=True)


# ---------------------------------------------------------------------------------------------
# 16-bit decoders: every bit pattern, against library conversions.
# ---------------------------------------------------------------------------------------------

def test_decode_binary16_all_patterns():
    raw = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(raw, "f16")
    want = raw.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def test_decode_bfloat16_all_patterns():
    raw = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(raw.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    got = oracle.decode(raw, "bf16")
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


# ---------------------------------------------------------------------------------------------
# Library routine: torch fp64 SDPA with an explicit bottom-right mask.
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("case", list(small_cases()), ids=lambda b: b.name)
def test_matches_torch_sdpa(case):
    o, lse = oracle.run(**case.oracle_kwargs(), nthreads=3)
    ro, rl = sdpa_reference(case)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_sm_scale_override():
    b = W.tiny_ragged_prefill()
    o, lse = oracle.run(**b.oracle_kwargs(), sm_scale=0.37)
    ro, rl = sdpa_reference(b, sm_scale=0.37)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_thread_count_does_not_change_bits():
    b = W.tiny_ragged_prefill()
    o1, l1 = oracle.run(**b.oracle_kwargs(), nthreads=1)
    o7, l7 = oracle.run(**b.oracle_kwargs(), nthreads=7)
    assert np.array_equal(o1, o7) and np.array_equal(l1, l7)


def test_row_subset_equals_full():
    b = W.tiny_ragged_prefill()
    o, lse = oracle.run(**b.oracle_kwargs())
    rows = [0, 5, 16, 17, 25]
    os_, ls = oracle.run(**b.oracle_kwargs(), rows=rows)
    assert np.array_equal(os_[rows], o[rows]) and np.array_equal(ls[rows], lse[rows])
    others = np.setdiff1d(np.arange(b.total_q), rows)
    assert np.isnan(os_[others]).all()


# ---------------------------------------------------------------------------------------------
# Closed forms.
# ---------------------------------------------------------------------------------------------

def _set(t, values):
    t.copy_(torch.as_tensor(values).to(t.dtype))


def test_single_visible_key_returns_that_value():
    # q_len 1, kv_len 1: one visible key, weight 1: O = V_0 exactly, LSE = s_0.
    b = W.make_batch("one", [1], [1], num_qo_heads=2, num_kv_heads=1, head_dim=8, dtype="f16", seed=3)
    o, lse = oracle.run(**b.oracle_kwargs())
    pg = b.kv_page_indices[0]
    v0 = b.kv_cache[pg, 1, 0, 0].double().numpy()
    k0 = b.kv_cache[pg, 0, 0, 0].double().numpy()
    for h in range(2):
        assert np.array_equal(o[0, h], v0)
        s0 = float(np.dot(b.q[0, h].double().numpy(), k0)) / math.sqrt(8)
        assert abs(lse[0, h] - s0) < 1e-14


def test_first_prompt_row_sees_only_its_own_token():
    # Causal prefill with q_len == kv_len: row 0 of each sequence attends to key 0 only.
    b = W.make_batch("rows0", [5, 9], [5, 9], num_qo_heads=4, num_kv_heads=2, head_dim=16,
                     dtype="bf16", seed=4)
    o, _ = oracle.run(**b.oracle_kwargs())
    for s in range(2):
        pg = b.kv_page_indices[b.kv_page_indptr[s]]
        for h in range(4):
            assert np.array_equal(o[b.qo_indptr[s], h], b.kv_cache[pg, 1, 0, h // 2].double().numpy())


def test_zero_query_gives_mean_of_visible_values():
    # Q = 0: every visible score is 0, weights 1/n: O = mean of the n visible V, LSE = ln n.
    b = W.make_batch("q0", [3, 2], [20, 35], num_qo_heads=2, num_kv_heads=1, head_dim=8,
                     dtype="f16", seed=5)
    b.q.zero_()
    o, lse = oracle.run(**b.oracle_kwargs())
    for s in range(2):
        _, v = W.contiguous_kv(b, s)
        ql, kl = int(b.q_lens[s]), int(b.kv_lens[s])
        for i in range(ql):
            n = kl - ql + i + 1
            want = v[:n, 0].double().mean(0).numpy()
            r = b.qo_indptr[s] + i
            np.testing.assert_allclose(o[r, 0], want, rtol=0, atol=1e-15)
            assert abs(lse[r, 0] - math.log(n)) < 1e-14


def test_constant_values_give_that_constant():
    b = W.make_batch("vc", [4], [29], num_qo_heads=4, num_kv_heads=1, head_dim=8, dtype="bf16", seed=6)
    b.kv_cache[:, 1] = 0.625  # exactly representable
    o, _ = oracle.run(**b.oracle_kwargs())
    np.testing.assert_allclose(o, 0.625, rtol=0, atol=1e-15)


def test_one_hot_key_selects_its_value():
    # K_{j*} = 16 q (exact in fp16) gives score 16 |q|^2 / sqrt(D), far above every other
    # score, so every other weight is below 2^-60: O equals V_{j*} to fp64 rounding.
    b = W.make_batch("onehot", [1], [40], num_qo_heads=1, num_kv_heads=1, head_dim=16, dtype="f16", seed=11)
    jstar = 23
    q = b.q[0, 0]
    q.copy_(torch.sign(q) * 2.0)  # |q|^2 = 64, score = 16*64/4 = 256
    pages = b.kv_page_indices
    b.kv_cache[pages[jstar // 16], 0, jstar % 16, 0] = 16 * q
    for j in range(40):
        if j != jstar:  # other keys small: |score| <= 16 * 2 * 2 / 4 = 16
            kk = b.kv_cache[pages[j // 16], 0, j % 16, 0]
            kk.copy_(torch.clamp(kk, -1, 1))
    o, lse = oracle.run(**b.oracle_kwargs())
    want = b.kv_cache[pages[jstar // 16], 1, jstar % 16, 0].double().numpy()
    np.testing.assert_allclose(o[0, 0], want, rtol=0, atol=1e-15)
    assert abs(lse[0, 0] - 256.0) < 1e-9


# ---------------------------------------------------------------------------------------------
# Invariants of the definition (bitwise in fp64: every output is computed in a fixed order
# that depends only on logical positions).
# ---------------------------------------------------------------------------------------------

def test_page_permutation_is_invisible():
    b = W.tiny_ragged_prefill(poison=True, spare_pages=4)
    p = W.permute_pages(b, seed=99)
    assert not np.array_equal(b.kv_page_indices, p.kv_page_indices)
    o1, l1 = oracle.run(**b.oracle_kwargs())
    o2, l2 = oracle.run(**p.oracle_kwargs())
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_padded_batch_gives_same_real_rows():
    base = W.make_batch("short", [7, 1, 19, 12], [7, 1, 19, 12], num_qo_heads=4, num_kv_heads=2,
                        head_dim=16, dtype="bf16", seed=12)
    pad = W.pad_to(base, 24, seed=13)
    o1, l1 = oracle.run(**base.oracle_kwargs())
    o2, l2 = oracle.run(**pad.oracle_kwargs())
    for s in range(base.batch):
        L = int(base.q_lens[s])
        a, c = base.qo_indptr[s], pad.qo_indptr[s]
        assert np.array_equal(o1[a:a + L], o2[c:c + L])
        assert np.array_equal(l1[a:a + L], l2[c:c + L])


def test_decode_row_equals_matching_prefill_row():
    # A prefill row at position p equals a q_len = 1 call over the first p + 1 tokens
    # (the page table truncated to them).
    b = W.make_batch("pf", [21], [37], num_qo_heads=4, num_kv_heads=1, head_dim=16, dtype="f16", seed=14)
    o, lse = oracle.run(**b.oracle_kwargs())
    for i in [0, 5, 16, 20]:
        pos = 37 - 21 + i
        npg = W.pages_for(pos + 1)
        d = W.Batch("dec", np.array([0, 1], np.int32), np.array([0, npg], np.int32),
                    b.kv_page_indices[:npg].copy(), np.array([W.last_page_len_for(pos + 1)], np.int32),
                    b.q[i:i + 1], b.kv_cache, 4, 1, 16, "f16")
        od, ld = oracle.run(**d.oracle_kwargs())
        assert np.array_equal(od[0], o[i]) and np.array_equal(ld[0], lse[i])


def test_shared_prefix_equals_duplicated_prefix():
    kw = dict(n_req=3, prefix=40, suffix=7, decode_steps=2, num_qo_heads=4, num_kv_heads=2,
              head_dim=16, dtype="bf16")
    sh = W.shared_prefix_suffix(**kw)
    du = W.shared_prefix_suffix(duplicated=True, **kw)
    # shared layout really shares: request 0 and 1 reference the same first pages
    n_sh = 40 // 16
    assert np.array_equal(sh.kv_page_indices[:n_sh], sh.kv_page_indices[sh.kv_page_indptr[1]:][:n_sh])
    o1, l1 = oracle.run(**sh.oracle_kwargs())
    o2, l2 = oracle.run(**du.oracle_kwargs())
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_cascade_halves_merge_to_the_whole():
    # Keys split into a shared prefix (attended non-causally by every request's
    # queries at once) and each request's private rest (causal): merging the two
    # results with weights exp(LSE_x - max LSE) gives the attention over all keys,
    # an exact identity of the softmax (vLLM issue #227's sharing as a cascade).
    kw = dict(n_req=4, prefix=40, suffix=7, decode_steps=0, num_qo_heads=8, num_kv_heads=2,
              head_dim=32, dtype="bf16")
    b = W.shared_prefix_suffix(**kw)
    shared, private = W.cascade_view(b, prefix=40)
    assert shared.batch == 1 and shared.q_lens[0] == b.total_q and shared.kv_lens[0] == 40
    assert (private.kv_lens == 7).all() and private.causal and not shared.causal
    o, lse = oracle.run(**b.oracle_kwargs())
    om, lm = oracle.merge_states(*oracle.run(**shared.oracle_kwargs()), *oracle.run(**private.oracle_kwargs()))
    assert np.abs(om - o).max() < 1e-12 and np.abs(lm - lse).max() < 1e-12
    # merging is symmetric, and merging with an empty state (LSE = -inf) is the identity
    om2, lm2 = oracle.merge_states(*oracle.run(**private.oracle_kwargs()), *oracle.run(**shared.oracle_kwargs()))
    assert np.abs(om2 - o).max() < 1e-12 and np.abs(lm2 - lse).max() < 1e-12
    oe, le = oracle.merge_states(o, lse, np.full_like(o, np.nan), np.full_like(lse, -np.inf))
    assert np.array_equal(oe, o) and np.array_equal(le, lse)
    oz, lz = oracle.merge_states(o, np.full_like(lse, -np.inf), o, np.full_like(lse, -np.inf))
    assert (oz == 0).all() and np.isneginf(lz).all()
    # decode rows after appending tokens split the same way
    d = W.decode_step(W.shared_prefix_suffix(**dict(kw, decode_steps=3)), 3)
    shared, private = W.cascade_view(d, prefix=40)
    o, lse = oracle.run(**d.oracle_kwargs())
    om, lm = oracle.merge_states(*oracle.run(**shared.oracle_kwargs()), *oracle.run(**private.oracle_kwargs()))
    assert np.abs(om - o).max() < 1e-12 and np.abs(lm - lse).max() < 1e-12


def test_gqa_equals_expanded_mha():
    b = W.make_batch("gqa", [6, 2], [6, 30], num_qo_heads=6, num_kv_heads=2, head_dim=8, dtype="bf16", seed=15)
    G = 3
    mha_kv = b.kv_cache.repeat_interleave(G, dim=3).contiguous()
    m = W.Batch("mha", b.qo_indptr, b.kv_page_indptr, b.kv_page_indices, b.kv_last_page_len, b.q,
                mha_kv, 6, 6, 8, "bf16")
    o1, l1 = oracle.run(**b.oracle_kwargs())
    o2, l2 = oracle.run(**m.oracle_kwargs())
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_rows_depend_only_on_their_own_sequence():
    b = W.make_batch("iso", [3, 4, 2], [10, 20, 18], num_qo_heads=2, num_kv_heads=1, head_dim=8,
                     dtype="f16", seed=16, permute=True)
    o1, l1 = oracle.run(**b.oracle_kwargs())
    # perturb sequence 1's Q and its pages
    b.q[b.qo_indptr[1]:b.qo_indptr[2]] += 1
    for p in b.kv_page_indices[b.kv_page_indptr[1]:b.kv_page_indptr[2]]:
        b.kv_cache[p] *= -1
    o2, l2 = oracle.run(**b.oracle_kwargs())
    for s in (0, 2):
        sl = slice(b.qo_indptr[s], b.qo_indptr[s + 1])
        assert np.array_equal(o1[sl], o2[sl]) and np.array_equal(l1[sl], l2[sl])
    sl = slice(b.qo_indptr[1], b.qo_indptr[2])
    assert not np.array_equal(o1[sl], o2[sl])


def test_sequence_order_permutes_rows():
    b = W.make_batch("ord", [3, 4, 2, 1], [10, 20, 18, 5], num_qo_heads=2, num_kv_heads=1,
                     head_dim=8, dtype="f16", seed=17)
    order = [2, 0, 3, 1]
    r = W.reorder_sequences(b, order)
    o1, l1 = oracle.run(**b.oracle_kwargs())
    o2, l2 = oracle.run(**r.oracle_kwargs())
    rows = W.row_permutation(b, order)
    assert np.array_equal(o2, o1[rows]) and np.array_equal(l2, l1[rows])


def test_unowned_slots_are_never_read():
    clean = W.tiny_ragged_prefill(spare_pages=4)
    dirty = W.tiny_ragged_prefill(spare_pages=4, poison=True)
    assert torch.isnan(dirty.kv_cache.float()).any()
    o1, l1 = oracle.run(**clean.oracle_kwargs())
    o2, l2 = oracle.run(**dirty.oracle_kwargs())
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---------------------------------------------------------------------------------------------
# Rejected inputs.
# ---------------------------------------------------------------------------------------------

def _bad(b, **over):
    kw = b.oracle_kwargs()
    kw.update(over)
    with pytest.raises(ValueError) as e:
        oracle.run(**kw)
    return str(e.value)


def test_rejects_invalid_page_tables():
    b = W.tiny_ragged_prefill()
    assert "E_LAST_PAGE_LEN" in _bad(b, kv_last_page_len=np.array([1, 0, 5, 16], np.int32))
    assert "E_LAST_PAGE_LEN" in _bad(b, kv_last_page_len=np.array([1, 17, 5, 16], np.int32))
    assert "E_QLEN_GT_KVLEN" in _bad(b, kv_last_page_len=np.array([1, 14, 4, 16], np.int32))
    # non-causal: more queries than keys is allowed, queries without any key are not
    nc = W.make_batch("nc", [3, 2], [1, 0], num_qo_heads=2, num_kv_heads=1, head_dim=8, dtype="f16",
                      seed=4, causal=False)
    assert "E_QLEN_GT_KVLEN" in _bad(nc)
    bad_idx = b.kv_page_indices.copy()
    bad_idx[3] = b.num_pages
    assert "E_PAGE_OOB" in _bad(b, kv_page_indices=bad_idx)
    assert "E_INDPTR" in _bad(b, qo_indptr=np.array([1, 17, 20, 25, 26], np.int32))
    assert "E_INDPTR" in _bad(b, kv_page_indptr=np.array([0, 2, 1, 5, 8], np.int32))
    assert "E_ARG" in _bad(b, num_kv_heads=3)
