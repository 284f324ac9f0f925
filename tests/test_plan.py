"""CPU tests of the C-ABI library: exported symbols, the host planner and its
error codes.  Nothing here launches a kernel (no GPU needed): the planner is
host-only and the library loads without a device.
"""
import ctypes
import math

import numpy as np
import torch
import pytest

import paged_kv_attention_ragged_amd as rpa
import workloads as W

F = dict(q_row0=0, q_count=1, pos0=2, kv_len=3, page_base=4, kv_head=5, kv_begin=6, kv_end=7, part=8,
         seq=9, split=10, n_splits=11, kind=12)


def make_plan(b: W.Batch, **kw):
    return rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=b.num_qo_heads,
                    num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, dtype=b.dtype, causal=b.causal, **kw)


def lengths_batch(q_lens, kv_lens, H=8, Hk=1, D=128, causal=True):
    """Page table only (no tensors needed by the planner)."""
    q_lens, kv_lens = list(q_lens), list(kv_lens)
    B = len(q_lens)
    qo = np.zeros(B + 1, np.int32)
    qo[1:] = np.cumsum(q_lens)
    npg = [W.pages_for(k) for k in kv_lens]
    kp = np.zeros(B + 1, np.int32)
    kp[1:] = np.cumsum(npg)
    last = np.array([W.last_page_len_for(k) for k in kv_lens], np.int32)
    return W.Batch("lengths", qo, kp, np.arange(kp[-1], dtype=np.int32), last, None, None, H, Hk, D, "f16", causal)


def test_library_exports_every_declared_function():
    lib = rpa.load()
    names = rpa.declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert rpa.version().count(".") == 2


def check_schedule(b: W.Batch, plan):
    """Properties every schedule must have, whatever the split decisions."""
    t = plan.tiles()
    info = plan.info
    G = b.num_qo_heads // b.num_kv_heads
    TQ = info["tokens_per_tile"]
    BN = info["block_n"]
    assert TQ == 128 // G and BN == 32
    q_lens, kv_lens = b.q_lens, b.kv_lens
    # 1. every (sequence, kv head, token) appears in exactly one query tile, and each query
    #    tile's pieces cover [0, kv_end) exactly once, in order, block-aligned
    seen = {}
    for rec in t:
        if rec[F["q_count"]] == 0:  # empty padding tile (XCD alignment of wide tiles)
            assert rec[F["kind"]] == 0 and rec[F["part"]] == -1 and rec[F["kv_end"]] == rec[F["kv_begin"]]
            continue
        key = (rec[F["seq"]], rec[F["kv_head"]], rec[F["q_row0"]])
        seen.setdefault(key, []).append(rec)
    covered = np.zeros((b.total_q, b.num_kv_heads), np.int32)
    n_part_rows = 0
    part_ranges = []
    for (s, hk, r0), recs in seen.items():
        recs = sorted(recs, key=lambda r: r[F["split"]])
        qc = recs[0][F["q_count"]]
        assert all(r[F["q_count"]] == qc for r in recs)
        assert qo_row_in_seq(b, s, r0) and r0 + qc <= b.qo_indptr[s + 1]
        assert (r0 - b.qo_indptr[s]) % TQ == 0 and 1 <= qc <= TQ
        covered[r0:r0 + qc, hk] += 1
        ql, kl = int(q_lens[s]), int(kv_lens[s])
        pos0 = kl - ql + (r0 - b.qo_indptr[s])
        assert recs[0][F["pos0"]] == pos0 and recs[0][F["kv_len"]] == kl
        assert recs[0][F["page_base"]] == b.kv_page_indptr[s]
        want_end = min(kl, pos0 + qc) if b.causal else kl  # causal tail skipped
        ns = len(recs)
        assert all(r[F["n_splits"]] == ns for r in recs)
        assert [r[F["split"]] for r in recs] == list(range(ns))
        assert recs[0][F["kv_begin"]] == 0 and recs[-1][F["kv_end"]] == want_end
        for a, c in zip(recs, recs[1:]):
            assert a[F["kv_end"]] == c[F["kv_begin"]]
        for r in recs:
            assert r[F["kv_begin"]] % BN == 0 and r[F["kv_begin"]] < r[F["kv_end"]] or want_end == 0
        if ns == 1:
            assert recs[0][F["part"]] == -1
        else:
            rows = qc * G
            for i, r in enumerate(recs):
                assert r[F["part"]] == recs[0][F["part"]] + i * rows
            part_ranges.append((recs[0][F["part"]], recs[0][F["part"]] + ns * rows))
            n_part_rows += ns * rows
    want = np.zeros_like(covered)
    for s in range(b.batch):
        want[b.qo_indptr[s]:b.qo_indptr[s + 1], :] = 1
    assert np.array_equal(covered, want)
    # 2. partial rows of different split tiles never overlap
    part_ranges.sort()
    for (a0, a1), (c0, c1) in zip(part_ranges, part_ranges[1:]):
        assert a1 <= c0
    assert info["partial_rows"] == n_part_rows
    # 3. tile kind, chosen per sequence: narrow (decode-like path) exactly for the tiles
    #    of sequences whose q_len * G rows fit one narrow tile (16 rows; 8 on the VALU
    #    kernel), unless the plan has wide tiles and the narrow ones carry at most 8 MiB
    #    of K/V: then they run as wide tiles too
    thr = 8 if plan.params.narrow_kernel == 1 else 16
    real = [r for r in t if r[F["q_count"]] > 0]
    narrow_seq = [int(q_lens[r[F["seq"]]]) * G <= thr for r in real]
    if any(narrow_seq) and not any(r[F["kind"]] == 1 for r in t):
        assert plan.params.narrow_kernel == 0 and not all(narrow_seq)
        assert fold_bytes([r for r, n in zip(real, narrow_seq) if n], b.head_dim) <= FOLD_BYTES
    else:
        assert [int(r[F["kind"]]) for r in real] == [int(n) for n in narrow_seq]
        if any(narrow_seq) and not all(narrow_seq) and plan.params.narrow_kernel == 0:
            assert fold_bytes([r for r, n in zip(real, narrow_seq) if n], b.head_dim) > FOLD_BYTES
    # 4. launch order: all wide tiles (one kernel), then all narrow tiles (another).
    #    Narrow tiles go longest first (keys walked, rounded to 64).  Wide tiles go
    #    longest first in small launches; in larger ones, launch slot i runs on XCD
    #    i % 8 and each XCD's slots hold each (sequence, kv head) stream as one
    #    contiguous, longest-first run.
    #    A plan with both kinds runs them in one launch instead: narrow tiles in blocks of
    #    8 between blocks of 8 wide ones, so each wide tile keeps its slot modulo 8.
    kinds = [int(r[F["kind"]]) for r in t]
    if 0 in kinds and 1 in kinds:
        wide_slots = [i for i, k in enumerate(kinds) if k == 0]
        assert all(i % 8 == j % 8 for j, i in enumerate(wide_slots))
        narrow_slots = [i for i, k in enumerate(kinds) if k == 1]
        assert all(i % 8 == j % 8 for j, i in enumerate(narrow_slots[:len(narrow_slots) // 8 * 8]))
    else:
        assert kinds == sorted(kinds)

    def cost(r, gran):
        return -(-(r[F["kv_end"]] - r[F["kv_begin"]]) // gran) * gran

    narrow = [cost(r, 64) for r in t if r[F["kind"]] == 1]
    assert all(x >= y for x, y in zip(narrow, narrow[1:]))
    wide = [r for r in t if r[F["kind"]] == 0]
    if len(wide) < 32:
        c = [cost(r, BN) for r in wide]
        assert all(x >= y for x, y in zip(c, c[1:])) and all(r[F["q_count"]] > 0 for r in wide)
    else:
        assert wide[-1][F["q_count"]] > 0
        for x in range(8):
            lane = [r for r in wide[x::8] if r[F["q_count"]] > 0]
            streams = [(int(r[F["seq"]]), int(r[F["kv_head"]])) for r in lane]
            starts = [s for i, s in enumerate(streams) if i == 0 or streams[i - 1] != s]
            assert len(starts) == len(set(starts)), "a stream is split within one XCD's slots"
            for a, c in zip(lane, lane[1:]):
                if (a[F["seq"]], a[F["kv_head"]]) == (c[F["seq"]], c[F["kv_head"]]):
                    assert cost(a, BN) >= cost(c, BN)
    # 5. split pieces start at multiples of 256 keys
    assert all(r[F["kv_begin"]] % 256 == 0 for r in t)
    # 6. work counts
    vis = sum((int(kv_lens[s]) - int(q_lens[s])) * int(q_lens[s]) + int(q_lens[s]) * (int(q_lens[s]) + 1) // 2
              if b.causal else int(q_lens[s]) * int(kv_lens[s]) for s in range(b.batch))
    assert info["visible_pairs"] == vis * b.num_qo_heads
    assert info["total_q"] == b.total_q
    return t


FOLD_BYTES = 8 << 20


def fold_bytes(recs, D):
    """K/V bytes of narrow tiles as the planner counts them for the fold rule."""
    return sum(int(r[F["kv_end"]] - r[F["kv_begin"]]) for r in recs) * D * 4


def test_small_narrow_work_joins_the_wide_launch():
    # short ragged prompts: every tile is wide, the partial last tiles of long prompts
    # (<= 16 rows) and the prompts of at most 4 tokens (4 heads per kv head) included
    lens = W.short_prompt_lengths() + [1, 2, 4]
    b = lengths_batch(lens, lens, H=32, Hk=8)
    t = make_plan(b).tiles()
    assert (t[:, F["kind"]] == 0).all() and ((t[:, F["q_count"]] * 4 <= 16) & (t[:, F["q_count"]] > 0)).any()
    # the same without any prompt of more than 16 rows: all narrow (no wide launch to join)
    s = lengths_batch([1, 2, 4, 3], [1, 2, 4, 3], H=32, Hk=8)
    assert (make_plan(s).tiles()[:, F["kind"]] == 1).all()
    # a partial last tile of a long prompt is wide even when narrow tiles keep their kernel
    m = lengths_batch([8192 + 2] * 4 + [1] * 256, [8192 + 2] * 4 + [4096] * 256, H=64, Hk=8)
    tm = make_plan(m).tiles()
    part = tm[(tm[:, F["q_count"]] == 2)]
    assert len(part) == 32 and (part[:, F["kind"]] == 0).all()
    # decode rows beside long prompts carry much K/V: they keep the narrow kernel
    assert ((tm[:, F["kind"]] == 1) == ((tm[:, F["q_count"]] == 1))).all()
    # so do decode-only batches
    tc = make_plan(lengths_batch([1] * 128, [1024] * 128)).tiles()
    assert (tc[:, F["kind"]] == 1).all()
    # the VALU decode kernel (a comparison) keeps every sequence of its size (q_len * G <= 8)
    v = rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=32, num_kv_heads=8,
                 head_dim=128, dtype="bf16", narrow_kernel="valu")
    tv = v.tiles()
    ql = np.array(lens)[tv[:, F["seq"]]]
    assert ((tv[:, F["kind"]] == 1) == ((tv[:, F["q_count"]] > 0) & (ql * 4 <= 8))).all()
    assert (tv[:, F["kind"]] == 1).sum() >= 8 * 2  # at least the added prompts of 1 and 2 tokens


def qo_row_in_seq(b, s, r0):
    return b.qo_indptr[s] <= r0 < b.qo_indptr[s + 1]


@pytest.mark.parametrize("case", [
    lengths_batch([17, 3, 5, 1], [17, 30, 5, 48], H=8, Hk=1, D=64),
    lengths_batch([1] * 128, [1024] * 128),
    lengths_batch([200, 1, 37, 0, 64], [200, 999, 300, 5, 64], H=32, Hk=8),
    lengths_batch([30] * 256, [230] * 256, H=32, Hk=8),
    lengths_batch([1] * 7, [5000, 17, 1, 16, 33, 4096, 64], H=64, Hk=8),
    lengths_batch([8192] * 4 + [1] * 256, [8192] * 4 + list(range(512, 8192, 30))[:256], H=64, Hk=8),
    lengths_batch([3, 9], [40, 9], H=6, Hk=2, D=64, causal=False),
    lengths_batch([5, 1], [5, 1], H=12, Hk=1),  # G = 12 does not divide 128
    lengths_batch([7680], [200], H=32, Hk=8, causal=False),  # cascade: shared prefix, all queries
    lengths_batch([256, 1, 40], [200, 3, 0 + 17], H=8, Hk=1, causal=False),
], ids=["tiny", "decode", "ragged", "suffix", "decode_mixed", "mixed_long", "noncausal", "g12",
        "cascade_shared", "noncausal_q_gt_kv"])
@pytest.mark.parametrize("max_kv_splits", [0, 1, 3])
def test_schedule_properties(case, max_kv_splits):
    plan = make_plan(case, max_kv_splits=max_kv_splits)
    t = check_schedule(case, plan)
    check_schedule(case, make_plan(case, max_kv_splits=max_kv_splits, narrow_kernel="valu"))
    if max_kv_splits == 1:
        assert (t[:, F["n_splits"]] == 1).all()
    if max_kv_splits == 3:
        assert (t[:, F["n_splits"]] <= 3).all()


@pytest.mark.parametrize("B,L,tiles,groups", [
    (128, 1024, 128, 0),   # balanced: the longest range is twice the fair share -> no split
    (256, 1024, 256, 0),
    (256, 4096, 256, 0),
    (127, 1024, 508, 127),  # just unbalanced: 256-key pieces, at least one per CU
    (64, 1024, 256, 64),    # one piece per CU: 4 x 256 keys each
    (64, 4096, 256, 64),    # 4 x 1024
    (32, 8192, 256, 32),    # 8 x 1024
    (16, 1024, 64, 16),     # 256-key pieces cannot make more
])
def test_decode_batch_split_rule(B, L, tiles, groups):
    b = lengths_batch([1] * B, [L] * B)
    info = make_plan(b).info
    assert (info["num_tiles"], info["num_split_groups"]) == (tiles, groups)
    check_schedule(b, make_plan(b))
    assert make_plan(b, max_kv_splits=1).info["num_tiles"] == B


def test_unbalanced_batches_are_split():
    # one long decode row among short ones: its range is far above a CU's share
    b = lengths_batch([1] * 200, [8192] + [64] * 199)
    t = make_plan(b).tiles()
    assert t[t[:, F["seq"]] == 0, F["n_splits"]].max() > 1
    assert (t[t[:, F["seq"]] != 0, F["n_splits"]] == 1).all()
    # a single 2048-token prompt (128 wide tiles, the last one walking every key): split
    p = make_plan(lengths_batch([2048], [2048])).info
    assert p["num_split_groups"] > 0
    # the long prompts of a mixed batch are balanced by themselves: never split
    assert make_plan(lengths_batch([8192] * 4, [8192] * 4, H=64, Hk=8)).info["num_split_groups"] == 0


def test_schedule_depends_only_on_lengths():
    b = W.tiny_ragged_prefill(spare_pages=4)
    p = W.permute_pages(b, seed=5)
    assert np.array_equal(make_plan(b).tiles(), make_plan(p).tiles())


def test_fully_masked_tail_blocks_are_never_scheduled():
    # a 4096-token prompt: tile i covers tokens [16i, 16i+16) and must stop at key 16i+16
    b = lengths_batch([4096], [4096], H=64, Hk=8)
    t = make_plan(b, max_kv_splits=1).tiles()
    ends = t[:, F["kv_end"]] - (t[:, F["pos0"]] + t[:, F["q_count"]])
    assert (ends == 0).all()
    # total blocks walked ~ half of the dense square
    BN = 64
    blocks = ((t[:, F["kv_end"]] + BN - 1) // BN).sum()
    dense = len(t) * (4096 // BN)
    assert blocks < 0.53 * dense


@pytest.mark.parametrize("bad,code", [
    (dict(qo_indptr=[1, 17, 20, 25, 26]), "RPA_E_INDPTR"),
    (dict(qo_indptr=[0, 17, 16, 25, 26]), "RPA_E_INDPTR"),
    (dict(kv_page_indptr=[0, 2, 1, 5, 8]), "RPA_E_INDPTR"),
    (dict(kv_last_page_len=[1, 0, 5, 16]), "RPA_E_LAST_PAGE_LEN"),
    (dict(kv_last_page_len=[1, 17, 5, 16]), "RPA_E_LAST_PAGE_LEN"),
    (dict(kv_last_page_len=[1, 14, 4, 16]), "RPA_E_QLEN_GT_KVLEN"),
    (dict(num_kv_heads=3), "RPA_E_SHAPE"),
    (dict(head_dim=96), "RPA_E_SHAPE"),
    (dict(page_size=32), "RPA_E_SHAPE"),
    (dict(dtype=7), "RPA_E_ARG"),
    (dict(max_kv_splits=-1), "RPA_E_ARG"),
])
def test_plan_rejects_bad_input(bad, code):
    b = W.tiny_ragged_prefill()
    kw = dict(qo_indptr=b.qo_indptr, kv_page_indptr=b.kv_page_indptr, kv_last_page_len=b.kv_last_page_len,
              num_qo_heads=8, num_kv_heads=1, head_dim=64, page_size=16, dtype="f16", max_kv_splits=0)
    kw.update(bad)
    if isinstance(kw["dtype"], int):
        p = rpa._Params(kw["num_qo_heads"], kw["num_kv_heads"], kw["head_dim"], 16, kw["dtype"], 1, 0.0, 0, 0)
        h = ctypes.c_void_p()
        qo, kp, kl = (rpa._host_i32(kw[k]) for k in ("qo_indptr", "kv_page_indptr", "kv_last_page_len"))
        rc = rpa.load().rpa_plan_create(ctypes.byref(p), 4, qo.ctypes.data, kp.ctypes.data, kl.ctypes.data,
                                        ctypes.byref(h))
        assert rpa.STATUS[rc] == code and rpa.load().rpa_last_error()
        return
    with pytest.raises(rpa.RPAError) as e:
        rpa.Plan(kw.pop("qo_indptr"), kw.pop("kv_page_indptr"), kw.pop("kv_last_page_len"), **kw)
    assert e.value.status == code
    assert len(str(e.value)) > len(code) + 5


def test_plan_rejects_bad_kv_shared():
    b = W.tiny_ragged_prefill()
    p = rpa._Params(8, 1, 64, 16, 0, 1, 0.0, 0, 0, 0, 2)
    h = ctypes.c_void_p()
    qo, kp, kl = (rpa._host_i32(a) for a in (b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len))
    rc = rpa.load().rpa_plan_create(ctypes.byref(p), 4, qo.ctypes.data, kp.ctypes.data, kl.ctypes.data,
                                    ctypes.byref(h))
    assert rpa.STATUS[rc] == "RPA_E_ARG" and b"kv_shared" in rpa.load().rpa_last_error()


def test_noncausal_may_have_more_queries_than_keys():
    # non-causal: q_len > kv_len is a valid request (every query sees all keys) ...
    info = make_plan(lengths_batch([40, 3], [5, 2], causal=False)).info
    assert info["visible_pairs"] == (40 * 5 + 3 * 2) * 8
    # ... but a causal one is not, and neither are queries with no key at all
    with pytest.raises(rpa.RPAError) as e:
        make_plan(lengths_batch([40, 3], [5, 2], causal=True))
    assert e.value.status == "RPA_E_QLEN_GT_KVLEN"
    with pytest.raises(rpa.RPAError) as e:
        make_plan(lengths_batch([2, 3], [0, 2], causal=False))
    assert e.value.status == "RPA_E_QLEN_GT_KVLEN"


def test_merge_states_rejects_bad_arguments_without_launching():
    lib = rpa.load()
    P = 256  # a 16-byte aligned stand-in address; these calls fail validation before any launch
    assert lib.rpa_merge_states(0, 8, 128, 1, None, None, None, None, None, None, None) == 0  # nothing to do
    assert rpa.STATUS[lib.rpa_merge_states(4, 8, 96, 1, P, P, P, P, P, P, None)] == "RPA_E_SHAPE"
    assert rpa.STATUS[lib.rpa_merge_states(4, 8, 128, 5, P, P, P, P, P, P, None)] == "RPA_E_ARG"
    assert rpa.STATUS[lib.rpa_merge_states(4, 8, 128, 1, None, P, P, P, P, P, None)] == "RPA_E_ARG"
    assert rpa.STATUS[lib.rpa_merge_states(4, 8, 128, 1, P + 2, P, P, P, P, P, None)] == "RPA_E_ARG"
    assert rpa.STATUS[lib.rpa_merge_states(-1, 8, 128, 1, P, P, P, P, P, P, None)] == "RPA_E_ARG"


def test_plan_update_keeps_the_launch_shape():
    # a decode step: every sequence one token longer, same tiles (no split change)
    b0 = lengths_batch([1] * 256, [231] * 256, H=32, Hk=8)
    b1 = lengths_batch([1] * 256, [232] * 256, H=32, Hk=8)
    p = make_plan(b0)
    n0 = p.info["num_tiles"]
    p.update(b1.qo_indptr, b1.kv_page_indptr, b1.kv_last_page_len)
    fresh = make_plan(b1)
    assert p.info["num_tiles"] == n0 and p.info["visible_pairs"] == fresh.info["visible_pairs"]
    assert np.array_equal(p.tiles(), fresh.tiles())
    check_schedule(b1, p)
    # lengths that need another launch shape are refused; the plan is left as it was
    b2 = lengths_batch([1] * 64, [1024] * 64)
    b3 = lengths_batch([1] * 64, [1100] * 64)  # 5 split pieces per sequence instead of 4
    p2 = make_plan(b2)
    before = p2.tiles().copy()
    with pytest.raises(rpa.RPAError) as e:
        p2.update(b3.qo_indptr, b3.kv_page_indptr, b3.kv_last_page_len)
    assert e.value.status == "RPA_E_UNSUPPORTED"
    assert np.array_equal(p2.tiles(), before)


def test_trim_page_table_keeps_the_real_tokens_of_a_padded_prefill():
    # llama.cpp discussion #15958: prompts padded to 200, real tokens first; trimming
    # each sequence back to its real length leaves exactly the ragged batch's tokens
    rag = W.short_prompt_prefill(n=8)
    pad = W.short_prompt_prefill(n=8, padded=True)
    ip, ix, kl = rpa.trim_page_table(pad.kv_page_indptr, pad.kv_page_indices, pad.kv_last_page_len, rag.kv_lens)
    t = W.Batch("trimmed", np.zeros(rag.batch + 1, np.int32), ip, ix, kl, None, pad.kv_cache,
                pad.num_qo_heads, pad.num_kv_heads, pad.head_dim, pad.dtype)
    assert np.array_equal(t.kv_lens, rag.kv_lens)
    assert np.array_equal(np.diff(ip), [-(-int(L) // 16) for L in rag.kv_lens])
    for s in range(rag.batch):
        k1, v1 = W.contiguous_kv(t, s)
        k2, v2 = W.contiguous_kv(rag, s)
        assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
        assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))
        # the kept pages are the padded sequence's first pages, in order
        assert np.array_equal(ix[ip[s]:ip[s + 1]], pad.kv_page_indices[pad.kv_page_indptr[s]:][:ip[s + 1] - ip[s]])
    with pytest.raises(rpa.RPAError) as e:
        rpa.trim_page_table(pad.kv_page_indptr, pad.kv_page_indices, pad.kv_last_page_len, pad.kv_lens + 1)
    assert e.value.status == "RPA_E_ARG"
    ip0, ix0, kl0 = rpa.trim_page_table(pad.kv_page_indptr, pad.kv_page_indices, pad.kv_last_page_len,
                                        np.zeros(pad.batch, np.int32))
    assert (ip0 == 0).all() and len(ix0) == 0


def test_append_kv_rejects_bad_arguments_without_launching():
    lib = rpa.load()
    P = 256  # aligned stand-in address; these calls fail validation before any launch
    assert lib.rpa_append_kv(4, 0, 8, 128, None, None, None, None, None, None, 10, None, None) == 0
    assert rpa.STATUS[lib.rpa_append_kv(0, 3, 8, 128, P, P, P, P, P, P, 10, None, None)] == "RPA_E_ARG"
    assert rpa.STATUS[lib.rpa_append_kv(4, 3, 8, 96, P, P, P, P, P, P, 10, None, None)] == "RPA_E_SHAPE"
    assert rpa.STATUS[lib.rpa_append_kv(4, 3, 8, 128, P, None, P, P, P, P, 10, None, None)] == "RPA_E_ARG"
    assert rpa.STATUS[lib.rpa_append_kv(4, 3, 8, 128, P, P, P, P, P + 4, P, 10, None, None)] == "RPA_E_ARG"
    assert rpa.STATUS[lib.rpa_plan_upload(None, None)] == "RPA_E_ARG"


def test_valu_narrow_kernel_takes_tiles_of_at_most_8_rows():
    b = lengths_batch([1, 2, 1, 3], [40, 50, 1000, 300], H=8, Hk=2)  # G = 4: rows 4, 8, 4, 12
    p = rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=8, num_kv_heads=2,
                 head_dim=128, dtype="bf16", narrow_kernel="valu")
    t = p.tiles()
    rows = t[:, F["q_count"]] * 4
    assert ((t[:, F["kind"]] == 1) == ((rows > 0) & (rows <= 8))).all()
    assert (t[t[:, F["kind"]] == 1][:, F["kv_begin"]] % 32 == 0).all()
    m = make_plan(b).tiles()  # the MFMA narrow kernel takes up to 16 rows
    assert ((m[:, F["kind"]] == 1) == ((m[:, F["q_count"]] * 4 > 0) & (m[:, F["q_count"]] * 4 <= 16))).all()
    with pytest.raises(KeyError):
        rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=8, num_kv_heads=2,
                 head_dim=128, narrow_kernel="tensor")


def test_validate_page_table():
    b = W.tiny_ragged_prefill(spare_pages=2)
    rpa.validate_page_table(b.kv_page_indptr, b.kv_page_indices, b.num_pages)
    bad = b.kv_page_indices.copy()
    bad[-1] = b.num_pages
    with pytest.raises(rpa.RPAError) as e:
        rpa.validate_page_table(b.kv_page_indptr, bad, b.num_pages)
    assert e.value.status == "RPA_E_PAGE_OOB"
    bad[-1] = -1
    with pytest.raises(rpa.RPAError):
        rpa.validate_page_table(b.kv_page_indptr, bad, b.num_pages)


def test_run_rejects_unbound_plan():
    b = W.tiny_ragged_prefill()
    plan = make_plan(b)
    lib = rpa.load()
    rc = lib.rpa_run(plan._h, 1, 1, 1, None, None)
    assert rpa.STATUS[rc] == "RPA_E_ARG" and b"bind" in lib.rpa_last_error()


def test_empty_batch_and_zero_query_sequences():
    b = lengths_batch([], [])
    assert make_plan(b).info["num_tiles"] == 0
    b = lengths_batch([0, 0], [5, 0])
    info = make_plan(b).info
    assert info["num_tiles"] == 0 and info["total_q"] == 0


def test_planner_buffer_reuse_leaves_no_stale_state():
    """The planner keeps its work buffers between calls (per thread) and reuses the
    buffers of schedules replaced by rpa_plan_update: plans built in any order, and a
    plan updated back and forth, equal freshly built ones."""
    cases = [lengths_batch([8192] * 4 + [1] * 256, [8192] * 4 + [4096] * 256, H=64, Hk=8),
             lengths_batch([1] * 128, [1024] * 128),
             lengths_batch(W.short_prompt_lengths(), W.short_prompt_lengths(), H=32, Hk=8),
             lengths_batch([17, 3, 5, 1], [17, 30, 5, 48], D=64)]
    fresh = [make_plan(c).tiles() for c in cases]
    for c, f in list(zip(cases, fresh))[::-1] + list(zip(cases, fresh)):
        assert np.array_equal(make_plan(c).tiles(), f)
    # decode steps: every sequence one token longer, then back
    a = lengths_batch([1] * 64, [300] * 64, H=32, Hk=8)
    b2 = lengths_batch([1] * 64, [301] * 64, H=32, Hk=8)
    p = make_plan(a)
    ta, tb = p.tiles(), make_plan(b2).tiles()
    for _ in range(3):
        p.update(b2.qo_indptr, b2.kv_page_indptr, b2.kv_last_page_len)
        assert np.array_equal(p.tiles(), tb)
        p.update(a.qo_indptr, a.kv_page_indptr, a.kv_last_page_len)
        assert np.array_equal(p.tiles(), ta)


# ----------------------------------------------------------------------------------------------
# Workspace bound: rpa_workspace_bytes(batch, total_q, total_pages) covers every plan of
# those totals.
# ----------------------------------------------------------------------------------------------

def bound_of(b: W.Batch, **kw):
    return rpa.workspace_bytes(b.batch, b.total_q, int(b.kv_page_indptr[-1]), num_qo_heads=b.num_qo_heads,
                               num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, causal=b.causal, **kw)


from hypothesis import given, settings, strategies as st  # noqa: E402

SHAPES_WS = [(8, 1, 128), (32, 8, 128), (64, 8, 128), (8, 8, 64), (12, 1, 128), (16, 2, 64)]


@settings(max_examples=80, deadline=None)
@given(data=st.data())
def test_workspace_bound_covers_random_batches(data):
    H, Hk, D = data.draw(st.sampled_from(SHAPES_WS))
    causal = data.draw(st.booleans())
    kw = dict(max_kv_splits=data.draw(st.sampled_from([0, 1, 2, 3])),
              num_cus=data.draw(st.sampled_from([0, 0, 4, 64, 1024])),
              narrow_kernel=data.draw(st.sampled_from(["mfma", "valu"])))
    B = data.draw(st.integers(1, 24))
    q = data.draw(st.lists(st.integers(0, 300), min_size=B, max_size=B))
    extra = data.draw(st.lists(st.sampled_from([0, 1, 15, 16, 200, 1000, 5000]), min_size=B, max_size=B))
    kv = [qq + e if causal else max(1, e) if qq else e for qq, e in zip(q, extra)]
    b = lengths_batch(q, kv, H=H, Hk=Hk, D=D, causal=causal)
    need = make_plan(b, **kw).info["workspace_bytes"]
    assert need <= bound_of(b, **kw)


@pytest.mark.parametrize("num_cus", [0, 32])
def test_workspace_bound_covers_adversarial_length_mixes(num_cus):
    """Fixed totals, lengths placed to maximise each term of the bound: one long
    sequence holding every query (largest split tiles), every query a decode row over
    one long sequence's pages, and one very long prompt beside many one-token prompts
    (the longest XCD padding run)."""
    for H, Hk in ((8, 1), (32, 8), (64, 8)):
        B, T, P = 64, 64 * 16, 64 * 300
        cases = [
            ([T] + [0] * (B - 1), [16 * P] + [0] * (B - 1)),                       # one sequence has all
            ([16] * B, [16 * 300] * B),                                            # even
            ([1] * (B - 1) + [T - B + 1], [16] * (B - 1) + [16 * (P - B + 1)]),    # one long prompt
            ([T // B] * B, [16 * (P - B + 1)] + [16] * (B - 1)),                   # keys on one sequence
        ]
        for q, kv in cases:
            assert sum(q) == T and sum(W.pages_for(k) for k in kv) == P
            b = lengths_batch(q, kv, H=H, Hk=Hk)
            for splits in (0, 1, 4):
                need = make_plan(b, max_kv_splits=splits, num_cus=num_cus).info["workspace_bytes"]
                assert need <= bound_of(b, max_kv_splits=splits, num_cus=num_cus), (H, q[:3], kv[:3], splits)


def test_workspace_bound_of_the_decode_workload_is_usable():
    # the flashinfer #323 repro's shape: 128 decode rows over 64 pages each
    b = lengths_batch([1] * 128, [1024] * 128)
    need, bound = make_plan(b).info["workspace_bytes"], bound_of(b)
    assert need <= bound <= 128 << 20  # within the repro's 128 MiB workspace
    with pytest.raises(rpa.RPAError) as e:
        rpa.workspace_bytes(4, 10, 10, num_qo_heads=8, num_kv_heads=3, head_dim=128)
    assert e.value.status == "RPA_E_SHAPE"
    with pytest.raises(rpa.RPAError) as e:
        rpa.workspace_bytes(-1, 10, 10, num_qo_heads=8, num_kv_heads=1, head_dim=128)
    assert e.value.status == "RPA_E_ARG"


def test_plan_update_refuses_another_kernel_configuration():
    """A captured graph replays the launch configured for the bound schedule; update
    must refuse lengths that would need another kernel: the VALU kernel's row
    capacity (2 -> 4 rows per tile) here, with the tile counts unchanged."""
    b1 = lengths_batch([1] * 8, [700] * 8, H=4, Hk=2)  # 2 rows per tile
    b2 = lengths_batch([2] * 8, [700] * 8, H=4, Hk=2)  # 4 rows per tile
    p = make_plan(b1, narrow_kernel="valu", max_kv_splits=1)
    before = p.tiles().copy()
    with pytest.raises(rpa.RPAError) as e:
        p.update(b2.qo_indptr, b2.kv_page_indptr, b2.kv_last_page_len)
    assert e.value.status == "RPA_E_UNSUPPORTED" and "kernel" in str(e.value)
    assert np.array_equal(p.tiles(), before)
    # the MFMA narrow kernel takes both row counts with one configuration
    m = make_plan(b1, max_kv_splits=1)
    m.update(b2.qo_indptr, b2.kv_page_indptr, b2.kv_last_page_len)
    assert np.array_equal(m.tiles(), make_plan(b2, max_kv_splits=1).tiles())


def test_benchmark_floors_library_loads():
    """The benchmark's microkernel library is built beside librpa.so and exports its
    four floors (launched only by bench.py, on a GPU)."""
    import os
    path = os.path.join(os.path.dirname(rpa.LIB_PATH), "librpa_floors.so")
    lib = ctypes.CDLL(path)
    for name in ("rpa_floor_empty", "rpa_floor_stream", "rpa_floor_gather", "rpa_floor_mfma"):
        assert hasattr(lib, name), name


# ----------------------------------------------------------------------------------------------
# Shared-prefix plans (rpa_plan_create_shared): decode rows grouped over the prefix.
# ----------------------------------------------------------------------------------------------

def check_groups(b, plan, shared_pages):
    """Group tiles of a shared-prefix plan: every eligible decode row (q_len 1, kv_len at
    least the prefix) of every kv head is in exactly one tile of its own kind, group
    members are consecutive sequences (consecutive query rows), a tile holds at most 16
    rows, and its virtual steps cover the prefix and each member's own keys."""
    t = plan.tiles()
    G = b.num_qo_heads // b.num_kv_heads
    Ks = 16 * shared_pages
    grp = t[t[:, F["kind"]] == 2]
    covered = {}
    for r in grp:
        n, b0, hk = int(r[F["q_count"]]), int(r[F["seq"]]), int(r[F["kv_head"]])
        assert 2 <= n and n * G <= 16 and r[F["kv_len"]] == Ks and r[F["n_splits"]] == 1 and r[F["part"]] == -1
        pm = int(r[F["pos0"]])  # private 16-key pages per member, two pages per 32-key step
        assert r[F["kv_begin"]] == 0 and r[F["kv_end"]] == 32 * -(-(shared_pages + n * pm) // 2)
        assert r[F["q_row0"]] == b.qo_indptr[b0] and r[F["page_base"]] == b.kv_page_indptr[b0]
        for i in range(n):
            s = b0 + i
            assert b.q_lens[s] == 1 and b.kv_lens[s] >= Ks and b.qo_indptr[s] == b.qo_indptr[b0] + i
            assert 16 * pm >= b.kv_lens[s] - Ks
            assert (s, hk) not in covered
            covered[(s, hk)] = True
    # ungrouped rows keep ordinary tiles: every (token, kv head) exactly once overall
    cov = np.zeros((b.total_q, b.num_kv_heads), np.int32)
    for r in t:
        if r[F["q_count"]] == 0:
            continue
        if r[F["kind"]] == 2:
            cov[r[F["q_row0"]]:r[F["q_row0"]] + r[F["q_count"]], r[F["kv_head"]]] += 1
        elif r[F["split"]] == 0:
            cov[r[F["q_row0"]]:r[F["q_row0"]] + r[F["q_count"]], r[F["kv_head"]]] += 1
    assert (cov == 1).all()
    return grp


def test_shared_prefix_decode_rows_are_grouped():
    # the shared-prefix decode step: 256 requests, 12 shared pages (192 tokens), kv 231,
    # 4 query heads per kv head: four requests per tile, 512 tiles instead of 2048
    b = lengths_batch([1] * 256, [231] * 256, H=32, Hk=8)
    p = make_plan(b, shared_pages=12)
    grp = check_groups(b, p, 12)
    # 39 own keys per request: 3 pages, so 12 shared + 4 x 3 private pages = 12 steps
    assert len(grp) == 512 and (grp[:, F["q_count"]] == 4).all() and (grp[:, F["pos0"]] == 3).all()
    assert (grp[:, F["kv_end"]] == 32 * 12).all()
    assert p.info["num_tiles"] == 512 and p.info["visible_pairs"] == make_plan(b).info["visible_pairs"]
    # 8 query heads per kv head: pairs; 16 or more: nothing to group
    assert (check_groups(lengths_batch([1] * 9, [300] * 9), make_plan(lengths_batch([1] * 9, [300] * 9),
                                                                     shared_pages=5), 5)[:, F["q_count"]] <= 2).all()
    b16 = lengths_batch([1] * 8, [300] * 8, H=16, Hk=1)
    assert not (make_plan(b16, shared_pages=5).tiles()[:, F["kind"]] == 2).any()
    # the VALU decode kernel does not take group tiles
    assert not (make_plan(b, shared_pages=12, narrow_kernel="valu").tiles()[:, F["kind"]] == 2).any()


def test_shared_prefix_grouping_rules():
    # prefill rows, rows that do not see the whole prefix, and lone rows keep ordinary
    # tiles; a group ends rather than pad a short member to a long one
    q = [1, 1, 30, 1, 1, 1, 1, 1, 1, 1, 1, 1]
    kv = [231, 240, 230, 231, 100, 231, 232, 900, 231, 233, 235, 1500]
    b = lengths_batch(q, kv, H=32, Hk=8)
    p = make_plan(b, shared_pages=12)
    grp = check_groups(b, p, 12)
    members = sorted({int(r[F["seq"]]) + i for r in grp for i in range(int(r[F["q_count"]]))})
    assert 2 not in members and 4 not in members  # prefill; kv_len below the prefix
    assert 7 not in members or 6 not in members  # 900 keys padded beside 232 wastes too much
    for extra in (0, 3):
        bb = lengths_batch([1] * 40, [16 * 7 + 5 + (i * extra) % 200 for i in range(40)], H=8, Hk=2)
        check_groups(bb, make_plan(bb, shared_pages=7), 7)
    # odd prefix page counts: the last shared page and the first private one share a step
    bo = lengths_batch([1] * 12, [16 * 5 + 9] * 12, H=16, Hk=4)
    go = check_groups(bo, make_plan(bo, shared_pages=5), 5)
    assert len(go) > 0 and (go[:, F["kv_end"]] == 32 * ((5 + go[:, F["q_count"]] * 1 + 1) // 2)).all()


def test_shared_prefix_plan_update_and_bounds():
    b0 = lengths_batch([1] * 256, [231] * 256, H=32, Hk=8)
    b1 = lengths_batch([1] * 256, [232] * 256, H=32, Hk=8)
    p = make_plan(b0, shared_pages=12)
    p.update(b1.qo_indptr, b1.kv_page_indptr, b1.kv_last_page_len)
    assert np.array_equal(p.tiles(), make_plan(b1, shared_pages=12).tiles())
    for b in (b0, b1, lengths_batch([1, 1, 40, 1], [300, 200, 250, 999], H=32, Hk=8)):
        need = make_plan(b, shared_pages=12).info["workspace_bytes"]
        assert need <= bound_of(b)
    with pytest.raises(rpa.RPAError) as e:
        make_plan(b0, shared_pages=-1)
    assert e.value.status == "RPA_E_ARG"


def test_binding_refuses_host_tensors_before_any_call():
    """The C ABI takes raw device pointers; the binding refuses host (CPU) tensors and
    wrong shapes itself, before anything reaches the library."""
    b = W.tiny_ragged_prefill()
    plan = make_plan(b)
    T, H, D = b.total_q, b.num_qo_heads, b.head_dim
    idx = torch.from_numpy(b.kv_page_indices.astype(np.int32))
    with pytest.raises(ValueError, match="kv_page_indices"):
        plan.bind(idx, num_pages=b.num_pages)
    with pytest.raises(ValueError, match="q must be"):
        plan.run(b.q, b.kv_cache)
    with pytest.raises(ValueError, match="q must be"):
        plan.run_noalloc(b.q, b.kv_cache, idx, torch.empty_like(b.q))
    new = torch.zeros((1, 2, 1, D), dtype=b.kv_cache.dtype)
    i32 = lambda *v: torch.tensor(v, dtype=torch.int32)
    with pytest.raises(ValueError, match="kv_cache"):
        rpa.append_kv(new, b.kv_cache, i32(0, 1), i32(0, 2), i32(0, 1), i32(5))
    o = torch.zeros((T, H, D), dtype=torch.float16)
    l = torch.zeros((T, H), dtype=torch.float32)
    with pytest.raises(ValueError, match="o_a and o_b"):
        rpa.merge_states(o, l, o, l)
    plan.close()
