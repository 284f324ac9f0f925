"""The planner's schedules, executed in binary64 on the CPU (tests/tile_interp.py),
against the oracle.

Each case plans a batch with the C-ABI planner (host-only, no GPU), runs every
work item the plan lists over the batch's own inputs, merges the split pieces,
and requires the oracle's O and LSE to within 1e-12 (summation order is the
only difference).  This checks, over whole schedules, that every (row, head)
sees exactly its visible keys once: no piece dropped or repeated, no key range
cut short, no mask or page base wrong, the kGroup members' private keys all
walked.  The last tests plant mistakes in a schedule and require the executor
to notice them.
"""
import numpy as np
import pytest

import oracle
import paged_kv_attention_ragged_amd as rpa
import workloads as W

from tests.tile_interp import execute, ScheduleError, KIND, KGROUP, POS0, N_SPLITS, KV_END, KV_BEGIN, KV_LEN, Q_COUNT, PART

TOL = 1e-12


def plan_for(b, **kw):
    return rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=b.num_qo_heads,
                    num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, dtype=b.dtype, causal=b.causal, **kw)


def assert_schedule_matches_oracle(b, plan):
    recs = plan.tiles()
    O, LSE = execute(b, recs)
    Oo, Lo = oracle.run(**b.oracle_kwargs())
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(LSE))
    eo = np.abs(O - Oo) / (1 + np.abs(Oo))
    el = np.abs(LSE - Lo) / (1 + np.abs(Lo))
    assert eo.max() <= TOL, eo.max()
    assert el.max() <= TOL, el.max()
    return recs


def test_tiny_ragged_prefill_schedules():
    b = W.tiny_ragged_prefill(poison=True, spare_pages=5)
    for kw in ({}, {"num_cus": 4096}, {"narrow_kernel": "valu"}):
        assert_schedule_matches_oracle(b, plan_for(b, **kw))


def test_decode_batch_split_and_valu():
    b = W.make_batch("decode", [1] * 12, [1024, 17, 300, 1, 999, 512, 513, 64, 2000, 31, 257, 700],
                     num_qo_heads=8, num_kv_heads=1, head_dim=128, dtype="f16", seed=11, poison=True, spare_pages=3)
    r = assert_schedule_matches_oracle(b, plan_for(b))
    assert (r[:, N_SPLITS] > 1).any()
    assert_schedule_matches_oracle(b, plan_for(b, narrow_kernel="valu"))
    assert_schedule_matches_oracle(b, plan_for(b, max_kv_splits=1))


def test_short_prompt_batch():
    b = W.make_batch("short", W.short_prompt_lengths(24, hi=200, seed=5), W.short_prompt_lengths(24, hi=200, seed=5),
                     num_qo_heads=16, num_kv_heads=4, head_dim=64, dtype="bf16", seed=12, poison=True)
    assert_schedule_matches_oracle(b, plan_for(b))
    assert_schedule_matches_oracle(b, plan_for(b, num_cus=2048))


def test_mixed_prompts_and_decode_rows_one_launch():
    q = [700, 1] + [1] * 20 + [333]
    kv = [700, 1500] + [40 + 37 * i for i in range(20)] + [333]
    b = W.make_batch("mixed", q, kv, num_qo_heads=8, num_kv_heads=1, head_dim=128, dtype="bf16", seed=13)
    for cus in (0, 8):
        p = plan_for(b, num_cus=cus)
        r = assert_schedule_matches_oracle(b, p)
    kinds = set(r[r[:, Q_COUNT] > 0, KIND].tolist())
    assert kinds <= {0, 1}


def test_suffix_rows_after_a_cached_prefix():
    # q_len < kv_len prefill (a suffix after cached tokens), several tiles per sequence
    b = W.make_batch("suffix", [30, 200, 5, 129], [230, 260, 500, 129], num_qo_heads=4, num_kv_heads=2,
                     head_dim=128, dtype="f16", seed=14, poison=True, spare_pages=2)
    for kw in ({}, {"num_cus": 4096}, {"narrow_kernel": "valu"}):
        assert_schedule_matches_oracle(b, plan_for(b, **kw))


def test_non_causal_queries_outnumbering_keys():
    b = W.make_batch("cascade_prefix", [40, 3, 300], [25, 200, 16], num_qo_heads=8, num_kv_heads=2,
                     head_dim=64, dtype="f16", seed=15, causal=False)
    assert_schedule_matches_oracle(b, plan_for(b))
    assert_schedule_matches_oracle(b, plan_for(b, num_cus=4096))


RAGGED_SHAPES = [(1, 2, 64), (4, 1, 128), (16, 1, 64), (2, 3, 128)]


def random_ragged_batches(G, Hk, D):
    """[(batch, [plan kwargs ...]), ...]: three random ragged batches (prefill rows,
    suffixes, decode rows; poisoned unowned slots) with a plan as made, one for a
    random machine size and one with forced splits of at most 2.  Also used by the
    GPU tests."""
    rng = np.random.default_rng(100 * G + Hk + D)
    out = []
    for trial in range(3):
        B = int(rng.integers(1, 9))
        kv = rng.integers(1, 600, B)
        q = np.array([int(rng.integers(1, k + 1)) if rng.random() < 0.6 else 1 for k in kv])
        b = W.make_batch("rand_g%d_hk%d_d%d_%d" % (G, Hk, D, trial), q.tolist(), kv.tolist(), num_qo_heads=G * Hk,
                         num_kv_heads=Hk, head_dim=D, dtype=("f16", "bf16")[trial % 2],
                         seed=int(rng.integers(1 << 30)), poison=True, spare_pages=int(rng.integers(0, 4)))
        out.append((b, [{}, {"num_cus": int(rng.choice([1, 4, 4096]))}, {"max_kv_splits": 2, "num_cus": 4096}]))
    return out


@pytest.mark.parametrize("G,Hk,D", RAGGED_SHAPES)
def test_random_ragged_batches(G, Hk, D):
    for b, kws in random_ragged_batches(G, Hk, D):
        for kw in kws:
            assert_schedule_matches_oracle(b, plan_for(b, **kw))


def _shared_decode(n_req=12, G=8, Hk=2, D=64):
    base = W.shared_prefix_suffix(n_req=n_req, prefix=200, suffix=30, decode_steps=70, num_qo_heads=G * Hk,
                                  num_kv_heads=Hk, head_dim=D, dtype="f16")
    return base


def test_grouped_decode_over_a_shared_prefix():
    base = _shared_decode()
    for step in (1, 40):
        d = W.decode_step(base, step)
        p = plan_for(d, shared_pages=12)
        r = assert_schedule_matches_oracle(d, p)
        assert (r[:, KIND] == KGROUP).any()


def test_grouped_members_of_different_lengths():
    # members' own keys differ: trim some sequences so the group pads its private steps
    base = _shared_decode(n_req=10, G=4, Hk=1, D=128)
    d = W.decode_step(base, 50)
    lens = d.kv_lens.copy()
    lens[1::3] -= 37
    lens[2::4] -= 5
    q_lens = [1] * d.batch
    qo, kp, ki, last = [0], [0], [], []
    for s in range(d.batch):
        n = W.pages_for(lens[s])
        ki.extend(d.kv_page_indices[d.kv_page_indptr[s]:d.kv_page_indptr[s] + n])
        kp.append(kp[-1] + n)
        qo.append(qo[-1] + q_lens[s])
        last.append(W.last_page_len_for(lens[s]))
    t = W.Batch("trimmed", np.array(qo, np.int32), np.array(kp, np.int32), np.array(ki, np.int32),
                np.array(last, np.int32), d.q, d.kv_cache, d.num_qo_heads, d.num_kv_heads, d.head_dim, d.dtype)
    r = assert_schedule_matches_oracle(t, plan_for(t, shared_pages=12))
    assert (r[:, KIND] == KGROUP).any()


def random_config_batch(seed):
    """(batch, [plan kwargs ...]): a random configuration -- G 1..16, 1..8 kv heads,
    D 64 / 128, fp16 / bf16, causal or not (non-causal rows may outnumber their keys),
    sequences with no queries among them, poisoned unowned slots -- with plans on the
    MFMA and the VALU narrow kernel, cacheable or streamed K/V, as made or split.
    Also used by the GPU tests."""
    rng = np.random.default_rng(900 + seed)
    G = int(rng.choice([1, 2, 4, 8, 16]))
    Hk = int(rng.choice([1, 2, 4, 8]))
    while G * Hk > 64:
        Hk //= 2
    D = int(rng.choice([64, 128]))
    causal = bool(rng.random() < 0.7)
    B = int(rng.integers(1, 16))
    q, kv = [], []
    for _ in range(B):
        r = rng.random()
        k = int(rng.integers(1, 400))
        if r < 0.1:
            q.append(0)                          # a sequence with no queries this call
        elif r < 0.55:
            q.append(1)                          # decode row
        elif causal:
            q.append(int(rng.integers(1, k + 1)))  # prefill or suffix
        else:
            q.append(int(rng.integers(1, k + k // 2 + 2)))  # may outnumber the keys
        kv.append(k)
    b = W.make_batch("cfg%d" % seed, q, kv, num_qo_heads=G * Hk, num_kv_heads=Hk, head_dim=D,
                     dtype=("f16", "bf16")[int(rng.integers(0, 2))], seed=1000 + seed, poison=True,
                     spare_pages=int(rng.integers(0, 3)), causal=causal)
    kws = [{}, {"narrow_kernel": "valu"}, {"kv_shared": True, "num_cus": int(rng.choice([2, 64, 4096]))}]
    return b, kws


@pytest.mark.parametrize("seed", range(12))
def test_random_configurations(seed):
    b, kws = random_config_batch(seed)
    for kw in kws:
        kw = {k: v for k, v in kw.items() if k != "kv_shared"}  # a caching hint: no effect on the plan
        assert_schedule_matches_oracle(b, plan_for(b, **kw))


def _share_prefix(b, pages):
    """The first `pages` page ids of every sequence with that many pages point at the
    first sequence's pages (a prefix stored once; layout only)."""
    idx = b.kv_page_indices.copy()
    first = idx[:pages].copy()
    for s in range(b.batch):
        a = int(b.kv_page_indptr[s])
        if int(b.kv_page_indptr[s + 1]) - a >= pages:
            idx[a:a + pages] = first
    return W.Batch(b.name + "_shared", b.qo_indptr, b.kv_page_indptr, idx, b.kv_last_page_len, b.q, b.kv_cache,
                   b.num_qo_heads, b.num_kv_heads, b.head_dim, b.dtype, b.causal)


def random_grouped_batch(seed):
    """(batch, P): a random mix over a declared shared prefix of P pages -- decode rows
    that see the whole prefix, decode rows shorter than it, prefill rows and suffixes;
    G from 1 to 8, poisoned unowned slots.  Also used by the GPU tests."""
    rng = np.random.default_rng(500 + seed)
    P = int(rng.integers(1, 7))
    Ks = 16 * P
    G = int(rng.choice([1, 2, 4, 8]))
    Hk = int(rng.choice([1, 2]))
    B = int(rng.integers(4, 40))
    q, kv = [1], [Ks + int(rng.integers(0, 80))]
    for _ in range(B - 1):
        r = rng.random()
        if r < 0.6:
            q.append(1)
            kv.append(Ks + int(rng.integers(0, 150)))
        elif r < 0.75:
            q.append(1)
            kv.append(int(rng.integers(1, Ks + 1)))
        else:
            k = int(rng.integers(1, Ks + 200))
            q.append(int(rng.integers(1, k + 1)))
            kv.append(k)
    b = _share_prefix(W.make_batch("grp_rand%d" % seed, q, kv, num_qo_heads=G * Hk, num_kv_heads=Hk,
                                   head_dim=int(rng.choice([64, 128])), dtype=("f16", "bf16")[seed % 2],
                                   seed=600 + seed, poison=True, spare_pages=2), P)
    return b, P


def grouped_page_edges_batch(dtype="bf16"):
    """(batch, P): decode rows over an odd shared prefix (P = 5 pages, 80 keys), 4 query
    heads per kv head, so 4 requests per group tile: a group with no keys of its own
    (no private page slots: the last shared page shares its step with nothing), and
    groups whose members own 1, 2, 15, 16, 17, 30-33 or 47 keys, so that a 32-key step
    holds the last page of one member and the first of the next, or a member's empty
    padding page.  Also used by the GPU tests."""
    P = 5
    own = [0, 0, 0, 0, 16, 17, 20, 30, 1, 16, 2, 15, 31, 32, 33, 47]
    b = W.make_batch("grp_edges_" + dtype, [1] * len(own), [16 * P + k for k in own], num_qo_heads=8,
                     num_kv_heads=2, head_dim=128, dtype=dtype, seed=77, poison=True, spare_pages=3)
    return _share_prefix(b, P), P


def test_grouped_page_slot_edges():
    """grouped_page_edges_batch on the CPU executor: group tiles with zero and with
    several private pages per member, each against the oracle."""
    b, P = grouped_page_edges_batch()
    plan = plan_for(b, shared_pages=P)
    r = plan.tiles()
    grp = r[r[:, KIND] == KGROUP]
    assert len(grp) > 0 and (grp[:, POS0] == 0).any() and (grp[:, POS0] >= 2).any()
    # no private pages: the 5 shared pages take 3 steps
    assert (grp[grp[:, POS0] == 0][:, KV_END] == 96).all()
    assert_schedule_matches_oracle(b, plan)


@pytest.mark.parametrize("seed", range(6))
def test_random_grouped_batches(seed):
    """random_grouped_batch plans, with and without forced splits, executed on the CPU."""
    b, P = random_grouped_batch(seed)
    for kw in ({}, {"num_cus": 4096}):
        assert_schedule_matches_oracle(b, plan_for(b, shared_pages=P, **kw))


def test_tail_skip_switch(monkeypatch):
    b = W.make_batch("prompts", [400, 129, 77], [400, 300, 77], num_qo_heads=8, num_kv_heads=1, head_dim=128,
                     dtype="bf16", seed=16, poison=True)
    on = plan_for(b, max_kv_splits=1).tiles()
    monkeypatch.setenv("RPA_DISABLE_TAIL_SKIP", "1")
    p_off = plan_for(b, max_kv_splits=1)
    off = assert_schedule_matches_oracle(b, p_off)
    assert_schedule_matches_oracle(b, plan_for(b))
    real_on, real_off = on[on[:, Q_COUNT] > 0], off[off[:, Q_COUNT] > 0]
    # without the skip every tile walks to kv_len; with it, the earlier tiles of a prompt stop sooner
    assert (real_off[:, KV_END] == real_off[:, KV_LEN]).all()
    assert (real_on[:, KV_END] - real_on[:, KV_BEGIN]).sum() < (real_off[:, KV_END] - real_off[:, KV_BEGIN]).sum()
    assert_schedule_matches_oracle(b, plan_for(b, num_cus=4096))
    # update keeps the setting of the plan it updates, whatever the environment says now
    monkeypatch.delenv("RPA_DISABLE_TAIL_SKIP")
    p_off.update(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len)
    assert (p_off.tiles() == off).all()


def test_plan_log_line(capfd, monkeypatch):
    b = W.tiny_ragged_prefill()
    plan_for(b)
    assert "rpa:" not in capfd.readouterr().err
    monkeypatch.setenv("RPA_LOG", "1")
    p = plan_for(b, num_cus=4096)
    err = capfd.readouterr().err
    assert err.startswith("rpa: create batch=4 total_q=26 tiles=%d " % p.info["num_tiles"])
    assert "split_groups=%d " % p.info["num_split_groups"] in err
    assert "workspace=%d B" % p.info["workspace_bytes"] in err
    p.update(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len)
    assert capfd.readouterr().err.startswith("rpa: update batch=4")


# ---- the executor notices a broken schedule ---------------------------------------------

def _broken(recs, how):
    r = recs.copy()
    real = np.nonzero(r[:, Q_COUNT] > 0)[0]
    if how == "drop_piece":
        i = real[np.nonzero(r[real, N_SPLITS] > 1)[0][1]]
        return np.delete(r, i, axis=0)
    if how == "repeat_tile":
        return np.concatenate([r, r[real[:1]]])
    if how == "short_range":
        i = real[np.argmax(r[real, KV_END] - r[real, KV_BEGIN])]
        r[i, KV_END] -= 16
        return r
    if how == "shifted_range":
        i = real[np.argmax(r[real, KV_END] - r[real, KV_BEGIN])]
        r[i, KV_BEGIN] += 1
        r[i, KV_END] += 1
        return r
    if how == "part_overlap":
        sp = real[r[real, N_SPLITS] > 1]
        r[sp[-1], PART] = r[sp[0], PART]
        return r
    raise ValueError(how)


@pytest.mark.parametrize("how", ["drop_piece", "repeat_tile", "short_range", "shifted_range", "part_overlap"])
def test_executor_rejects_broken_schedules(how):
    b = W.make_batch("dec", [1, 1, 3, 40], [900, 700, 600, 800], num_qo_heads=8, num_kv_heads=1, head_dim=64,
                     dtype="f16", seed=17)
    recs = plan_for(b, num_cus=4096).tiles()
    assert (recs[:, N_SPLITS] > 1).sum() >= 4
    Oo, Lo = oracle.run(**b.oracle_kwargs())
    try:
        O, L = execute(b, _broken(recs, how))
    except (ScheduleError, IndexError):
        return
    err = max(np.nanmax(np.abs(O - Oo)), np.nanmax(np.abs(L - Lo)))
    assert err > 1e-6 or np.isnan(O).any()
