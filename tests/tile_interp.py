"""Binary64 CPU executor of a plan's work items: the test suite's stand-in backend.

It runs every record that ``rpa_plan_tiles`` reports with the scope the kernels
give it (query rows, kv head, key range, split piece, kGroup members) and then
combines each split query tile's pieces by their log-sum-exp, the way the fused
merge does.  All arithmetic is numpy float64, so the only difference from the
oracle (one pass over all visible keys in binary64) is summation order.  A
schedule that drops, repeats, misplaces or mis-masks work therefore misses the
oracle by far more than rounding, while a correct one agrees to about 1e-14.

The record fields are those rpa.h documents for rpa_plan_tiles.  Inputs are the
test's own Batch (host page table, CPU fp16 / bf16 tensors); the planner only
sees lengths, so every page access here goes through the batch's page table.
"""
import math
from collections import defaultdict

import numpy as np
import torch

# record fields (rpa_plan_tiles)
Q_ROW0, Q_COUNT, POS0, KV_LEN, PAGE_BASE, KV_HEAD, KV_BEGIN, KV_END, PART, SEQ, SPLIT, N_SPLITS, KIND, GROUP = range(14)
WIDE, NARROW, KGROUP = 0, 1, 2


class ScheduleError(AssertionError):
    pass


def _state(qh, keys, vals, visible, scale):
    """Softmax state of query rows qh [R, D] over keys [n, D]: running max m [R]
    (-inf where no key is visible), sum l [R] and unnormalised output acc [R, D]."""
    R = qh.shape[0]
    if keys.shape[0] == 0 or not visible.any():
        return np.full(R, -np.inf), np.zeros(R), np.zeros((R, qh.shape[1]))
    s = scale * (qh @ keys.T)
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1)
    ms = np.where(np.isfinite(m), m, 0.0)
    p = np.where(visible, np.exp(s - ms[:, None]), 0.0)
    return m, p.sum(axis=1), p @ vals


def _combine(states):
    """Merge softmax states [(m, l, acc), ...] of the same rows."""
    m = np.max(np.stack([s[0] for s in states]), axis=0)
    ms = np.where(np.isfinite(m), m, 0.0)
    l = np.zeros_like(m)
    acc = np.zeros_like(states[0][2])
    for mi, li, ai in states:
        w = np.where(np.isfinite(mi), np.exp(mi - ms), 0.0)
        l += w * li
        acc += w[:, None] * ai
    return m, l, acc


class Executor:
    def __init__(self, batch, sm_scale=None):
        b = batch
        self.b = b
        self.H, self.Hk, self.D = b.num_qo_heads, b.num_kv_heads, b.head_dim
        self.G = self.H // self.Hk
        self.ps = b.page_size
        self.scale = 1.0 / math.sqrt(self.D) if sm_scale is None else float(sm_scale)
        self.q = b.q.to(torch.float64).numpy()
        self.kv = b.kv_cache.to(torch.float64).numpy()
        self.idx = np.asarray(b.kv_page_indices, dtype=np.int64)
        self.kv_lens = np.asarray(b.kv_lens, dtype=np.int64)
        self.q_lens = np.asarray(b.q_lens, dtype=np.int64)
        T = b.total_q
        self.O = np.full((T, self.H, self.D), np.nan)
        self.LSE = np.full((T, self.H), np.nan)
        self.written = np.zeros(T, dtype=np.int64)  # (row, kv head) writes, as a count per row
        self.pieces = defaultdict(dict)

    def _kv(self, page_base, j, hk):
        """K and V rows of keys j (int array) through the page table from entry page_base."""
        ent = page_base + j // self.ps
        if len(j) and (ent.min() < 0 or ent.max() >= len(self.idx)):
            raise ScheduleError("key outside the page table (entries %d..%d of %d)" % (ent.min(), ent.max(), len(self.idx)))
        pg = self.idx[ent]
        sl = j % self.ps
        return self.kv[pg, 0, sl, hk], self.kv[pg, 1, sl, hk]

    def _rows(self, rows, hk):
        """Query rows [len(rows) * G, D], token-major then head (the tiles' row order)."""
        return self.q[rows][:, hk * self.G:(hk + 1) * self.G].reshape(-1, self.D)

    def _emit(self, rec, rows, hk, st):
        m, l, acc = st
        if rec[PART] < 0:
            self._write(rows, hk, m, l, acc)
        else:
            g = int(rec[GROUP])
            if int(rec[SPLIT]) in self.pieces[g]:
                raise ScheduleError("split group %d piece %d scheduled twice" % (g, rec[SPLIT]))
            self.pieces[g][int(rec[SPLIT])] = (tuple(rows), hk, int(rec[N_SPLITS]), int(rec[PART]), st)

    def _write(self, rows, hk, m, l, acc):
        G = self.G
        if np.any(l <= 0):
            raise ScheduleError("a query row of kv head %d saw no key" % hk)
        o = acc / l[:, None]
        lse = m + np.log(l)
        for i, r in enumerate(rows):
            if not np.all(np.isnan(self.LSE[r, hk * G:(hk + 1) * G])):
                raise ScheduleError("row %d, kv head %d written twice" % (r, hk))
            self.O[r, hk * G:(hk + 1) * G] = o[i * G:(i + 1) * G]
            self.LSE[r, hk * G:(hk + 1) * G] = lse[i * G:(i + 1) * G]
            self.written[r] += 1

    def run_tile(self, rec):
        n = int(rec[Q_COUNT])
        if n == 0:  # empty XCD padding slot
            if rec[KV_END] != rec[KV_BEGIN] or rec[PART] != -1:
                raise ScheduleError("padding slot with work: %s" % rec[:14])
            return
        hk = int(rec[KV_HEAD])
        if int(rec[KIND]) == KGROUP:
            self._run_group(rec, hk, n)
            return
        rows = list(range(int(rec[Q_ROW0]), int(rec[Q_ROW0]) + n))
        pos = int(rec[POS0]) + np.arange(n)
        # keys of the piece that exist (past kv_len there may be no page to read)
        j = np.arange(int(rec[KV_BEGIN]), min(int(rec[KV_END]), int(rec[KV_LEN])))
        vis = np.ones((n, len(j)), dtype=bool)
        if self.b.causal:
            vis &= j[None, :] <= pos[:, None]
        K, V = self._kv(int(rec[PAGE_BASE]), j, hk)
        st = _state(self._rows(rows, hk), K, V, np.repeat(vis, self.G, axis=0), self.scale)
        self._emit(rec, rows, hk, st)

    def _run_group(self, rec, hk, n):
        """kGroup tile: n consecutive decode sequences from rec[SEQ]; the first rec[KV_LEN]
        keys (the declared shared prefix) through the first member's page table, then
        rec[POS0] 16-key pages of each member's own keys through its own, all of them
        walked two pages per 32-key step up to rec[KV_END]."""
        seq0 = int(rec[SEQ])
        shared = int(rec[KV_LEN])
        pages = int(rec[POS0])
        if rec[PART] != -1:
            raise ScheduleError("kGroup tiles are never split")
        if shared % 16 or int(rec[KV_END]) != 32 * -(-(shared // 16 + n * pages) // 2):
            raise ScheduleError("kGroup tile's key range %d does not hold its %d shared keys and %d x %d pages"
                                % (rec[KV_END], shared, n, pages))
        for mbr in range(n):
            s = seq0 + mbr
            if self.q_lens[s] != 1:
                raise ScheduleError("kGroup member %d has q_len %d" % (s, self.q_lens[s]))
            row = int(self.b.qo_indptr[s])
            if row != int(rec[Q_ROW0]) + mbr:
                raise ScheduleError("kGroup member %d is not at row %d" % (s, int(rec[Q_ROW0]) + mbr))
            L = int(self.kv_lens[s])
            if shared + 16 * pages < L:
                raise ScheduleError("kGroup member %d: %d pages do not cover its %d own keys" % (s, pages, L - shared))
            js = np.arange(0, shared)
            jp = np.arange(shared, min(L, shared + 16 * pages))
            K0, V0 = self._kv(int(rec[PAGE_BASE]), js, hk)
            K1, V1 = self._kv(int(self.b.kv_page_indptr[s]), jp, hk)
            K, V = np.concatenate([K0, K1]), np.concatenate([V0, V1])
            j = np.concatenate([js, jp])
            vis = np.ones((self.G, len(j)), dtype=bool)
            if self.b.causal:
                vis &= (j <= L - 1)[None, :]
            self._write([row], hk, *_state(self._rows([row], hk), K, V, vis, self.scale))

    def finish(self):
        """Combine split pieces; returns (O [T, H, D], LSE [T, H]) in float64."""
        parts = []
        for g, ps in self.pieces.items():
            rows, hk, ns, _, _ = next(iter(ps.values()))
            if sorted(ps) != list(range(ns)):
                raise ScheduleError("split group %d has pieces %s of %d" % (g, sorted(ps), ns))
            for s, (r, h, n2, part, _) in ps.items():
                if r != rows or h != hk or n2 != ns:
                    raise ScheduleError("split group %d mixes query tiles" % g)
                parts.append((part, part + len(rows) * self.G))
            self._write(list(rows), hk, *_combine([ps[s][4] for s in range(ns)]))
        parts.sort()
        for (a0, a1), (b0, _) in zip(parts, parts[1:]):
            if b0 < a1:
                raise ScheduleError("partial rows [%d, %d) and [%d, ..) overlap" % (a0, a1, b0))
        return self.O, self.LSE


def execute(batch, records, sm_scale=None):
    """Run every record of a plan over `batch` in binary64; returns (O, LSE)."""
    ex = Executor(batch, sm_scale)
    for rec in records:
        ex.run_tile(rec)
    O, LSE = ex.finish()
    if np.any(ex.written != batch.num_kv_heads):
        raise ScheduleError("query rows %s not written once per kv head" % np.nonzero(ex.written != batch.num_kv_heads)[0][:8])
    return O, LSE
