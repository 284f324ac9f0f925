"""Seeded synthetic inputs for ragged attention over a paged KV cache.

This module only builds inputs: lengths, page tables, and N(0,1) Q / K / V
tensors in fp16 or bf16.  It holds none of the attention arithmetic and
imports neither the GPU library nor the oracle; both of those consume what
it produces.

Recipe (shared by every workload):
  * one ``torch.Generator('cpu')`` per workload, seeded from the workload;
  * draw order: lengths -> physical page placement -> Q -> K/V -> padding /
    poison values;
  * values are drawn as fp32 N(0,1) and rounded to nearest-even to the
    storage dtype;
  * a sequence of kv_len tokens owns ceil(kv_len / page_size) pages, all full
    except the last, which holds (kv_len - 1) % page_size + 1 tokens
    (flashinfer issue #323 requires 1 <= kv_last_page_len <= page_size);
  * the cache is [num_pages, 2, page_size, num_kv_heads, head_dim] ("NHD"
    pages, index 0 of the size-2 axis is K and 1 is V), as in the same issue's
    repro; Q is [total_q, num_qo_heads, head_dim], packed by qo_indptr.
  * with ``poison=True`` every slot that no sequence owns (the tail of a last
    page, spare pages) holds NaN, so a reader that touches it shows up.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np
import torch

PAGE_SIZE = 16
_DT = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass
class Batch:
    """One ragged batch: host int32 page table + CPU fp16/bf16 tensors."""
    name: str
    qo_indptr: np.ndarray          # int32 [B+1]
    kv_page_indptr: np.ndarray     # int32 [B+1]
    kv_page_indices: np.ndarray    # int32 [nnz_pages]
    kv_last_page_len: np.ndarray   # int32 [B]
    q: torch.Tensor                # [total_q, H_qo, D]
    kv_cache: torch.Tensor         # [num_pages, 2, page_size, H_kv, D]
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                     # 'f16' | 'bf16'
    causal: bool = True
    page_size: int = PAGE_SIZE

    @property
    def batch(self) -> int:
        return len(self.qo_indptr) - 1

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.qo_indptr).astype(np.int64)

    @property
    def kv_lens(self) -> np.ndarray:
        np_ = np.diff(self.kv_page_indptr).astype(np.int64)
        last = self.kv_last_page_len.astype(np.int64)
        return np.where(np_ == 0, 0, (np_ - 1) * self.page_size + last)

    @property
    def total_q(self) -> int:
        return int(self.qo_indptr[-1])

    @property
    def num_pages(self) -> int:
        return int(self.kv_cache.shape[0])

    def oracle_kwargs(self):
        return dict(qo_indptr=self.qo_indptr, kv_page_indptr=self.kv_page_indptr,
                    kv_page_indices=self.kv_page_indices, kv_last_page_len=self.kv_last_page_len,
                    q=self.q, kv_cache=self.kv_cache, num_qo_heads=self.num_qo_heads,
                    num_kv_heads=self.num_kv_heads, head_dim=self.head_dim,
                    page_size=self.page_size, dtype=self.dtype, causal=self.causal)


def pages_for(kv_len: int, page_size: int = PAGE_SIZE) -> int:
    return -(-int(kv_len) // page_size)


def last_page_len_for(kv_len: int, page_size: int = PAGE_SIZE) -> int:
    return 0 if kv_len == 0 else (int(kv_len) - 1) % page_size + 1


def _randn(gen: torch.Generator, shape, dtype: str, chunk_rows: int = 4096) -> torch.Tensor:
    """N(0,1) fp32 draws rounded to `dtype`, on the generator's device, generated
    in leading-axis chunks of `chunk_rows` so that very large pools never need a
    whole fp32 copy in memory."""
    out = torch.empty(shape, dtype=_DT[dtype], device=gen.device)
    n0 = shape[0] if len(shape) else 1
    for s in range(0, n0, chunk_rows):
        e = min(n0, s + chunk_rows)
        out[s:e] = torch.randn((e - s,) + tuple(shape[1:]), generator=gen, dtype=torch.float32,
                               device=gen.device).to(_DT[dtype])
    return out


def value_generator(gen: torch.Generator, device=None) -> torch.Generator:
    """Generator for Q / K / V values.  On the CPU it is `gen` itself; on another
    device it is that device's generator, seeded by the next draw of `gen` (so
    the draw order stays lengths -> placement -> values).  CPU and GPU generators
    give different values for the same seed; a run on a device reads its values
    back from that device."""
    if device is None or torch.device(device).type == "cpu":
        return gen
    seed = int(torch.randint(0, 2 ** 62, (1,), generator=gen))
    return torch.Generator(torch.device(device)).manual_seed(seed)


def make_batch(name: str, q_lens: Sequence[int], kv_lens: Sequence[int], *, num_qo_heads: int,
               num_kv_heads: int, head_dim: int, dtype: str, seed: int = 0,
               gen: Optional[torch.Generator] = None, permute: bool = True, spare_pages: int = 0,
               poison: bool = False, causal: bool = True, page_size: int = PAGE_SIZE,
               device=None) -> Batch:
    """Ragged batch with private pages per sequence, placed at random physical
    pages of a pool of (owned + spare_pages) pages when `permute`, else in order.
    Q / K / V are drawn on `device` (CPU when None)."""
    q_lens = [int(x) for x in q_lens]
    kv_lens = [int(x) for x in kv_lens]
    assert len(q_lens) == len(kv_lens)
    if gen is None:
        gen = torch.Generator("cpu").manual_seed(seed)
    B = len(q_lens)
    n_pages = [pages_for(k, page_size) for k in kv_lens]
    nnz = int(sum(n_pages))
    pool = nnz + int(spare_pages)
    if permute and pool > 0:
        phys = torch.randperm(pool, generator=gen)[:nnz].numpy().astype(np.int32)
    else:
        phys = np.arange(nnz, dtype=np.int32)
    qo_indptr = np.zeros(B + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(q_lens)
    kv_page_indptr = np.zeros(B + 1, dtype=np.int32)
    kv_page_indptr[1:] = np.cumsum(n_pages)
    last = np.array([last_page_len_for(k, page_size) for k in kv_lens], dtype=np.int32)
    T = int(qo_indptr[-1])
    vgen = value_generator(gen, device)
    q = _randn(vgen, (T, num_qo_heads, head_dim), dtype)
    kv = _randn(vgen, (pool, 2, page_size, num_kv_heads, head_dim), dtype)
    if poison:
        _poison_unowned(kv, phys, kv_page_indptr, last)
    return Batch(name, qo_indptr, kv_page_indptr, phys, last, q, kv, num_qo_heads, num_kv_heads,
                 head_dim, dtype, causal, page_size)


def _poison_unowned(kv: torch.Tensor, phys: np.ndarray, kv_page_indptr: np.ndarray, last: np.ndarray):
    """NaN into every slot no sequence owns (slots past kv_last_page_len of a
    last page, and pages referenced by no sequence)."""
    page_size = kv.shape[2]
    owned = np.zeros((kv.shape[0], page_size), dtype=bool)
    for b in range(len(last)):
        pages = phys[kv_page_indptr[b]:kv_page_indptr[b + 1]]
        if len(pages) == 0:
            continue
        owned[pages[:-1], :] = True
        owned[pages[-1], :last[b]] = True
    pg, sl = np.nonzero(~owned)
    if len(pg):
        kv[torch.from_numpy(pg).to(kv.device), :, torch.from_numpy(sl).to(kv.device)] = float("nan")


def poison_unowned(batch: Batch) -> Batch:
    _poison_unowned(batch.kv_cache, batch.kv_page_indices, batch.kv_page_indptr, batch.kv_last_page_len)
    return batch


# ----------------------------------------------------------------------------------------------
# The five workloads.  Seeds are 1000 + k for workload k.
# ----------------------------------------------------------------------------------------------

def tiny_ragged_prefill(poison: bool = False, spare_pages: int = 0) -> Batch:
    """4 sequences, q_len {17,3,5,1}, kv_len {17,30,5,48}, 8 qo / 1 kv heads, D 64,
    fp16, pages randomly permuted."""
    return make_batch("tiny_ragged_prefill", [17, 3, 5, 1], [17, 30, 5, 48], num_qo_heads=8,
                      num_kv_heads=1, head_dim=64, dtype="f16", seed=1001, poison=poison,
                      spare_pages=spare_pages)


def decode_b128_kv1024(batch: int = 128, kv_len: int = 1024, dtype: str = "f16", device=None) -> Batch:
    """batch 128 x q_len 1 x kv_len 1024, 8 qo / 1 kv heads, D 128, fp16; 64 pages
    per sequence laid out contiguously (kv_page_indices = arange)."""
    return make_batch("decode_b%d_kv%d" % (batch, kv_len), [1] * batch, [kv_len] * batch,
                      num_qo_heads=8, num_kv_heads=1, head_dim=128, dtype=dtype, seed=1002,
                      permute=False, device=device)


def short_prompt_lengths(n: int = 64, lo: int = 1, hi: int = 200, seed: int = 1003) -> List[int]:
    gen = torch.Generator("cpu").manual_seed(seed)
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=gen)]


def short_prompt_prefill(n: int = 64, max_len: int = 200, padded: bool = False,
                         poison: bool = False, num_qo_heads: int = 32, num_kv_heads: int = 8) -> Batch:
    """64 prompts, lengths uniform in [1, 200], q_len = kv_len, causal, 32 qo / 8 kv
    heads, D 128, bf16, random page placement.

    padded=True gives the padded twin: every sequence has q_len = kv_len = max_len;
    its first L tokens (Q, K, V) equal the un-padded batch's, the pad tokens are
    finite N(0,1) from a separate stream (seed 2003)."""
    gen = torch.Generator("cpu").manual_seed(1003)
    lens = [int(x) for x in torch.randint(1, max_len + 1, (n,), generator=gen)]
    base = make_batch("short_prompt_prefill", lens, lens, num_qo_heads=num_qo_heads,
                      num_kv_heads=num_kv_heads, head_dim=128, dtype="bf16", gen=gen,
                      poison=poison and not padded)
    if not padded:
        return base
    return pad_to(base, max_len, seed=2003)


def pad_to(base: Batch, length: int, seed: int) -> Batch:
    """Padded twin of a q_len == kv_len batch: real tokens first, unchanged; pad
    tokens after them, drawn from their own seeded stream; fresh page placement."""
    gen = torch.Generator("cpu").manual_seed(seed)
    B = base.batch
    padded = make_batch(base.name + "_padded%d" % length, [length] * B, [length] * B,
                        num_qo_heads=base.num_qo_heads, num_kv_heads=base.num_kv_heads,
                        head_dim=base.head_dim, dtype=base.dtype, gen=gen, causal=base.causal)
    ps = base.page_size
    for b in range(B):
        L = int(base.q_lens[b])
        assert L == int(base.kv_lens[b]) and L <= length
        padded.q[padded.qo_indptr[b]:padded.qo_indptr[b] + L] = base.q[base.qo_indptr[b]:base.qo_indptr[b] + L]
        for t in range(L):
            src = base.kv_page_indices[base.kv_page_indptr[b] + t // ps]
            dst = padded.kv_page_indices[padded.kv_page_indptr[b] + t // ps]
            padded.kv_cache[dst, :, t % ps] = base.kv_cache[src, :, t % ps]
    return padded


def shared_prefix_suffix(n_req: int = 256, prefix: int = 200, suffix: int = 30, decode_steps: int = 50,
                         duplicated: bool = False, num_qo_heads: int = 32, num_kv_heads: int = 8,
                         head_dim: int = 128, dtype: str = "bf16", seed: int = 1004) -> Batch:
    """Shared-prefix suffix prefill: every request's first `prefix` tokens are the
    same; each adds `suffix` private tokens (q_len = suffix, kv_len = prefix + suffix).

    Shared layout: the prefix's full pages (prefix // 16 = 12) are physically
    shared; the page holding the prefix's last partial page (tokens 192..199)
    is copied into a private page per request, whose remaining slots hold that
    request's first suffix tokens; further private pages follow.  The pool is
    sized so each request can append `decode_steps` more tokens in place.

    duplicated=True: the same token values, but every request owns private
    copies of all its pages (the reference layout for the sharing invariance).
    """
    ps = PAGE_SIZE
    gen = torch.Generator("cpu").manual_seed(seed)
    kv_len = prefix + suffix
    max_len = kv_len + decode_steps
    pages_req = pages_for(max_len)
    n_shared = prefix // ps if not duplicated else 0
    n_priv = pages_req - n_shared
    pool = n_shared + n_req * n_priv
    # token values come first, from `gen`, so both layouts hold the same values;
    # physical placement has a stream of its own (one per layout)
    pre_kv = _randn(gen, (prefix, 2, num_kv_heads, head_dim), dtype)
    q = _randn(gen, (n_req * suffix, num_qo_heads, head_dim), dtype)
    suf_kv = _randn(gen, (n_req, suffix, 2, num_kv_heads, head_dim), dtype)
    gen_place = torch.Generator("cpu").manual_seed(seed + (2000 if duplicated else 3000))
    phys = torch.randperm(pool, generator=gen_place).numpy().astype(np.int32)
    shared_pages = phys[:n_shared]
    priv = phys[n_shared:].reshape(n_req, n_priv)
    kv = torch.zeros((pool, 2, ps, num_kv_heads, head_dim), dtype=_DT[dtype])
    # slots beyond kv_len (room for decode) get finite N(0,1) from their own stream
    gen_fill = torch.Generator("cpu").manual_seed(seed + 1000)
    kv.copy_(_randn(gen_fill, kv.shape, dtype))
    n_used = pages_for(kv_len)
    indices = np.zeros((n_req, n_used), dtype=np.int32)
    for r in range(n_req):
        pages_r = np.concatenate([shared_pages, priv[r]])[:pages_req]
        indices[r] = pages_r[:n_used]
        for t in range(kv_len):
            if t < n_shared * ps and r > 0:
                continue  # shared page already written by request 0
            val = pre_kv[t] if t < prefix else suf_kv[r, t - prefix]
            kv[pages_r[t // ps], :, t % ps] = val
    b = Batch("shared_prefix_suffix" + ("_dup" if duplicated else ""),
              np.arange(0, n_req * suffix + 1, suffix, dtype=np.int32),
              np.arange(0, n_req * n_used + 1, n_used, dtype=np.int32),
              indices.reshape(-1).copy(), np.full(n_req, last_page_len_for(kv_len), dtype=np.int32),
              q, kv, num_qo_heads, num_kv_heads, head_dim, dtype, True, ps)
    b.extra = dict(priv=priv, shared=shared_pages, pages_req=pages_req, prefix=prefix, suffix=suffix)
    return b


def decode_step(base: Batch, step: int, seed: int = 5004) -> Batch:
    """Decode step `step` (1-based) after a shared_prefix_suffix prefill: every
    request appends one token at position kv_len0 + step - 1 (fresh seeded K/V
    written into its page slot of base.kv_cache, in place) and issues one query
    (fresh seeded Q).  Returns the q_len = 1 batch that reads kv_len0 + step tokens."""
    ex = base.extra
    ps = base.page_size
    n_req = base.batch
    kv_len0 = ex["prefix"] + ex["suffix"]
    pos = kv_len0 + step - 1
    gen = torch.Generator("cpu").manual_seed(seed + step)
    new_kv = _randn(gen, (n_req, 2, base.num_kv_heads, base.head_dim), base.dtype)
    q = _randn(gen, (n_req, base.num_qo_heads, base.head_dim), base.dtype)
    n_shared = len(ex["shared"])
    n_used = pages_for(pos + 1)
    indices = np.zeros((n_req, n_used), dtype=np.int32)
    for r in range(n_req):
        pages_r = np.concatenate([ex["shared"], ex["priv"][r]])
        assert pos // ps >= n_shared, "decode tokens go to private pages"
        base.kv_cache[pages_r[pos // ps], :, pos % ps] = new_kv[r]
        indices[r] = pages_r[:n_used]
    b = Batch(base.name + "_decode%d" % step, np.arange(n_req + 1, dtype=np.int32),
              np.arange(0, n_req * n_used + 1, n_used, dtype=np.int32), indices.reshape(-1).copy(),
              np.full(n_req, last_page_len_for(pos + 1), dtype=np.int32), q, base.kv_cache,
              base.num_qo_heads, base.num_kv_heads, base.head_dim, base.dtype, True, ps)
    return b


def cascade_view(b: Batch, prefix: int, poison: bool = True):
    """The same token values in the layout of a two-level cascade: one copy of the
    `prefix` tokens every sequence shares, in pages of their own (the last one
    partly filled), plus each sequence's remaining tokens in private pages (vLLM
    issue #227: many requests over one system prompt).  Returns (shared, private):
      shared  -- one non-causal sequence holding every query row of b (q_len =
                 b.total_q) over the prefix (kv_len = prefix);
      private -- b's sequences and queries over their own tokens past the prefix
                 (kv_len - prefix each), with b's causal flag.
    Both index one new pool; unused slots are NaN when `poison`.  Every query must
    sit at or after the prefix, so that it sees all of it.  Layout only: token
    values are copied, never combined."""
    ps = b.page_size
    kvl, ql = b.kv_lens, b.q_lens
    assert b.batch > 0 and (kvl >= prefix).all() and (kvl - ql >= prefix).all()

    def tokens(seq):  # [kv_len, 2, Hkv, D] through the page table
        L = int(kvl[seq])
        pg = b.kv_page_indices[b.kv_page_indptr[seq]:b.kv_page_indptr[seq + 1]]
        t = np.arange(L)
        idx = torch.from_numpy(pg[t // ps].astype(np.int64)).to(b.kv_cache.device)
        sl = torch.from_numpy((t % ps).astype(np.int64)).to(b.kv_cache.device)
        return b.kv_cache[idx, :, sl]

    pre = tokens(0)[:prefix]
    n_sh = pages_for(prefix)
    priv_len = [int(kvl[s]) - prefix for s in range(b.batch)]
    n_pr = [pages_for(L) for L in priv_len]
    pool = n_sh + sum(n_pr)
    kv = torch.empty((pool, 2, ps, b.num_kv_heads, b.head_dim), dtype=b.kv_cache.dtype, device=b.kv_cache.device)
    kv.fill_(float("nan") if poison else 0.0)

    def put(first_page, vals):  # vals [L, 2, Hkv, D] into consecutive pages from first_page
        L = vals.shape[0]
        t = np.arange(L)
        idx = torch.from_numpy(first_page + t // ps).to(kv.device)
        sl = torch.from_numpy(t % ps).to(kv.device)
        kv[idx, :, sl] = vals

    put(0, pre)
    priv_idx, nxt = [], n_sh
    for s in range(b.batch):
        full = tokens(s)
        assert torch.equal(full[:prefix].view(torch.int16), pre.view(torch.int16)), "prefix differs at %d" % s
        put(nxt, full[prefix:])
        priv_idx.append(np.arange(nxt, nxt + n_pr[s], dtype=np.int32))
        nxt += n_pr[s]
    shared = Batch(b.name + "_cascade_shared", np.array([0, b.total_q], np.int32),
                   np.array([0, n_sh], np.int32), np.arange(n_sh, dtype=np.int32),
                   np.array([last_page_len_for(prefix)], np.int32), b.q, kv,
                   b.num_qo_heads, b.num_kv_heads, b.head_dim, b.dtype, False, ps)
    private = Batch(b.name + "_cascade_private", b.qo_indptr.copy(),
                    np.concatenate([[0], np.cumsum(n_pr)]).astype(np.int32),
                    np.concatenate(priv_idx).astype(np.int32) if priv_idx else np.zeros(0, np.int32),
                    np.array([last_page_len_for(L) if L else 1 for L in priv_len], np.int32), b.q, kv,
                    b.num_qo_heads, b.num_kv_heads, b.head_dim, b.dtype, b.causal, ps)
    return shared, private


def mixed_long_lengths(n_prompts: int = 4, prompt_len: int = 8192, n_decode: int = 256,
                       lo: int = 512, hi: int = 8192, seed: int = 1005):
    gen = torch.Generator("cpu").manual_seed(seed)
    dec = [int(x) for x in torch.randint(lo, hi + 1, (n_decode,), generator=gen)]
    q_lens = [prompt_len] * n_prompts + [1] * n_decode
    kv_lens = [prompt_len] * n_prompts + dec
    return gen, q_lens, kv_lens


def mixed_long_batch(n_prompts: int = 4, prompt_len: int = 8192, n_decode: int = 256,
                     lo: int = 512, hi: int = 8192, part: str = "all", device=None) -> Batch:
    """4 causal prompts of 8192 tokens plus 256 decode rows (q_len 1, kv_len uniform
    in [512, 8192]) in one ragged batch; 64 qo / 8 kv heads, D 128, bf16, random
    page placement.  part='prompts' or 'decode' keeps only that part of the same
    draw (same lengths, same seed)."""
    gen, q_lens, kv_lens = mixed_long_lengths(n_prompts, prompt_len, n_decode, lo, hi)
    if part == "prompts":
        q_lens, kv_lens = q_lens[:n_prompts], kv_lens[:n_prompts]
    elif part == "decode":
        q_lens, kv_lens = q_lens[n_prompts:], kv_lens[n_prompts:]
    return make_batch("mixed_long_" + part, q_lens, kv_lens, num_qo_heads=64, num_kv_heads=8,
                      head_dim=128, dtype="bf16", gen=gen, device=device)


# ----------------------------------------------------------------------------------------------
# Transformations used by invariance tests (structure only, no arithmetic).
# ----------------------------------------------------------------------------------------------

def permute_pages(b: Batch, seed: int) -> Batch:
    """Same logical content, pages moved to new physical slots of the pool."""
    gen = torch.Generator("cpu").manual_seed(seed)
    perm = torch.randperm(b.num_pages, generator=gen)
    new_kv = torch.empty_like(b.kv_cache)
    new_kv[perm] = b.kv_cache
    new_idx = perm.numpy().astype(np.int32)[b.kv_page_indices]
    return dataclasses.replace(b, name=b.name + "_perm", kv_page_indices=new_idx, kv_cache=new_kv)


def reorder_sequences(b: Batch, order: Sequence[int]) -> Batch:
    """The same sequences listed in another order (rows of Q move with them)."""
    order = list(order)
    q_lens = b.q_lens[order]
    np_ = np.diff(b.kv_page_indptr)[order]
    qo = np.zeros(len(order) + 1, dtype=np.int32)
    qo[1:] = np.cumsum(q_lens)
    kp = np.zeros(len(order) + 1, dtype=np.int32)
    kp[1:] = np.cumsum(np_)
    idx = np.concatenate([b.kv_page_indices[b.kv_page_indptr[s]:b.kv_page_indptr[s + 1]] for s in order]
                         ).astype(np.int32) if len(order) else np.zeros(0, np.int32)
    q = torch.cat([b.q[b.qo_indptr[s]:b.qo_indptr[s + 1]] for s in order]) if len(order) else b.q[:0]
    return dataclasses.replace(b, name=b.name + "_reordered", qo_indptr=qo, kv_page_indptr=kp,
                               kv_page_indices=idx, kv_last_page_len=b.kv_last_page_len[order].copy(), q=q)


def row_permutation(b: Batch, order: Sequence[int]) -> np.ndarray:
    """Token rows of `b` in the order reorder_sequences(b, order) lists them."""
    return np.concatenate([np.arange(b.qo_indptr[s], b.qo_indptr[s + 1]) for s in order]).astype(np.int64)


def contiguous_kv(b: Batch, seq: int):
    """K and V of sequence `seq` as contiguous [kv_len, H_kv, D] tensors, read
    through the page table (a layout change, no arithmetic)."""
    ps = b.page_size
    L = int(b.kv_lens[seq])
    pages = b.kv_page_indices[b.kv_page_indptr[seq]:b.kv_page_indptr[seq + 1]]
    k = torch.stack([b.kv_cache[pages[t // ps], 0, t % ps] for t in range(L)]) if L else None
    v = torch.stack([b.kv_cache[pages[t // ps], 1, t % ps] for t in range(L)]) if L else None
    return k, v


REGISTRY = {
    "tiny_ragged_prefill": tiny_ragged_prefill,
    "decode_b128_kv1024": decode_b128_kv1024,
    "short_prompt_prefill": short_prompt_prefill,
    "shared_prefix_suffix": shared_prefix_suffix,
    "mixed_long_batch": mixed_long_batch,
}
