"""GPU parity of the cascade path: a prefix shared by many requests attended once,
non-causally, for all of their queries, plus each request's private tokens, joined
by rpa_merge_states (vLLM issue #227, "Question about efficient memory sharing";
the merge is the split-KV merge of flashinfer issue #323 applied to whole
outputs).  References come from the oracle: the merge kernel against
oracle.merge_states, the cascade against the oracle's attention over the whole
(unsplit) sequences."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_ragged_amd as rpa
import workloads as W
from tests.gpu_util import assert_close, say

pytestmark = pytest.mark.gpu


def ref(b, rows=None):
    say("oracle %s rows=%s" % (b.name, "all" if rows is None else len(rows)))
    return oracle.run(**b.oracle_kwargs(), rows=rows)


def plan_for(b):
    p = rpa.Plan(b.qo_indptr, b.kv_page_indptr, b.kv_last_page_len, num_qo_heads=b.num_qo_heads,
                 num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, dtype=b.dtype, causal=b.causal)
    p.bind(torch.from_numpy(b.kv_page_indices).cuda(), num_pages=b.kv_cache.shape[0])
    return p


def run_cascade(shared, private, q, kv):
    """O, LSE of the cascade: shared-prefix state, private state, merged in place."""
    say("cascade %s (shared T=%d kv=%d) + %s" % (shared.name, shared.total_q, int(shared.kv_lens[0]), private.name))
    pa, pb = plan_for(shared), plan_for(private)
    oa, la = pa.run(q, kv, return_lse=True)
    ob, lb = pb.run(q, kv, return_lse=True)
    o, lse = rpa.merge_states(oa, la, ob, lb, out=oa, lse_out=la)
    torch.cuda.synchronize()
    pa.check()
    pb.check()
    pa.close()
    pb.close()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_merge_states_matches_oracle(dtype, head_dim):
    say("merge_states %s D=%d" % (dtype, head_dim))
    g = torch.Generator("cpu").manual_seed(77)
    rows, H = 1000, 12
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    oa = torch.randn(rows, H, head_dim, generator=g).to(tdt)
    ob = torch.randn(rows, H, head_dim, generator=g).to(tdt)
    la = (torch.randn(rows, H, generator=g) * 4).float()
    lb = (torch.randn(rows, H, generator=g) * 4).float()
    la[::7, 0] = -float("inf")          # no visible key in A: B alone
    lb[::11, 1] = -float("inf")         # no visible key in B: A alone
    la[::13, 2] = lb[::13, 2] = -float("inf")  # neither: O = 0, LSE = -inf
    ob[::11, 1] = float("nan")          # a weight-0 state's O is never read
    lb[5, 3] = la[5, 3] + 60.0          # weights of very different size
    ro, rl = oracle.merge_states(oa.double().numpy(), la.double().numpy(), ob.double().numpy(), lb.double().numpy())
    dev = [t.cuda() for t in (oa, la, ob, lb)]
    o, lse = rpa.merge_states(*dev)
    torch.cuda.synchronize()
    o64, l64 = o.double().cpu().numpy(), lse.double().cpu().numpy()
    fin = np.isfinite(rl)
    assert np.array_equal(np.isneginf(l64), ~fin) and (o64[~fin] == 0).all()
    assert_close(o64[fin], l64[fin], ro[fin], rl[fin], what="merge_states %s D%d" % (dtype, head_dim))
    # in place (into A) gives the same bits
    oa_d, la_d = dev[0].clone(), dev[1].clone()
    rpa.merge_states(oa_d, la_d, dev[2], dev[3], out=oa_d, lse_out=la_d)
    torch.cuda.synchronize()
    assert torch.equal(oa_d.cpu().view(torch.int16), o.cpu().view(torch.int16))
    assert torch.equal(la_d.cpu(), lse.cpu())


def test_cascade_suffix_prefill_matches_oracle():
    """256 requests x (200 shared + 30 own tokens): the shared prefix is attended
    once for all 7680 suffix queries, the own tokens causally per request."""
    b = W.shared_prefix_suffix()
    shared, private = W.cascade_view(b, prefix=200)
    q, kv = b.q.cuda(), shared.kv_cache.cuda()
    o, lse = run_cascade(shared, private, q, kv)
    rows = list(range(0, b.total_q, 3)) + list(range(b.total_q - 64, b.total_q))
    rows = sorted(set(rows))
    ro, rl = ref(b, rows=rows)
    assert_close(o, lse, ro, rl, rows=rows, what="cascade suffix prefill")


def test_cascade_decode_steps_match_oracle():
    """Decode after the suffix prefill: each request appends one token per step
    (private pages); the cascade splits every step into the shared prefix and the
    request's own 30 + step tokens."""
    base = W.shared_prefix_suffix()
    for step in range(1, 51):
        d = W.decode_step(base, step)
        if step not in (1, 2, 17, 50):
            continue
        shared, private = W.cascade_view(d, prefix=200)
        assert (private.kv_lens == 30 + step).all()
        o, lse = run_cascade(shared, private, d.q.cuda(), shared.kv_cache.cuda())
        ro, rl = ref(d)
        assert_close(o, lse, ro, rl, what="cascade decode step %d" % step)
