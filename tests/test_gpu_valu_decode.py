"""GPU parity of the VALU narrow kernel (decode tiles without MFMA: the pages'
CUDA-core decode design, flashinfer issue #323) against the oracle: every row
capacity (2, 4, 8), both head dims and dtypes, causal multi-token rows, key ranges
ending mid-step and mid-page, the split path, NaN-poisoned unused slots."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_util import assert_close, run, say

pytestmark = pytest.mark.gpu


def ref(b, rows=None):
    say("oracle %s" % b.name)
    return oracle.run(**b.oracle_kwargs(), rows=rows)


@pytest.mark.parametrize("shape", [(8, 1, 128, "f16"), (8, 2, 128, "bf16"), (4, 4, 64, "bf16"), (2, 1, 64, "f16"),
                                   (16, 8, 128, "bf16"), (4, 1, 128, "f16")],
                         ids=lambda s: "h%d_kv%d_d%d_%s" % s)
def test_valu_narrow_tiles(shape):
    H, Hk, D, dt = shape
    G = H // Hk
    tq = max(1, 8 // G)
    q_lens = [1, tq, 1, tq, 1]
    kv_lens = [1, 77, 1000, 2049, 5000]
    b = W.make_batch("valu", q_lens, kv_lens, num_qo_heads=H, num_kv_heads=Hk, head_dim=D, dtype=dt, seed=41,
                     spare_pages=3, poison=True)
    ro, rl = ref(b)
    for splits, cus in ((1, 0), (0, 0), (0, 4096)):
        o, l, info = run(b, max_kv_splits=splits, num_cus=cus, narrow_kernel="valu")
        assert_close(o, l, ro, rl, what="valu %s splits=%d cus=%d" % (shape, splits, cus))


def test_valu_decode_b128_kv1024():
    b = W.decode_b128_kv1024()
    ro, rl = ref(b)
    o, l, info = run(b, narrow_kernel="valu")
    assert info["num_split_groups"] == 0  # 128 equal rows: balanced, not split
    assert_close(o, l, ro, rl, what="valu decode_b128_kv1024")
    o, l, info = run(b, narrow_kernel="valu", num_cus=1024)
    assert info["num_split_groups"] == 128
    assert_close(o, l, ro, rl, what="valu decode_b128_kv1024 split")


def test_valu_mixed_batch_decode_rows():
    b = W.mixed_long_batch(part="decode", device="cuda")
    import torch
    rows = list(range(0, b.total_q, 5))
    o, l, _ = run(b, dev=(b.q, b.kv_cache, torch.from_numpy(b.kv_page_indices).cuda()), narrow_kernel="valu")
    ro, rl = ref(b, rows=rows)
    assert_close(o, l, ro, rl, rows=rows, what="valu mixed decode rows (sampled)")
