"""Plant plausible mistakes in a copy of the oracle and check the pins catch each.

Every mutation edits one line of a temporary copy of oracle/rpa_oracle.c
(the oracle itself is never modified), builds it with gcc, swaps it in for
the real library and runs the pin tests of test_oracle.py against it.  At
least one pin must fail for every mutation, otherwise the pins would not
protect the oracle against that class of mistake.
"""
import inspect
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import tests.test_oracle as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(os.path.dirname(oracle.__file__), "rpa_oracle.c")

MUTATIONS = {
    # causal alignment: queries at the first q_len positions instead of the last
    "top_left_causal": ("const int32_t pos = kv_len - q_len + i;", "const int32_t pos = i;"),
    # causal off by one: the diagonal key is hidden
    "causal_excludes_diagonal": ("J->causal ? pos + 1 : kv_len", "J->causal ? pos : kv_len"),
    # GQA: interleaved instead of contiguous head groups
    "gqa_modulo": ("const int32_t hk = h / group;", "const int32_t hk = h % J->num_kv_heads;"),
    # scores read V instead of K
    "scores_from_v": ("decode(qrow[d], J->dtype) * kv_elem(J, b, j, 0, hk, d)",
                      "decode(qrow[d], J->dtype) * kv_elem(J, b, j, 1, hk, d)"),
    # wrong slot within a page
    "slot_shift": ("int64_t slot = t % J->page_size;", "int64_t slot = (t + 1) % J->page_size;"),
    # K/V axis folded into the page stride
    "page_stride": ("(((page * 2 + kv) * J->page_size", "(((page + kv) * J->page_size"),
    # sequence length ignores kv_last_page_len
    "full_last_page": ("(np - 1) * J->page_size + J->kv_last_page_len[b];", "np * J->page_size;"),
    # Q head stride transposed
    "q_head_major": ("J->q + (r * J->num_qo_heads + h) * (int64_t)D", "J->q + (h * J->total_q + r) * (int64_t)D"),
    # softmax scale dropped
    "no_scale": ("s[j] = J->sm_scale * dot;", "s[j] = dot;"),
    # normalisation dropped
    "no_normalise": ("orow[d] /= l;", "orow[d] /= 1.0;"),
    # log-sum-exp in base 2
    "lse_log2": ("m + log(l)", "m + log2(l)"),
    # log-sum-exp without the max
    "lse_no_max": ("= m + log(l);", "= log(l);"),
    # bfloat16 exponent bias off by one
    "bf16_bias": ("v = ldexp((double)(f + 128), e - 134);", "v = ldexp((double)(f + 128), e - 133);"),
    # binary16 subnormals scaled wrongly
    "f16_subnormal": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    # sign bit ignored for binary16
    "f16_sign": ("return sign ? -v : v;\n}\n\n/* bfloat16", "return v;\n}\n\n/* bfloat16"),
    # non-causal sequences with more queries than keys rejected like causal ones
    "noncausal_q_gt_kv_rejected": ("if (causal ? q_len > kv_len : (q_len > 0 && kv_len == 0))",
                                   "if (q_len > kv_len)"),
}


def _pin_tests():
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        cases = [None]
        for m in getattr(fn, "pytestmark", []):
            if m.name == "parametrize":
                cases = list(m.args[1])
        for c in cases:
            out.append((name, fn, c))
    return out


def run_pins_against(lib_path):
    """Run every pin of test_oracle.py with the oracle library at `lib_path`;
    return the names of the pins that failed."""
    oracle._lib = oracle.load_library(lib_path)
    failed = []
    for name, fn, case in _pin_tests():
        try:
            fn(case) if case is not None else fn()
        except (AssertionError, ValueError, IndexError, RuntimeError, pytest.fail.Exception):
            failed.append(name)
    return failed


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_every_planted_mistake_fails_a_pin(mutation, tmp_path):
    old, new = MUTATIONS[mutation]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor must match exactly once: %r" % old
    mutated_src = tmp_path / "mutant.c"
    mutated_src.write_text(src.replace(old, new))
    so = oracle.build(force=True, src=str(mutated_src), out=str(tmp_path / "mutant.so"))
    # A mutant may also crash (e.g. write past a buffer sized for the true
    # lengths): run it in a child process; a crash counts as caught.
    code = ("import sys; sys.path.insert(0, %r); import tests.test_oracle_mutations as m; "
            "f = m.run_pins_against(%r); print('FAILED_PINS', len(f), ' '.join(sorted(set(f))))"
            % (ROOT, so))
    p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    if p.returncode != 0:
        return  # crashed: caught
    line = [l for l in p.stdout.splitlines() if l.startswith("FAILED_PINS")][-1]
    assert int(line.split()[1]) > 0, "no pin caught the planted mistake %r" % mutation


# Planted mistakes in oracle.merge_states (numpy): the cascade pin must catch each.
def _merge_unweighted(o_a, lse_a, o_b, lse_b):
    o, lse = _true_merge(o_a, lse_a, o_b, lse_b)
    return (np.asarray(o_a, np.float64) + np.asarray(o_b, np.float64)) / 2, lse


def _merge_swapped(o_a, lse_a, o_b, lse_b):
    return _true_merge(o_b, lse_a, o_a, lse_b)


def _merge_lse_is_max(o_a, lse_a, o_b, lse_b):
    o, _ = _true_merge(o_a, lse_a, o_b, lse_b)
    return o, np.maximum(lse_a, lse_b)


def _merge_log2(o_a, lse_a, o_b, lse_b):
    m = np.maximum(lse_a, lse_b)
    wa, wb = np.exp2(lse_a - m), np.exp2(lse_b - m)
    return (wa[..., None] * o_a + wb[..., None] * o_b) / (wa + wb)[..., None], m + np.log2(wa + wb)


_true_merge = oracle.merge_states
MERGE_MUTANTS = {"unweighted": _merge_unweighted, "swapped_outputs": _merge_swapped,
                 "lse_is_max": _merge_lse_is_max, "base2_weights": _merge_log2}


@pytest.mark.parametrize("mutant", sorted(MERGE_MUTANTS))
def test_every_planted_merge_mistake_fails_the_cascade_pin(mutant, monkeypatch):
    monkeypatch.setattr(oracle, "merge_states", MERGE_MUTANTS[mutant])
    with pytest.raises(AssertionError):
        pins.test_cascade_halves_merge_to_the_whole()
