"""GPU parity of hqq_quantize_ex: every stop rule against the oracle run with the same rule, a
chosen tiny-range threshold, and the debug flags that switch off the solver's exact shortcuts
(fixed-point skip, zero fast path of the shrink), whose results must not change by one bit.

Inputs: seeded N(0, 0.02) weights with 0.1 % outliers at +/-10 sigma (fp16), a tensor that
reaches a fixed point and stops early (the oracle pin's N(0, 0.02) 8 x 64 tensor at 30 rounds),
2-bit groups of 16 (the early-stopping configuration of the Laplace layer set) and sigma = 1
weights at 2 bits (shrink active).  Comparisons as in the quantizer parity tests.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import compare_quant, gpu_quantize, say

pytestmark = pytest.mark.gpu


def _stopping_tensor():
    return np.random.default_rng(23).normal(0, 0.02, (8, 64)).astype(np.float16)


@pytest.mark.parametrize("rule", [0, 1, 2, 4, 5, 6])
def test_stop_rules_on_a_stopping_tensor(rule):
    W = _stopping_tensor()
    ref = oracle.get().quantize(W.astype(np.float64), nbits=4, group_size=64, axis=1, iters=30, stop_rule=rule)
    assert ref["rounds"] < 30  # the loop stops: the rule decides the kept zero
    say("stop rule", rule, "k_out", ref["kout"])
    gq = gpu_quantize(W, 4, 64, 1, 30, meta="f64", stop_rule=rule)
    compare_quant(W, ref, gq, 4, 64, 1)


EX_CASES = [(2, 16, 1, 37, 192), (2, 64, 1, 21, 128), (4, 64, 1, 64, 256), (2, 16, 0, 64, 72), (3, 128, 0, 256, 104)]


@pytest.mark.parametrize("rule", [1, 2, 4, 6])
@pytest.mark.parametrize("nbits,g,axis,rows,cols", EX_CASES, ids=lambda v: str(v))
def test_stop_rules(rule, nbits, g, axis, rows, cols):
    W = synth.weight_normal(rows, cols, 0.02, 3000 + rows + cols + nbits, 0.001, 10.0)
    ref = oracle.get().quantize(W.astype(np.float64), nbits=nbits, group_size=g, axis=axis, iters=20,
                                stop_rule=rule)
    gq = gpu_quantize(W, nbits, g, axis, 20, meta="f64", stop_rule=rule)
    compare_quant(W, ref, gq, nbits, g, axis)


def test_tiny_range():
    """Groups whose range lies between the default threshold and the chosen one start with s = 1."""
    r = np.random.default_rng(5)
    W = r.normal(0, 0.02, (16, 128)).astype(np.float16)
    W[3, :64] = np.float16(0.25)
    W[3, 7] = np.float16(0.25 + 2 ** -9)   # range 2^-9 ~ 2e-3
    W[9, 64:] = np.float16(-0.125)
    W[9, 70] = np.float16(-0.125 + 2 ** -11)  # range 2^-11 ~ 4.9e-4
    for tiny in (1e-4, 1e-3, 5e-3):
        ref = oracle.get().quantize(W.astype(np.float64), nbits=4, group_size=64, axis=1, iters=20, tiny=tiny)
        gq = gpu_quantize(W, 4, 64, 1, 20, meta="f64", tiny_range=tiny)
        compare_quant(W, ref, gq, 4, 64, 1)
    assert ref["s"][3 * 2] == 1.0 and ref["s"][9 * 2 + 1] == 1.0  # both groups take s = 1 at tiny = 5e-3


def _same(a, b):
    for k in ("packed", "delta", "zero", "stop"):
        assert np.array_equal(a[k], b[k]), k
    assert np.array_equal(np.nan_to_num(a["mae"], nan=-1.0), np.nan_to_num(b["mae"], nan=-1.0)), "mae"


@pytest.mark.parametrize("flags", [1, 2, 3, 4])
@pytest.mark.parametrize("nbits,g,axis,rows,cols", EX_CASES[:3] + [(4, 128, 0, 256, 200)], ids=lambda v: str(v))
def test_debug_flags_change_nothing(flags, nbits, g, axis, rows, cols):
    W = synth.weight_normal(rows, cols, 0.02, 3100 + rows + cols + nbits, 0.001, 10.0)
    _same(gpu_quantize(W, nbits, g, axis, 20, meta="f64"), gpu_quantize(W, nbits, g, axis, 20, meta="f64",
                                                                         debug_flags=flags))


@pytest.mark.parametrize("flags", [1, 2, 3])
def test_debug_flags_with_the_shrink_active(flags):
    W = synth.weight_normal(48, 256, 1.0, seed=9)
    _same(gpu_quantize(W, 2, 64, 1, 20, meta="f64"), gpu_quantize(W, 2, 64, 1, 20, meta="f64", debug_flags=flags))


def test_fixed_point_tensor_without_the_skip():
    """The stopping tensor reaches a fixed point (frozen groups): without the skip every round
    is computed, with the same result."""
    W = _stopping_tensor()
    _same(gpu_quantize(W, 4, 64, 1, 30, meta="f64"), gpu_quantize(W, 4, 64, 1, 30, meta="f64", debug_flags=1))
