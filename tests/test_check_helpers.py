"""The comparison helpers the GPU parity tests use, exercised on the CPU
with values whose distance from the fp64 oracle is known: what they must
accept and what they must reject."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import oracle  # noqa: E402
from gpu_util import check_log  # noqa: E402
from row_wise_online_amd import workloads as wl  # noqa: E402


def _fp32_log_softmax(xf):
    """(x - m) - log d evaluated in fp32, the stable form of the row LSE."""
    m = xf.max(1, keepdims=True)
    d = np.exp(xf - m).sum(1, keepdims=True, dtype=np.float32)
    return (xf - m) - np.log(d).astype(np.float32)


def _expect_fail(fn):
    try:
        fn()
    except AssertionError:
        return
    raise AssertionError("the helper accepted a planted error")


def test_log_bf16_dominant_element():
    # One element 20 above seven others: the others sum to 7 e^-20 < 2^-24
    # of the max term, so d rounds to 1 in fp32 and log p of the max element
    # comes out 0 where the exact value is -1.45e-8, thousands of bf16 steps
    # away but within fp32's absolute error.  The helper accepts it.
    x = wl.f32_to_bf16_bits(np.array([[0.0] + [-20.0] * 7], np.float32))
    ref = oracle.log_softmax(x)
    y = _fp32_log_softmax(oracle.bf16_bits_to_f64(x).astype(np.float32))
    got = oracle.round_f64_to_bf16_bits(y.astype(np.float64))
    assert got[0, 0] == 0 and -1.5e-8 < ref[0, 0] < -1.4e-8
    assert oracle.bf16_ulp_distance(got[0, 0], oracle.round_f64_to_bf16_bits(ref[0, 0])) > 1000
    check_log(got, ref, "dominant")


def test_log_bf16_fp32_evaluation_of_a_wide_row():
    # scale 30 rows: many log-probabilities within fp32 rounding of 0
    x = wl.normal(16, 3000, scale=30.0, offset=50.0, seed=77, dtype="bf16")
    ref = oracle.log_softmax(x)
    y = _fp32_log_softmax(oracle.bf16_bits_to_f64(x).astype(np.float32))
    check_log(oracle.round_f64_to_bf16_bits(y.astype(np.float64)), ref, "wide")


def test_log_bf16_planted_errors_fail():
    x = wl.normal(4, 500, scale=2.0, seed=5, dtype="bf16")
    ref = oracle.log_softmax(x)
    good = oracle.round_f64_to_bf16_bits(ref)
    check_log(good, ref, "exact")
    # two steps away at |ref| ~ 1 and beyond
    i = int(np.argmin(np.abs(ref + 1.0)))
    bad = good.copy()
    bad.flat[i] += 2
    _expect_fail(lambda: check_log(bad, ref, "two steps"))
    # near 0 the allowance is absolute and small: 1e-4 off fails
    near = np.array([[-3e-6, -5.0]])
    off = oracle.round_f64_to_bf16_bits(near + np.array([[-1e-4, 0.0]]))
    _expect_fail(lambda: check_log(off, near, "near zero"))
    # an infinity out of place fails
    inf = good.copy()
    inf.flat[0] = 0xFF80
    _expect_fail(lambda: check_log(inf, ref, "infinity"))
