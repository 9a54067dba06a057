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
    """(x - m) - log d evaluated in fp32 with d summed whole, the form that
    loses the log-probabilities near 0 (d rounds to 1)."""
    m = xf.max(1, keepdims=True)
    d = np.exp(xf - m).sum(1, keepdims=True, dtype=np.float32)
    return (xf - m) - np.log(d).astype(np.float32)


def _fp32_log_softmax_r(xf):
    """(x - m) - log1p(r) in fp32 with r = d - 1 summed apart from the max
    term's 1 (each further element equal to the max adds 1): the form the
    kernels evaluate."""
    m = xf.max(1, keepdims=True)
    t = np.exp(xf - m).astype(np.float32)
    eq = xf == m
    r = np.where(eq, np.float32(0), t).sum(1, keepdims=True, dtype=np.float32)
    r = r + (eq.sum(1, keepdims=True) - 1).astype(np.float32)
    return (xf - m) - np.log1p(r).astype(np.float32)


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
    # away.  The helper rejects that; r = d - 1 summed apart keeps the value.
    x = wl.f32_to_bf16_bits(np.array([[0.0] + [-20.0] * 7], np.float32))
    ref = oracle.log_softmax(x)
    xf = oracle.bf16_bits_to_f64(x).astype(np.float32)
    got = oracle.round_f64_to_bf16_bits(_fp32_log_softmax(xf).astype(np.float64))
    assert got[0, 0] == 0 and -1.5e-8 < ref[0, 0] < -1.4e-8
    assert oracle.bf16_ulp_distance(got[0, 0], oracle.round_f64_to_bf16_bits(ref[0, 0])) > 1000
    _expect_fail(lambda: check_log(got, ref, "dominant, d form"))
    good = oracle.round_f64_to_bf16_bits(_fp32_log_softmax_r(xf).astype(np.float64))
    check_log(good, ref, "dominant, r form")


def test_log_bf16_fp32_evaluation_of_a_wide_row():
    # scale 30 rows: many log-probabilities near 0; the r form in fp32 is
    # within one bf16 step of every one
    x = wl.normal(16, 3000, scale=30.0, offset=50.0, seed=77, dtype="bf16")
    ref = oracle.log_softmax(x)
    y = _fp32_log_softmax_r(oracle.bf16_bits_to_f64(x).astype(np.float32))
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
    # near 0 the bar is still one bf16 step: 1e-4 off fails
    near = np.array([[-3e-6, -5.0]])
    off = oracle.round_f64_to_bf16_bits(near + np.array([[-1e-4, 0.0]]))
    _expect_fail(lambda: check_log(off, near, "near zero"))
    # an infinity out of place fails
    inf = good.copy()
    inf.flat[0] = 0xFF80
    _expect_fail(lambda: check_log(inf, ref, "infinity"))
