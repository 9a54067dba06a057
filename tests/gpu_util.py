"""Helpers shared by the GPU parity tests: moving the seeded numpy inputs to
the device and comparing device results with fp64 oracle values at the
accuracy the method promises.

Accuracy bar (fp32 arithmetic against the fp64 oracle):
  * y fp32:   |y - y_ref| <= 1e-6 + 1e-5 |y_ref|, every element;
  * y bf16:   at most 1 bf16 step from round_to_nearest_even(y_ref);
  * m:        bit-exact (the row max is an input element);
  * d:        relative error <= 1e-5;
  * lse:      |lse - lse_ref| <= 1e-5 + one fp32 ulp at lse_ref (an fp32
              result cannot be closer than half an ulp, which exceeds 1e-5
              beyond |lse| = 128); for |lse| < 64 this is within 1e-5 + 7.6e-6.
"""
import numpy as np
import torch

import oracle

Y_ABS = 1e-6
Y_REL = 1e-5
D_REL = 1e-5
LSE_ABS = 1e-5


def to_device(arr):
    """numpy fp32 / uint16(bf16 bits) matrix (possibly a strided view into a
    wider padded buffer) -> torch GPU tensor with the same row stride."""
    arr = np.asarray(arr)
    M, N = arr.shape
    ld = arr.strides[0] // arr.itemsize
    base = arr
    if ld != N:
        base = arr.base
        assert base is not None and base.shape == (M, ld), "need padded base"
    if base.dtype == np.float32:
        t = torch.from_numpy(np.ascontiguousarray(base))
    else:
        t = torch.from_numpy(np.ascontiguousarray(base).view(np.int16)).view(
            torch.bfloat16)
    t = t.cuda()
    return t[:, :N]


def to_host(t):
    """GPU tensor -> numpy fp32 or uint16 bf16 bits."""
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def empty_like_rows(x_dev, ld=None):
    M, N = x_dev.shape
    ld = ld or N
    return torch.empty((M, ld), dtype=x_dev.dtype, device=x_dev.device)[:, :N]


def check_y(y_host, y_ref, what=""):
    """Return (max_abs, max_rel / max_ulp) and assert the accuracy bar."""
    if y_host.dtype == np.uint16:
        want = oracle.round_f64_to_bf16_bits(y_ref)
        dist = oracle.bf16_ulp_distance(y_host, want)
        bad = np.argwhere(dist > 1)
        assert bad.size == 0, (
            f"{what}: {len(bad)} bf16 values more than 1 ulp off, first at "
            f"{tuple(bad[0])}: got {y_host[tuple(bad[0])]:#06x} want "
            f"{want[tuple(bad[0])]:#06x}")
        return float(np.max(np.abs(oracle.bf16_bits_to_f64(y_host) - y_ref))), \
            int(dist.max())
    y = y_host.astype(np.float64)
    err = np.abs(y - y_ref)
    ok = err <= Y_ABS + Y_REL * np.abs(y_ref)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(
            f"{what}: {int((~ok).sum())} fp32 values outside tolerance, first "
            f"at {i}: got {y[i]!r} want {y_ref[i]!r}")
    rel = err / np.maximum(np.abs(y_ref), 1e-30)
    return float(err.max()), float(rel[y_ref > 1e-30].max(initial=0.0))


def check_m(m_host, m_ref, what=""):
    assert np.array_equal(m_host.astype(np.float64), m_ref), \
        f"{what}: m not bit-exact"


def check_d(d_host, d_ref, what=""):
    rel = np.abs(d_host.astype(np.float64) - d_ref) / d_ref
    assert np.all(rel <= D_REL), f"{what}: d rel err {rel.max():.3e}"
    return float(rel.max())


def check_lse(l_host, l_ref, what=""):
    err = np.abs(l_host.astype(np.float64) - l_ref)
    tol = LSE_ABS + oracle.f32_ulp(l_ref)
    assert np.all(err <= tol), f"{what}: lse err {err.max():.3e}"
    return float(err.max())


def check_log(y_host, y_ref, what=""):
    """log-softmax / loss values: fp32 within 1e-5 + 2 ulp(y_ref) (the
    output's own rounding plus that of x - m), bf16 within one bf16 step of
    round_to_nearest_even(y_ref), near 0 included (the kernels take
    log d as log1p(d - 1) with d - 1 summed apart, so a log-probability
    near 0 keeps full relative precision); infinities and NaNs must sit
    where the oracle has them."""
    if y_host.dtype == np.uint16:
        yf = oracle.bf16_bits_to_f64(y_host)
    else:
        yf = y_host.astype(np.float64)
    special = ~np.isfinite(y_ref)
    assert np.array_equal(np.isnan(yf), np.isnan(y_ref)), f"{what}: NaN layout"
    inf = np.isinf(y_ref)
    assert np.array_equal(yf[inf], y_ref[inf]), f"{what}: infinities"
    fin = ~special
    if y_host.dtype == np.uint16:
        want = oracle.round_f64_to_bf16_bits(y_ref[fin])
        dist = oracle.bf16_ulp_distance(y_host[fin], want)
        bad = dist > 1
        if bad.any():
            i = int(np.argmax(dist))
            raise AssertionError(
                f"{what}: {int(bad.sum())} bf16 values more than 1 step off, "
                f"worst {int(dist[i])} steps: got {yf[fin][i]!r} want "
                f"{y_ref[fin][i]!r}")
        return float(dist.max(initial=0))
    err = np.abs(yf[fin] - y_ref[fin])
    tol = 1e-5 + 2 * oracle.f32_ulp(y_ref[fin])
    bad = err > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} values off, worst "
                           f"{err.max():.3e}")
    return float(err.max(initial=0))
