"""The seeded input recipe: every workload is reproducible byte for byte and
has the structure its description states (scale, offsets, ascending trend,
planted maxima, bf16 rounding, attention layouts).  CPU only."""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from row_wise_online_amd import workloads as wl  # noqa: E402


def _f64(name, x):
    if wl.WORKLOADS[name].dtype == "f32":
        return x.astype(np.float64)
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_reproducible_bytes(name):
    a, b = wl.generate(name), wl.generate(name)
    assert a.dtype == b.dtype and a.shape == b.shape
    assert a.tobytes() == b.tobytes()
    w = wl.WORKLOADS[name]
    assert a.shape == (w.M, w.N)
    assert a.dtype == (np.float32 if w.dtype == "f32" else np.uint16)


def test_c1_offsets_and_scale():
    x = _f64("c1", wl.generate("c1"))
    assert abs(x[0].mean() - 80.0) < 0.5 and abs(x[1].mean() + 80.0) < 0.5
    rest = x[2:]
    assert abs(rest.mean()) < 0.05
    assert abs(rest.std() - 3.0) < 0.05


def test_c2_standard_normal():
    x = _f64("c2", wl.generate("c2"))
    assert abs(x.mean()) < 2e-3 and abs(x.std() - 1.0) < 2e-3
    # fp32 values are the fp64 normals rounded once
    z = np.random.default_rng(wl.WORKLOADS["c2"].seed).standard_normal((4, 4096))
    assert np.array_equal(wl.generate("c2")[:4], z.astype(np.float32))


def test_c3_bf16_is_rne_of_fp32():
    x = wl.generate("c3")
    z = 2.0 * np.random.default_rng(wl.WORKLOADS["c3"].seed).standard_normal((8, 1024))
    f = z.astype(np.float32).view(np.uint32).astype(np.uint64)
    # round to nearest even on the top 16 bits
    r = ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(x[:8], r)
    xv = _f64("c3", x)
    assert abs(xv.std() - 2.0) < 5e-3


def test_c4_ascending_trend():
    x = _f64("c4", wl.generate("c4"))
    j = np.arange(x.shape[1])
    col_mean = x.mean(axis=0)
    slope = np.polyfit(j, col_mean, 1)[0]
    assert abs(slope - 0.01) < 1e-5
    resid = x - 0.01 * j[None, :]
    assert abs(resid.std() - 0.1) < 2e-3
    # a sequential scan finds a new running max at about 1 element in 6;
    # a lane that reads every 64th element finds one at nearly every element
    rises = np.mean(np.diff(np.maximum.accumulate(x[:8], axis=1), axis=1) > 0)
    assert 0.12 < rises < 0.22
    lane = x[:8].reshape(8, -1, 64).transpose(0, 2, 1)      # [row, lane, t]
    lane_rises = np.mean(np.diff(np.maximum.accumulate(lane, axis=2), axis=2) > 0)
    assert lane_rises > 0.99


def test_c5_planted_maxima():
    x = wl.generate("c5")
    cols = wl.planted_columns()
    w = wl.WORKLOADS["c5"]
    assert cols.shape == (w.M,) and np.all((cols >= 0) & (cols < w.N))
    assert np.all(x[np.arange(w.M), cols] == np.float32(20.0))
    assert np.array_equal(np.argmax(x, axis=1), cols)
    # the columns are drawn after the normals, from the same generator
    rng = np.random.default_rng(w.seed)
    rng.standard_normal((w.M, w.N))
    assert np.array_equal(rng.integers(0, w.N, size=w.M), cols)


def test_generic_inputs_with_padding():
    x = wl.normal(5, 70, scale=2.0, offset=1.0, seed=3, ld=80)
    assert x.shape == (5, 70)
    assert x.strides[0] == 80 * 4
    base = np.lib.stride_tricks.as_strided(x, shape=(5, 80), strides=x.strides)
    assert np.all(np.isnan(base[:, 70:]))
    assert np.array_equal(x, wl.normal(5, 70, scale=2.0, offset=1.0, seed=3, ld=80))


@pytest.mark.parametrize("layout", ["bhsd", "bshd"])
def test_attention_inputs(layout):
    q, k, v = wl.attention_inputs(2, 3, 17, 19, 64, seed=5, q_scale=2.0, layout=layout)
    assert q.shape == (2, 3, 17, 64) and k.shape == (2, 3, 19, 64) and v.shape == k.shape
    q2, k2, v2 = wl.attention_inputs(2, 3, 17, 19, 64, seed=5, q_scale=2.0)
    # the same values whatever the layout; bshd is a [B, H, S, D] view of [B, S, H, D]
    assert np.array_equal(q, q2) and np.array_equal(k, k2) and np.array_equal(v, v2)
    if layout == "bshd":
        assert q.base is not None and q.strides[2] == 3 * 64 * 2
    qf = (q.astype(np.uint32) << 16).view(np.float32)
    kf = (k.astype(np.uint32) << 16).view(np.float32)
    assert 1.6 < qf.std() < 2.4 and 0.8 < kf.std() < 1.2
