"""Pins for the fp64 attention oracle (CPU only).

The oracle's attention (the three-pass definition and the tiled online
recurrence) is checked against values printed on the pages (the two worked
attention examples of "从原始Softmax到在线Softmax"), against scipy's softmax
and logsumexp composed with a numpy product, and against closed forms:
constant value rows, a zero query, a single key, two keys (logistic
weights), a dominant key, the first row under a causal mask, key
permutations.  A dropped scale, a wrong stride, a missing rescale or
normalisation, an off-by-one mask or an LSE without its max each fails at
least one of these (the mutation test plants them).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from row_wise_online_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _golden():
    with open(os.path.join(GOLDEN, "p3_worked_examples.json")) as f:
        return json.load(f)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _widen(a):
    a = np.asarray(a)
    return oracle.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def _scipy_attention(q, k, v, scale, causal=-1):
    """softmax(scale q k^T) v and logsumexp through scipy and numpy."""
    q, k, v = _widen(q), _widen(k), _widen(v)
    s = scale * (q @ k.T)
    if causal >= 0:
        i = np.arange(s.shape[0])[:, None]
        j = np.arange(s.shape[1])[None, :]
        s = np.where(j <= i + causal, s, -np.inf)
    p = scipy.special.softmax(s, axis=1)
    return p @ v, scipy.special.logsumexp(s, axis=1)


# ---------------------------------------------------------------------------
# Values printed on the pages
# ---------------------------------------------------------------------------

def test_worked_attention_example():
    g = _golden()["attention_examples"][0]
    Q, K, V = _f32(g["Q"]), _f32(g["K"]), _f32(g["V"])
    scale = 1.0 / math.sqrt(2.0)
    o, lse = oracle.attention(Q, K, V)
    assert np.allclose(o, g["O"], atol=g["tol"], rtol=0)
    # LSE = row max + log(sum of exponentials), both printed on the page
    want = np.array(g["row_max"]) + np.log(g["row_sum_exp"])
    assert np.allclose(lse, want, atol=1e-4, rtol=0)
    # the probabilities: with V the identity (Q and K padded by a zero
    # column so that d stays 2 in the scale) the output rows are P
    pad = lambda a: _f32(np.hstack([a, np.zeros((3, 1))]))
    P, _ = oracle.attention(pad(Q), pad(K), _f32(np.eye(3)), scale=scale)
    assert np.allclose(P, g["P"], atol=1e-4, rtol=0)
    # the scores: attention over the single key j has LSE = s_ij
    S = np.empty((3, 3))
    for j in range(3):
        S[:, j] = oracle.attention(Q, K[j:j + 1], V[j:j + 1], scale=scale)[1]
    assert np.allclose(S, g["S"], atol=1e-4, rtol=0)
    assert np.allclose(np.exp(S - S.max(1, keepdims=True)).sum(1),
                       g["row_sum_exp"], atol=g["tol"], rtol=0)


def _online_example():
    g = _golden()["attention_online_examples"][0]
    s = np.array(g["scores"])
    q = _f32([[1.0, 0.0]])
    k = _f32(np.stack([s, np.zeros_like(s)], axis=1))
    return g, q, k, _f32(g["V"])


def test_worked_online_merge_example():
    g, q, k, v = _online_example()
    o, lse = oracle.attention(q, k, v, scale=1.0)
    assert np.allclose(o[0], g["o_standard"], atol=g["tol"], rtol=0)
    assert abs(lse[0] - (g["merged"]["m"] + math.log(g["merged"]["l"]))) < 1e-4
    o2, lse2 = oracle.attention(q, k, v, scale=1.0, online_block=g["block"])
    assert np.allclose(o2[0], g["o_online"], atol=g["tol_online"], rtol=0)
    assert np.allclose(o2, o, atol=1e-15, rtol=0) and abs(lse2[0] - lse[0]) < 1e-15
    # each block alone: its state (m, l) and its normalised output
    for name, sl in (("block1", slice(0, 2)), ("block2", slice(2, 4))):
        ob, lb = oracle.attention(q, k[sl], v[sl], scale=1.0)
        b = g[name]
        assert np.allclose(ob[0], b["o"], atol=g["tol"], rtol=0)
        assert abs(lb[0] - (b["m"] + math.log(b["l"]))) < 1e-4
    # the factor applied to the first block's state when the second raises
    # the max: e^(m1 - m2)
    assert abs(math.exp(g["block1"]["m"] - g["block2"]["m"])
               - g["merged"]["scale_old"]) < 1e-4


# ---------------------------------------------------------------------------
# Library routine: scipy softmax / logsumexp and a numpy product
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("Sq,Sk,D,causal,dtype,seed", [
    (5, 7, 4, -1, "f32", 1), (17, 33, 16, -1, "bf16", 2),
    (33, 17, 8, -1, "f32", 3), (20, 20, 8, 0, "bf16", 4),
    (12, 30, 8, 18, "f32", 5), (9, 40, 128, 3, "bf16", 6),
])
def test_matches_scipy(Sq, Sk, D, causal, dtype, seed):
    rng = np.random.default_rng(seed)
    mk = lambda S, sc: wl.from_values(sc * rng.standard_normal((S, D)), dtype)
    q, k, v = mk(Sq, 2.0), mk(Sk, 1.0), mk(Sk, 1.0)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attention(q, k, v, causal=causal)
    o_ref, lse_ref = _scipy_attention(q, k, v, scale, causal)
    assert np.allclose(o, o_ref, atol=1e-13, rtol=1e-12)
    assert np.allclose(lse, lse_ref, atol=1e-13, rtol=1e-13)


def test_strides_are_honoured():
    # K and V in wider NaN-padded rows, Q dense: any read of the padding
    # or any use of the wrong row stride poisons or changes the result
    rng = np.random.default_rng(11)
    D = 8
    q = wl.from_values(rng.standard_normal((6, D)))
    k = wl.from_values(rng.standard_normal((9, D)), ld=13)
    v = wl.from_values(rng.standard_normal((9, D)), ld=21)
    o, lse = oracle.attention(q, k, v)
    o_ref, lse_ref = _scipy_attention(q, np.array(k), np.array(v),
                                      1 / math.sqrt(D))
    assert np.all(np.isfinite(o))
    assert np.allclose(o, o_ref, atol=1e-13) and np.allclose(lse, lse_ref,
                                                             atol=1e-13)


def test_bhsd_and_bshd_layouts_agree():
    qa, ka, va = wl.attention_inputs(2, 3, 5, 7, 8, seed=3)
    qb, kb, vb = wl.attention_inputs(2, 3, 5, 7, 8, seed=3, layout="bshd")
    oa, la = oracle.attention_bhsd(qa, ka, va)
    ob, lb = oracle.attention_bhsd(qb, kb, vb)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)
    o_ref, l_ref = _scipy_attention(qa[1, 2], ka[1, 2], va[1, 2], 8 ** -0.5)
    assert np.allclose(oa[1, 2], o_ref, atol=1e-13)
    assert np.allclose(la[1, 2], l_ref, atol=1e-13)


# ---------------------------------------------------------------------------
# Closed forms and special cases
# ---------------------------------------------------------------------------

def test_constant_value_rows():
    rng = np.random.default_rng(5)
    q = wl.from_values(rng.standard_normal((4, 6)))
    k = wl.from_values(3 * rng.standard_normal((50, 6)))
    c = np.array([1.5, -2.0, 0.25, 7.0, 0.0, -0.125])
    v = wl.from_values(np.tile(c, (50, 1)))
    o, _ = oracle.attention(q, k, v)
    assert np.allclose(o, c[None, :], atol=1e-13, rtol=0)


def test_zero_query_averages_values():
    rng = np.random.default_rng(6)
    Sk, D = 37, 5
    q = wl.from_values(np.zeros((3, D)))
    k = wl.from_values(rng.standard_normal((Sk, D)))
    v = wl.from_values(rng.standard_normal((Sk, D)))
    o, lse = oracle.attention(q, k, v)
    assert np.allclose(o, np.asarray(v, np.float64).mean(0), atol=1e-14)
    assert np.allclose(lse, math.log(Sk), atol=1e-14)


def test_single_key():
    q = wl.from_values([[0.5, -1.0, 2.0]])
    k = wl.from_values([[1.0, 0.25, 0.5]])
    v = wl.from_values([[3.0, 4.0, -5.0]])
    o, lse = oracle.attention(q, k, v, scale=0.75)
    assert np.array_equal(o[0], [3.0, 4.0, -5.0])
    assert lse[0] == pytest.approx(0.75 * (0.5 - 0.25 + 1.0), abs=1e-15)


def test_two_keys_logistic_weights():
    q = wl.from_values([[1.0, 2.0]])
    k = wl.from_values([[0.5, 0.25], [-1.0, 1.5]])
    v = wl.from_values([[1.0, 0.0], [0.0, 1.0]])
    scale = 0.6
    s0, s1 = scale * (0.5 + 0.5), scale * (-1.0 + 3.0)
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    o, lse = oracle.attention(q, k, v, scale=scale)
    assert np.allclose(o[0], [w0, 1.0 - w0], atol=1e-15)
    assert lse[0] == pytest.approx(max(s0, s1) + math.log1p(math.exp(-abs(s1 - s0))),
                                   abs=1e-14)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(8)
    D = 4
    q = wl.from_values([[1.0, 1.0, 1.0, 1.0]])
    k = wl.from_values(0.1 * rng.standard_normal((20, D)))
    kk = np.asarray(k, np.float64).copy()
    kk[13] = 200.0                       # score 400 against ~0.2
    v = wl.from_values(rng.standard_normal((20, D)))
    o, lse = oracle.attention(q, wl.from_values(kk), v, scale=0.5)
    assert np.allclose(o[0], np.asarray(v, np.float64)[13], atol=1e-15)
    assert lse[0] == pytest.approx(400.0, abs=1e-12)


def test_causal_first_rows_and_offsets():
    rng = np.random.default_rng(9)
    Sq, Sk, D = 6, 10, 3
    q = wl.from_values(rng.standard_normal((Sq, D)))
    k = wl.from_values(rng.standard_normal((Sk, D)))
    v = wl.from_values(rng.standard_normal((Sk, D)))
    o, lse = oracle.attention(q, k, v, causal=0)
    # row 0 sees key 0 only
    assert np.array_equal(o[0], np.asarray(v, np.float64)[0])
    s00 = float(np.dot(np.asarray(q, np.float64)[0], np.asarray(k, np.float64)[0]))
    assert lse[0] == pytest.approx(s00 / math.sqrt(D), abs=1e-15)
    # row i under offset c equals unmasked attention over the first i+c+1 keys
    for c in (0, 2, 4):
        oc, lc = oracle.attention(q, k, v, causal=c)
        for i in range(Sq):
            n = min(Sk, i + c + 1)
            oi, li = oracle.attention(q[i:i + 1], k[:n], v[:n])
            assert np.array_equal(oc[i], oi[0]) and lc[i] == li[0]
    # an offset reaching past the last key is no mask
    assert np.array_equal(oracle.attention(q, k, v, causal=Sk)[0],
                          oracle.attention(q, k, v)[0])


def test_key_permutation_invariance():
    rng = np.random.default_rng(10)
    q = wl.from_values(rng.standard_normal((5, 8)))
    k = wl.from_values(rng.standard_normal((64, 8)))
    v = wl.from_values(rng.standard_normal((64, 8)))
    perm = rng.permutation(64)
    o, lse = oracle.attention(q, k, v)
    op, lp = oracle.attention(q, np.ascontiguousarray(k[perm]),
                              np.ascontiguousarray(v[perm]))
    assert np.allclose(o, op, atol=1e-14) and np.allclose(lse, lp, atol=1e-14)


def test_large_logits_do_not_overflow():
    # scores of several thousand: a naive e^s overflows fp64 near 709
    rng = np.random.default_rng(12)
    q = wl.from_values(60 * rng.standard_normal((4, 16)))
    k = wl.from_values(60 * rng.standard_normal((30, 16)))
    v = wl.from_values(rng.standard_normal((30, 16)))
    o, lse = oracle.attention(q, k, v)
    o_ref, l_ref = _scipy_attention(q, k, v, 0.25)
    assert np.all(np.isfinite(o)) and np.max(np.abs(lse)) > 1000
    assert np.allclose(o, o_ref, atol=1e-12) and np.allclose(lse, l_ref, rtol=1e-14)


@pytest.mark.parametrize("Bc", [1, 3, 16, 64, 333])
@pytest.mark.parametrize("causal", [-1, 0, 5])
def test_online_recurrence_equals_definition(Bc, causal):
    q, k, v = (a[0, 0] for a in wl.attention_inputs(1, 1, 40, 333, 16, seed=Bc,
                                                   q_scale=3.0))
    o, lse = oracle.attention(q, k, v, causal=causal)
    o2, lse2 = oracle.attention(q, k, v, causal=causal, online_block=Bc)
    assert np.allclose(o, o2, atol=1e-13, rtol=0)
    assert np.allclose(lse, lse2, atol=1e-13, rtol=0)


def test_selected_rows_equal_full_rows():
    q, k, v = (a[0, 0] for a in wl.attention_inputs(1, 1, 50, 70, 8, seed=4))
    rows = [49, 0, 17, 17, 3]
    o, lse = oracle.attention(q, k, v, causal=2)
    os_, ls = oracle.attention(q, k, v, causal=2, rows=rows)
    assert np.array_equal(os_, o[rows]) and np.array_equal(ls, lse[rows])


def test_special_values():
    q = wl.from_values([[1.0, 0.0], [0.0, 1.0]])
    k = wl.from_values([[1.0, np.nan], [0.5, 0.5], [2.0, 1.0]])
    v = wl.from_values([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])
    o, lse = oracle.attention(q, k, v)
    # q0 . k0 = 1 + 0*NaN = NaN, q1 . k0 = 0*1 + NaN: both rows see a NaN score
    assert np.all(np.isnan(o)) and np.all(np.isnan(lse))
    k2 = wl.from_values([[np.inf, 0.0], [0.5, 0.5]])
    o2, lse2 = oracle.attention(q, k2, v[:2])
    assert np.all(np.isnan(o2[0])) and np.isnan(lse2[0])     # +inf score
    assert np.all(np.isnan(o2[1]))                           # 0 * inf = NaN


def test_argument_errors():
    q = wl.from_values(np.ones((2, 4)))
    k = wl.from_values(np.ones((3, 4)))
    with pytest.raises(ValueError):
        oracle.attention(q, k[:0], k[:0])                     # Sk = 0
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, rows=[2])                   # row out of range
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, online_block=0)
    with pytest.raises(TypeError):
        oracle.attention(q, wl.from_values(np.ones((3, 4)), "bf16"), k)
    with pytest.raises(ValueError):
        oracle.attention(q, k, wl.from_values(np.ones((4, 4))))
    o, lse = oracle.attention(q[:0], k, k)                    # Sq = 0
    assert o.shape == (0, 4) and lse.shape == (0,)
