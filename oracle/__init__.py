"""fp64 CPU oracle for row-wise softmax -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
import this package.  The product path (``row_wise_online_amd``) never does.

This module is a ctypes wrapper around ``liboracle.so`` (built from
``oracle.c`` by ``oracle/build.py``) plus the comparison helpers the parity
tests use.  See ``oracle.c`` for the cited definitions.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB lets the mutation test load a deliberately broken build.
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i64, i32, dp = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                            ctypes.c_void_p)
        lib.oracle_softmax.argtypes = [vp, i64, i64, i64, i32, dp, dp, dp, dp]
        lib.oracle_softmax.restype = i32
        lib.oracle_state.argtypes = [vp, i64, i64, i64, i32, dp, dp]
        lib.oracle_state.restype = i32
        lib.oracle_merge2.argtypes = [ctypes.c_double] * 4 + [
            ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
        lib.oracle_merge2.restype = None
        lib.oracle_merge.argtypes = [dp, dp, i64, i64, i64, dp, dp, dp]
        lib.oracle_merge.restype = i32
        lib.oracle_log_softmax.argtypes = [vp, i64, i64, i64, i32, dp]
        lib.oracle_log_softmax.restype = i32
        lib.oracle_normalize.argtypes = [vp, i64, i64, i64, i32, dp, dp, i64,
                                         i32, dp]
        lib.oracle_normalize.restype = i32
        lib.oracle_cross_entropy.argtypes = [vp, i64, i64, i64, i32, vp, dp,
                                             dp]
        lib.oracle_cross_entropy.restype = i32
        lib.oracle_softmax_masked.argtypes = [vp, i64, i64, i64, i32, vp, i64,
                                              dp, dp, dp, dp, dp]
        lib.oracle_softmax_masked.restype = i32
        lib.oracle_attention.argtypes = [vp, i64, vp, i64, vp, i64, i32, i64,
                                         i64, i64, ctypes.c_double, i64, vp,
                                         i64, dp, dp]
        lib.oracle_attention.restype = i32
        lib.oracle_attention_online.argtypes = [vp, i64, vp, i64, vp, i64, i32,
                                                i64, i64, i64, ctypes.c_double,
                                                i64, i64, vp, i64, dp, dp]
        lib.oracle_attention_online.restype = i32
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _as_input(x):
    """Return (array, dtype code).  fp32 arrays are fp32; bf16 inputs are
    uint16 arrays holding the raw bf16 bit patterns."""
    x = np.asarray(x)
    if x.dtype == np.float32:
        code = F32
    elif x.dtype == np.uint16:
        code = BF16
    else:
        raise TypeError("oracle input must be float32 or uint16 (bf16 bits)")
    if x.ndim == 1:
        x = x[None, :]
    if x.ndim != 2 or x.strides[1] != x.itemsize:
        raise ValueError("oracle input must be a 2-D array with unit column stride")
    if x.strides[0] % x.itemsize:
        raise ValueError("row stride must be a whole number of elements")
    return x, code


def softmax(x, want_y=True):
    """Three-pass fp64 safe softmax of every row of ``x``.

    Returns (y [M,N] fp64 or None, m [M], d [M], lse [M])."""
    x, code = _as_input(x)
    M, N = x.shape
    ld = x.strides[0] // x.itemsize
    y = np.empty((M, N), np.float64) if want_y else None
    m = np.empty(M, np.float64)
    d = np.empty(M, np.float64)
    lse = np.empty(M, np.float64)
    rc = _load().oracle_softmax(_ptr(x), ld, M, N, code, _ptr(y), _ptr(m),
                                _ptr(d), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_softmax rejected its arguments")
    return y, m, d, lse


def state(x):
    """The element-by-element online (m, d) fold of every row of ``x``."""
    x, code = _as_input(x)
    M, N = x.shape
    ld = x.strides[0] // x.itemsize
    m = np.empty(M, np.float64)
    d = np.empty(M, np.float64)
    rc = _load().oracle_state(_ptr(x), ld, M, N, code, _ptr(m), _ptr(d))
    if rc != 0:
        raise ValueError("oracle_state rejected its arguments")
    return m, d


def merge2(a, b):
    """Merge two states a = (m_a, d_a), b = (m_b, d_b)."""
    m = ctypes.c_double()
    d = ctypes.c_double()
    _load().oracle_merge2(float(a[0]), float(a[1]), float(b[0]), float(b[1]),
                          ctypes.byref(m), ctypes.byref(d))
    return m.value, d.value


def merge(m_in, d_in):
    """Left-fold merge of the K states of each row: m_in, d_in are [M,K]
    (any float dtype; widened to fp64).  Returns (m, d, lse) fp64 [M]."""
    m_in = np.ascontiguousarray(m_in, dtype=np.float64)
    d_in = np.ascontiguousarray(d_in, dtype=np.float64)
    if m_in.ndim == 1:
        m_in, d_in = m_in[None, :], d_in[None, :]
    M, K = m_in.shape
    m = np.empty(M, np.float64)
    d = np.empty(M, np.float64)
    lse = np.empty(M, np.float64)
    rc = _load().oracle_merge(_ptr(m_in), _ptr(d_in), K, M, K, _ptr(m),
                              _ptr(d), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_merge rejected its arguments")
    return m, d, lse


def log_softmax(x):
    """log p = z - LSE(z) for every row of ``x`` (fp64 [M, N])."""
    x, code = _as_input(x)
    M, N = x.shape
    ld = x.strides[0] // x.itemsize
    y = np.empty((M, N), np.float64)
    rc = _load().oracle_log_softmax(_ptr(x), ld, M, N, code, _ptr(y))
    if rc != 0:
        raise ValueError("oracle_log_softmax rejected its arguments")
    return y


def normalize(x, m, d, log=False):
    """Pass 2 of every row of ``x`` for the given row states (m, d) [M]
    (any float dtype, widened to fp64): e^(x - m) / d, or with log=True
    (x - m) - log d; fp64 [M, N].  The exact value for that state."""
    x, code = _as_input(x)
    M, N = x.shape
    ld = x.strides[0] // x.itemsize
    m = np.ascontiguousarray(m, dtype=np.float64).reshape(-1)
    d = np.ascontiguousarray(d, dtype=np.float64).reshape(-1)
    if m.shape != (M,) or d.shape != (M,):
        raise ValueError("one state per row")
    y = np.empty((M, N), np.float64)
    rc = _load().oracle_normalize(_ptr(x), ld, M, N, code, _ptr(m), _ptr(d),
                                  1, 1 if log else 0, _ptr(y))
    if rc != 0:
        raise ValueError("oracle_normalize rejected its arguments")
    return y


def cross_entropy(x, labels):
    """Per-row cross-entropy (fp64 [M]) and the mean over rows whose
    label is not negative."""
    x, code = _as_input(x)
    M, N = x.shape
    ld = x.strides[0] // x.itemsize
    labels = np.ascontiguousarray(labels, dtype=np.int64)
    if labels.shape != (M,):
        raise ValueError("one label per row")
    loss = np.empty(M, np.float64)
    mean = np.empty(1, np.float64)
    rc = _load().oracle_cross_entropy(_ptr(x), ld, M, N, code, _ptr(labels),
                                      _ptr(loss), _ptr(mean))
    if rc != 0:
        raise ValueError("oracle_cross_entropy rejected its arguments")
    return loss, float(mean[0])


def softmax_masked(x, row_len=None, causal=-1):
    """Softmax and log-softmax of each row over its first n_i columns
    (n_i from row_len and/or the causal offset).  Returns
    (y, log_y, m, d, lse), fp64."""
    x, code = _as_input(x)
    M, N = x.shape
    ld = x.strides[0] // x.itemsize
    rl = None if row_len is None else np.ascontiguousarray(row_len,
                                                            dtype=np.int32)
    if rl is not None and rl.shape != (M,):
        raise ValueError("one length per row")
    y = np.empty((M, N), np.float64)
    log_y = np.empty((M, N), np.float64)
    m = np.empty(M, np.float64)
    d = np.empty(M, np.float64)
    lse = np.empty(M, np.float64)
    rc = _load().oracle_softmax_masked(_ptr(x), ld, M, N, code, _ptr(rl),
                                       int(causal), _ptr(y), _ptr(log_y),
                                       _ptr(m), _ptr(d), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_softmax_masked rejected its arguments")
    return y, log_y, m, d, lse


def _attn_inputs(q, k, v):
    (q, cq), (k, ck), (v, cv) = _as_input(q), _as_input(k), _as_input(v)
    if not (cq == ck == cv):
        raise TypeError("q, k and v must share one dtype")
    if k.shape != v.shape or q.shape[1] != k.shape[1]:
        raise ValueError("q [Sq, D], k and v [Sk, D]")
    ld = lambda a: a.strides[0] // a.itemsize
    return q, k, v, cq, ld(q), ld(k), ld(v)


def attention(q, k, v, scale=None, causal=-1, rows=None, online_block=None):
    """Attention of one (batch, head) slice: q [Sq, D], k and v [Sk, D]
    (fp32, or uint16 bf16 bits).  scale defaults to 1/sqrt(D); causal >= 0
    admits key j for query i when j <= i + causal.  rows: the query rows to
    evaluate (default all).  online_block: evaluate by the tiled online
    recurrence with key blocks of that size instead of the definition.
    Returns (o fp64 [nrows, D], lse fp64 [nrows])."""
    q, k, v, code, ldq, ldk, ldv = _attn_inputs(q, k, v)
    Sq, D = q.shape
    Sk = k.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = Sq if r is None else r.shape[0]
    o = np.empty((n, D), np.float64)
    lse = np.empty(n, np.float64)
    lib = _load()
    if online_block is None:
        rc = lib.oracle_attention(_ptr(q), ldq, _ptr(k), ldk, _ptr(v), ldv,
                                  code, Sq, Sk, D, float(scale), int(causal),
                                  _ptr(r), n, _ptr(o), _ptr(lse))
    else:
        rc = lib.oracle_attention_online(_ptr(q), ldq, _ptr(k), ldk, _ptr(v),
                                         ldv, code, Sq, Sk, D, float(scale),
                                         int(causal), int(online_block),
                                         _ptr(r), n, _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_attention rejected its arguments")
    return o, lse


def attention_bhsd(q, k, v, scale=None, causal=-1, rows=None):
    """attention() for every (batch, head) of q [B, H, Sq, D] and
    k, v [B, H, Sk, D] (any layout whose last axis is contiguous).
    Returns (o fp64 [B, H, nrows, D], lse fp64 [B, H, nrows])."""
    B, H = q.shape[:2]
    n = q.shape[2] if rows is None else len(rows)
    o = np.empty((B, H, n, q.shape[3]), np.float64)
    lse = np.empty((B, H, n), np.float64)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = attention(q[b, h], k[b, h], v[b, h], scale,
                                           causal, rows)
    return o, lse


# ---------------------------------------------------------------------------
# Comparison helpers used by the parity tests.  They compare a result against
# fp64 oracle values; they never compute a softmax themselves.
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits):
    """Exact widening of raw bf16 bit patterns (uint16) to fp64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_f64_to_bf16_bits(v):
    """Round fp64 values to the nearest bf16 (ties to even), returning raw
    uint16 bit patterns.  Rounding is done once, directly from fp64 (no
    intermediate fp32 rounding).  Finite values only; NaN maps to a quiet
    NaN pattern and values beyond the bf16 range to +-inf."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    flat_v = v.ravel()
    flat_o = out.ravel()
    sign = np.signbit(flat_v)
    a = np.abs(flat_v)
    nan = np.isnan(flat_v)
    # bf16: 8 significant bits, min normal 2^-126, subnormal quantum 2^-133
    _, e = np.frexp(np.where(a > 0, a, 1.0))    # a = f * 2^e, f in [0.5, 1)
    e = np.maximum(e, -125)                      # subnormal range: fixed quantum
    quantum = np.ldexp(1.0, e - 8)
    q = np.rint(a / quantum) * quantum           # exact in fp64; rint is RNE
    q32 = q.astype(np.float32)                   # exact: q has <= 8 bits
    bits = (q32.view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(q > 3.3895313892515355e38, np.uint16(0x7F80), bits)
    bits = np.where(sign, bits | np.uint16(0x8000), bits)
    bits = np.where(nan, np.uint16(0x7FC0), bits)
    flat_o[:] = bits
    return out


def bf16_ulp_distance(a_bits, b_bits):
    """Distance in representable bf16 steps between two raw bf16 patterns
    (ordered-integer distance; +0 and -0 are the same point)."""
    def ordered(b):
        b = np.asarray(b, dtype=np.uint16).astype(np.int32)
        mag = b & 0x7FFF
        return np.where(b & 0x8000, -mag, mag)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def f32_ulp(v):
    """The fp32 unit in the last place at |v| (spacing to the next float)."""
    v = np.abs(np.asarray(v, dtype=np.float32))
    return np.spacing(v).astype(np.float64)
