"""Seeded synthetic inputs for the row-wise softmax workloads.

This module only draws and stores input values; it contains none of the
softmax arithmetic.  The same stored bytes feed the fp64 oracle and the HIP
path, so both sides see identical inputs.

Recipe (for every workload): ``numpy.random.default_rng(seed)`` (PCG64),
fp64 standard normals in row-major order, scaled and given their structure
in fp64, then rounded to fp32 with round-to-nearest-even; bf16 inputs are
rounded once more, fp32 -> bf16, to nearest-even at the bit level.  bf16
arrays are returned as ``uint16`` arrays of raw bit patterns.

The five named workloads:

=====  ===========  =====  ============================================
name   M x N        dtype  values
=====  ===========  =====  ============================================
c1     64 x 1000    fp32   3 N(0,1); row 0 += 80, row 1 -= 80
c2     4096 x 4096  fp32   N(0,1)
c3     32768 x 1024 bf16   2 N(0,1)
c4     1024 x 32768 fp32   0.01 j + 0.1 N(0,1)  (ascending in j)
c5     16 x 4194304 fp32   N(0,1), then x[i, c_i] = 20 for a seeded c_i
=====  ===========  =====  ============================================

Attention inputs (the online softmax inside key tiles): Q, K and V are
drawn in that order, each [B, H, S, D] in row-major order, as
``q_scale`` N(0,1) for Q and N(0,1) for K and V, rounded to bf16 as above.
With the default scale 1/sqrt(D) the scores are then about N(0, q_scale^2).
The named attention workloads:

=====  ===============================  ======  =======================
name   B x H x Sq x Sk x D              causal  values
=====  ===============================  ======  =======================
a1     2 x 3 x 300 x 333 x 128          no      N(0,1)
a2     1 x 1 x 131072 x 131072 x 128    no      N(0,1)
a3     1 x 1 x 131072 x 131072 x 128    0       N(0,1)
a4     1 x 1 x 131072 x 131072 x 64     no      N(0,1)
a5     1 x 1 x 131072 x 131072 x 32     no      N(0,1)
=====  ===============================  ======  =======================
"""
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    dtype: str            # "f32" or "bf16"
    seed: int
    outputs: tuple        # which outputs the workload asks for
    desc: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def esize(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS = {
    "c1": Workload("c1", 64, 1000, "f32", 1001, ("y", "lse"),
                   "fp32 64x1000, 3N(0,1), row0 +80, row1 -80"),
    "c2": Workload("c2", 4096, 4096, "f32", 1002, ("y", "m", "d"),
                   "fp32 4096x4096, N(0,1)"),
    "c3": Workload("c3", 32768, 1024, "bf16", 1003, ("y",),
                   "bf16 32768x1024, 2N(0,1)"),
    "c4": Workload("c4", 1024, 32768, "f32", 1004, ("y",),
                   "fp32 1024x32768, 0.01j + 0.1N(0,1) ascending"),
    "c5": Workload("c5", 16, 4194304, "f32", 1005, ("y", "m", "d", "lse"),
                   "fp32 16x4194304, N(0,1) with a planted +20 per row"),
}


def f32_to_bf16_bits(a):
    """Round fp32 values to bf16 (nearest, ties to even) at the bit level.
    Returns raw uint16 patterns.  Inputs are finite here."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _store(v64, dtype, ld=None, pad_value=np.nan):
    """Round fp64 values to the storage dtype; optionally embed them in a
    wider row stride ``ld`` whose padding holds ``pad_value`` (NaN by
    default, so that any read of the padding would poison a result)."""
    f32 = v64.astype(np.float32)
    store = f32 if dtype == "f32" else f32_to_bf16_bits(f32)
    if ld is None or ld == v64.shape[1]:
        return store
    M, N = v64.shape
    if dtype == "f32":
        buf = np.full((M, ld), pad_value, np.float32)
    else:
        buf = np.full((M, ld), f32_to_bf16_bits(np.float32([pad_value]))[0],
                      np.uint16)
    buf[:, :N] = store
    return buf[:, :N]


def generate(name: str):
    """The stored input of a named workload (fp32 array or bf16 bit array)."""
    w = WORKLOADS[name]
    rng = np.random.default_rng(w.seed)
    z = rng.standard_normal((w.M, w.N))
    if name == "c1":
        v = 3.0 * z
        v[0] += 80.0
        v[1] -= 80.0
    elif name == "c2":
        v = z
    elif name == "c3":
        v = 2.0 * z
    elif name == "c4":
        j = np.arange(w.N, dtype=np.float64)
        v = 0.01 * j[None, :] + 0.1 * z
    elif name == "c5":
        v = z
        cols = rng.integers(0, w.N, size=w.M)   # drawn after the normals
        v[np.arange(w.M), cols] = 20.0
    else:
        raise KeyError(name)
    return _store(v, w.dtype)


def planted_columns(name: str = "c5"):
    """The seeded planted-max columns of the long-row workload."""
    w = WORKLOADS[name]
    rng = np.random.default_rng(w.seed)
    rng.standard_normal((w.M, w.N))
    return rng.integers(0, w.N, size=w.M)


def normal(M, N, *, scale=1.0, offset=0.0, seed=0, dtype="f32", ld=None):
    """Generic seeded input: offset + scale * N(0,1), rounded to ``dtype``.
    With ``ld`` > N the rows sit in a wider buffer padded with NaN."""
    rng = np.random.default_rng(seed)
    v = offset + scale * rng.standard_normal((M, N))
    return _store(v, dtype, ld)


def ascending(M, N, *, slope=0.01, noise=0.1, seed=0, dtype="f32"):
    """Seeded adversarial-order input: slope * j + noise * N(0,1)."""
    rng = np.random.default_rng(seed)
    j = np.arange(N, dtype=np.float64)
    v = slope * j[None, :] + noise * rng.standard_normal((M, N))
    return _store(v, dtype)


def from_values(v, dtype="f32", ld=None):
    """Store explicit fp64 values (special values allowed) in ``dtype``."""
    v = np.asarray(v, dtype=np.float64)
    if v.ndim == 1:
        v = v[None, :]
    return _store(v, dtype, ld)


@dataclass(frozen=True)
class AttnWorkload:
    name: str
    B: int
    H: int
    Sq: int
    Sk: int
    D: int
    causal: int           # -1: none; >= 0: key j admitted when j <= i + causal
    seed: int
    desc: str = ""

    def flops(self) -> float:
        """2 Sq Sk D multiply-adds for each of Q K^T and P V, per head; a
        causal mask with offset c admits sum_i min(Sk, i + c + 1) keys."""
        if self.causal < 0:
            pairs = self.Sq * self.Sk
        else:
            i = np.arange(self.Sq, dtype=np.int64)
            pairs = int(np.minimum(self.Sk, i + self.causal + 1).sum())
        return 4.0 * self.B * self.H * pairs * self.D


ATTN_WORKLOADS = {
    "a1": AttnWorkload("a1", 2, 3, 300, 333, 128, -1, 2001,
                       "bf16 2x3 heads, 300 queries x 333 keys, d=128"),
    "a2": AttnWorkload("a2", 1, 1, 131072, 131072, 128, -1, 2002,
                       "bf16 one head, 131072 queries x 131072 keys, d=128"),
    "a3": AttnWorkload("a3", 1, 1, 131072, 131072, 128, 0, 2003,
                       "bf16 one head, 131072^2, d=128, causal"),
    "a4": AttnWorkload("a4", 1, 1, 131072, 131072, 64, -1, 2004,
                       "bf16 one head, 131072^2, d=64"),
    "a5": AttnWorkload("a5", 1, 1, 131072, 131072, 32, -1, 2005,
                       "bf16 one head, 131072^2, d=32"),
}


def attention_inputs(B, H, Sq, Sk, D, *, seed=0, q_scale=1.0, layout="bhsd"):
    """Seeded bf16 Q [B,H,Sq,D], K and V [B,H,Sk,D] (uint16 bit arrays).

    layout "bhsd" stores each tensor densely in that order; "bshd" stores
    it as [B,S,H,D] and returns the [B,H,S,D] view (same values)."""
    rng = np.random.default_rng(seed)
    out = []
    for S, sc in ((Sq, q_scale), (Sk, 1.0), (Sk, 1.0)):
        v = sc * rng.standard_normal((B, H, S, D))
        bits = f32_to_bf16_bits(v.astype(np.float32))
        if layout == "bshd":
            buf = np.ascontiguousarray(bits.transpose(0, 2, 1, 3))
            bits = buf.transpose(0, 2, 1, 3)
        elif layout != "bhsd":
            raise ValueError(layout)
        out.append(bits)
    return tuple(out)


def attention_workload(name: str):
    """(q, k, v) of a named attention workload."""
    w = ATTN_WORKLOADS[name]
    return attention_inputs(w.B, w.H, w.Sq, w.Sk, w.D, seed=w.seed)
