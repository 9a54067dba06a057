"""GPU parity of the attention forward (os_attention_fwd) against the fp64
oracle, through the C ABI.

Accuracy bar, derived from the arithmetic (fp32 = unit roundoff u = 2^-24;
the kernel multiplies bf16 operands exactly and accumulates in fp32):
  * score error: q.k sums D exact products in fp32, so
    |ds| <= D u sum_c |q_c k_c|; with the fma that forms t = s c - m2 and the
    rounding of m2 the exponent of each p is off by at most
    dt = c D u max_j sum_c |q_c k_jc| + 2 ulp(max |t|), and each p by a
    factor 2^(+-2 dt), i.e. relatively by Delta = 2 ln2 dt (first order);
  * the probabilities enter P.V rounded to bf16 (8 significant bits, unit
    roundoff 2^-8): a relative 2^-8 each;
  * o~ accumulates Sk/16 MFMA partial sums and is rescaled at most once per
    64-key tile; l sums 32 values per lane per tile, rescaled once per tile:
    together at most n_acc = Sk/16 + 2 Sk/64 + 64 roundings;
  so with w = max over admitted keys of |v_jd|,
    |o - o_ref| <= (2^-8 + 2 Delta + n_acc u) w  (+ 2^-8 |o_ref| for bf16 o)
    |lse - lse_ref| <= Delta + n_acc u + 2 ulp(lse_ref).
This bound on o is worst-case; a lost key or a missing rescale shows in
lse (tight) or as an O(1) error in o, and the structured cases below check
single probabilities to 2^-8.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import row_wise_online_amd as rwo
from row_wise_online_amd import workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.filterwarnings("ignore::RuntimeWarning")]

U = 2.0 ** -24
LOG2E = 1.4426950408889634


def _dev(bits):
    """numpy bf16 bits [B, H, S, D] -> GPU bf16 tensor of the same strides
    order (dense BHSD, or a BHSD view of a dense BSHD buffer)."""
    if bits.flags.c_contiguous:
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    buf = np.ascontiguousarray(bits.transpose(0, 2, 1, 3))
    t = torch.from_numpy(buf.view(np.int16)).view(torch.bfloat16).cuda()
    return t.permute(0, 2, 1, 3)


def _host(t):
    if t.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(
            t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.contiguous().cpu().numpy().astype(np.float64)


def _w(a):
    return oracle.bf16_bits_to_f64(np.asarray(a))


def run(q, k, v, *, causal=-1, scale=None, out=torch.bfloat16, o_layout=None):
    qd, kd, vd = _dev(q), _dev(k), _dev(v)
    B, H, Sq, D = q.shape
    if o_layout == "bshd":
        o = torch.empty((B, Sq, H, D), dtype=out, device="cuda").permute(0, 2, 1, 3)
    else:
        o = torch.empty((B, H, Sq, D), dtype=out, device="cuda")
    o.fill_(float("nan"))
    lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device="cuda")
    rwo.attention_fwd(qd, kd, vd, o, lse=lse, scale=scale, causal_offset=causal)
    torch.cuda.synchronize()
    return _host(o), lse.cpu().numpy().astype(np.float64)


def bounds(q2, k2, v2, rows, o_ref, lse_ref, scale, causal, bf16_out):
    """Tolerances for one (batch, head) slice at the given query rows."""
    rows = np.asarray(rows)
    qf, kf, vf = _w(q2)[rows], _w(k2), _w(v2)
    Sk, D = kf.shape
    c = scale * LOG2E
    ka = np.abs(kf).T
    amax = np.empty(len(rows))
    for r0 in range(0, len(rows), 64):           # [rows, Sk] in blocks
        dot_abs = np.abs(qf[r0:r0 + 64]) @ ka
        if causal >= 0:                          # admitted keys only
            j = np.arange(Sk)[None, :]
            dot_abs = np.where(j <= rows[r0:r0 + 64, None] + causal, dot_abs, 0.0)
        amax[r0:r0 + 64] = dot_abs.max(axis=1)
    tmax = c * amax
    dt = c * D * U * amax + 2 * oracle.f32_ulp(np.maximum(tmax, 1.0))
    delta = 2 * math.log(2) * dt
    n_acc = Sk / 16 + 2 * Sk / 64 + 64
    # the largest |v| over the keys each row admits: a running max down
    # the keys, read at the row's last admitted key
    vmax = np.maximum.accumulate(np.abs(vf), axis=0)
    last = np.full(len(rows), Sk - 1) if causal < 0 else np.minimum(Sk - 1, rows + causal)
    wmax = vmax[last]
    tol_o = (2.0 ** -8 + 2 * delta[:, None] + n_acc * U) * wmax
    if bf16_out:
        tol_o = tol_o + 2.0 ** -8 * np.abs(o_ref)
    tol_lse = delta + n_acc * U + 2 * oracle.f32_ulp(lse_ref)
    return tol_o, tol_lse


def _oracle_rows(q2, k2, v2, scale, causal, rows):
    """oracle.attention at the given rows, on several host threads when the
    rows are many (the C call releases the interpreter lock)."""
    rows = list(rows)
    if len(rows) <= 64:
        return oracle.attention(q2, k2, v2, scale, causal, rows)
    from concurrent.futures import ThreadPoolExecutor
    T = max(1, min(8, os.cpu_count() or 1))
    parts = [rows[i::T] for i in range(T) if rows[i::T]]
    with ThreadPoolExecutor(len(parts)) as ex:
        res = list(ex.map(lambda r: oracle.attention(q2, k2, v2, scale, causal, r),
                          parts))
    o = np.empty((len(rows), q2.shape[1]))
    lse = np.empty(len(rows))
    for i, (oo, ll) in enumerate(res):
        o[i::len(parts)] = oo
        lse[i::len(parts)] = ll
    return o, lse


def check(q, k, v, o, lse, *, causal=-1, scale=None, bf16_out=True, rows=None,
          what=""):
    B, H, Sq, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    rows = list(range(Sq)) if rows is None else list(rows)
    worst = (0.0, 0.0)
    for b in range(B):
        for h in range(H):
            o_ref, l_ref = _oracle_rows(q[b, h], k[b, h], v[b, h], scale,
                                        causal, rows)
            tol_o, tol_l = bounds(q[b, h], k[b, h], v[b, h], rows, o_ref,
                                  l_ref, scale, causal, bf16_out)
            err_o = np.abs(o[b, h][rows] - o_ref)
            err_l = np.abs(lse[b, h][rows] - l_ref)
            bad = np.argwhere(~(err_o <= tol_o))
            assert bad.size == 0, (
                f"{what} b{b} h{h}: {len(bad)} outputs off, first row "
                f"{rows[bad[0][0]]} col {bad[0][1]}: got "
                f"{o[b, h][rows[bad[0][0]], bad[0][1]]!r} want "
                f"{o_ref[tuple(bad[0])]!r} tol {tol_o[tuple(bad[0])]:.3g}")
            badl = np.argwhere(~(err_l <= tol_l))
            assert badl.size == 0, (
                f"{what} b{b} h{h}: lse off at row {rows[badl[0][0]]}: got "
                f"{lse[b, h][rows[badl[0][0]]]!r} want {l_ref[badl[0][0]]!r}")
            worst = (max(worst[0], float(err_o.max(initial=0))),
                     max(worst[1], float(err_l.max(initial=0))))
    return worst


# ---------------------------------------------------------------------------
# Small shapes: every output element against the oracle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_a1_shape_every_element(D, out):
    w = wl.ATTN_WORKLOADS["a1"]
    q, k, v = wl.attention_inputs(w.B, w.H, w.Sq, w.Sk, D, seed=w.seed)
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    print(f"a1 shape D={D} out={out}", flush=True)
    o, lse = run(q, k, v, out=odt)
    check(q, k, v, o, lse, bf16_out=out == "bf16", what=f"a1 D{D} {out}")


@pytest.mark.parametrize("causal", [0, 5, 33, 200, 332, 1000])
def test_causal_offsets(causal):
    q, k, v = wl.attention_inputs(1, 2, 300, 333, 128, seed=40 + causal)
    print(f"causal offset {causal}", flush=True)
    o, lse = run(q, k, v, causal=causal, out=torch.float32)
    check(q, k, v, o, lse, causal=causal, bf16_out=False, what=f"causal {causal}")


@pytest.mark.parametrize("Sq,Sk", [(1, 1), (1, 64), (1, 65), (31, 7), (129, 1),
                                   (128, 64), (70, 192), (257, 200), (64, 1000),
                                   (5, 4097)])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_ragged_shapes(Sq, Sk, D):
    q, k, v = wl.attention_inputs(1, 1, Sq, Sk, D, seed=Sq * 7 + Sk)
    print(f"ragged Sq={Sq} Sk={Sk} D={D}", flush=True)
    o, lse = run(q, k, v, out=torch.float32)
    check(q, k, v, o, lse, bf16_out=False, what=f"{Sq}x{Sk}")
    oc, lc = run(q, k, v, causal=0, out=torch.float32)
    check(q, k, v, oc, lc, causal=0, bf16_out=False, what=f"{Sq}x{Sk} causal")


def test_large_logits_rescale():
    # scores about N(0, 64): the running max keeps rising across tiles
    q, k, v = wl.attention_inputs(1, 2, 200, 700, 128, seed=77, q_scale=8.0)
    o, lse = run(q, k, v, out=torch.float32)
    assert np.max(np.abs(lse)) > 20
    check(q, k, v, o, lse, bf16_out=False, what="large logits")
    # ascending keys: every tile raises the max of every row
    rng = np.random.default_rng(5)
    base = np.linspace(-30, 30, 700)[None, None, :, None] * np.ones((1, 1, 1, 64))
    kk = wl.f32_to_bf16_bits((base + 0.1 * rng.standard_normal(base.shape))
                             .astype(np.float32))
    qq = wl.f32_to_bf16_bits(np.ones((1, 1, 50, 64), np.float32))
    vv = wl.attention_inputs(1, 1, 1, 700, 64, seed=6)[2]
    o, lse = run(qq, kk, vv, out=torch.float32)
    check(qq, kk, vv, o, lse, bf16_out=False, what="ascending keys")


def test_scale_argument():
    q, k, v = wl.attention_inputs(2, 1, 100, 150, 64, seed=3)
    o, lse = run(q, k, v, scale=0.37, out=torch.float32)
    check(q, k, v, o, lse, scale=0.37, bf16_out=False, what="scale 0.37")


def test_bshd_layout_matches_bhsd_bitwise():
    qa, ka, va = wl.attention_inputs(2, 3, 150, 170, 128, seed=9)
    qb, kb, vb = wl.attention_inputs(2, 3, 150, 170, 128, seed=9, layout="bshd")
    oa, la = run(qa, ka, va)
    ob, lb = run(qb, kb, vb, o_layout="bshd")
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)
    check(qb, kb, vb, ob, lb, what="bshd")


def test_kv_shared_across_heads():
    q, k, v = wl.attention_inputs(1, 4, 130, 90, 64, seed=12)
    qd = _dev(q)
    kd = _dev(k[:, :1]).expand(1, 4, 90, 64)       # head stride 0
    vd = _dev(v[:, :1]).expand(1, 4, 90, 64)
    o = torch.empty((1, 4, 130, 64), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, 4, 130), dtype=torch.float32, device="cuda")
    rwo.attention_fwd(qd, kd, vd, o, lse=lse)
    torch.cuda.synchronize()
    kk = np.ascontiguousarray(np.broadcast_to(k[:, :1], k.shape))
    vv = np.ascontiguousarray(np.broadcast_to(v[:, :1], v.shape))
    check(q, kk, vv, _host(o), lse.cpu().numpy().astype(np.float64),
          bf16_out=False, what="shared kv")


def test_constant_value_rows():
    q, k, _ = wl.attention_inputs(1, 1, 100, 300, 64, seed=21, q_scale=3.0)
    c = np.linspace(-4, 4, 64).astype(np.float32)
    v = wl.f32_to_bf16_bits(np.tile(c, (1, 1, 300, 1)))
    o, _ = run(q, k, v, out=torch.float32)
    cw = _w(v[0, 0, 0])
    # o = c * sum(bf16(p)) / sum(p): within 2^-8 of c, plus fp32 sums
    assert np.all(np.abs(o[0, 0] - cw) <= (2.0 ** -8 + 1e-4) * np.abs(cw) + 1e-7)


def test_one_hot_values_expose_probabilities():
    # V = identity: o_ij = bf16(p_ij) / l_i, each probability to 2^-8 (its
    # bf16 rounding) plus the score and sum errors (1e-5 here)
    D = 64
    q, k, _ = wl.attention_inputs(1, 1, 70, D, D, seed=22, q_scale=2.0)
    v = wl.f32_to_bf16_bits(np.eye(D, dtype=np.float32)[None, None])
    o, _ = run(q, k, v, out=torch.float32)
    p_ref, _ = oracle.attention(q[0, 0], k[0, 0], v[0, 0])
    err = np.abs(o[0, 0] - p_ref)
    assert np.all(err <= (2.0 ** -8 + 1e-5) * p_ref + 1e-12)
    assert np.allclose(o[0, 0].sum(1), 1.0, atol=2.0 ** -8)


def test_nan_key_poisons_the_rows_that_admit_it():
    q, k, v = wl.attention_inputs(1, 1, 90, 100, 64, seed=23)
    k = k.copy()
    k[0, 0, 40, 3] = 0x7FC0                                   # NaN
    o, lse = run(q, k, v, out=torch.float32)
    assert np.all(np.isnan(o[0, 0])) and np.all(np.isnan(lse[0, 0]))
    oc, lc = run(q, k, v, causal=0, out=torch.float32)
    assert np.all(np.isfinite(oc[0, 0, :40])) and np.all(np.isnan(oc[0, 0, 40:]))
    check(q[:, :, :40], k, v, oc[:, :, :40], lc[:, :, :40], causal=0,
          bf16_out=False, what="rows before the NaN key")


def test_empty_calls_touch_nothing():
    q, k, v = wl.attention_inputs(1, 1, 4, 8, 64, seed=1)
    qd, kd, vd = _dev(q), _dev(k), _dev(v)
    o = torch.full((1, 1, 0, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    rwo.attention_fwd(qd[:, :, :0], kd, vd, o)
    o2 = torch.full((0, 1, 4, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    rwo.attention_fwd(qd[:0], kd[:0], vd[:0], o2)
    torch.cuda.synchronize()


def test_repeat_calls_are_bit_identical():
    q, k, v = wl.attention_inputs(2, 2, 300, 500, 128, seed=31)
    a = run(q, k, v, causal=7)
    b = run(q, k, v, causal=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_graph_replay_matches_eager():
    q, k, v = wl.attention_inputs(1, 2, 256, 384, 128, seed=32)
    qd, kd, vd = _dev(q), _dev(k), _dev(v)
    o = torch.empty((1, 2, 256, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 2, 256), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call = rwo.prepare_attention(qd, kd, vd, o, lse=lse, stream=s)
        call()
    torch.cuda.synchronize()
    want_o, want_l = o.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        rwo.prepare_attention(qd, kd, vd, o, lse=lse,
                              stream=torch.cuda.current_stream())()
    for i in range(3):
        o.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, want_o) and torch.equal(lse, want_l), f"replay {i}"


# ---------------------------------------------------------------------------
# Full-size workloads (one head of 131072 x 131072): sampled query rows
# ---------------------------------------------------------------------------

def _sample_rows(Sq, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 127, 128, 4095, Sq // 2, Sq - 129, Sq - 1]
    return sorted(set(fixed) | set(rng.integers(0, Sq, 14).tolist()))


@pytest.mark.parametrize("D,causal", [(32, -1), (64, -1), (128, -1), (128, 0),
                                      (64, 1000)])
def test_4096_square_every_row(D, causal):
    # one head of 4096 queries x 4096 keys: 16 query blocks (8 workgroups
    # under the causal pairing) over 64 key tiles (32 at d = 32), every row
    # and every output element against the fp64 oracle, bf16 O
    q, k, v = wl.attention_inputs(1, 1, 4096, 4096, D, seed=4096 + D + causal)
    print(f"4096^2 every row D={D} causal={causal}", flush=True)
    o, lse = run(q, k, v, causal=causal)
    check(q, k, v, o, lse, causal=causal, what=f"4096^2 D{D} c{causal}")


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("causal", [-1, 0, 700])
def test_many_heads_medium_sampled(D, causal):
    # a grid of many workgroups over several (batch, head) pairs, a ragged
    # query count, more keys than queries, BSHD input and output layouts;
    # sampled rows of every (batch, head) against the oracle
    B, H, Sq, Sk = 2, 3, 2049, 3001
    q, k, v = wl.attention_inputs(B, H, Sq, Sk, D, seed=900 + D + causal,
                                  layout="bshd")
    print(f"many heads D={D} causal={causal}", flush=True)
    o, lse = run(q, k, v, causal=causal, out=torch.float32, o_layout="bshd")
    rows = [r for r in _sample_rows(Sq, D) if r < Sq]
    check(q, k, v, o, lse, causal=causal, bf16_out=False, rows=rows,
          what=f"many heads D{D} c{causal}")


def _all_rows_check(q, k, v, o, lse, causal, what, chunk=4096):
    """Every query row of head (0, 0) against the definition computed again
    in fp32 with torch on the GPU, in row chunks (scores, logsumexp,
    probabilities, P V).  The reference carries roundings of the same kinds
    as the kernel, so the tolerance is twice the bound of the module
    docstring, with Delta from the row's largest sum_c |q_c k_jc| and w
    from the largest |v| over the keys it admits.  This is a check of
    every row for gross errors (a wrong block, tile or head, an unwritten
    row); the fp64 oracle checks the sampled rows to the bound itself."""
    f32 = lambda a: torch.from_numpy(_w(a).astype(np.float32)).cuda()
    Q, K, V = f32(q[0, 0]), f32(k[0, 0]), f32(v[0, 0])
    O = torch.from_numpy(o[0, 0].astype(np.float32)).cuda()
    L = torch.from_numpy(lse[0, 0].astype(np.float32)).cuda()
    Sq, D = Q.shape
    Sk = K.shape[0]
    scale = 1.0 / math.sqrt(D)
    c = scale * LOG2E
    Kt, Kat = K.t().contiguous(), K.abs().t().contiguous()
    vabs = V.abs()
    wpre = torch.cummax(vabs, dim=0).values if causal >= 0 else None
    wall = vabs.max(dim=0).values
    cols = torch.arange(Sk, device="cuda")[None, :]
    n_acc = Sk / 16 + 2 * Sk / 64 + 64
    for r0 in range(0, Sq, chunk):
        r1 = min(Sq, r0 + chunk)
        S = (Q[r0:r1] @ Kt) * scale
        A = Q[r0:r1].abs() @ Kat
        if causal >= 0:
            rows = torch.arange(r0, r1, device="cuda")[:, None]
            masked = cols > rows + causal
            S.masked_fill_(masked, float("-inf"))
            A.masked_fill_(masked, 0.0)
            w = wpre[torch.clamp(torch.arange(r0, r1, device="cuda") + causal, max=Sk - 1)]
        else:
            w = wall[None, :].expand(r1 - r0, D)
        lref = torch.logsumexp(S, dim=1)
        oref = torch.exp(S - lref[:, None]) @ V
        del S
        amax = A.max(dim=1).values.double()
        del A
        dt = c * D * U * amax + 2 * torch.clamp(c * amax, min=1.0) * 2.0 ** -23
        delta = 2 * math.log(2) * dt
        tol_l = 2 * (delta + n_acc * U + 2 * lref.double().abs().clamp(min=1.0) * 2.0 ** -23)
        tol_o = 2 * ((2.0 ** -8 + 2 * delta[:, None] + n_acc * U) * w.double()
                     + 2.0 ** -8 * oref.double().abs())
        err_l = (L[r0:r1].double() - lref.double()).abs()
        err_o = (O[r0:r1].double() - oref.double()).abs()
        assert bool((err_l <= tol_l).all()), (
            f"{what}: lse off in rows {r0}..{r1}: worst {float(err_l.max()):.3g}")
        assert bool((err_o <= tol_o).all()), (
            f"{what}: o off in rows {r0}..{r1}: worst {float((err_o - tol_o).max()):.3g} past")


@pytest.mark.parametrize("name", ["a2", "a3", "a4", "a5"])
def test_full_size_sampled_rows(name):
    # the fp64 oracle on one row of every 256-row query block (every
    # workgroup's output; the row's place in its block varies) and the
    # sampled rows; every row against the fp32 re-computation below
    w = wl.ATTN_WORKLOADS[name]
    print(f"full size {name}: {w.desc}", flush=True)
    q, k, v = wl.attention_workload(name)
    o, lse = run(q, k, v, causal=w.causal)
    per_block = [b * 256 + (b * 37) % 256 for b in range(w.Sq // 256)]
    rows = sorted(set(_sample_rows(w.Sq, w.seed)) | set(per_block))
    check(q, k, v, o, lse, causal=w.causal, rows=rows, what=name)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    if w.causal == 0:                        # row 0 sees key 0 alone
        assert np.array_equal(o[0, 0, 0], _w(v[0, 0, 0]))
    _all_rows_check(q, k, v, o, lse, w.causal, name)
    if name == "a2":
        # the all-rows check has teeth: one wrong row of o, or of lse, fails it
        bad = o.copy()
        bad[0, 0, w.Sq // 3, 5] += 0.25
        with pytest.raises(AssertionError):
            _all_rows_check(q, k, v, bad, lse, w.causal, "planted o error")
        bad = lse.copy()
        bad[0, 0, 2 * w.Sq // 3] += 0.01
        with pytest.raises(AssertionError):
            _all_rows_check(q, k, v, o, bad, w.causal, "planted lse error")
