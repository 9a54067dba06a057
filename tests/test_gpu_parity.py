"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Every test calls the library via the ctypes binding on seeded inputs from
row_wise_online_amd.workloads and compares with oracle values computed
from the same stored bytes.  Shapes span several tiles and ragged tails;
each path is forced on every shape it accepts, in fp32 and bf16, with
16-byte-aligned and misaligned rows.
"""
import math
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import row_wise_online_amd as rw  # noqa: E402
from row_wise_online_amd import workloads as wl  # noqa: E402

from gpu_util import (check_d, check_lse, check_m, check_y, empty_like_rows,  # noqa: E402
                      to_device, to_host)


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rw.load()
    yield
    torch.cuda.synchronize()


def _run_fwd(x_host, path="auto", ld_y=None, stats=True):
    x = to_device(x_host)
    M, N = x.shape
    y = empty_like_rows(x, ld_y)
    z = lambda: torch.full((M,), float("nan"), device="cuda")
    m, d, lse = (z(), z(), z()) if stats else (None, None, None)
    rw.softmax_fwd(x, y, m=m, d=d, lse=lse, path=path)
    torch.cuda.synchronize()
    out = to_host(y)
    if stats:
        return out, m.cpu().numpy(), d.cpu().numpy(), lse.cpu().numpy()
    return out, None, None, None


def _check_all(x_host, res, what):
    y, m, d, lse = res
    y_ref, m_ref, d_ref, l_ref = oracle.softmax(x_host)
    check_y(y, y_ref, what)
    if m is not None:
        check_m(m, m_ref, what)
        check_d(d, d_ref, what)
        check_lse(lse, l_ref, what)


# ---------------------------------------------------------------------------
# Each path forced on shapes spanning tiles and ragged tails
# ---------------------------------------------------------------------------

SHAPES = [(3, 1), (5, 2), (7, 3), (4, 63), (4, 64), (4, 65), (9, 1000),
          (3, 1023), (3, 1025), (5, 4096), (2, 4097), (2, 8191), (3, 16385),
          (2, 32768)]
LONG_SHAPES = [(3, 20000), (2, 70001), (1, 300000)]


def _input(M, N, dtype, seed, misalign):
    # misaligned rows: an odd row stride, so 16-byte vectors are illegal
    ld = N + 1 if misalign else None
    return wl.normal(M, N, scale=3.0, seed=seed, dtype=dtype, ld=ld)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("misalign", [False, True])
@pytest.mark.parametrize("path", ["resident", "stream", "split"])
def test_paths_on_shapes(path, dtype, misalign):
    for i, (M, N) in enumerate(SHAPES + (LONG_SHAPES if path != "resident" else [])):
        what = f"{path} {dtype} misalign={misalign} M={M} N={N}"
        _say(what)
        x = _input(M, N, dtype, seed=100 + i, misalign=misalign)
        _check_all(x, _run_fwd(x, path), what)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_misaligned_base_column_window(dtype):
    # x starts one element into each row: the base pointer is misaligned
    full = wl.normal(6, 1500, scale=2.0, seed=7, dtype=dtype)
    xw = full[:, 1:]
    xd = to_device(full)[:, 1:]
    for path in ("resident", "stream", "split"):
        y = torch.empty((6, 1499), dtype=xd.dtype, device="cuda")
        rw.softmax_fwd(xd, y, path=path)
        torch.cuda.synchronize()
        y_ref, *_ = oracle.softmax(np.ascontiguousarray(xw))
        check_y(to_host(y), y_ref, f"window {path} {dtype}")


def test_padded_output_stride():
    x = wl.normal(5, 777, scale=2.0, seed=8)
    for path in ("resident", "stream", "split"):
        res = _run_fwd(x, path, ld_y=800)
        _check_all(x, res, f"ld_y {path}")


# ---------------------------------------------------------------------------
# The five workloads at full size, on the path the library picks
# ---------------------------------------------------------------------------

def _oracle_blocks(fn, x_host, rows=512):
    """Oracle results over blocks of rows (the oracle's fp64 outputs of a
    whole 16 x 4194304 matrix would take 512 MiB at once; blocks bound the
    host memory of each comparison)."""
    M = x_host.shape[0]
    for r0 in range(0, M, rows):
        yield r0, min(M, r0 + rows), fn(np.ascontiguousarray(x_host[r0:r0 + rows]))


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_workload_full_size(name):
    # every element of every row against the oracle, at the bench's launch
    w = wl.WORKLOADS[name]
    _say(f"workload {name}: {w.desc} path={rw.select_path(w.M, w.N, w.dtype)}")
    x_host = wl.generate(name)
    x = to_device(x_host)
    y = torch.empty_like(x)
    m = torch.empty(w.M, device="cuda")
    d = torch.empty(w.M, device="cuda")
    lse = torch.empty(w.M, device="cuda")
    rw.softmax_fwd(x, y, m=m, d=d, lse=lse)
    torch.cuda.synchronize()

    # properties over every row, as extra checks
    ysum = y.double().sum(dim=1).cpu().numpy()
    # each bf16 value is within one bf16 step (relative 2^-7) of the exact
    # value, so a row sum is within 2^-7 of 1; fp32 values are far closer
    tol = 2.0 ** -7 if w.dtype == "bf16" else 1e-4
    assert np.all(np.abs(ysum - 1.0) < tol), f"{name}: row sums"
    m_h = m.cpu().numpy()
    assert np.array_equal(m_h, x.float().max(dim=1).values.cpu().numpy())
    assert torch.isfinite(y).all()

    # the oracle on every row: y element by element, m, d and lse per row
    y_h = to_host(y)
    d_h, l_h = d.cpu().numpy(), lse.cpu().numpy()
    worst_abs, worst_rel = 0.0, 0.0
    bs = max(1, (1 << 22) // w.N)
    for r0, r1, (y_ref, m_ref, d_ref, l_ref) in _oracle_blocks(
            oracle.softmax, x_host, bs):
        what = f"{name} rows {r0}..{r1 - 1}"
        err = check_y(y_h[r0:r1], y_ref, what)
        worst_abs, worst_rel = max(worst_abs, err[0]), max(worst_rel, err[1])
        check_m(m_h[r0:r1], m_ref, what)
        check_d(d_h[r0:r1], d_ref, what)
        check_lse(l_h[r0:r1], l_ref, what)
        if name != "c4":
            # the workloads whose LSE stays below 128 meet the plain 1e-5
            assert np.all(np.abs(l_h[r0:r1] - l_ref) <= 1e-5), what
    _say(f"  {name}: all {w.M} rows; max abs err {worst_abs:.3e}, "
         f"max rel/ulp {worst_rel}")
    if name == "c5":
        cols = wl.planted_columns("c5")
        assert np.all(m_h == 20.0)
        assert np.all(np.argmax(y_h, axis=1) == cols)


# ---------------------------------------------------------------------------
# Statistics, column windows and the state merge
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("path", ["stream", "split"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_stats(path, dtype):
    for (M, N), inc in [((5, 1000), 1), ((3, 70001), 3), ((600, 130), 2),
                        ((2, 4096), 1)]:
        x_h = wl.normal(M, N, scale=4.0, seed=N, dtype=dtype)
        x = to_device(x_h)
        buf = torch.full((3, M * inc), float("nan"), device="cuda")
        rw.softmax_stats(x, buf[0], buf[1], buf[2], inc=inc, path=path)
        torch.cuda.synchronize()
        h = buf.cpu().numpy()[:, ::inc]
        _, m_ref, d_ref, l_ref = oracle.softmax(x_h, want_y=False)
        what = f"stats {path} {dtype} {M}x{N} inc={inc}"
        check_m(h[0], m_ref, what)
        check_d(h[1], d_ref, what)
        check_lse(h[2], l_ref, what)
        # untouched gaps between strided outputs
        if inc > 1:
            assert np.all(np.isnan(buf.cpu().numpy()[:, 1::inc]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_read_only_auto_streams_long_rows(dtype):
    # with many rows longer than 16384, AUTO streams the statistics (the
    # forward stays resident); the result equals the forced stream path
    M, N = 600, 20000
    assert rw.select_path(M, N, dtype, op="stats") == "stream"
    assert rw.select_path(M, N, dtype, op="cross_entropy") == "stream"
    assert rw.select_path(M, N, dtype) == "resident"
    x_h = wl.normal(M, N, scale=4.0, seed=21, dtype=dtype)
    x = to_device(x_h)
    auto = torch.empty((3, M), device="cuda")
    forced = torch.empty((3, M), device="cuda")
    rw.softmax_stats(x, auto[0], auto[1], auto[2])
    rw.softmax_stats(x, forced[0], forced[1], forced[2], path="stream")
    torch.cuda.synchronize()
    assert torch.equal(auto, forced)
    _, m_ref, d_ref, l_ref = oracle.softmax(x_h, want_y=False)
    h = auto.cpu().numpy()
    what = f"stats auto {dtype} {M}x{N}"
    check_m(h[0], m_ref, what)
    check_d(h[1], d_ref, what)
    check_lse(h[2], l_ref, what)


def test_column_windows_merge_to_row_state():
    # the state of each column window, merged, is the state of the row
    M, N, Wn = 7, 50000, 6
    x_h = wl.normal(M, N, scale=2.0, seed=9)
    x = to_device(x_h)
    edges = np.linspace(0, N, Wn + 1).astype(int)
    ms = torch.empty((M, Wn), device="cuda")
    ds = torch.empty((M, Wn), device="cuda")
    for k in range(Wn):
        a, b = edges[k], edges[k + 1]
        rw.softmax_stats(x[:, a:b], ms[:, k], ds[:, k], inc=Wn)
    mo = torch.empty(M, device="cuda")
    do = torch.empty(M, device="cuda")
    lo = torch.empty(M, device="cuda")
    rw.state_merge(ms, ds, mo, do, lo)
    torch.cuda.synchronize()
    _, m_ref, d_ref, l_ref = oracle.softmax(x_h, want_y=False)
    check_m(mo.cpu().numpy(), m_ref, "windows")
    check_d(do.cpu().numpy(), d_ref, "windows")
    check_lse(lo.cpu().numpy(), l_ref, "windows")


@pytest.mark.parametrize("K", [1, 5, 64, 65, 1000])
def test_state_merge_against_oracle(K):
    rng = np.random.default_rng(K)
    M = 37
    m_in = rng.uniform(-100.0, 100.0, (M, K)).astype(np.float32)
    d_in = rng.uniform(0.5, 1000.0, (M, K)).astype(np.float32)
    ident = rng.random((M, K)) < 0.2        # identity states (-inf, 0)
    m_in[ident] = -np.inf
    d_in[ident] = 0.0
    m_in[3, :] = -np.inf                    # a row of identities only
    d_in[3, :] = 0.0
    mo = torch.empty(M, device="cuda")
    do = torch.empty(M, device="cuda")
    lo = torch.empty(M, device="cuda")
    rw.state_merge(torch.from_numpy(m_in).cuda(), torch.from_numpy(d_in).cuda(),
                   mo, do, lo)
    torch.cuda.synchronize()
    m_ref, d_ref, l_ref = oracle.merge(m_in, d_in)
    mh, dh, lh = mo.cpu().numpy(), do.cpu().numpy(), lo.cpu().numpy()
    assert np.array_equal(mh.astype(np.float64), m_ref)
    fin = np.isfinite(m_ref)
    rel = np.abs(dh[fin] - d_ref[fin]) / d_ref[fin]
    assert rel.max() <= 1e-5
    assert dh[3] == 0.0 and mh[3] == -np.inf and lh[3] == -np.inf
    assert np.all(np.abs(lh[fin] - l_ref[fin]) <= 1e-5 + oracle.f32_ulp(l_ref[fin]))


def test_state_merge_strided_rows():
    M, K, ld = 9, 13, 20
    rng = np.random.default_rng(3)
    m_full = rng.uniform(-5, 5, (M, ld)).astype(np.float32)
    d_full = rng.uniform(1, 3, (M, ld)).astype(np.float32)
    m_full[:, K:] = np.nan                   # padding must not be read
    d_full[:, K:] = np.nan
    mo = torch.empty(M, device="cuda")
    do = torch.empty(M, device="cuda")
    rw.state_merge(torch.from_numpy(m_full).cuda()[:, :K],
                   torch.from_numpy(d_full).cuda()[:, :K], mo, do)
    torch.cuda.synchronize()
    m_ref, d_ref, _ = oracle.merge(m_full[:, :K], d_full[:, :K])
    assert np.array_equal(mo.cpu().numpy().astype(np.float64), m_ref)
    assert np.all(np.abs(do.cpu().numpy() - d_ref) / d_ref <= 1e-5)


# ---------------------------------------------------------------------------
# Edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("offset", [80.0, -80.0, 1e4, -1e4, 1e30, -1e30])
@pytest.mark.parametrize("path", ["resident", "stream", "split"])
def test_large_offsets(offset, path):
    x = wl.normal(4, 3000, scale=3.0, offset=offset, seed=11)
    res = _run_fwd(x, path)
    assert np.all(np.isfinite(res[0]))
    _check_all(x, res, f"offset {offset} {path}")


@pytest.mark.parametrize("path", ["resident", "stream", "split"])
def test_all_equal_and_single(path):
    for N, c in [(1, 5.0), (1000, -3.25), (4096, 80.0), (9999, 0.0)]:
        x = wl.from_values(np.full((3, N), c))
        y, m, d, lse = _run_fwd(x, path)
        assert np.all(np.abs(y.astype(np.float64) - 1.0 / N) <= 1e-6 + 1e-5 / N)
        assert np.all(m == np.float32(c))
        assert np.all(np.abs(d - N) <= 1e-5 * N)


@pytest.mark.parametrize("path", ["resident", "stream", "split"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_special_values(path, dtype):
    inf, nan = math.inf, math.nan
    N = 300
    rows = np.random.default_rng(4).standard_normal((5, N))
    rows[0, ::3] = -inf                     # masked elements
    rows[1, :] = -inf                       # fully masked row
    rows[2, 17] = nan                       # NaN element
    rows[3, 200] = inf                      # +inf element
    x = wl.from_values(rows, dtype=dtype)
    y, m, d, lse = _run_fwd(x, path)
    y_ref, m_ref, d_ref, l_ref = oracle.softmax(x)
    yf = y.astype(np.float64) if y.dtype == np.float32 else oracle.bf16_bits_to_f64(y)
    # masked row 0 behaves like the row without the masked elements
    check_y(y[0:1], y_ref[0:1], f"masked {path}")
    check_m(m[0:1], m_ref[0:1])
    check_d(d[0:1], d_ref[0:1])
    assert np.all(yf[0, ::3] == 0)
    # fully masked: m = -inf, d = 0, lse = -inf, y NaN
    assert m[1] == -inf and d[1] == 0 and lse[1] == -inf
    assert np.all(np.isnan(yf[1]))
    # NaN / +inf rows: NaN d, lse and y, as the oracle
    for r in (2, 3):
        assert np.isnan(d[r]) and np.isnan(lse[r]) and np.all(np.isnan(yf[r]))
        assert np.isnan(d_ref[r])
    assert m[2] == m_ref[2] and m[3] == inf
    check_y(y[4:5], y_ref[4:5], f"plain row {path}")


@pytest.mark.parametrize("path", ["resident", "stream", "split"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_in_place(path, dtype):
    x_h = wl.normal(6, 5000, scale=2.0, seed=12, dtype=dtype)
    x = to_device(x_h)
    rw.softmax_fwd(x, x, path=path)
    torch.cuda.synchronize()
    y_ref, *_ = oracle.softmax(x_h)
    check_y(to_host(x), y_ref, f"in place {path} {dtype}")


@pytest.mark.parametrize("path", ["resident", "stream", "split"])
def test_deterministic(path):
    x_h = wl.normal(64, 4096, seed=13)
    a = _run_fwd(x_h, path)
    b = _run_fwd(x_h, path)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint32), v.view(np.uint32))


def test_empty_rows_noop():
    x = torch.empty((0, 16), device="cuda")
    y = torch.empty((0, 16), device="cuda")
    rw.softmax_fwd(x, y)
    torch.cuda.synchronize()


def test_adversarial_order_small():
    # every element a new running max along the row
    x_h = wl.ascending(8, 32768, seed=14)
    for path in ("resident", "stream", "split"):
        _check_all(x_h, _run_fwd(x_h, path), f"ascending {path}")


@pytest.mark.parametrize("path", ["resident", "stream", "split"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_wide_range_rows_keep_subnormal_outputs(path, dtype):
    # rows spanning ~0 .. -95: e^(x - m) reaches below 2^-126, where bf16
    # still has subnormals down to 2^-133; bf16 outputs must stay within one
    # step there, fp32 outputs within the absolute tolerance
    rng = np.random.default_rng(15)
    N = 3000
    rows = -95.0 * rng.random((4, N))
    rows[:, 7] = 0.0
    rows[1] = np.sort(rows[1])          # ascending: every value a new max
    x = wl.from_values(rows, dtype=dtype)
    _check_all(x, _run_fwd(x, path), f"wide range {path} {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [17000, 32768])
def test_resident_row_loop_many_rows(dtype, N):
    # more rows than the persistent grid: workgroups walk 2-3 rows each with
    # the next row's loads in flight; check rows on both sides of the grid
    # stride and every row's sum
    M = 1100
    x_h = wl.normal(M, N, scale=2.0, seed=16, dtype=dtype)
    x = to_device(x_h)
    y = torch.empty_like(x)
    m = torch.empty(M, device="cuda")
    d = torch.empty(M, device="cuda")
    rw.softmax_fwd(x, y, m=m, d=d, path="resident")
    torch.cuda.synchronize()
    rows = np.array([0, 1, 511, 512, 513, 587, 1023, 1024, 1025, 1099])
    xs = np.ascontiguousarray(x_h[rows])
    y_ref, m_ref, d_ref, _ = oracle.softmax(xs)
    check_y(to_host(y[torch.as_tensor(rows, device="cuda")]), y_ref, "row loop")
    check_m(m.cpu().numpy()[rows], m_ref)
    check_d(d.cpu().numpy()[rows], d_ref)
    tol = 2.0 ** -7 if dtype == "bf16" else 1e-4
    assert np.all(np.abs(y.double().sum(dim=1).cpu().numpy() - 1.0) < tol)


# ---------------------------------------------------------------------------
# Log-softmax and cross-entropy
# ---------------------------------------------------------------------------

from gpu_util import check_log  # noqa: E402

LOG_SHAPES = [(3, 1), (7, 3), (4, 65), (9, 1000), (3, 1025), (5, 4096),
              (2, 8191), (2, 32768)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("misalign", [False, True])
@pytest.mark.parametrize("path", ["resident", "stream", "split"])
def test_log_softmax_paths(path, dtype, misalign):
    shapes = LOG_SHAPES + ([(3, 70001)] if path != "resident" else [])
    for i, (M, N) in enumerate(shapes):
        what = f"log {path} {dtype} misalign={misalign} {M}x{N}"
        _say(what)
        x_h = _input(M, N, dtype, seed=300 + i, misalign=misalign)
        x = to_device(x_h)
        y = empty_like_rows(x)
        lse = torch.empty(M, device="cuda")
        rw.log_softmax_fwd(x, y, lse=lse, path=path)
        torch.cuda.synchronize()
        check_log(to_host(y), oracle.log_softmax(x_h), what)
        _, _, _, l_ref = oracle.softmax(x_h, want_y=False)
        check_lse(lse.cpu().numpy(), l_ref, what)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_log_softmax_workloads(name):
    # every element of every row against the oracle
    w = wl.WORKLOADS[name]
    _say(f"log-softmax workload {name}: {w.desc}")
    x_h = wl.generate(name)
    x = to_device(x_h)
    y = torch.empty_like(x)
    rw.log_softmax_fwd(x, y)
    torch.cuda.synchronize()
    y_h = to_host(y)
    bs = max(1, (1 << 22) // w.N)
    for r0, r1, ref in _oracle_blocks(oracle.log_softmax, x_h, bs):
        check_log(y_h[r0:r1], ref, f"{name} rows {r0}..{r1 - 1}")


def _dominant_rows(M, N, seed):
    """Rows whose max term dominates: every other term below 2^-24 of it for
    most rows, so d rounds to 1 in fp32 and log d to 0 unless d - 1 is kept
    apart.  Row 0: others near -20 (d - 1 ~ 1e-5 N); rows 1, 2: near -25
    and -32; row 3: two maxima (d >= 2); row 4: every other element -inf
    (d = 1 exactly); row 5 onwards: normals."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((M, N))
    for i, off in enumerate([-20.0, -25.0, -32.0, -25.0]):
        v[i] = v[i] * 0.5 + off
    v[4, :] = -np.inf
    cols = rng.integers(0, N, size=M)
    for i in range(5):
        v[i, cols[i]] = 0.0
    v[3, (cols[3] + N // 2) % N] = 0.0
    return v, cols


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("path", ["resident", "stream", "split"])
def test_log_probabilities_near_zero(path, dtype):
    # the max element's log-probability, -log1p(d - 1) ~ -1e-8, and the
    # log-softmax's log-sum-exp - m keep full relative precision: within
    # one bf16 step (bf16) and 1e-5 relative (fp32), where log d of a
    # rounded d would give 0; the cross-entropy and statistics on the same
    # rows meet their absolute fp32 bar
    shapes = [(6, 3000), (6, 20000)] if path == "resident" else \
        [(6, 3000), (6, 70001)]
    for M, N in shapes:
        what = f"near 0 {path} {dtype} {M}x{N}"
        _say(what)
        v, cols = _dominant_rows(M, N, seed=N)
        x_h = wl.from_values(v, dtype=dtype)
        x = to_device(x_h)
        y = torch.empty_like(x)
        m = torch.empty(M, device="cuda")
        lse = torch.empty(M, device="cuda")
        rw.log_softmax_fwd(x, y, m=m, lse=lse, path=path)
        labels = torch.from_numpy(cols.astype(np.int64)).cuda()
        loss = torch.empty(M, device="cuda")
        lse2 = torch.empty(M, device="cuda")
        rw.cross_entropy_fwd(x, labels, loss, lse=lse2, path=path)
        sm, sd, sl = (torch.empty(M, device="cuda") for _ in range(3))
        rw.softmax_stats(x, sm, sd, sl, path=path)
        torch.cuda.synchronize()
        ref = oracle.log_softmax(x_h)
        y_h = to_host(y)
        check_log(y_h, ref, what)
        l_ref, _ = oracle.cross_entropy(x_h, cols)
        check_log(loss.cpu().numpy(), l_ref, what)
        # the max element's log-probability in closed form: -log1p(s), s the
        # sum of every other term e^(x_j - m) taken apart from the max's 1
        # (fp64, relative error below N 2^-53).  The oracle's d = 1 + s
        # summed whole carries an absolute error up to N 2^-53, too coarse
        # for a relative check of values near 1e-11.
        xf = (x_h.astype(np.float64) if dtype == "f32"
              else oracle.bf16_bits_to_f64(x_h))
        mx = xf.max(axis=1)
        terms = np.exp(xf - mx[:, None])
        rows = np.arange(5)              # the rows whose max sits at cols
        mx = mx[rows]
        terms = terms[rows]
        terms[rows, cols[rows]] = 0.0
        s_apart = terms.sum(axis=1)
        top = -np.log1p(s_apart)
        assert np.all(mx == 0.0)
        yf = (y_h.astype(np.float64) if dtype == "f32"
              else oracle.bf16_bits_to_f64(y_h))
        got = yf[rows, cols[rows]]
        if dtype == "f32":
            assert np.all(np.abs(got - top) <= 1e-5 * np.abs(top)), (got, top)
        else:
            want = oracle.round_f64_to_bf16_bits(top)
            assert np.all(oracle.bf16_ulp_distance(y_h[rows, cols[rows]],
                                                   want) <= 1), what
        # log-softmax's lse - m is log1p(s): 1e-5 relative
        lh = lse.cpu().numpy().astype(np.float64)[rows]
        assert np.all(np.abs((lh - mx) - (-top)) <= 1e-5 * np.abs(top)), what
        # the cross-entropy and the statistics keep d: their fp32 bar is
        # absolute (1e-5 plus fp32 rounding)
        _, _, _, l2_ref = oracle.softmax(x_h, want_y=False)
        check_lse(lse2.cpu().numpy(), l2_ref, what)
        check_lse(sl.cpu().numpy(), l2_ref, what)


@pytest.mark.parametrize("path", ["resident", "stream", "split"])
def test_log_softmax_special_values_and_in_place(path):
    inf, nan = math.inf, math.nan
    rows = np.random.default_rng(7).standard_normal((4, 500))
    rows[0, ::4] = -inf
    rows[1, :] = -inf
    rows[2, 3] = nan
    x_h = wl.from_values(rows)
    x = to_device(x_h)
    y = torch.empty_like(x)
    rw.log_softmax_fwd(x, y, path=path)
    torch.cuda.synchronize()
    check_log(to_host(y), oracle.log_softmax(x_h), f"log special {path}")
    rw.log_softmax_fwd(x, x, path=path)            # in place
    torch.cuda.synchronize()
    check_log(to_host(x), oracle.log_softmax(x_h), f"log in place {path}")


def _labels(M, N, seed):
    rng = np.random.default_rng(seed)
    lab = rng.integers(0, N, size=M).astype(np.int64)
    if M > 4:
        lab[1] = -100          # ignored
        lab[3] = N - 1         # last column
        lab[4] = 0             # first column
    return lab


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("misalign", [False, True])
@pytest.mark.parametrize("path", ["resident", "stream", "split"])
def test_cross_entropy_paths(path, dtype, misalign):
    shapes = [(9, 1000), (6, 63), (5, 4096), (3, 16385), (7, 32768)]
    if path != "resident":
        shapes += [(3, 70001)]
    for i, (M, N) in enumerate(shapes):
        what = f"ce {path} {dtype} misalign={misalign} {M}x{N}"
        _say(what)
        x_h = _input(M, N, dtype, seed=400 + i, misalign=misalign)
        lab = _labels(M, N, 400 + i)
        x = to_device(x_h)
        labels = torch.from_numpy(lab).cuda()
        loss = torch.full((M,), float("nan"), device="cuda")
        lse = torch.empty(M, device="cuda")
        mean = torch.empty(1, device="cuda")
        rw.cross_entropy_fwd(x, labels, loss, lse=lse, mean=mean, path=path)
        torch.cuda.synchronize()
        l_ref, mean_ref = oracle.cross_entropy(x_h, lab)
        check_log(loss.cpu().numpy(), l_ref, what)
        _, _, _, lse_ref = oracle.softmax(x_h, want_y=False)
        check_lse(lse.cpu().numpy(), lse_ref, what)
        assert abs(mean.item() - mean_ref) <= 1e-5 + 1e-5 * abs(mean_ref), what


def test_cross_entropy_label_edge_cases():
    M, N = 6, 300
    x_h = wl.normal(M, N, scale=2.0, seed=17)
    x = to_device(x_h)
    for lab, note in [(np.array([-1, -100, -1, -5, -1, -1]), "all ignored"),
                      (np.array([0, N, 5, -1, 7, 2]), "one out of range")]:
        labels = torch.from_numpy(lab.astype(np.int64)).cuda()
        for path in ("resident", "stream", "split"):
            loss = torch.empty(M, device="cuda")
            mean = torch.empty(1, device="cuda")
            rw.cross_entropy_fwd(x, labels, loss, mean=mean, path=path)
            torch.cuda.synchronize()
            l_ref, mean_ref = oracle.cross_entropy(x_h, lab)
            check_log(loss.cpu().numpy(), l_ref, f"{note} {path}")
            assert np.isnan(mean.item()) and np.isnan(mean_ref), note


@pytest.mark.parametrize("M", [1, 3, 4, 5, 4095, 4097, 32771, 70001])
@pytest.mark.parametrize("offset", [0, 1])
def test_cross_entropy_mean_shapes(M, offset):
    # the mean over row counts around the 4-row groups and the kernel's
    # batch of 1024 x 4 x 8 rows, with loss and labels 16-byte aligned
    # (offset 0) or one element off (offset 1: one row at a time); the
    # oracle's mean over its own losses
    N = 40
    x_h = wl.normal(M, N, scale=2.0, seed=26 + M)
    lab = np.random.default_rng(M).integers(-2, N, size=M).astype(np.int64)
    x = to_device(x_h)
    lab_d = torch.empty(M + offset, dtype=torch.int64, device="cuda")
    lab_d[offset:] = torch.from_numpy(lab).cuda()
    loss = torch.empty(M + offset, device="cuda")
    mean = torch.empty(1, device="cuda")
    rw.cross_entropy_fwd(x, lab_d[offset:], loss[offset:], mean=mean)
    torch.cuda.synchronize()
    l_ref, mean_ref = oracle.cross_entropy(x_h, lab)
    check_log(loss[offset:].cpu().numpy(), l_ref, f"loss M={M}")
    if np.isnan(mean_ref):
        assert np.isnan(mean.item())
    else:
        # fp32 sums of up to 70001 losses of about 4: relative 1e-5
        assert abs(mean.item() - mean_ref) <= 1e-5 * abs(mean_ref), (mean.item(), mean_ref)


@pytest.mark.parametrize("path", ["resident", "stream", "split"])
def test_cross_entropy_ignored_rows_marked_by_negative_zero(path):
    # ignored rows carry -0.0 (equal to 0); a row whose loss is exactly +0
    # (label on the max, every other term below 2^-24 of it) still counts
    # in the mean, which is taken over the losses alone
    M, N = 7, 300
    v = np.random.default_rng(27).standard_normal((M, N))
    v[3, :] = -200.0
    v[3, 5] = 0.0
    x_h = wl.from_values(v)
    lab = np.array([4, -1, 10, 5, -7, 0, -1], np.int64)
    x = to_device(x_h)
    mean = torch.empty(1, device="cuda")
    loss = rw.cross_entropy_fwd(x, torch.from_numpy(lab).cuda(), mean=mean,
                                path=path)
    torch.cuda.synchronize()
    bits = loss.cpu().numpy().view(np.uint32)
    assert np.all(bits[lab < 0] == 0x80000000)
    assert bits[3] == 0 and np.all(bits[lab >= 0] != 0x80000000)
    l_ref, mean_ref = oracle.cross_entropy(x_h, lab)
    check_log(loss.cpu().numpy(), l_ref, f"ignored rows {path}")
    assert abs(mean.item() - mean_ref) <= 1e-6 * abs(mean_ref)


def test_cross_entropy_worked_example():
    # "从原始Softmax到在线Softmax": logits [2, 1, 0.1], class 0 -> loss 0.4170
    x = torch.tensor([[2.0, 1.0, 0.1]], device="cuda")
    labels = torch.tensor([0], dtype=torch.int64, device="cuda")
    mean = torch.empty(1, device="cuda")
    loss = rw.cross_entropy_fwd(x, labels, mean=mean)
    torch.cuda.synchronize()
    assert abs(loss.item() - 0.4170) <= 5e-5
    assert abs(mean.item() - 0.4170) <= 5e-5


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_cross_entropy_workloads(name):
    # the loss of every row against the oracle
    w = wl.WORKLOADS[name]
    _say(f"cross-entropy workload {name}: {w.desc}")
    x_h = wl.generate(name)
    lab = _labels(w.M, w.N, 18)
    x = to_device(x_h)
    labels = torch.from_numpy(lab).cuda()
    mean = torch.empty(1, device="cuda")
    loss = rw.cross_entropy_fwd(x, labels, mean=mean)
    torch.cuda.synchronize()
    l_ref, mean_ref = oracle.cross_entropy(x_h, lab)
    check_log(loss.cpu().numpy(), l_ref, name)
    assert abs(mean.item() - mean_ref) <= 1e-5 * abs(mean_ref), name
    # the mean against the device losses summed in fp64 (order-free check)
    lh = loss.cpu().numpy().astype(np.float64)
    keep = lab >= 0
    assert abs(mean.item() - lh[keep].mean()) <= 1e-5 * abs(lh[keep].mean())


# ---------------------------------------------------------------------------
# Masked rows: valid lengths and causal offsets
# ---------------------------------------------------------------------------

def _lengths(M, N, seed):
    rng = np.random.default_rng(seed)
    rl = rng.integers(0, N + 1, size=M).astype(np.int32)
    rl[0] = 0                      # fully masked row
    if M > 1:
        rl[1] = N + 100            # longer than the row: no mask
    if M > 2:
        rl[2] = -7                 # negative: fully masked
    if M > 3:
        rl[3] = 1
    return rl


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("path", ["resident", "stream", "split"])
def test_masked_paths(path, dtype):
    shapes = [(7, 65), (9, 1000), (6, 4096), (5, 8191), (5, 32768)]
    if path != "resident":
        shapes += [(5, 70001)]
    for i, (M, N) in enumerate(shapes):
        for misalign in (False, True):
            x_h = _input(M, N, dtype, seed=500 + i, misalign=misalign)
            x = to_device(x_h)
            for case, (rl, causal) in enumerate([
                    (_lengths(M, N, 500 + i), None),
                    (None, 0), (None, N // 3),
                    (_lengths(M, N, 600 + i), N // 2)]):
                what = (f"masked {path} {dtype} {M}x{N} misalign={misalign} "
                        f"case={case}")
                rl_t = None if rl is None else torch.from_numpy(rl).cuda()
                y = empty_like_rows(x)
                ly = empty_like_rows(x)
                m = torch.empty(M, device="cuda")
                d = torch.empty(M, device="cuda")
                lse = torch.empty(M, device="cuda")
                rw.softmax_fwd(x, y, m=m, d=d, lse=lse, path=path,
                               row_len=rl_t, causal=causal)
                rw.log_softmax_fwd(x, ly, path=path, row_len=rl_t,
                                   causal=causal)
                torch.cuda.synchronize()
                y_ref, ly_ref, m_ref, d_ref, l_ref = oracle.softmax_masked(
                    x_h, rl, -1 if causal is None else causal)
                yh = to_host(y)
                ok = ~np.isnan(y_ref[:, 0])          # rows with columns
                yf = yh.astype(np.float64) if yh.dtype == np.float32 else \
                    oracle.bf16_bits_to_f64(yh)
                assert np.all(np.isnan(yf[~ok])), what
                check_y(yh[ok], y_ref[ok], what)
                check_log(to_host(ly), ly_ref, what)
                mh, dh, lh = m.cpu().numpy(), d.cpu().numpy(), lse.cpu().numpy()
                check_m(mh, m_ref, what)
                assert np.all(dh[~ok] == 0) and np.all(lh[~ok] == -np.inf), what
                check_d(dh[ok], d_ref[ok], what)
                check_lse(lh[ok], l_ref[ok], what)


@pytest.mark.parametrize("path", ["resident", "stream", "split"])
def test_masked_in_place_and_reads(path):
    # masked columns are never read: NaN there must not leak into the row
    M, N = 6, 3000
    v = np.random.default_rng(19).standard_normal((M, N)) * 2.0
    rl = np.array([3000, 2999, 1500, 1, 64, 0], np.int32)
    for i, n in enumerate(rl):
        v[i, n:] = np.nan
    x_h = wl.from_values(v)
    x = to_device(x_h)
    rw.softmax_fwd(x, x, path=path, row_len=torch.from_numpy(rl).cuda())
    torch.cuda.synchronize()
    y_ref, *_ = oracle.softmax_masked(x_h, rl)
    yh = to_host(x)
    check_y(yh[:5], y_ref[:5], f"masked in place {path}")
    assert np.all(np.isnan(yh[5]))


@pytest.mark.parametrize("path", ["resident", "stream", "split"])
def test_causal_offset_beyond_the_row_is_no_mask(path):
    # an offset of N - 1 or more admits every column of every row, up to the
    # largest int64 (where row + offset would not fit without the clamp)
    M, N = 40, 3000
    x_h = wl.normal(M, N, scale=2.0, seed=77)
    x = to_device(x_h)
    y_ref, *_ = oracle.softmax(x_h)
    for off in (N - 1, N, 2 ** 40, 2 ** 63 - 1):
        y = rw.softmax_fwd(x, path=path, causal=off)
        ly = rw.log_softmax_fwd(x, path=path, causal=off)
        torch.cuda.synchronize()
        check_y(to_host(y), y_ref, f"causal {off} {path}")
        check_log(to_host(ly), oracle.log_softmax(x_h), f"log causal {off} {path}")


# ---------------------------------------------------------------------------
# Streaming statistics: windows folded into a running state
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("path", ["auto", "resident", "stream", "split"])
def test_stats_update_streams_windows(path, dtype):
    M, N = 9, 40000
    x_h = wl.normal(M, N, scale=3.0, seed=21, dtype=dtype)
    x = to_device(x_h)
    rng = np.random.default_rng(21)
    cuts = np.sort(rng.choice(np.arange(1, N), size=7, replace=False))
    edges = [0, *cuts.tolist(), N]
    inc = 2
    m = torch.full((M * inc,), float("-inf"), device="cuda")
    d = torch.zeros(M * inc, device="cuda")
    lse = torch.empty(M * inc, device="cuda")
    for a, b in zip(edges[:-1], edges[1:]):
        p = path
        if path == "resident" and b - a > 32768:
            p = "stream"
        rw.softmax_stats_update(x[:, a:b], m, d, lse, inc=inc, path=p)
    torch.cuda.synchronize()
    _, m_ref, d_ref, l_ref = oracle.softmax(x_h, want_y=False)
    what = f"stream windows {path} {dtype}"
    check_m(m.cpu().numpy()[::inc], m_ref, what)
    check_d(d.cpu().numpy()[::inc], d_ref, what)
    check_lse(lse.cpu().numpy()[::inc], l_ref, what)


def test_stats_update_from_identity_equals_stats():
    x_h = wl.normal(33, 2000, scale=2.0, seed=22)
    x = to_device(x_h)
    m = torch.full((33,), float("-inf"), device="cuda")
    d = torch.zeros(33, device="cuda")
    rw.softmax_stats_update(x, m, d)
    m2 = torch.empty(33, device="cuda")
    d2 = torch.empty(33, device="cuda")
    rw.softmax_stats(x, m2, d2)
    torch.cuda.synchronize()
    # merging into the identity leaves the window state unchanged
    assert torch.equal(m, m2) and torch.equal(d, d2)


# ---------------------------------------------------------------------------
# Pass 2 alone with a held row state: column windows normalised with the
# state merged from their statistics
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,N", [(9, 40000), (3000, 700), (5, 300001), (1, 1)])
def test_windows_normalized_with_the_row_state(M, N, dtype):
    # the statistics of random column windows (some starting off the 16-byte
    # grid) merged into one state per row, then each window normalised with
    # it: together they are the row's softmax and log-softmax
    x_h = wl.normal(M, N, scale=3.0, seed=24, dtype=dtype)
    x = to_device(x_h)
    rng = np.random.default_rng(24)
    cuts = sorted(rng.choice(np.arange(1, N), size=min(6, N - 1),
                             replace=False).tolist()) if N > 1 else []
    edges = [0, *cuts, N]
    inc = 2
    m = torch.full((M * inc,), float("-inf"), device="cuda")
    d = torch.zeros(M * inc, device="cuda")
    for a, b in zip(edges[:-1], edges[1:]):
        rw.softmax_stats_update(x[:, a:b], m, d, inc=inc)
    y = torch.full_like(x, float("nan"))
    ly = torch.full_like(x, float("nan"))
    for a, b in zip(edges[:-1], edges[1:]):
        rw.softmax_normalize(x[:, a:b], m, d, y[:, a:b], inc=inc)
        rw.softmax_normalize(x[:, a:b], m, d, ly[:, a:b], inc=inc, log=True)
    torch.cuda.synchronize()
    what = f"normalize {M}x{N} {dtype} windows {edges}"
    y_ref, m_ref, d_ref, _ = oracle.softmax(x_h)
    check_m(m[0::inc].cpu().numpy(), m_ref, what)
    check_d(d[0::inc].cpu().numpy(), d_ref, what)
    check_y(to_host(y), y_ref, what)
    # the log form of pass 2 for the fp32 state it was given: its exact
    # value for that state (log d of an fp32 d is what a held state fixes)
    mh, dh = m[0::inc].cpu().numpy(), d[0::inc].cpu().numpy()
    check_log(to_host(ly), oracle.normalize(x_h, mh, dh, log=True), what)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_normalize_in_place_and_special_rows(dtype):
    # in place, with the state from os_softmax_stats; a row of only -inf
    # (state (-inf, 0)) comes out NaN, as from the full softmax
    M, N = 6, 5000
    v = np.random.default_rng(25).standard_normal((M, N)) * 2.0
    v[2, :] = -np.inf
    v[4, 100:] = -np.inf
    x_h = wl.from_values(v, dtype=dtype)
    x = to_device(x_h)
    m = torch.empty(M, device="cuda")
    d = torch.empty(M, device="cuda")
    rw.softmax_stats(x, m, d)
    rw.softmax_normalize(x, m, d, x)
    torch.cuda.synchronize()
    y_ref, *_ = oracle.softmax(x_h)
    yh = to_host(x)
    keep = [0, 1, 3, 4, 5]
    check_y(yh[keep], y_ref[keep], f"normalize in place {dtype}")
    yf = yh.astype(np.float64) if dtype == "f32" else oracle.bf16_bits_to_f64(yh)
    assert np.all(np.isnan(yf[2]))


# ---------------------------------------------------------------------------
# Host threads and streams: the library keeps no host state, so concurrent
# calls from several threads, each on its own stream, give the bits of the
# same calls made one after another
# ---------------------------------------------------------------------------

def test_concurrent_threads_and_streams():
    import threading
    shapes = [(300, 5000, "f32", "split"), (700, 1000, "bf16", "resident"),
              (64, 40000, "f32", "stream"), (2000, 4096, "f32", "auto")]
    xs = [to_device(wl.normal(M, N, scale=2.0, seed=30 + i, dtype=dt))
          for i, (M, N, dt, _) in enumerate(shapes)]

    def work(i, stream, reps):
        M, N, dt, path = shapes[i]
        x = xs[i]
        with torch.cuda.stream(stream):
            m = torch.empty(M, device="cuda")
            d = torch.empty(M, device="cuda")
            ws = torch.empty(max(rw.workspace_bytes(M, N, x.dtype, path), 1),
                             dtype=torch.uint8, device="cuda")
            y = torch.empty_like(x)
            for _ in range(reps):
                rw.softmax_fwd(x, y, m=m, d=d, ws=ws, path=path, stream=stream)
                z = rw.softmax_normalize(x, m, d, stream=stream)
        return y, m, d, z

    # one after another on the default stream
    want = [work(i, torch.cuda.current_stream(), 1) for i in range(len(shapes))]
    torch.cuda.synchronize()
    got = [None] * len(shapes)
    streams = [torch.cuda.Stream() for _ in shapes]

    def run(i):
        got[i] = work(i, streams[i], 20)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(shapes))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        for a, b in zip(got[i], want[i]):
            assert torch.equal(a, b), f"thread {i} ({shapes[i]}) differs"


def test_binding_allocations_follow_the_launch_stream():
    # stream= given outside any stream context, with the workspace and the
    # outputs left to the binding: what it allocates belongs to the launch
    # stream, so blocks the current stream allocates and fills while the
    # launch stream is still busy (a bounded spin kernel) cannot be the
    # call's workspace or outputs.  Every result must equal the same call
    # made on the current stream.
    M, N = 16, 300000            # AUTO takes the split path: a workspace
    assert rw.select_path(M, N, "f32") == "split"
    assert rw.select_path(M, N, "f32", op="stats") == "split"
    x = to_device(wl.normal(M, N, scale=2.0, seed=31))
    lab = torch.from_numpy(_labels(M, N, 31)).cuda()
    want_y = rw.softmax_fwd(x)
    want_l = rw.cross_entropy_fwd(x, lab)
    want_m, want_d = torch.empty(M, device="cuda"), torch.empty(M, device="cuda")
    rw.softmax_stats(x, want_m, want_d)
    torch.cuda.synchronize()
    need = rw.workspace_bytes(M, N, "f32")
    s = torch.cuda.Stream()
    got = []
    for _ in range(3):
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            torch.cuda._sleep(5_000_000)
        m, d = torch.empty(M, device="cuda"), torch.empty(M, device="cuda")
        s.wait_stream(torch.cuda.current_stream())
        y = rw.softmax_fwd(x, stream=s)
        loss = rw.cross_entropy_fwd(x, lab, stream=s)
        rw.softmax_stats(x, m, d, stream=s)
        junk = [torch.full((need // 4 + 64,), float("nan"), device="cuda")
                for _ in range(4)]
        junk.append(torch.full_like(x, float("nan")))
        got.append((y, loss, m, d))
        del junk
    torch.cuda.synchronize()
    for y, loss, m, d in got:
        assert torch.equal(y, want_y)
        assert torch.equal(loss, want_l)
        assert torch.equal(m, want_m) and torch.equal(d, want_d)


# ---------------------------------------------------------------------------
# HIP graph replay: the row ops captured once, replayed on new inputs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("path", ["resident", "stream", "split"])
def test_graph_replay_rows(path):
    # softmax with its statistics, log-softmax, statistics alone and the
    # cross-entropy with its mean (two launches), captured in one graph;
    # each replay runs on inputs written eagerly just before it and must
    # give the bits of the same calls made eagerly
    M, N = 300, 5000
    x = torch.empty(M, N, device="cuda")
    labels = torch.empty(M, dtype=torch.int64, device="cuda")
    outs = dict(y=torch.empty(M, N, device="cuda"),
                ly=torch.empty(M, N, device="cuda"),
                m=torch.empty(M, device="cuda"), d=torch.empty(M, device="cuda"),
                lse=torch.empty(M, device="cuda"),
                sm=torch.empty(M, device="cuda"), sd=torch.empty(M, device="cuda"),
                loss=torch.empty(M, device="cuda"),
                mean=torch.empty(1, device="cuda"))
    need = max(rw.workspace_bytes(M, N, torch.float32, path), 1)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def calls(stream):
        o = outs
        return [rw.prepare_fwd(x, o["y"], m=o["m"], d=o["d"], lse=o["lse"],
                               ws=ws, path=path, stream=stream),
                rw.prepare_fwd(x, o["ly"], ws=ws, path=path, stream=stream,
                               log=True),
                rw.prepare_stats(x, o["sm"], o["sd"], ws=ws, path=path,
                                 stream=stream),
                rw.prepare_cross_entropy(x, labels, o["loss"], mean=o["mean"],
                                         ws=ws, path=path, stream=stream)]

    def inputs(seed):
        x.copy_(torch.from_numpy(wl.normal(M, N, scale=3.0, seed=seed)))
        labels.copy_(torch.from_numpy(_labels(M, N, seed)))

    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    inputs(70)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        for c in calls(torch.cuda.current_stream()):
            c()
    eager = calls(None)
    for i, seed in enumerate((71, 72, 73)):
        inputs(seed)
        for c in eager:
            c()
        torch.cuda.synchronize()
        want = {k: v.clone() for k, v in outs.items()}
        for v in outs.values():
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v, want[k]) or (
                torch.isnan(v).equal(torch.isnan(want[k]))
                and torch.equal(v.nan_to_num(), want[k].nan_to_num())), \
                f"replay {i} ({path}): {k} differs from the eager call"
        # and the eager result is the oracle's
        if i == 0:
            x_h = wl.normal(M, N, scale=3.0, seed=seed)
            y_ref, m_ref, d_ref, l_ref = oracle.softmax(x_h)
            check_y(want["y"].cpu().numpy(), y_ref, f"graph {path}")
            check_m(want["m"].cpu().numpy(), m_ref, f"graph {path}")
            check_lse(want["lse"].cpu().numpy(), l_ref, f"graph {path}")
