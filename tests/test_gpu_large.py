"""Problems larger than one launch: a dispatch counts its grid in 32-bit
work-items, so row calls of more than 2^22 rows and attention calls of more
than 2^22 workgroups are issued in parts.  These cases put part boundaries
inside the problem and compare every row (or sampled heads, including those
on each side of a boundary) with the fp64 oracle.  A per-row pointer left
unmoved, or a causal offset not taken relative to the part, shows up in the
rows after a boundary."""
import numpy as np
import pytest
import torch

import oracle
import row_wise_online_amd as rw
from row_wise_online_amd import workloads as wl
from gpu_util import check_d, check_log, check_lse, check_m, check_y, to_device, to_host
import test_gpu_attention as ta

pytestmark = [pytest.mark.gpu,
              pytest.mark.filterwarnings("ignore::RuntimeWarning")]

LIMIT = 1 << 22           # rows / attention workgroups per launch
M_BIG = LIMIT + 3         # two parts of 2097154 and 2097153 rows
EDGE = (M_BIG + 1) // 2   # first row of the second part
N = 8


def _x(seed, dtype="f32"):
    return wl.normal(M_BIG, N, scale=3.0, seed=seed, dtype=dtype)


@pytest.mark.parametrize("path", ["resident", "stream", "split"])
def test_softmax_rows_beyond_one_launch(path):
    x_h = _x(900)
    x = to_device(x_h)
    m, d, lse = (torch.empty(M_BIG, device="cuda") for _ in range(3))
    print(f"softmax {M_BIG}x{N} path={path}", flush=True)
    y = rw.softmax_fwd(x, m=m, d=d, lse=lse, path=path)
    torch.cuda.synchronize()
    y_ref, m_ref, d_ref, l_ref = oracle.softmax(x_h)
    what = f"softmax {path}"
    check_y(to_host(y), y_ref, what)
    check_m(m.cpu().numpy(), m_ref, what)
    check_d(d.cpu().numpy(), d_ref, what)
    check_lse(lse.cpu().numpy(), l_ref, what)


@pytest.mark.parametrize("path", ["resident", "stream", "split"])
def test_masked_rows_beyond_one_launch(path):
    # lengths per row and causal offset 0: row i keeps min(len_i, i + 1)
    # columns, so the first rows of the problem are masked by the offset and
    # the rows after the part boundary are not
    x_h = _x(901, "bf16")
    rl = np.random.default_rng(5).integers(-1, N + 2, size=M_BIG).astype(np.int32)
    rl[EDGE:EDGE + 8] = N
    x = to_device(x_h)
    print(f"masked log-softmax {M_BIG}x{N} path={path}", flush=True)
    ly = rw.log_softmax_fwd(x, path=path, row_len=torch.from_numpy(rl).cuda(),
                            causal=0)
    torch.cuda.synchronize()
    _, ly_ref, _, _, _ = oracle.softmax_masked(x_h, rl, 0)
    check_log(to_host(ly), ly_ref, f"masked {path}")


def test_cross_entropy_rows_beyond_one_launch():
    x_h = _x(902)
    lab = np.random.default_rng(6).integers(-1, N, size=M_BIG).astype(np.int64)
    x = to_device(x_h)
    mean = torch.empty(1, device="cuda")
    print(f"cross-entropy {M_BIG}x{N}", flush=True)
    loss = rw.cross_entropy_fwd(x, torch.from_numpy(lab).cuda(), mean=mean,
                                path="resident")
    torch.cuda.synchronize()
    l_ref, _ = oracle.cross_entropy(x_h, lab)
    check_log(loss.cpu().numpy(), l_ref, "cross-entropy")
    keep = lab >= 0
    assert abs(mean.item() - l_ref[keep].mean()) <= 1e-5 * abs(l_ref[keep].mean())


def test_stats_update_strided_beyond_one_launch():
    # statistics at index row * 2, merged into a running state in place
    x_h = _x(903)
    x = to_device(x_h)
    m = torch.full((2 * M_BIG,), float("-inf"), device="cuda")
    d = torch.zeros(2 * M_BIG, device="cuda")
    print(f"stats update {M_BIG}x{N} inc=2", flush=True)
    rw.softmax_stats_update(x[:, :3], m, d, inc=2, path="stream")
    rw.softmax_stats_update(x[:, 3:], m, d, inc=2, path="stream")
    torch.cuda.synchronize()
    _, m_ref, d_ref, _ = oracle.softmax(x_h, want_y=False)
    mh, dh = m.cpu().numpy(), d.cpu().numpy()
    check_m(mh[0::2], m_ref, "stats update m")
    check_d(dh[0::2], d_ref, "stats update d")
    assert np.all(mh[1::2] == -np.inf) and np.all(dh[1::2] == 0)


def test_normalize_rows_beyond_one_launch():
    # the state of each row at index row * 2, from the statistics entry
    # point, then pass 2 alone over all rows
    x_h = _x(905, "bf16")
    x = to_device(x_h)
    m = torch.empty(2 * M_BIG, device="cuda")
    d = torch.empty(2 * M_BIG, device="cuda")
    print(f"normalize {M_BIG}x{N} inc=2", flush=True)
    rw.softmax_stats(x, m, d, inc=2)
    y = rw.softmax_normalize(x, m, d, inc=2)
    ly = rw.softmax_normalize(x, m, d, inc=2, log=True)
    torch.cuda.synchronize()
    y_ref, *_ = oracle.softmax(x_h)
    check_y(to_host(y), y_ref, "normalize")
    # the log form for the fp32 state it was given (its exact value)
    check_log(to_host(ly), oracle.normalize(x_h, m[0::2].cpu().numpy(),
                                            d[0::2].cpu().numpy(), log=True),
              "log normalize")


def test_state_merge_rows_beyond_one_launch():
    K = 3
    rng = np.random.default_rng(7)
    m_in = rng.uniform(-50.0, 50.0, (M_BIG, K)).astype(np.float32)
    d_in = rng.uniform(0.5, 100.0, (M_BIG, K)).astype(np.float32)
    ident = rng.random((M_BIG, K)) < 0.2
    m_in[ident] = -np.inf
    d_in[ident] = 0.0
    mo, do, lo = (torch.empty(M_BIG, device="cuda") for _ in range(3))
    print(f"state merge {M_BIG}x{K}", flush=True)
    rw.state_merge(torch.from_numpy(m_in).cuda(), torch.from_numpy(d_in).cuda(),
                   mo, do, lo)
    torch.cuda.synchronize()
    m_ref, d_ref, l_ref = oracle.merge(m_in, d_in)
    mh, dh, lh = mo.cpu().numpy(), do.cpu().numpy(), lo.cpu().numpy()
    assert np.array_equal(mh.astype(np.float64), m_ref)
    fin = np.isfinite(m_ref)
    assert np.all(np.abs(dh[fin] - d_ref[fin]) <= 1e-5 * d_ref[fin])
    assert np.all(dh[~fin] == 0) and np.all(lh[~fin] == -np.inf)
    assert np.all(np.abs(lh[fin] - l_ref[fin]) <= 1e-5 + oracle.f32_ulp(l_ref[fin]))


@pytest.mark.parametrize("B,H,D,causal,out", [
    (1, LIMIT + 5, 32, -1, torch.float32),    # runs of heads of one batch
    (3, 1398102, 64, 0, torch.bfloat16),      # whole batches, 2 + 1
])
def test_attention_heads_beyond_one_launch(B, H, D, causal, out):
    # one query row per head (one workgroup each), keys and values shared
    # by every head through zero strides
    Sk = 17
    G = B * H
    q, k, v = wl.attention_inputs(1, 1, G, Sk, D, seed=903 + D)
    qd = ta._dev(q).view(B, H, 1, D)
    kd = ta._dev(k).expand(B, H, Sk, D)
    vd = ta._dev(v).expand(B, H, Sk, D)
    o = torch.empty((B, H, 1, D), dtype=out, device="cuda")
    lse = torch.empty((B, H, 1), dtype=torch.float32, device="cuda")
    print(f"attention B{B} H{H} Sq1 Sk{Sk} D{D} causal={causal}", flush=True)
    rw.attention_fwd(qd, kd, vd, o, lse=lse, causal_offset=causal)
    torch.cuda.synchronize()
    edges = [0, 1, LIMIT - 1, LIMIT, LIMIT + 1, 2 * H - 1, 2 * H, G - 1]
    rng = np.random.default_rng(11)
    heads = sorted({g for g in edges if 0 <= g < G} |
                   set(rng.integers(0, G, size=40).tolist()))
    n = len(heads)
    qs = np.ascontiguousarray(q[0, 0][heads].reshape(1, n, 1, D))
    ks = np.ascontiguousarray(np.broadcast_to(k, (1, n, Sk, D)))
    vs = np.ascontiguousarray(np.broadcast_to(v, (1, n, Sk, D)))
    oh = ta._host(o.view(G, D)[heads]).reshape(1, n, 1, D)
    lh = lse.view(G)[heads].cpu().numpy().astype(np.float64).reshape(1, n, 1)
    ta.check(qs, ks, vs, oh, lh, causal=causal, bf16_out=out == torch.bfloat16,
             what=f"attention B{B} H{H}")


@pytest.mark.parametrize("dtype,path", [("f32", "auto"), ("bf16", "stream")])
def test_longest_row(dtype, path):
    # one row of N = 2^30 elements, the largest the entry points take (4 GiB
    # in fp32), with a planted maximum in the middle; the oracle evaluates
    # the whole row and sampled columns are compared, including the planted
    # one, the ends and the split path's chunk edges
    N = 1 << 30
    planted = 123_456_789
    g = torch.Generator(device="cuda").manual_seed(904)
    x = torch.randn(1, N, device="cuda", generator=g)
    x.mul_(2.0)
    if dtype == "bf16":
        x = x.to(torch.bfloat16)
    x[0, planted] = 30.0
    m, d, lse = (torch.empty(1, device="cuda") for _ in range(3))
    print(f"softmax 1x{N} {dtype} path={path}", flush=True)
    y = rw.softmax_fwd(x, m=m, d=d, lse=lse, path=path)
    torch.cuda.synchronize()
    x_h = to_host(x)
    y_ref, m_ref, d_ref, l_ref = oracle.softmax(x_h)
    rng = np.random.default_rng(12)
    chunk = 1 << 19                                 # the split path's chunk length here
    edges = [k * chunk + e for k in (1, 2, 1000, 2047) for e in (-1, 0)]
    cols = sorted(set(rng.integers(0, N, size=4000).tolist())
                  | {0, 1, planted - 1, planted, planted + 1, N - 2, N - 1}
                  | set(edges))
    ct = torch.tensor(cols, device="cuda")
    what = f"longest row {dtype} {path}"
    check_y(to_host(y[:, ct]), y_ref[:, cols], what)
    check_m(m.cpu().numpy(), m_ref, what)
    check_d(d.cpu().numpy(), d_ref, what)
    check_lse(lse.cpu().numpy(), l_ref, what)
    # every element: non-negative, and the row sums to 1 within the
    # per-element relative bar (fp32 1e-5, bf16 one step of 2^-8)
    total = float(y.double().sum())
    assert float(y.min()) >= 0.0
    assert abs(total - 1.0) <= (1e-5 if dtype == "f32" else 2.0 ** -8), total


def test_attention_long_key_sequence():
    # 2^24 keys (262144 tiles of 64, 1 GiB each for K and V at D = 32) for
    # 300 queries in two blocks: tile indices far past the bench shapes and
    # a running max that moves over the whole sequence; sampled rows
    # against the oracle at the derived bound
    Sq, Sk, D = 300, 1 << 24, 32
    g = torch.Generator(device="cuda").manual_seed(906)
    bits = lambda t: t.to(torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
    q = bits(2.0 * torch.randn(1, 1, Sq, D, device="cuda", generator=g))
    k = bits(torch.randn(1, 1, Sk, D, device="cuda", generator=g))
    v = bits(torch.randn(1, 1, Sk, D, device="cuda", generator=g))
    print(f"attention Sq{Sq} Sk{Sk} D{D}", flush=True)
    o, lse = ta.run(q, k, v, out=torch.float32)
    ta.check(q, k, v, o, lse, bf16_out=False, rows=[0, 255, 256, 299],
             what="long key sequence")


def test_most_rows():
    # M = 2^31 - 1, the largest row count the entry points take, with one
    # element per row (8 GiB of x): 512 launches of about 2^22 rows.  A
    # one-element row has the closed form y = 1, m = x, d = 1, lse = x and
    # log-softmax 0, checked on every row on the device
    M = (1 << 31) - 1
    g = torch.Generator(device="cuda").manual_seed(907)
    x = torch.randn(M, 1, device="cuda", generator=g)
    m, d, lse = (torch.empty(M, device="cuda") for _ in range(3))
    print(f"softmax {M}x1", flush=True)
    y = rw.softmax_fwd(x, m=m, d=d, lse=lse)
    torch.cuda.synchronize()
    assert bool((y == 1.0).all())
    assert torch.equal(m, x[:, 0]) and bool((d == 1.0).all()) and torch.equal(lse, x[:, 0])
    del y
    ly = rw.log_softmax_fwd(x)
    torch.cuda.synchronize()
    assert bool((ly == 0.0).all())
    del ly
    # statistics, pass 2 alone and the merge of one state per row
    m.fill_(0.0)
    d.fill_(0.0)
    rw.softmax_stats(x, m, d)
    z = rw.softmax_normalize(x, m, d)
    torch.cuda.synchronize()
    assert torch.equal(m, x[:, 0]) and bool((d == 1.0).all())
    assert bool((z == 1.0).all())
    del z
    mo, do = torch.empty_like(m), torch.empty_like(d)
    rw.state_merge(m.view(M, 1), d.view(M, 1), mo, do, lse)
    torch.cuda.synchronize()
    assert torch.equal(mo, m) and torch.equal(do, d) and torch.equal(lse, m)
    del mo, do
    # cross-entropy: label 0 is the row's only element, loss (x - x) + log 1
    # = +0; every third row ignored (-0.0); the mean of the rest is 0
    labels = torch.zeros(M, dtype=torch.int64, device="cuda")
    labels[::3] = -1
    mean = torch.empty(1, device="cuda")
    loss = rw.cross_entropy_fwd(x, labels, mean=mean)
    torch.cuda.synchronize()
    bits = loss.view(torch.int32)
    assert bool((bits[::3] == -(1 << 31)).all())        # -0.0
    assert bool((bits[1::3] == 0).all()) and bool((bits[2::3] == 0).all())
    assert mean.item() == 0.0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_row_stride_beyond_32_bits(dtype):
    # three rows 2^31 + 16 elements apart (the last one starts 2^32 + 32
    # elements, 16 or 8 GiB, into the buffer): every row offset must be
    # formed in 64 bits, on every path and entry point.  Only the rows'
    # first N columns are written; the rest of the buffer is never read.
    M3, N3, ld = 3, 1000, (1 << 31) + 16
    x_h = wl.normal(M3, N3, scale=3.0, seed=903, dtype=dtype)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    print(f"row stride {ld} {dtype}: {M3} rows of {N3}", flush=True)
    buf = torch.empty(M3 * ld, dtype=tdt, device="cuda")
    x = buf.view(M3, ld)[:, :N3]
    x.copy_(to_device(x_h))
    try:
        _, m_ref, d_ref, l_ref = oracle.softmax(x_h, want_y=False)
        y_ref = oracle.softmax(x_h)[0]
        for path in ("resident", "stream", "split"):
            what = f"stride {ld} {dtype} {path}"
            m, d, lse = (torch.empty(M3, device="cuda") for _ in range(3))
            y = rw.softmax_fwd(x, m=m, d=d, lse=lse, path=path)
            ly = rw.log_softmax_fwd(x, path=path)
            torch.cuda.synchronize()
            check_y(to_host(y), y_ref, what)
            check_log(to_host(ly), oracle.log_softmax(x_h), what)
            check_m(m.cpu().numpy(), m_ref, what)
            check_d(d.cpu().numpy(), d_ref, what)
            check_lse(lse.cpu().numpy(), l_ref, what)
            m2, d2 = (torch.empty(M3, device="cuda") for _ in range(2))
            rw.softmax_stats(x, m2, d2, path=path)
            torch.cuda.synchronize()
            check_m(m2.cpu().numpy(), m_ref, what + " stats")
            check_d(d2.cpu().numpy(), d_ref, what + " stats")
        # pass 2 alone, in place, on the strided rows
        rw.softmax_normalize(x, m2, d2, x)
        torch.cuda.synchronize()
        check_y(to_host(x), y_ref, f"stride {ld} {dtype} normalize in place")
    finally:
        del x, buf
        torch.cuda.empty_cache()
