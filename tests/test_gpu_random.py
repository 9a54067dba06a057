"""Randomised parity cases: each case draws its own shape, dtype, row
stride, path, value scale and offset, operation (softmax, log-softmax,
masked rows, statistics, pass 2 alone over column windows, cross-entropy
with its mean) or attention configuration (batch, heads, query
and key lengths, head dimension, causal offset, layout, output dtype) from
a generator seeded by the case number, and checks the HIP path against the
fp64 oracle at the same accuracy bars as the fixed cases.  The draws cover
shapes the fixed lists do not name: odd row counts, every tail length,
padded strides and offsets that put all mass on few elements."""
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

N_CASES = 160


def _row_case(rng, k):
    M = int(rng.integers(1, 300))
    N = int(rng.choice([int(rng.integers(1, 200)), int(rng.integers(200, 5000)),
                        int(rng.integers(5000, 70000))]))
    dtype = str(rng.choice(["f32", "bf16"]))
    ld = N + int(rng.choice([0, 0, 1, 7, 64]))
    path = str(rng.choice(["auto", "resident", "stream", "split"]))
    if path == "resident" and N > 32768:
        path = "auto"
    scale = float(rng.choice([1.0, 4.0, 30.0]))
    offset = float(rng.choice([0.0, 50.0, -1e3]))
    op = str(rng.choice(["softmax", "log_softmax", "masked", "stats",
                         "normalize", "cross_entropy"]))
    what = (f"case {k}: {op} {dtype} {M}x{N} ld={ld} path={path} "
            f"scale={scale} offset={offset}")
    print(what, flush=True)
    x_h = wl.normal(M, N, scale=scale, offset=offset, seed=50000 + k,
                    dtype=dtype, ld=ld if ld != N else None)
    x = to_device(x_h)
    m, d, lse = (torch.empty(M, device="cuda") for _ in range(3))
    if op == "stats":
        rw.softmax_stats(x, m, d, lse, path=path)
        torch.cuda.synchronize()
        _, m_ref, d_ref, l_ref = oracle.softmax(x_h, want_y=False)
    elif op == "normalize":
        # statistics of random column windows merged at a stride, then each
        # window normalised with the merged state
        cuts = sorted(rng.choice(np.arange(1, N), size=min(3, N - 1),
                                 replace=False).tolist()) if N > 1 else []
        edges = [0, *cuts, N]
        inc = int(rng.integers(1, 3))
        mm = torch.full((M * inc,), float("-inf"), device="cuda")
        dd = torch.zeros(M * inc, device="cuda")
        for a, b in zip(edges[:-1], edges[1:]):
            rw.softmax_stats_update(x[:, a:b], mm, dd, inc=inc)
        y = torch.full_like(x, float("nan"))
        ly = torch.full_like(x, float("nan"))
        for a, b in zip(edges[:-1], edges[1:]):
            rw.softmax_normalize(x[:, a:b], mm, dd, y[:, a:b], inc=inc)
            rw.softmax_normalize(x[:, a:b], mm, dd, ly[:, a:b], inc=inc, log=True)
        torch.cuda.synchronize()
        what += f" windows {edges} inc={inc}"
        y_ref, m_ref, d_ref, _ = oracle.softmax(x_h)
        check_y(to_host(y), y_ref, what)
        # the log form for the fp32 state it was given (its exact value)
        check_log(to_host(ly), oracle.normalize(
            x_h, mm[0::inc].cpu().numpy(), dd[0::inc].cpu().numpy(),
            log=True), what)
        check_m(mm[0::inc].cpu().numpy(), m_ref, what)
        check_d(dd[0::inc].cpu().numpy(), d_ref, what)
        return
    elif op == "cross_entropy":
        lab = rng.integers(-2, N, size=M).astype(np.int64)
        mean = torch.empty(1, device="cuda")
        loss = rw.cross_entropy_fwd(x, torch.from_numpy(lab).cuda(), lse=lse,
                                    mean=mean, path=path)
        torch.cuda.synchronize()
        l_ref, mean_ref = oracle.cross_entropy(x_h, lab)
        check_log(loss.cpu().numpy(), l_ref, what)
        if np.isnan(mean_ref):
            assert np.isnan(mean.item()), what
        else:
            assert abs(mean.item() - mean_ref) <= 1e-5 * abs(mean_ref) + 1e-6, \
                (what, mean.item(), mean_ref)
        _, _, _, l2 = oracle.softmax(x_h, want_y=False)
        check_lse(lse.cpu().numpy(), l2, what)
        return
    elif op == "masked":
        causal = int(rng.integers(0, N + 5)) if rng.random() < 0.5 else None
        rl = (rng.integers(-2, N + 3, size=M).astype(np.int32)
              if rng.random() < 0.6 else None)
        if causal is None and rl is None:
            causal = 0
        what += f" causal={causal} row_len={'yes' if rl is not None else 'no'}"
        rl_d = None if rl is None else torch.from_numpy(rl).cuda()
        y = rw.softmax_fwd(x, m=m, d=d, lse=lse, path=path, row_len=rl_d,
                           causal=causal)
        ly = rw.log_softmax_fwd(x, path=path, row_len=rl_d, causal=causal)
        torch.cuda.synchronize()
        y_ref, ly_ref, m_ref, d_ref, l_ref = oracle.softmax_masked(
            x_h, rl, -1 if causal is None else causal)
        # rows with no valid column: y NaN, d = 0, lse = -inf
        ok = ~np.isnan(y_ref[:, 0])
        yh = to_host(y)
        yf = (yh.astype(np.float64) if yh.dtype == np.float32
              else oracle.bf16_bits_to_f64(yh))
        assert np.all(np.isnan(yf[~ok])), what
        if ok.any():
            check_y(yh[ok], y_ref[ok], what)
        check_log(to_host(ly), ly_ref, what)
        dh, lh = d.cpu().numpy(), lse.cpu().numpy()
        check_m(m.cpu().numpy(), m_ref, what)
        assert np.all(dh[~ok] == 0) and np.all(lh[~ok] == -np.inf), what
        if ok.any():
            check_d(dh[ok], d_ref[ok], what)
            check_lse(lh[ok], l_ref[ok], what)
        return
    elif op == "softmax":
        y = rw.softmax_fwd(x, m=m, d=d, lse=lse, path=path)
        torch.cuda.synchronize()
        y_ref, m_ref, d_ref, l_ref = oracle.softmax(x_h)
        check_y(to_host(y), y_ref, what)
    else:
        y = rw.log_softmax_fwd(x, m=m, d=d, lse=lse, path=path)
        torch.cuda.synchronize()
        check_log(to_host(y), oracle.log_softmax(x_h), what)
        _, m_ref, d_ref, l_ref = oracle.softmax(x_h, want_y=False)
    check_m(m.cpu().numpy(), m_ref, what)
    check_d(d.cpu().numpy(), d_ref, what)
    check_lse(lse.cpu().numpy(), l_ref, what)


def _attention_case(rng, k):
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    Sq, Sk = int(rng.integers(1, 700)), int(rng.integers(1, 1500))
    D = int(rng.choice([32, 64, 128]))
    causal = int(rng.choice([-1, -1, 0, int(rng.integers(0, 400))]))
    layout = str(rng.choice(["bhsd", "bshd"]))
    qs = float(rng.choice([1.0, 1.0, 4.0]))
    out = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    what = (f"case {k}: attention B{B} H{H} Sq{Sq} Sk{Sk} D{D} causal={causal} "
            f"{layout} q_scale={qs} out={out}")
    print(what, flush=True)
    q, kk, v = wl.attention_inputs(B, H, Sq, Sk, D, seed=60000 + k, q_scale=qs,
                                   layout=layout)
    o, lse = ta.run(q, kk, v, causal=causal, out=out,
                    o_layout="bshd" if layout == "bshd" else None)
    rows = sorted(set(rng.integers(0, Sq, size=min(Sq, 12)).tolist()) | {0, Sq - 1})
    ta.check(q, kk, v, o, lse, causal=causal, bf16_out=out == torch.bfloat16,
             rows=rows, what=what)


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_case(k):
    rng = np.random.default_rng([7, k])
    (_attention_case if rng.random() < 0.4 else _row_case)(rng, k)
