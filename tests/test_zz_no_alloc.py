"""The entry point that allocates nothing, os_softmax_fwd_noalloc (through
the C ABI), against os_softmax_fwd_path with a caller-allocated workspace
on the same inputs: the same kernels and plan, so the results must be
bit-identical, and both within the oracle's bar.  Two calls in a row, the
second on a smaller input, reuse the device's fixed array; a HIP graph that
captures the call replays it on new inputs."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import row_wise_online_amd as rw  # noqa: E402
from row_wise_online_amd import workloads as wl  # noqa: E402

from gpu_util import check_d, check_lse, check_m, check_y, to_device, to_host  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rw.load()
    yield
    torch.cuda.synchronize()


def _pair(x, path):
    """(noalloc outputs, workspace outputs) of one softmax call each."""
    M, N = x.shape
    res = []
    for noalloc in (True, False):
        y = torch.full_like(x, float("nan"))
        st = [torch.full((M,), float("nan"), device="cuda") for _ in range(3)]
        if noalloc:
            rw.softmax_fwd_noalloc(x, y, m=st[0], d=st[1], lse=st[2], path=path)
        else:
            ws = torch.empty(max(rw.workspace_bytes(M, N, x.dtype, path), 1),
                             dtype=torch.uint8, device="cuda")
            rw.softmax_fwd(x, y, m=st[0], d=st[1], lse=st[2], ws=ws, path=path)
        torch.cuda.synchronize()
        res.append((y, *st))
    return res


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_two_calls_in_a_row_second_smaller(dtype):
    # AUTO takes the split path on both shapes (few long rows), so both
    # calls run in the fixed array; the second is smaller and must not be
    # disturbed by what the first left there
    cases = [(16, 1 << 20, 40), (5, 300001, 41)]
    for M, N, seed in cases:
        assert rw.select_path(M, N, dtype) == "split"
        x_h = wl.normal(M, N, scale=3.0, seed=seed, dtype=dtype)
        x = to_device(x_h)
        got, want = _pair(x, "auto")
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"{dtype} {M}x{N}: differs from the workspace call"
        y_ref, m_ref, d_ref, l_ref = oracle.softmax(x_h)
        what = f"noalloc {dtype} {M}x{N}"
        check_y(to_host(got[0]), y_ref, what)
        check_m(got[1].cpu().numpy(), m_ref, what)
        check_d(got[2].cpu().numpy(), d_ref, what)
        check_lse(got[3].cpu().numpy(), l_ref, what)


def test_every_path_and_a_forced_split():
    # resident and stream need no workspace; a forced split on many short
    # rows uses the array too
    for M, N, path in [(300, 1000, "resident"), (40, 20000, "stream"),
                       (600, 5000, "split"), (3, 70001, "auto")]:
        x_h = wl.normal(M, N, scale=2.0, seed=M + N)
        x = to_device(x_h)
        got, want = _pair(x, path)
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"{M}x{N} {path}"
        y_ref, *_ = oracle.softmax(x_h)
        check_y(to_host(got[0]), y_ref, f"noalloc {M}x{N} {path}")


def test_plan_beyond_the_array_is_refused():
    # a forced split over 32768 rows needs 4 tables of 32768 floats
    # (512 KiB): refused with OS_ERR_WORKSPACE before anything is enqueued
    M, N = 32768, 4096
    x = torch.zeros((M, N), device="cuda")
    y = torch.full_like(x, 7.0)
    with pytest.raises(rw.OsError, match="WORKSPACE"):
        rw.softmax_fwd_noalloc(x, y, path="split")
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
    # the same shape on AUTO (resident) needs no workspace and runs
    rw.softmax_fwd_noalloc(x, y)
    torch.cuda.synchronize()
    assert bool((y == 1.0 / N).all())


def test_graph_capture_and_replay():
    # the callers this entry point is for: a HIP graph captures the call
    # (it allocates nothing, and the split path's scratch is the fixed
    # array), and each replay on new inputs gives the bits of the eager call
    # with a caller workspace
    M, N = 8, 300001
    assert rw.select_path(M, N, "f32") == "split"
    x = torch.empty(M, N, device="cuda")
    y = torch.empty_like(x)
    st = [torch.empty(M, device="cuda") for _ in range(3)]

    def fill(seed):
        x.copy_(torch.from_numpy(wl.normal(M, N, scale=3.0, seed=seed)))

    fill(80)
    # one eager call first, as a caller warms up before capturing: the
    # device's array address is read on the first call on a device
    rw.softmax_fwd_noalloc(x, y, m=st[0], d=st[1], lse=st[2])
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        rw.softmax_fwd_noalloc(x, y, m=st[0], d=st[1], lse=st[2])
    for i, seed in enumerate((81, 82, 83)):
        fill(seed)
        eager = _pair(x, "auto")[1]
        want_y, want = eager[0], eager[1:]
        for t in (y, *st):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want_y), f"replay {i}: y differs from the eager call"
        for a, b in zip(st, want):
            assert torch.equal(a, b), f"replay {i}: a row statistic differs"
        if i == 0:
            x_h = wl.normal(M, N, scale=3.0, seed=seed)
            y_ref, m_ref, d_ref, l_ref = oracle.softmax(x_h)
            check_y(to_host(y), y_ref, "graph replay")
            check_m(st[0].cpu().numpy(), m_ref, "graph replay")
            check_d(st[1].cpu().numpy(), d_ref, "graph replay")
            check_lse(st[2].cpu().numpy(), l_ref, "graph replay")
