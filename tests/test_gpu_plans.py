"""The launch plan on the GPU: the path AUTO takes and the workspace size
the library asks for on the current device equal os_softmax_plan's for the
device's CU count (the pure host function the CPU tests check), and a
workspace one byte short of it is refused before anything is written."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import row_wise_online_amd as rw  # noqa: E402
from row_wise_online_amd import _lib  # noqa: E402
from row_wise_online_amd import workloads as wl  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rw.load()
    yield
    torch.cuda.synchronize()


SHAPES = [(64, 1000), (4096, 4096), (32768, 1024), (1024, 32768),
          (16, 4194304), (511, 16385), (512, 16385), (4096, 65536), (3, 70001),
          (1, 1 << 22), (0, 100)]


def test_plan_matches_the_device():
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    assert cus >= 1
    for M, N in SHAPES:
        for dt in ("f32", "bf16"):
            for op in ("softmax", "stats"):
                plan = rw.softmax_plan(M, N, dt, cus, op=op)
                if M > 0:
                    assert rw.select_path(M, N, dt, op=op) == plan["path"], (M, N, dt, op)
            for path in ("auto", "stream", "split"):
                plan = rw.softmax_plan(M, N, dt, cus, path=path)
                assert rw.workspace_bytes(M, N, dt, path) == plan["workspace_bytes"], \
                    (M, N, dt, path)


@pytest.mark.parametrize("M,N", [(16, 300000), (3, 70001)])
def test_workspace_one_byte_short_is_refused(M, N):
    x = torch.from_numpy(wl.normal(M, N, seed=M)).cuda()
    need = rw.workspace_bytes(M, N, "f32")
    assert need > 0 and rw.select_path(M, N, "f32") == "split"
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y = torch.full_like(x, 5.0)
    with pytest.raises(rw.OsError, match="WORKSPACE"):
        rw.softmax_fwd(x, y, ws=ws[:need - 1])
    m, d = torch.empty(M, device="cuda"), torch.empty(M, device="cuda")
    with pytest.raises(rw.OsError, match="WORKSPACE"):
        rw.softmax_stats(x, m, d, ws=ws[:need - 1])
    torch.cuda.synchronize()
    assert bool((y == 5.0).all())
    # the exact size works
    rw.softmax_fwd(x, y, ws=ws)
    torch.cuda.synchronize()
    s = y.double().sum(dim=1).cpu().numpy()
    assert np.all(np.abs(s - 1.0) < 1e-4)


def test_device_is_usable():
    # the planning queries answer on a gfx950
    lib = rw.load()
    assert lib.os_softmax_select_path(4, 4, 0) == _lib.PATHS["resident"]
