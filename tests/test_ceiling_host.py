"""The benchmark's ceiling kernels (ceiling/ceiling.hip) on the host: the
library loads, and shapes the kernels do not tile exactly (or misaligned
buffers) are refused before any launch, so every access of an accepted
launch stays inside rows x pitch bytes.  The launch shapes bench.py picks
match the resident kernels of the workloads.  No GPU needed."""
import ctypes
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import ceiling  # noqa: E402
from row_wise_online_amd import workloads as wl  # noqa: E402

pytestmark = pytest.mark.skipif(not os.path.exists(ceiling.LIB_PATH),
                                reason="libos_ceiling.so not built")

A = ctypes.c_void_p(0x10000)       # 16-byte aligned, never dereferenced
B = ctypes.c_void_p(0x20000)
ODD = ctypes.c_void_p(0x10008)


@pytest.fixture(scope="module")
def lib():
    return ceiling.load()


@pytest.mark.parametrize("args", [
    (A, B, 0, 16384, 16384, 8, 2),          # no rows
    (A, B, (1 << 22) + 1, 16384, 16384, 8, 2),
    (A, B, 4, 16000, 16384, 8, 2),          # row not 64 * waves * spl vectors
    (A, B, 4, 16384, 16000, 8, 2),          # pitch below the row
    (A, B, 4, 16384, 16392, 8, 2),          # pitch not a multiple of 16
    (ODD, B, 4, 16384, 16384, 8, 2),        # misaligned source
    (A, ODD, 4, 16384, 16384, 8, 2),        # misaligned destination
    (A, B, 4, 3 * 1024 * 2, 3 * 1024 * 2, 3, 2),   # 3 waves: not built
    (A, B, 4, 8192 * 3, 8192 * 3, 8, 3),    # 3 vectors per lane: not built
])
def test_copy_and_read_refuse_untiled_shapes(lib, args):
    s = None
    assert lib.ceil_copy(*args, s) == 1
    assert lib.ceil_read(*args, s) == 1


def test_write_and_empty_refusals(lib):
    assert lib.ceil_write(ODD, 4, 16384, 16384, 8, 2, None) == 1
    assert lib.ceil_write(A, 4, 16384, 16384, 4, 2, None) == 1
    assert lib.ceil_read(A, None, 4, 16384, 16384, 8, 2, None) == 1
    assert lib.ceil_empty(0, 64, None) == 1
    assert lib.ceil_empty(4, 0, None) == 1
    assert lib.ceil_empty(4, 2048, None) == 1
    assert lib.ceil_memcpy(None, A, 16, None) == 1


def test_launch_shapes_of_the_workloads():
    # the resident kernel's workgroup and vectors per lane for each row
    # length: fp32 4096 -> 8 waves x 2 vectors; bf16 1024 -> 1 wave x 2;
    # fp32 32768 -> 8 waves x 16; 1000 columns do not tile
    W = wl.WORKLOADS
    assert bench.resident_shape(W["c2"]) == (8, 2)
    assert bench.resident_shape(W["c3"]) == (1, 2)
    assert bench.resident_shape(W["c4"]) == (8, 16)
    assert bench.resident_shape(W["c1"]) is None
    assert bench.resident_shape(W["c5"]) is None
    assert bench.ceiling_shape(W["c2"]) == (4096, 16384, 8, 2)
    assert bench.ceiling_shape(W["c3"]) == (32768, 2048, 1, 2)
    # the read-only passes take 2 waves x 8 vectors at 4096 fp32 columns
    assert bench.resident_shape(W["c2"], read_only=True) == (2, 8)
    assert bench.ceiling_shape(W["c2"], read_only=True) == (4096, 16384, 2, 8)
    assert bench.resident_shape(W["c3"], read_only=True) == (1, 2)
    # long rows: x cut into 128 KiB rows
    assert bench.ceiling_shape(W["c5"]) == (2048, 131072, 8, 16)
    for name in ("c2", "c3", "c4", "c5"):
        for ro in (False, True):
            rows, rb, waves, spl = bench.ceiling_shape(W[name], read_only=ro)
            assert rb == 16 * 64 * waves * spl
            assert rows * rb == W[name].M * W[name].N * W[name].esize
            assert waves in ceiling.WAVES and spl in ceiling.VECTORS_PER_LANE


def test_sweep_shapes_are_built():
    # every shape bench.py's copy sweep asks for has an instantiation
    for waves, spl in bench.COPY_SHAPES:
        assert waves in ceiling.WAVES and spl in ceiling.VECTORS_PER_LANE
