"""Bandwidth and launch ceilings for the benchmark (``libos_ceiling.so``,
built from ``ceiling.hip``): a copy, a read-only and a write-only kernel in
the launch shape of a softmax launch, an empty kernel, and the runtime's own
device-to-device copy.  Not part of the softmax library or its ABI; only
``bench.py`` uses it.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libos_ceiling.so")

# the launch shapes the kernels are built for (ceiling.hip): waves per
# workgroup and 16-byte vectors per lane
WAVES = (1, 2, 4, 8)
VECTORS_PER_LANE = (1, 2, 4, 8, 16)

_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python ceiling/build.py` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        for name in ("ceil_copy", "ceil_read"):
            fn = getattr(lib, name)
            fn.argtypes = [vp, vp, i64, i64, i64, i32, i32, vp]
            fn.restype = i32
        lib.ceil_write.argtypes = [vp, i64, i64, i64, i32, i32, vp]
        lib.ceil_write.restype = i32
        lib.ceil_empty.argtypes = [i64, i32, vp]
        lib.ceil_empty.restype = i32
        lib.ceil_memcpy.argtypes = [vp, vp, ctypes.c_size_t, vp]
        lib.ceil_memcpy.restype = i32
        _lib = lib
    return _lib


def check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what}: {'unsupported shape' if rc == 1 else 'launch failed'}")
