"""ctypes view of the C ABI in ``include/os_softmax.h`` and
``include/os_attention.h``.

Argument marshalling only: this module loads ``libos_softmax.so`` (built by
``row_wise_online_amd/build.py``) and declares each exported function's
signature.  There is no fallback: if the library is missing, loading fails
with an error that says how to build it.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libos_softmax.so")

# os_status
OS_OK = 0
STATUS_NAMES = {
    0: "OS_OK", 1: "OS_ERR_NULL", 2: "OS_ERR_SHAPE", 3: "OS_ERR_STRIDE",
    4: "OS_ERR_DTYPE", 5: "OS_ERR_WORKSPACE", 6: "OS_ERR_PATH",
    7: "OS_ERR_UNSUPPORTED", 8: "OS_ERR_HIP", 9: "OS_ERR_DEVICE",
}
# os_dtype
OS_F32 = 0
OS_BF16 = 1
# os_path
PATHS = {"auto": 0, "resident": 1, "stream": 2, "split": 3}
PATH_NAMES = {v: k for k, v in PATHS.items()}



class Plan(ctypes.Structure):
    """os_plan: the launch plan of a row-wise call."""
    _fields_ = [("path", ctypes.c_int), ("chunks_per_row", ctypes.c_int32),
                ("chunk_len", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_size_t)]


# Every function the header declares, with its ctypes signature.
_vp, _i64, _i32, _sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                        ctypes.c_size_t)
SIGNATURES = {
    "os_softmax_fwd": (_i32, [_vp, _i64, _vp, _i64, _i64, _i64, _i32,
                              _vp, _vp, _vp, _vp, _sz, _vp]),
    "os_softmax_fwd_path": (_i32, [_vp, _i64, _vp, _i64, _i64, _i64, _i32,
                                   _vp, _vp, _vp, _vp, _sz, _i32, _vp]),
    "os_softmax_fwd_noalloc": (_i32, [_vp, _i64, _vp, _i64, _i64, _i64,
                                      _i32, _vp, _vp, _vp, _i32, _vp]),
    "os_log_softmax_fwd": (_i32, [_vp, _i64, _vp, _i64, _i64, _i64, _i32,
                                  _vp, _vp, _vp, _vp, _sz, _vp]),
    "os_log_softmax_fwd_path": (_i32, [_vp, _i64, _vp, _i64, _i64, _i64,
                                       _i32, _vp, _vp, _vp, _vp, _sz, _i32,
                                       _vp]),
    "os_softmax_fwd_masked": (_i32, [_vp, _i64, _vp, _i64, _i64, _i64, _i32,
                                     _vp, _i64, _vp, _vp, _vp, _vp, _sz,
                                     _i32, _vp]),
    "os_log_softmax_fwd_masked": (_i32, [_vp, _i64, _vp, _i64, _i64, _i64,
                                         _i32, _vp, _i64, _vp, _vp, _vp, _vp,
                                         _sz, _i32, _vp]),
    "os_cross_entropy_fwd": (_i32, [_vp, _i64, _i64, _i64, _i32, _vp, _vp,
                                    _vp, _vp, _vp, _sz, _vp]),
    "os_cross_entropy_fwd_path": (_i32, [_vp, _i64, _i64, _i64, _i32, _vp,
                                         _vp, _vp, _vp, _vp, _sz, _i32,
                                         _vp]),
    "os_softmax_stats": (_i32, [_vp, _i64, _i64, _i64, _i32, _vp, _vp, _i64,
                                _vp, _vp, _sz, _vp]),
    "os_softmax_stats_path": (_i32, [_vp, _i64, _i64, _i64, _i32, _vp, _vp,
                                     _i64, _vp, _vp, _sz, _i32, _vp]),
    "os_softmax_stats_update": (_i32, [_vp, _i64, _i64, _i64, _i32, _vp, _vp,
                                       _i64, _vp, _vp, _sz, _i32, _vp]),
    "os_state_merge": (_i32, [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp,
                              _vp]),
    "os_softmax_normalize": (_i32, [_vp, _i64, _vp, _i64, _i64, _i64, _i32,
                                    _vp, _vp, _i64, _vp]),
    "os_log_softmax_normalize": (_i32, [_vp, _i64, _vp, _i64, _i64, _i64,
                                        _i32, _vp, _vp, _i64, _vp]),
    "os_softmax_workspace_bytes": (_sz, [_i64, _i64, _i32, _i32]),
    "os_softmax_plan": (_i32, [_i64, _i64, _i32, _i32, _i32, _i32,
                               ctypes.POINTER(Plan)]),
    "os_softmax_select_path": (_i32, [_i64, _i64, _i32]),
    "os_softmax_stats_select_path": (_i32, [_i64, _i64, _i32]),
    "os_status_string": (ctypes.c_char_p, [_i32]),
    "os_attention_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                _i64, _i64, _vp, _vp, _vp, _vp, _i32,
                                ctypes.c_float, _i64, _vp]),
}

_lib = None


class OsError(RuntimeError):
    """A non-OK os_status returned by the library."""

    def __init__(self, fn, status):
        self.status = status
        msg = _lib.os_status_string(status).decode() if _lib else str(status)
        super().__init__(f"{fn}: {msg}")


def load():
    """Load the HIP library (once) and return the ctypes handle."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python row_wise_online_amd/build.py` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(fn, status):
    if status != OS_OK:
        raise OsError(fn, status)
