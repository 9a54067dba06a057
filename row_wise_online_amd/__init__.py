"""Row-wise online softmax for AMD MI355X (gfx950) -- Python binding.

Thin wrapper over the C ABI of ``libos_softmax.so`` (``include/os_softmax.h``):
each function checks that its tensors are on the GPU with the layout the ABI
expects, passes their device pointers and the current HIP stream, and raises
``OsError`` on a non-OK status.  PyTorch supplies device memory and streams
only; every step of the computation runs in the library's HIP kernels, and
there is no fallback when the library is missing.

Same names as the C ABI, without the ``os_`` prefix:

* ``softmax_fwd(x, y=None, m=None, d=None, lse=None, ws=None, path="auto")``
* ``log_softmax_fwd(x, y=None, m=None, d=None, lse=None, ws=None, path="auto")``
* ``cross_entropy_fwd(x, labels, loss=None, lse=None, mean=None, ws=None,
  path="auto")``
* ``softmax_stats(x, m, d, lse=None, inc=1, ws=None, path="auto")``
* ``softmax_stats_update(x, m, d, lse=None, inc=1, ws=None, path="auto")``
* ``state_merge(m_in, d_in, m_out, d_out, lse_out=None)``
* ``workspace_bytes(M, N, dtype, path="auto")``, ``select_path(M, N, dtype, op)``
* ``attention_fwd(q, k, v, o=None, lse=None, scale=None, causal_offset=-1)``
  (``include/os_attention.h``), and ``prepare_attention`` for launch loops
"""
import ctypes
import math

from . import _lib
from ._lib import OsError, PATHS, PATH_NAMES  # noqa: F401

__all__ = ["softmax_fwd", "softmax_fwd_noalloc", "log_softmax_fwd", "cross_entropy_fwd",
           "prepare_fwd", "prepare_cross_entropy", "prepare_stats",
           "softmax_stats",
           "softmax_stats_update", "softmax_normalize", "prepare_normalize",
           "state_merge", "workspace_bytes", "select_path", "softmax_plan",
           "OsError", "load",
           "attention_fwd", "prepare_attention"]


def load():
    """Load the HIP library; raises ImportError if it has not been built."""
    return _lib.load()


def _torch():
    import torch
    return torch


def _dtype_code(dtype):
    torch = _torch()
    if dtype == torch.float32:
        return _lib.OS_F32
    if dtype == torch.bfloat16:
        return _lib.OS_BF16
    raise TypeError(f"unsupported dtype {dtype}: float32 or bfloat16")


def _dtype_code_any(dtype):
    if isinstance(dtype, str):
        return {"f32": _lib.OS_F32, "float32": _lib.OS_F32,
                "bf16": _lib.OS_BF16, "bfloat16": _lib.OS_BF16}[dtype]
    return _dtype_code(dtype)


def _matrix(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return t.data_ptr(), t.stride(0)


def _vec(t, name, M, inc=1):
    """Pointer of an fp32 GPU vector holding M values at stride inc: either a
    view whose own stride is inc, or a dense vector with room for them."""
    torch = _torch()
    if t is None:
        return None
    if t.dtype != torch.float32 or not t.is_cuda:
        raise ValueError(f"{name} must be a float32 GPU tensor")
    if t.dim() != 1:
        raise ValueError(f"{name} must be 1-D")
    if t.stride(0) == inc and t.numel() >= M:
        return t.data_ptr()
    if t.stride(0) == 1 and t.numel() >= (M - 1) * inc + 1:
        return t.data_ptr()
    raise ValueError(f"{name} must hold {M} values at stride {inc}")


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _on(stream):
    """Context in which tensors the binding allocates for a call belong to
    the stream the call is launched on.  PyTorch's caching allocator reuses
    a freed block only for allocations on the stream that owns it, in that
    stream's order, so a workspace (or output) freed after the call cannot
    be handed to other work while the call's kernels still use it."""
    import contextlib
    if stream is None:
        return contextlib.nullcontext()
    return _torch().cuda.stream(stream)


def _path_code(path):
    if isinstance(path, str):
        return _lib.PATHS[path]
    return int(path)


def workspace_bytes(M, N, dtype, path="auto"):
    return _lib.load().os_softmax_workspace_bytes(
        M, N, _dtype_code_any(dtype), _path_code(path))


def softmax_plan(M, N, dtype, cu_count, path="auto", op="softmax"):
    """The launch plan (os_softmax_plan) of a call of shape (M, N) on a
    device with cu_count compute units: a dict with the path, the split
    path's chunks per row and chunk length, and the workspace bytes.  op
    "stats" or "cross_entropy" takes the read-only entry points' rule."""
    plan = _lib.Plan()
    st = _lib.load().os_softmax_plan(
        int(M), int(N), _dtype_code_any(dtype), _path_code(path),
        1 if op in ("stats", "cross_entropy") else 0, int(cu_count),
        ctypes.byref(plan))
    _lib.check("os_softmax_plan", st)
    return {"path": _lib.PATH_NAMES[plan.path],
            "chunks_per_row": plan.chunks_per_row,
            "chunk_len": plan.chunk_len,
            "workspace_bytes": plan.workspace_bytes}


def select_path(M, N, dtype, op="softmax"):
    """The path AUTO takes at this shape: for softmax / log-softmax, or,
    with op "stats" or "cross_entropy", for the read-only entry points."""
    fn = ("os_softmax_stats_select_path" if op in ("stats", "cross_entropy")
          else "os_softmax_select_path")
    return _lib.PATH_NAMES[getattr(_lib.load(), fn)(
        int(M), int(N), _dtype_code_any(dtype))]


def _workspace(ws, need, device, stream=None):
    """(pointer, bytes, tensor) of the call's workspace: the caller's, or
    one allocated here on the launch stream when the path needs one.  The
    caller of this helper keeps the tensor referenced until the C call has
    returned (its kernels are then ordered on that stream)."""
    torch = _torch()
    if ws is None:
        if need == 0:
            return None, 0, None
        with _on(stream):
            ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws.data_ptr(), ws.numel() * ws.element_size(), ws


def _fwd(fn_name, x, y, m, d, lse, ws, path, stream, row_len=None,
         causal=None):
    torch = _torch()
    lib = _lib.load()
    dt = _dtype_code(x.dtype)
    if y is None:
        with _on(stream):
            y = torch.empty_like(x)
    if y.dtype != x.dtype or y.shape != x.shape:
        raise ValueError("y must have the dtype and shape of x")
    xp, ldx = _matrix(x, "x")
    yp, ldy = _matrix(y, "y")
    M, N = x.shape
    pc = _path_code(path)
    need = lib.os_softmax_workspace_bytes(M, N, dt, pc)
    wp, wb, ws = _workspace(ws, need, x.device, stream)
    if row_len is None and causal is None:
        st = getattr(lib, fn_name)(xp, ldx, yp, ldy, M, N, dt,
                                   _vec(m, "m", M), _vec(d, "d", M),
                                   _vec(lse, "lse", M), wp, wb, pc,
                                   _stream(stream))
    else:
        if row_len is not None and (
                row_len.dtype != torch.int32 or not row_len.is_cuda or
                row_len.dim() != 1 or row_len.numel() != M or
                row_len.stride(0) != 1):
            raise ValueError("row_len must be a contiguous int32 GPU vector "
                             "of M")
        fn_name = fn_name.replace("_path", "_masked")
        st = getattr(lib, fn_name)(
            xp, ldx, yp, ldy, M, N, dt,
            None if row_len is None else row_len.data_ptr(),
            -1 if causal is None else int(causal), _vec(m, "m", M),
            _vec(d, "d", M), _vec(lse, "lse", M), wp, wb, pc,
            _stream(stream))
    del ws  # released only now that the call's kernels are enqueued
    _lib.check(fn_name, st)
    return y


def softmax_fwd(x, y=None, *, m=None, d=None, lse=None, ws=None,
                path="auto", stream=None, row_len=None, causal=None):
    """y = softmax(x) along rows; optional fp32 row statistics m, d, lse.
    row_len (int32 [M] GPU tensor) and/or causal (offset >= 0) mask each
    row to its first columns (os_softmax_fwd_masked)."""
    return _fwd("os_softmax_fwd_path", x, y, m, d, lse, ws, path, stream,
                row_len, causal)


def softmax_fwd_noalloc(x, y, *, m=None, d=None, lse=None, path="auto",
                        stream=None):
    """softmax_fwd without allocation (os_softmax_fwd_noalloc): y is
    required and the split path's workspace is the library's fixed device
    array (256 KiB per device, shared by every call on the device: calls
    that overlap on one device race)."""
    lib = _lib.load()
    dt = _dtype_code(x.dtype)
    if y.dtype != x.dtype or y.shape != x.shape:
        raise ValueError("y must have the dtype and shape of x")
    xp, ldx = _matrix(x, "x")
    yp, ldy = _matrix(y, "y")
    M, N = x.shape
    st = lib.os_softmax_fwd_noalloc(xp, ldx, yp, ldy, M, N, dt,
                                    _vec(m, "m", M), _vec(d, "d", M),
                                    _vec(lse, "lse", M), _path_code(path),
                                    _stream(stream))
    _lib.check("os_softmax_fwd_noalloc", st)
    return y


def log_softmax_fwd(x, y=None, *, m=None, d=None, lse=None, ws=None,
                    path="auto", stream=None, row_len=None, causal=None):
    """y = log_softmax(x) = x - lse along rows; optional m, d, lse; masks
    as softmax_fwd."""
    return _fwd("os_log_softmax_fwd_path", x, y, m, d, lse, ws, path, stream,
                row_len, causal)


def cross_entropy_fwd(x, labels, loss=None, *, lse=None, mean=None, ws=None,
                      path="auto", stream=None):
    """Per-row cross-entropy of the logits x against int64 labels (negative
    label: ignored row, loss -0.0, which equals 0).  Returns the fp32 loss
    vector; ``mean`` (a 1-element fp32 tensor) receives the mean over
    non-ignored rows."""
    torch = _torch()
    lib = _lib.load()
    dt = _dtype_code(x.dtype)
    xp, ldx = _matrix(x, "x")
    M, N = x.shape
    if labels.dtype != torch.int64 or not labels.is_cuda or labels.dim() != 1 \
            or labels.numel() != M or labels.stride(0) != 1:
        raise ValueError("labels must be a contiguous int64 GPU vector of M")
    if loss is None:
        with _on(stream):
            loss = torch.empty(M, dtype=torch.float32, device=x.device)
    pc = _path_code(path)
    need = lib.os_softmax_workspace_bytes(M, N, dt, pc)
    wp, wb, ws = _workspace(ws, need, x.device, stream)
    st = lib.os_cross_entropy_fwd_path(
        xp, ldx, M, N, dt, labels.data_ptr(), _vec(loss, "loss", M),
        _vec(lse, "lse", M), _vec(mean, "mean", 1), wp, wb, pc,
        _stream(stream))
    del ws
    _lib.check("os_cross_entropy_fwd_path", st)
    return loss


def prepare_fwd(x, y, *, m=None, d=None, lse=None, ws=None, path="auto",
                stream=None, log=False, causal=None):
    """Marshal the arguments of one softmax_fwd (log=True: log_softmax_fwd)
    call once and return a function that repeats the call (same tensors,
    same stream) with only the ctypes call left per invocation -- for tight
    launch loops."""
    lib = _lib.load()
    dt = _dtype_code(x.dtype)
    if y.dtype != x.dtype or y.shape != x.shape:
        raise ValueError("y must have the dtype and shape of x")
    xp, ldx = _matrix(x, "x")
    yp, ldy = _matrix(y, "y")
    M, N = x.shape
    pc = _path_code(path)
    need = lib.os_softmax_workspace_bytes(M, N, dt, pc)
    if need and ws is None:
        raise ValueError(f"path needs a workspace of {need} bytes")
    wp, wb, ws = _workspace(ws, need, x.device)
    stats = (_vec(m, "m", M), _vec(d, "d", M), _vec(lse, "lse", M))
    name = "os_log_softmax_fwd_path" if log else "os_softmax_fwd_path"
    if causal is None:
        args = (xp, ldx, yp, ldy, M, N, dt, *stats, wp, wb, pc,
                _stream(stream))
    else:
        name = name.replace("_path", "_masked")
        args = (xp, ldx, yp, ldy, M, N, dt, None, int(causal), *stats, wp,
                wb, pc, _stream(stream))
    fn = getattr(lib, name)
    keep = (x, y, m, d, lse, ws)   # the tensors must outlive the closure

    def call():
        st = fn(*args)
        if st:
            _lib.check(name, st)
    call.tensors = keep
    return call


def prepare_cross_entropy(x, labels, loss, *, lse=None, mean=None, ws=None,
                          path="auto", stream=None):
    """cross_entropy_fwd's counterpart of prepare_fwd: marshal once, return
    a function that repeats the call."""
    torch = _torch()
    lib = _lib.load()
    dt = _dtype_code(x.dtype)
    xp, ldx = _matrix(x, "x")
    M, N = x.shape
    if labels.dtype != torch.int64 or not labels.is_cuda or \
            labels.numel() != M or labels.stride(0) != 1:
        raise ValueError("labels must be a contiguous int64 GPU vector of M")
    pc = _path_code(path)
    need = lib.os_softmax_workspace_bytes(M, N, dt, pc)
    if need and ws is None:
        raise ValueError(f"path needs a workspace of {need} bytes")
    wp, wb, ws = _workspace(ws, need, x.device)
    args = (xp, ldx, M, N, dt, labels.data_ptr(), _vec(loss, "loss", M),
            _vec(lse, "lse", M), _vec(mean, "mean", 1), wp, wb, pc,
            _stream(stream))
    fn = lib.os_cross_entropy_fwd_path
    keep = (x, labels, loss, lse, mean, ws)

    def call():
        st = fn(*args)
        if st:
            _lib.check("os_cross_entropy_fwd_path", st)
    call.tensors = keep
    return call


def prepare_stats(x, m, d, lse=None, *, ws=None, path="auto", stream=None):
    """softmax_stats's counterpart of prepare_fwd (inc = 1)."""
    lib = _lib.load()
    dt = _dtype_code(x.dtype)
    xp, ldx = _matrix(x, "x")
    M, N = x.shape
    pc = _path_code(path)
    need = lib.os_softmax_workspace_bytes(M, N, dt, pc)
    if need and ws is None:
        raise ValueError(f"path needs a workspace of {need} bytes")
    wp, wb, ws = _workspace(ws, need, x.device)
    args = (xp, ldx, M, N, dt, _vec(m, "m", M), _vec(d, "d", M), 1,
            _vec(lse, "lse", M), wp, wb, pc, _stream(stream))
    fn = lib.os_softmax_stats_path
    keep = (x, m, d, lse, ws)

    def call():
        st = fn(*args)
        if st:
            _lib.check("os_softmax_stats_path", st)
    call.tensors = keep
    return call


def softmax_stats(x, m, d, lse=None, *, inc=1, ws=None, path="auto",
                  stream=None):
    """Pass 1 only: each row's (m, d) (and lse) at index row * inc."""
    lib = _lib.load()
    dt = _dtype_code(x.dtype)
    xp, ldx = _matrix(x, "x")
    M, N = x.shape
    pc = _path_code(path)
    need = lib.os_softmax_workspace_bytes(M, N, dt, pc)
    wp, wb, ws = _workspace(ws, need, x.device, stream)
    st = lib.os_softmax_stats_path(xp, ldx, M, N, dt, _vec(m, "m", M, inc),
                                   _vec(d, "d", M, inc),
                                   inc, _vec(lse, "lse", M, inc), wp, wb, pc,
                                   _stream(stream))
    del ws
    _lib.check("os_softmax_stats_path", st)


def softmax_stats_update(x, m, d, lse=None, *, inc=1, ws=None, path="auto",
                         stream=None):
    """Merge the state of the column window x into the running per-row
    state (m, d) in place (start from m = -inf, d = 0)."""
    lib = _lib.load()
    dt = _dtype_code(x.dtype)
    xp, ldx = _matrix(x, "x")
    M, N = x.shape
    pc = _path_code(path)
    need = lib.os_softmax_workspace_bytes(M, N, dt, pc)
    wp, wb, ws = _workspace(ws, need, x.device, stream)
    st = lib.os_softmax_stats_update(xp, ldx, M, N, dt, _vec(m, "m", M, inc),
                                     _vec(d, "d", M, inc), inc,
                                     _vec(lse, "lse", M, inc), wp, wb, pc,
                                     _stream(stream))
    del ws
    _lib.check("os_softmax_stats_update", st)


def softmax_normalize(x, m, d, y=None, *, inc=1, log=False, stream=None):
    """Pass 2 alone with a row state the caller holds: y = e^(x - m) / d
    (log=True: (x - m) - log d) per row, m and d fp32 at index row * inc.
    x may be a column window of longer rows whose state (m, d) covers the
    whole row.  Returns y (allocated like x when not given)."""
    torch = _torch()
    lib = _lib.load()
    dt = _dtype_code(x.dtype)
    if y is None:
        with _on(stream):
            y = torch.empty_like(x)
    if y.dtype != x.dtype or y.shape != x.shape:
        raise ValueError("y must have the dtype and shape of x")
    xp, ldx = _matrix(x, "x")
    yp, ldy = _matrix(y, "y")
    M, N = x.shape
    name = "os_log_softmax_normalize" if log else "os_softmax_normalize"
    st = getattr(lib, name)(xp, ldx, yp, ldy, M, N, dt, _vec(m, "m", M, inc),
                            _vec(d, "d", M, inc), inc, _stream(stream))
    _lib.check(name, st)
    return y


def prepare_normalize(x, y, m, d, *, inc=1, log=False, stream=None):
    """softmax_normalize's counterpart of prepare_fwd: marshal once, return
    a function that repeats the call."""
    lib = _lib.load()
    dt = _dtype_code(x.dtype)
    if y.dtype != x.dtype or y.shape != x.shape:
        raise ValueError("y must have the dtype and shape of x")
    xp, ldx = _matrix(x, "x")
    yp, ldy = _matrix(y, "y")
    M, N = x.shape
    name = "os_log_softmax_normalize" if log else "os_softmax_normalize"
    args = (xp, ldx, yp, ldy, M, N, dt, _vec(m, "m", M, inc),
            _vec(d, "d", M, inc), inc, _stream(stream))
    fn = getattr(lib, name)
    keep = (x, y, m, d)

    def call():
        st = fn(*args)
        if st:
            _lib.check(name, st)
    call.tensors = keep
    return call


def state_merge(m_in, d_in, m_out, d_out, lse_out=None, *, stream=None):
    """Merge the K states of each row of m_in, d_in ([M, K], fp32)."""
    torch = _torch()
    lib = _lib.load()
    for t, n in ((m_in, "m_in"), (d_in, "d_in")):
        if t.dtype != torch.float32:
            raise ValueError(f"{n} must be float32")
    mp, ld = _matrix(m_in, "m_in")
    dp, ld2 = _matrix(d_in, "d_in")
    if ld != ld2 or m_in.shape != d_in.shape:
        raise ValueError("m_in and d_in must have the same shape and stride")
    M, K = m_in.shape
    st = lib.os_state_merge(mp, dp, ld, M, K, _vec(m_out, "m_out", M),
                            _vec(d_out, "d_out", M),
                            _vec(lse_out, "lse_out", M), _stream(stream))
    _lib.check("os_state_merge", st)


def _bhsd(t, name):
    """Pointer and (batch, head, row) element strides of a [B, H, S, D] GPU
    tensor whose last axis is contiguous."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError(f"{name} must be [B, H, S, D] with a contiguous last axis")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return t.data_ptr(), (ctypes.c_int64 * 3)(t.stride(0), t.stride(1),
                                              t.stride(2))


def prepare_attention(q, k, v, o, *, lse=None, scale=None, causal_offset=-1,
                      stream=None):
    """Marshal one os_attention_fwd call (q, k, v bf16 [B, H, S, D]; o bf16
    or fp32 of q's shape; lse fp32 [B, H, Sq] dense or None) and return a
    function that repeats it on the same tensors and stream."""
    torch = _torch()
    lib = _lib.load()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{n} must be bfloat16")
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if k.shape != (B, H, Sk, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B, H, Sk, D] matching q")
    if o.shape != q.shape:
        raise ValueError("o must have q's shape")
    od = _dtype_code(o.dtype)
    ptrs = [_bhsd(t, n) for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"))]
    lp = None
    if lse is not None:
        if (lse.dtype != torch.float32 or not lse.is_cuda
                or lse.shape != (B, H, Sq) or not lse.is_contiguous()):
            raise ValueError("lse must be a dense float32 GPU tensor [B, H, Sq]")
        lp = lse.data_ptr()
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    args = (ptrs[0][0], ptrs[1][0], ptrs[2][0], ptrs[3][0], lp, B, H, Sq, Sk,
            D, ptrs[0][1], ptrs[1][1], ptrs[2][1], ptrs[3][1], od,
            float(scale), int(causal_offset), _stream(stream))
    fn = lib.os_attention_fwd
    keep = (q, k, v, o, lse, ptrs)

    def call():
        st = fn(*args)
        if st:
            _lib.check("os_attention_fwd", st)
    call.tensors = keep
    return call


def attention_fwd(q, k, v, o=None, *, lse=None, scale=None, causal_offset=-1,
                  out_dtype=None, stream=None):
    """o = softmax(scale q k^T) v per (batch, head), with the online softmax
    inside key tiles (os_attention_fwd).  q, k, v: bf16 [B, H, S, D] GPU
    tensors with a contiguous last axis (any other strides); scale defaults
    to 1/sqrt(D); causal_offset >= 0 admits key j for query i when
    j <= i + causal_offset.  Returns o (allocated as out_dtype, default
    bf16, when not given)."""
    torch = _torch()
    if o is None:
        with _on(stream):
            o = torch.empty(q.shape, dtype=out_dtype or torch.bfloat16,
                            device=q.device)
    prepare_attention(q, k, v, o, lse=lse, scale=scale,
                      causal_offset=causal_offset, stream=stream)()
    return o
