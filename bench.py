#!/usr/bin/env python3
"""Throughput of the row-wise online softmax forward on one MI355X.

A step is one ``os_softmax_fwd`` call (the whole hot path: pass 1, the
state merges, pass 2) over one seeded synthetic input already resident in
HBM.  Inputs rotate over enough buffer sets (>= 1 GiB) that every step reads
from HBM rather than from the 256 MB Infinity Cache.  The timed region is
bracketed by device synchronisation and HIP events on the stream the
kernels are launched on.

Prints one JSON line on stdout (rank 0, N = 1).  ``value`` is algorithmic
GB/s: the bytes the path must move (x read once per read pass, y written
once, row statistics written) divided by the step time.

``--all`` also prints one JSON line per workload to stderr.

``--op attention`` (workloads a2, a3, a4, a5) times one ``os_attention_fwd``
call per step instead: the attention forward with the online softmax inside
key tiles; ``value`` is then TFLOP/s (4 Sq Sk D per head for Q K^T and P V,
over the admitted key pairs only under a causal mask), against the MI355X
dense bf16 matrix-core peak.
"""
import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("achieved HBM GB/s (% of peak) + rows/s, online softmax fwd fp32 "
          "4096×4096")
PEAK_GBS = 8000.0           # MI355X HBM3E, published peak
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published peak
# The pages' own figure for this metric and workload: their register-cached
# one-read kernel on fp32 4096 x 4096, on an A100 80GB SXM4 ("5.2 CUDA Online
# Softmax 实现优化" §8.1).  Another machine's number: context, not a target.
PAGES_C2_GBS = 1672.0
ROTATE_BYTES = 1 << 30      # rotating working set, 4x the Infinity Cache


def kernel_source_hash(family="softmax"):
    """Hash of the sources one kernel family is built from: "softmax" (every
    csrc file but the attention kernel) or "attention" (the attention kernel
    and the headers it includes).  A committed counter record applies only
    while this hash is unchanged."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "row_wise_online_amd",
                                           "csrc", "*"))):
        name = os.path.basename(p)
        if os.path.splitext(name)[1] not in (".hip", ".hpp", ".h"):
            continue  # sources only, not compiler temporaries
        is_attn = name.startswith("attention")
        if family == "softmax" and is_attn:
            continue
        if family == "attention" and not (is_attn or name in (
                "common.hpp", "chunks.hpp", "launch.hpp", "plan.hpp")):
            continue
        with open(p, "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def valid_elements(w, causal):
    """Elements a causal mask with this offset leaves in the workload."""
    if causal is None:
        return w.M * w.N
    i = __import__("numpy").arange(w.M, dtype="int64")
    return int(__import__("numpy").minimum(w.N, i + causal + 1).sum())


def device_cus():
    """Compute units of the current GPU (256 on MI355X), from torch."""
    import torch
    if torch.cuda.is_available():
        return torch.cuda.get_device_properties(
            torch.cuda.current_device()).multi_processor_count
    return 256


def algorithmic_bytes(w, path, n_stats, op="softmax", causal=None, cus=None):
    """Bytes the path must move for one step of workload w: x read once per
    read pass (only the unmasked part of each row), y written once (all of
    it), row statistics written; the cross-entropy reads x once and moves
    8 B of label + 4 B of loss per row (+ 4 B mean); pass 2 alone
    (normalize) reads x and the 8 B row state and writes y."""
    import row_wise_online_amd as rw
    xy = w.M * w.N * w.esize
    xr = valid_elements(w, causal) * w.esize
    if op == "cross_entropy":
        b = xy + 12 * w.M + 4
    elif op == "stats":
        b = xy + 12 * w.M
    elif op == "normalize":
        return 2 * xy + 8 * w.M
    else:
        reads = 1 if path == "resident" else 2
        b = reads * xr + xy + 4 * w.M * n_stats
    if path == "split":
        cus = device_cus() if cus is None else cus
        b += 2 * rw.softmax_plan(w.M, w.N, w.dtype, cus, "split")[
            "workspace_bytes"]  # partial and row states, written and read
    return b


def measure(w, steps, warmup, path="auto", rotate=True, graph=False,
            op="softmax", causal=None, trials=0, keep=False):
    """Average device time per step (ms), the rotation depth, the host time
    per launch (us), the spread of the launch time (or None) and the kept
    outputs (or None).  Steps cycle over R buffer sets; with graph=True the
    launches are captured once in a HIP graph and replayed.  With trials > 0
    (plain launches) that many further runs of up to 50 launches, each
    between its own pair of events, follow the timed steps; their
    per-launch times give the p10 / p50 / p90 spread.  With keep=True the
    outputs of the last step on buffer set 0 (every set holds the same x)
    are copied to the host and returned last, else None."""
    import numpy as np
    import torch
    import row_wise_online_amd as rw
    from row_wise_online_amd import workloads as wl

    x_host = wl.generate(w.name)
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    if w.dtype == "f32":
        x0 = torch.from_numpy(x_host).cuda()
    else:
        x0 = torch.from_numpy(x_host.view(np.int16)).view(tdt).cuda()
    ce = op == "cross_entropy"
    one_read = op in ("cross_entropy", "stats")
    per_set = (1 if one_read else 2) * w.M * w.N * w.esize
    R = max(2, -(-ROTATE_BYTES // per_set)) if rotate else 1
    xs = [x0] + [x0.clone() for _ in range(R - 1)]
    ys = [None if one_read else torch.empty_like(x0) for _ in range(R)]
    want = set(w.outputs)
    stat = lambda k: torch.empty(w.M, device="cuda") if k in want else None
    m, d, lse = stat("m"), stat("d"), stat("lse")
    ws_bytes = rw.workspace_bytes(w.M, w.N, w.dtype, path)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    if ce:
        labels = torch.from_numpy(np.random.default_rng(w.seed).integers(
            0, w.N, size=w.M)).cuda()
        loss = torch.empty(w.M, device="cuda")
        mean = torch.empty(1, device="cuda")

    if op == "stats":
        m = torch.empty(w.M, device="cuda")
        d = torch.empty(w.M, device="cuda")
        lse = torch.empty(w.M, device="cuda")
    if op == "normalize":
        # the row state every buffer set shares (they hold the same values),
        # taken once before the timed steps
        m_st = torch.empty(w.M, device="cuda")
        d_st = torch.empty(w.M, device="cuda")
        rw.softmax_stats(x0, m_st, d_st)
        m = d = lse = None

    def prepared():
        # the launch stream is taken here, so that under graph capture the
        # calls bind to the capturing stream
        strm = torch.cuda.current_stream()
        if op == "stats":
            return [rw.prepare_stats(xs[i], m, d, lse, ws=ws, path=path)
                    for i in range(R)]
        if op == "normalize":
            return [rw.prepare_normalize(xs[i], ys[i], m_st, d_st)
                    for i in range(R)]
        if ce:
            return [rw.prepare_cross_entropy(xs[i], labels, loss, mean=mean,
                                             ws=ws, path=path)
                    for i in range(R)]
        return [rw.prepare_fwd(xs[i], ys[i], m=m, d=d, lse=lse, ws=ws,
                               path=path, log=(op == "log_softmax"),
                               causal=causal, stream=strm)
                for i in range(R)]

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    strm = torch.cuda.current_stream()   # the stream the calls launch on
    dist = None
    if not graph:
        calls = prepared()
        for i in range(warmup):
            calls[i % R]()
        torch.cuda.synchronize()
        start.record(strm)
        t0 = time.perf_counter()
        for i in range(steps):
            calls[i % R]()
        host_us = (time.perf_counter() - t0) / steps * 1e6
        end.record(strm)
        end.synchronize()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / steps
        if trials:
            per = max(1, min(steps, 50))
            evs = [(torch.cuda.Event(enable_timing=True),
                    torch.cuda.Event(enable_timing=True))
                   for _ in range(trials)]
            k = 0
            for a, b in evs:
                a.record(strm)
                for _ in range(per):
                    calls[k % R]()
                    k += 1
                b.record(strm)
            torch.cuda.synchronize()
            us = sorted(a.elapsed_time(b) / per * 1e3 for a, b in evs)
            q = lambda f: round(us[int(f * (len(us) - 1) + 0.5)], 3)
            dist = {"trials": trials, "launches_each": per,
                    "us_p10": q(0.1), "us_p50": q(0.5), "us_p90": q(0.9)}
    else:
        per_graph = R * max(1, 32 // R)
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            calls = prepared()
            for i in range(per_graph):
                calls[i % R]()
        reps = max(1, -(-steps // per_graph))
        for _ in range(max(1, warmup // per_graph)):
            g.replay()
        torch.cuda.synchronize()
        start.record()
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        host_us = (time.perf_counter() - t0) / (reps * per_graph) * 1e6
        end.record()
        end.synchronize()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / (reps * per_graph)
        del g
    outs = None
    if keep:
        def host(t):
            if t is None:
                return None
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).cpu().numpy().view(np.uint16)
            return t.cpu().numpy()
        if op in ("softmax", "log_softmax", "normalize"):
            outs = {"y": host(ys[0]), "m": host(m), "d": host(d),
                    "lse": host(lse)}
        elif op == "stats":
            outs = {"m": host(m), "d": host(d), "lse": host(lse)}
        else:
            outs = {"loss": host(loss), "mean": float(mean.item())}
    del xs, ys
    return ms, R, host_us, dist, outs


def resident_shape(w, read_only=False):
    """(waves, 16-byte vectors per lane) of the resident kernel the library
    launches for this row length and dtype (one workgroup per row), if the
    row is a whole number of its tiles; else None.  read_only: the shape of
    the statistics / cross-entropy pass (2 waves x 32 at 4096 columns)."""
    E = 4 if w.dtype == "f32" else 8          # elements per 16-byte vector
    ladder = [(256, 1, 4), (512, 1, 8), (1024, 1, 16), (2048, 4, 8),
              (4096, 2 if read_only else 8, 32 if read_only else 8),
              (8192, 8, 16), (16384, 8, 32), (32768, 8, 64)]
    for n_max, waves, epl in ladder:
        if w.N <= n_max:
            if epl % E or w.N * w.esize != 16 * 64 * waves * (epl // E):
                return None
            return waves, epl // E
    return None


def ceiling_shape(w, read_only=False):
    """Rows, row bytes, waves and vectors per lane of the ceiling kernels for
    workload w: the resident kernel's launch shape (of the read-only passes
    with read_only) when it tiles the row exactly, else x cut into 128 KiB
    rows (512 lanes x 16 vectors)."""
    rs = resident_shape(w, read_only)
    nbytes = w.M * w.N * w.esize
    if rs is not None:
        waves, spl = rs
        return w.M, w.N * w.esize, waves, spl
    rb = 16 * 512 * 16
    if nbytes % rb == 0:
        return nbytes // rb, rb, 8, 16
    return None


def _time_launches(launch, R, steps, warmup, trials):
    """Mean device time per launch (us) over `steps` launches cycling over R
    buffer sets, bracketed by synchronisation and events on the current
    stream, and the p10 / p50 / p90 of `trials` further runs of up to 50."""
    import torch
    for i in range(warmup):
        launch(i % R)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        launch(i % R)
    b.record()
    b.synchronize()
    mean = a.elapsed_time(b) / steps * 1e3
    per = max(1, min(steps, 50))
    evs = [(torch.cuda.Event(enable_timing=True),
            torch.cuda.Event(enable_timing=True)) for _ in range(trials)]
    k = 0
    for e0, e1 in evs:
        e0.record()
        for _ in range(per):
            launch(k % R)
            k += 1
        e1.record()
    torch.cuda.synchronize()
    us = sorted(e0.elapsed_time(e1) / per * 1e3 for e0, e1 in evs)
    q = lambda f: round(us[int(f * (len(us) - 1) + 0.5)], 3) if us else None
    return mean, {"us_p10": q(0.1), "us_p50": q(0.5), "us_p90": q(0.9)}


def copy_gbps(nbytes, steps=50):
    """GB/s (read + write) of the in-tree copy kernel over nbytes, cut into
    128 KiB rows (512 lanes x 16 vectors), rotating over >= 1 GiB."""
    import torch
    import ceiling
    lib = ceiling.load()
    rb = 16 * 512 * 16
    rows = nbytes // rb
    if rows < 1:
        return None
    R = max(2, -(-ROTATE_BYTES // (2 * rows * rb)))
    src = [torch.ones(rows * rb // 4, device="cuda") for _ in range(R)]
    dst = [torch.empty(rows * rb // 4, device="cuda") for _ in range(R)]
    strm = torch.cuda.current_stream().cuda_stream
    mean, _ = _time_launches(lambda i: ceiling.check(lib.ceil_copy(
        src[i].data_ptr(), dst[i].data_ptr(), rows, rb, rb, 8, 16, strm),
        "ceil_copy"), R, steps, 10, 0)
    return round(2 * rows * rb / (mean * 1e-6) / 1e9, 1)


# Launch shapes (waves per workgroup, 16-byte vectors per lane) the copy
# sweep tries on the workload's bytes: one workgroup per 1 KiB to 128 KiB.
COPY_SHAPES = [(1, 1), (1, 2), (1, 4), (1, 8), (1, 16), (4, 1), (4, 2), (4, 4),
               (4, 8), (8, 1), (8, 2), (8, 4), (8, 8), (8, 16)]


def ceilings(w, steps=200, warmup=400, trials=20, full=True, read_only=False):
    """What this device reaches on the bytes of one softmax launch of
    workload w, cold (buffer sets rotating over >= 1 GiB), with no
    arithmetic: the in-tree copy, read-only and write-only kernels in the
    resident kernel's launch shape (ceiling/ceiling.hip), the same copy in
    every shape of COPY_SHAPES (the best one-launch copy of these bytes),
    the runtime's device-to-device copy, torch's copy, and the launch floor
    (an empty kernel back to back, one workgroup and the workload's grid).
    full=False: the same-shape copy alone (the counters' calibration
    kernel in profiler runs).  read_only: the launch shape of the
    statistics / cross-entropy pass in place of the softmax's."""
    import torch
    import ceiling
    lib = ceiling.load()
    shape = ceiling_shape(w, read_only)
    nbytes = w.M * w.N * w.esize
    R = max(2, -(-ROTATE_BYTES // (2 * nbytes)))
    src = [torch.full((nbytes // 4,), 1.0, device="cuda") for _ in range(R)]
    dst = [torch.empty(nbytes // 4, device="cuda") for _ in range(R)]
    sink = torch.zeros(max(shape[0] if shape else 1, 1), device="cuda")
    strm = torch.cuda.current_stream().cuda_stream
    out = {"rotating_sets": R}

    def rate(nb, us):
        return round(nb / (us * 1e-6) / 1e9, 1)

    if shape is not None:
        rows, rb, waves, spl = shape
        out["shape"] = {"grid": rows, "threads": 64 * waves,
                        "vectors_per_lane": spl, "row_bytes": rb}
        kern = {
            "copy": (lambda i: ceiling.check(lib.ceil_copy(
                src[i].data_ptr(), dst[i].data_ptr(), rows, rb, rb, waves,
                spl, strm), "ceil_copy"), 2 * nbytes),
            "read": (lambda i: ceiling.check(lib.ceil_read(
                src[i].data_ptr(), sink.data_ptr(), rows, rb, rb, waves, spl,
                strm), "ceil_read"), nbytes),
            "write": (lambda i: ceiling.check(lib.ceil_write(
                dst[i].data_ptr(), rows, rb, rb, waves, spl, strm),
                "ceil_write"), nbytes),
        }
        for k, (fn, nb) in kern.items():
            if not full and k != "copy":
                continue
            mean, dist = _time_launches(fn, R, steps, warmup, trials)
            out[k] = {"GBps": rate(nb, mean), "us": round(mean, 3),
                      "bytes": nb, **dist}
    if not full:
        del src, dst, sink
        torch.cuda.empty_cache()
        return out
    sweep = {}
    for waves, spl in COPY_SHAPES:
        rb = 16 * 64 * waves * spl
        if nbytes % rb:
            continue
        rows = nbytes // rb
        mean, _ = _time_launches(lambda i: ceiling.check(lib.ceil_copy(
            src[i].data_ptr(), dst[i].data_ptr(), rows, rb, rb, waves, spl,
            strm), "ceil_copy"), R, steps, warmup, 0)
        sweep[f"{rows}x{64 * waves}x{spl}"] = round(mean, 3)
    if sweep:
        best = min(sweep, key=sweep.get)
        out["copy_shapes_us"] = sweep
        out["best_copy"] = {"shape": best, "us": sweep[best],
                            "GBps": rate(2 * nbytes, sweep[best])}
    mean, dist = _time_launches(lambda i: ceiling.check(lib.ceil_memcpy(
        dst[i].data_ptr(), src[i].data_ptr(), nbytes, strm), "ceil_memcpy"),
        R, min(steps, 50), 10, trials)
    out["hip_memcpy_dtod"] = {"GBps": rate(2 * nbytes, mean),
                              "us": round(mean, 3), **dist}
    mean, dist = _time_launches(lambda i: dst[i].copy_(src[i]), R,
                                min(steps, 50), 10, trials)
    out["torch_copy"] = {"GBps": rate(2 * nbytes, mean), "us": round(mean, 3),
                         **dist}
    floor = {}
    grids = [(1, 64)]
    if shape is not None:
        grids.append((shape[0], 64 * shape[2]))
    for g, t in grids:
        mean, dist = _time_launches(lambda i: ceiling.check(
            lib.ceil_empty(g, t, strm), "ceil_empty"), 1, 1000, 1000, trials)
        floor[f"{g}x{t}"] = {"us": round(mean, 3), **dist}
    out["launch_floor"] = floor
    del src, dst, sink
    torch.cuda.empty_cache()
    return out


def host_threads():
    """Host cores this process may run on, at most 16 (one GPU's share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline_parallel(w, n_stats, budget_s):
    """The same fp64 softmax oracle called on T row blocks at once from T
    host threads (the C call releases the interpreter lock), until about
    budget_s seconds have passed: the oracle's rate on the host's cores."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    from row_wise_online_amd import workloads as wl
    x = wl.generate(w.name)
    T = min(host_threads(), w.M)
    blocks = [x[i * w.M // T:(i + 1) * w.M // T] for i in range(T)]
    b = 2 * w.M * w.N * w.esize + 4 * w.M * n_stats
    with ThreadPoolExecutor(T) as ex:
        reps, t0 = 0, time.perf_counter()
        while True:
            list(ex.map(oracle.softmax, blocks))
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 256:
                break
    per = el / reps
    return {"value": round(b / per / 1e9, 4), "unit": "GB/s", "cores": T,
            "kind": "oracle", "rows_per_s": round(w.M / per, 1),
            "sample": f"{reps} x full {w.M}x{w.N} {w.dtype} matrix, fp64 "
                      f"three-pass softmax oracle on {T} row blocks from "
                      f"{T} threads, {el:.1f} s"}


def cpu_baseline(w, n_stats, budget_s, op="softmax", causal=None):
    """The fp64 oracle, as it is, on this host: whole input matrices of the
    workload, repeated until about budget_s seconds have passed.  Returns
    the record and the oracle's result (the same every repetition)."""
    import numpy as np
    import oracle
    from row_wise_online_amd import workloads as wl
    x = wl.generate(w.name)
    if op == "cross_entropy":
        labels = np.random.default_rng(w.seed).integers(0, w.N, size=w.M)
        fn = lambda: oracle.cross_entropy(x, labels)
        what = "cross-entropy (loss, mean)"
        b = w.M * w.N * w.esize + 12 * w.M + 4
    elif op == "stats":
        fn = lambda: oracle.softmax(x, want_y=False)
        what = "row statistics (m, d, lse)"
        b = w.M * w.N * w.esize + 12 * w.M
    elif op == "normalize":
        # the oracle has no pass 2 of its own: its softmax forms the same y
        fn = lambda: oracle.softmax(x)
        what = "three-pass softmax (y, for pass 2 alone)"
        b = 2 * w.M * w.N * w.esize + 8 * w.M
    elif causal is not None:
        fn = lambda: oracle.softmax_masked(x, None, causal)
        what = f"causal (offset {causal}) softmax and log-softmax"
        b = (valid_elements(w, causal) + w.M * w.N) * w.esize
    elif op == "log_softmax":
        fn = lambda: oracle.log_softmax(x)
        what = "log-softmax"
        b = 2 * w.M * w.N * w.esize
    else:
        fn = lambda: oracle.softmax(x)
        what = "three-pass softmax (y, m, d, lse)"
        b = 2 * w.M * w.N * w.esize + 4 * w.M * n_stats
    reps, t0 = 0, time.perf_counter()
    while True:
        ref = fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 64:
            break
    per = el / reps
    return {"value": round(b / per / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "rows_per_s": round(w.M / per, 1),
            "sample": f"{reps} x full {w.M}x{w.N} {w.dtype} matrix, fp64 "
                      f"{what} oracle, 1 thread, {el:.1f} s"}, ref


def cpu_leg_accuracy(w, op, ref, outs):
    """How far the benched step's outputs (every row) are from the oracle's
    result that the CPU baseline just computed on the same input: max abs
    and max rel error of y (fp32) or its largest distance in bf16 steps
    from the correctly rounded value, the largest |lse - lse_ref|, whether
    m is bit-exact, the largest relative error of d, and of the loss."""
    import numpy as np
    import oracle
    acc = {"rows_checked": w.M, "reference": "fp64 oracle (cpu_baseline leg)"}

    def y_err(y, y_ref, log=False):
        fin = np.isfinite(y_ref)
        if y.dtype == np.uint16:
            want = oracle.round_f64_to_bf16_bits(y_ref[fin])
            acc["y_max_bf16_ulp"] = int(oracle.bf16_ulp_distance(
                y[fin], want).max(initial=0))
            yf = oracle.bf16_bits_to_f64(y[fin])
        else:
            yf = y[fin].astype(np.float64)
        err = np.abs(yf - y_ref[fin])
        acc["y_max_abs_err"] = float(err.max(initial=0.0))
        big = np.abs(y_ref[fin]) > (0.0 if log else 1e-30)
        acc["y_max_rel_err"] = float((err[big] / np.abs(y_ref[fin][big])).max(
            initial=0.0))

    if op == "softmax":
        if isinstance(ref, tuple) and len(ref) == 5:      # masked
            y_ref, _, m_ref, d_ref, l_ref = ref
        else:
            y_ref, m_ref, d_ref, l_ref = ref
        y_err(outs["y"], y_ref)
    elif op == "log_softmax":
        if isinstance(ref, tuple):
            _, y_ref, m_ref, d_ref, l_ref = ref
        else:
            y_ref, m_ref, d_ref, l_ref = ref, None, None, None
        y_err(outs["y"], y_ref, log=True)
    elif op == "normalize":
        y_ref, m_ref, d_ref, l_ref = ref
        y_err(outs["y"], y_ref)
        m_ref = d_ref = l_ref = None
    elif op == "stats":
        _, m_ref, d_ref, l_ref = ref
    else:
        l_ref, mean_ref = ref
        err = np.abs(outs["loss"].astype(np.float64) - l_ref)
        acc["loss_max_abs_err"] = float(err.max(initial=0.0))
        acc["mean_rel_err"] = float(abs(outs["mean"] - mean_ref) /
                                    abs(mean_ref))
        return acc
    if outs.get("m") is not None and m_ref is not None:
        acc["m_bit_exact"] = bool(np.array_equal(
            outs["m"].astype(np.float64), m_ref))
    if outs.get("d") is not None and d_ref is not None:
        acc["d_max_rel_err"] = float(np.max(np.abs(
            outs["d"].astype(np.float64) - d_ref) / d_ref))
    if outs.get("lse") is not None and l_ref is not None:
        acc["lse_max_abs_err"] = float(np.max(np.abs(
            outs["lse"].astype(np.float64) - l_ref)))
    return acc


def git_sha():
    """The commit the tree was built from, where git and the repository's
    history are at hand (a copy of the tree without .git gives None)."""
    import subprocess
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"],
                           capture_output=True, text=True, timeout=10)
    except (OSError, subprocess.SubprocessError):
        return None
    return r.stdout.strip() or None if r.returncode == 0 else None


def traffic_record(workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f).get(workload)
    family = "attention" if workload.startswith("a") else "softmax"
    if not rec or rec.get("kernel_hash") != kernel_source_hash(family):
        return None
    return rec.get("bytes_per_launch")


def run_workload(name, steps, warmup, path="auto", want_cpu=True,
                 cpu_budget=10.0, extras=True, op="softmax", causal=None):
    import row_wise_online_amd as rw
    from row_wise_online_amd import workloads as wl
    w = wl.WORKLOADS[name]
    if op == "normalize":
        resolved = "normalize"   # one kernel of its own, whatever the path
    else:
        resolved = rw.select_path(w.M, w.N, w.dtype, op=op) if path == "auto" else path
    n_stats = len(set(w.outputs) & {"m", "d", "lse"})
    if op == "cross_entropy":
        n_stats = 0
    if op == "stats":
        n_stats = 3
    if op == "normalize":
        n_stats = 0
        if causal is not None:
            raise ValueError("pass 2 alone takes no mask")
    if causal is not None and op == "cross_entropy":
        raise ValueError("the causal mask applies to softmax / log-softmax")
    # the ceilings first: they also bring the clocks up from idle before
    # the timed steps
    ro = op in ("stats", "cross_entropy")
    ceil = (ceilings(w, read_only=ro) if extras
            else ceilings(w, 50, 10, 0, full=False, read_only=ro))
    ms, R, host_us, dist, outs = measure(w, steps, warmup, path, op=op,
                                         causal=causal,
                                         trials=20 if extras else 0,
                                         keep=want_cpu)
    if extras:
        graph_ms = measure(w, steps, warmup, path, graph=True, op=op,
                           causal=causal)[0]
        warm_ms = measure(w, max(10, steps // 4), 3, path, rotate=False,
                          op=op, causal=causal)[0]
    nbytes = algorithmic_bytes(w, resolved, n_stats, op, causal)
    gbs = nbytes / (ms * 1e-3) / 1e9
    # the single-read minimum: x once and y once (x once for the read-only
    # passes), and the row statistics
    read_only = op in ("stats", "cross_entropy")
    eff = ((1 if read_only else 2) * w.M * w.N * w.esize + 4 * w.M * n_stats) \
        / (ms * 1e-3) / 1e9
    opname = {"softmax": "softmax", "log_softmax": "log-softmax",
              "cross_entropy": "cross-entropy",
              "stats": "row statistics (m, d, lse)",
              "normalize": "softmax pass 2 with a held row state"}[op]
    if causal is not None:
        opname = f"causal (offset {causal}) {opname}"
    rec = {
        "metric": METRIC if (name == "c2" and op == "softmax" and
                             causal is None) else
        f"achieved HBM GB/s (% of peak) + rows/s, online {opname} fwd "
        f"{w.dtype} {w.M}x{w.N}",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(gbs / PAGES_C2_GBS, 3) if (name == "c2" and op == "softmax"
                                                        and causal is None) else None),
        "dtype": "f32" if w.dtype == "f32" else "bf16",
        **({"vs_baseline_source": "the pages' register-cached one-read kernel, "
            "fp32 4096x4096, 1672 GB/s on an A100 80GB SXM4 (other hardware: "
            "context, not a target)"}
           if (name == "c2" and op == "softmax" and causal is None) else {}),
        "data": "synthetic (seeded numpy PCG64 normals, HBM-resident, "
                f"{R} rotating buffer sets)",
        "config": {"workload": w.desc, "M": w.M, "N": w.N, "op": op,
                   "causal_offset": causal,
                   "outputs": (["loss", "mean"] if op == "cross_entropy"
                               else ["m", "d", "lse"] if op == "stats"
                               else ["y"] if op == "normalize"
                               else list(w.outputs)), "path": resolved},
        "pct_of_peak": round(100.0 * gbs / PEAK_GBS, 2),
        "rows_per_s": round(w.M / (ms * 1e-3), 1),
        "effective_single_read_GBps": round(eff, 1),
        "effective_single_read_pct_of_peak": round(100.0 * eff / PEAK_GBS, 2),
        "bytes_counted": ("x read once, y written once, row statistics"
                          if resolved == "resident" or op in (
                              "stats", "cross_entropy", "normalize")
                          else "x read twice (pass 1 and pass 2; the second "
                               "read may be served by the Infinity Cache, so "
                               "value is not HBM bandwidth: the effective "
                               "single-read rate is), y written once, row "
                               "statistics" +
                               (", partial states" if resolved == "split"
                                else "")),
        "host_us_per_launch": round(host_us, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 1),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_GBS, 4),
            "traffic": traffic_record(name) if (op == "softmax" and
                                            causal is None) else None,
            "algorithmic_bytes_per_launch": nbytes,
            # split: partial states, then the normalise (or, for
            # statistics and cross-entropy, the state merge); the
            # cross-entropy adds its mean
            "kernel_launches_per_step": (2 if resolved == "split" else 1) +
                                        (1 if op == "cross_entropy" else 0),
        },
        "kernel_source": kernel_source_hash(),
    }
    if extras:
        if dist is not None:
            rec["per_launch_us"] = dist
        rec["warm_cache_GBps"] = round(nbytes / (warm_ms * 1e-3) / 1e9, 1)
        rec["graph_replay_GBps"] = round(nbytes / (graph_ms * 1e-3) / 1e9, 1)
    # the ceiling kernel of the same bytes: the copy (x read, y written), or
    # for the read-only passes the read-only kernel, in the resident
    # kernel's launch shape; and the best copy over the shapes tried
    ck = "read" if read_only else "copy"
    if ck in ceil:
        rec["copy_ceiling_GBps"] = ceil[ck]["GBps"]
        rec["roofline"]["ceiling_kernel"] = ck
        rec["roofline"]["frac_of_copy_ceiling"] = round(
            ceil[ck]["us"] / (ms * 1e3) * nbytes / ceil[ck]["bytes"], 4)
    if "best_copy" in ceil and not read_only:
        rec["roofline"]["frac_of_best_copy"] = round(
            ceil["best_copy"]["us"] / (ms * 1e3) * nbytes / (2 * w.M * w.N * w.esize), 4)
    if "launch_floor" in ceil:
        rec["launch_floor_us"] = {k: v["us"] for k, v in
                                  ceil["launch_floor"].items()}
    rec["ceilings"] = ceil
    rec["git_sha"] = git_sha()
    if want_cpu:
        base, ref = cpu_baseline(w, n_stats, cpu_budget, op, causal)
        rec["cpu_baseline"] = base
        if outs is not None:
            rec["accuracy"] = cpu_leg_accuracy(w, op, ref, outs)
        if op == "softmax" and causal is None and host_threads() > 1:
            rec["cpu_baseline_parallel"] = cpu_baseline_parallel(
                w, n_stats, cpu_budget / 2)
    return rec


def measure_attention(w, steps, warmup, graph=False):
    """Average device time per attention step (ms) and host time per launch
    (us) on the seeded inputs of attention workload w (bf16 output, fp32
    lse), timed with HIP events on the launch stream."""
    import numpy as np
    import torch
    import row_wise_online_amd as rw
    from row_wise_online_amd import workloads as wl
    dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = (dev(a) for a in wl.attention_workload(w.name))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device="cuda")
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    if not graph:
        call = rw.prepare_attention(q, k, v, o, lse=lse,
                                    causal_offset=w.causal)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        start.record()
        t0 = time.perf_counter()
        for _ in range(steps):
            call()
        host_us = (time.perf_counter() - t0) / steps * 1e6
        end.record()
        end.synchronize()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps, host_us
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call = rw.prepare_attention(q, k, v, o, lse=lse,
                                    causal_offset=w.causal,
                                    stream=torch.cuda.current_stream())
        for _ in range(steps):
            call()
    g.replay()
    torch.cuda.synchronize()
    start.record()
    t0 = time.perf_counter()
    g.replay()
    host_us = (time.perf_counter() - t0) / steps * 1e6
    end.record()
    end.synchronize()
    torch.cuda.synchronize()
    del g
    return start.elapsed_time(end) / steps, host_us


def cpu_baseline_attention(w, budget_s):
    """The fp64 attention oracle, as it is, on this host: whole query rows
    of the workload (each against all its admitted keys), one at a time,
    until about budget_s seconds have passed."""
    import numpy as np
    import oracle
    from row_wise_online_amd import workloads as wl
    q, k, v = wl.attention_workload(w.name)
    rng = np.random.default_rng(w.seed)
    rows = rng.integers(0, w.Sq, size=4096)
    flops, n, t0 = 0.0, 0, time.perf_counter()
    while True:
        i = int(rows[n % len(rows)])
        oracle.attention(q[0, 0], k[0, 0], v[0, 0], causal=w.causal, rows=[i])
        keys = w.Sk if w.causal < 0 else min(w.Sk, i + w.causal + 1)
        flops += 4.0 * keys * w.D
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": round(flops / el / 1e12, 8), "unit": "TFLOP/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{n} random query rows of {w.Sq}x{w.Sk} d={w.D} "
                      f"(head 0), fp64 definition oracle, 1 thread, "
                      f"{el:.1f} s"}


def cpu_baseline_attention_parallel(w, budget_s):
    """The same fp64 attention oracle on T host threads at once (the C call
    releases the interpreter lock), each taking its own random query rows,
    until about budget_s seconds have passed."""
    from concurrent.futures import ThreadPoolExecutor
    import numpy as np
    import oracle
    from row_wise_online_amd import workloads as wl
    q, k, v = wl.attention_workload(w.name)
    T = host_threads()
    t0 = time.perf_counter()

    def worker(t):
        rows = np.random.default_rng(w.seed + 1 + t).integers(0, w.Sq, size=4096)
        flops, n = 0.0, 0
        while True:
            i = int(rows[n % len(rows)])
            oracle.attention(q[0, 0], k[0, 0], v[0, 0], causal=w.causal, rows=[i])
            keys = w.Sk if w.causal < 0 else min(w.Sk, i + w.causal + 1)
            flops += 4.0 * keys * w.D
            n += 1
            if time.perf_counter() - t0 >= budget_s:
                return flops, n

    with ThreadPoolExecutor(T) as ex:
        res = list(ex.map(worker, range(T)))
    el = time.perf_counter() - t0
    flops = sum(r[0] for r in res)
    n = sum(r[1] for r in res)
    return {"value": round(flops / el / 1e12, 8), "unit": "TFLOP/s",
            "cores": T, "kind": "oracle",
            "sample": f"{n} random query rows of {w.Sq}x{w.Sk} d={w.D} "
                      f"(head 0), fp64 definition oracle, {T} threads, "
                      f"{el:.1f} s"}


def run_attention(name, steps, warmup, want_cpu=True, cpu_budget=10.0,
                  extras=True):
    from row_wise_online_amd import workloads as wl
    w = wl.ATTN_WORKLOADS[name]
    ms, host_us = measure_attention(w, steps, warmup)
    flops = w.flops()
    tf = flops / (ms * 1e-3) / 1e12
    rec = {
        "metric": f"attention fwd TFLOP/s, online softmax inside key tiles, "
                  f"bf16 {w.B}x{w.H}x{w.Sq}x{w.Sk} d={w.D}"
                  + (" causal" if w.causal >= 0 else ""),
        "value": round(tf, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded numpy PCG64 normals, HBM-resident)",
        "config": {"workload": w.desc, "B": w.B, "H": w.H, "Sq": w.Sq,
                   "Sk": w.Sk, "D": w.D, "causal_offset": w.causal,
                   "outputs": ["o (bf16)", "lse (fp32)"], "op": "attention"},
        "host_us_per_launch": round(host_us, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(tf, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_record(name),
            "algorithmic_flops_per_launch": flops,
            "kernel_launches_per_step": 1,
        },
        "kernel_source": kernel_source_hash("attention"),
    }
    if extras:
        gms, _ = measure_attention(w, steps, 1, graph=True)
        rec["graph_replay_TFLOPs"] = round(flops / (gms * 1e-3) / 1e12, 2)
    # a plain copy of Q's size (the in-tree copy kernel): the calibration
    # kernel for the HBM counters
    rec["copy_ceiling_GBps"] = copy_gbps(w.B * w.H * w.Sq * w.D * 2)
    if want_cpu:
        rec["cpu_baseline"] = cpu_baseline_attention(w, cpu_budget)
        if host_threads() > 1:
            rec["cpu_baseline_parallel"] = cpu_baseline_attention_parallel(
                w, cpu_budget / 2)
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 1000; 20 for attention)")
    # the clocks take ~10 ms of sustained launches to settle after setup
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps (default 2000; 3 for attention)")
    ap.add_argument("--workload", default=None,
                    choices=["c1", "c2", "c3", "c4", "c5", "a2", "a3", "a4",
                             "a5"],
                    help="default c2 (a2 for --op attention)")
    ap.add_argument("--path", default="auto",
                    choices=["auto", "resident", "stream", "split"])
    ap.add_argument("--op", default="softmax",
                    choices=["softmax", "log_softmax", "cross_entropy",
                             "stats", "normalize", "attention"])
    ap.add_argument("--causal", type=int, default=None,
                    help="causal mask offset (softmax / log-softmax)")
    ap.add_argument("--all", action="store_true",
                    help="also report every workload on stderr")
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the headline loop and the same-shape "
                         "copy (the counters' calibration; profiler runs)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build measures the "
              "single-GPU hot path (rows shard across GPUs with no "
              "communication, see the design notes); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    att = args.op == "attention"
    if args.workload is None:
        args.workload = "a2" if att else "c2"
    if att != args.workload.startswith("a"):
        print("--op attention takes workloads a2..a5; the row-wise ops "
              "c1..c5", file=sys.stderr)
        sys.exit(2)
    if args.steps is None:
        args.steps = 20 if att else 1000
    if args.warmup is None:
        args.warmup = 3 if att else 2000

    import torch
    import row_wise_online_amd as rw
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    rw.load()

    if args.all:
        for op in ["softmax", "log_softmax", "cross_entropy", "stats",
                   "normalize"]:
            for name in ["c1", "c2", "c3", "c4", "c5"]:
                print(f"[bench] {op} workload {name}", file=sys.stderr,
                      flush=True)
                r = run_workload(name, args.steps, args.warmup, "auto",
                                 want_cpu=False, extras=not args.no_extras,
                                 op=op)
                print(json.dumps(r), file=sys.stderr, flush=True)
        for name in ["c2", "c3"]:
            print(f"[bench] causal softmax workload {name}", file=sys.stderr,
                  flush=True)
            r = run_workload(name, args.steps, args.warmup, "auto",
                             want_cpu=False, extras=not args.no_extras,
                             causal=0)
            print(json.dumps(r), file=sys.stderr, flush=True)
        if not att:
            for name in ["a2", "a3", "a4", "a5"]:
                print(f"[bench] attention workload {name}", file=sys.stderr,
                      flush=True)
                r = run_attention(name, 20, 3, want_cpu=False,
                                  extras=not args.no_extras)
                print(json.dumps(r), file=sys.stderr, flush=True)
    print(f"[bench] headline workload {args.workload}", file=sys.stderr,
          flush=True)
    if att:
        rec = run_attention(args.workload, args.steps, args.warmup,
                            want_cpu=not args.no_cpu,
                            cpu_budget=args.cpu_budget,
                            extras=not args.no_extras)
        print(json.dumps(rec), flush=True)
        return
    rec = run_workload(args.workload, args.steps, args.warmup, args.path,
                       want_cpu=not args.no_cpu, cpu_budget=args.cpu_budget,
                       extras=not args.no_extras, op=args.op,
                       causal=args.causal)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
