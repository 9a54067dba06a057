/*
 * os_softmax -- row-wise online softmax for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every entry point takes plain device pointers, 64-bit sizes and a
 * hipStream_t; nothing here allocates device memory or keeps a pointer after
 * it returns.  All compute runs in the library's HIP kernels.
 *
 * What is computed (per row i of x[M,N]):
 *   m_i   = max_j x_ij                               (the running max)
 *   d_i   = sum_j e^(x_ij - m_i)                     (the normaliser)
 *   y_ij  = e^(x_ij - m_i) / d_i                     (softmax)
 *   lse_i = m_i + log d_i                            (log-sum-exp)
 *   y_ij  = x_ij - lse_i                             (log-softmax)
 *   loss_i = lse_i - x_{i,c_i}                       (cross-entropy, label c_i)
 * The pass that produces (m, d) keeps a running state and combines partial
 * states with the associative merge
 *   m = max(m_a, m_b),  d = d_a e^(m_a - m) + d_b e^(m_b - m),
 * as derived in "5.2 CUDA Online Softmax 实现优化" (AIInfraGuide), §2.1
 * (recurrence), §2.2 (two passes), §4.1 (merge); the same state and merge
 * appear in "Softmax 数值稳定性与 IO-Aware Attention：从在线归一化到
 * FlashAttention" §4 and §4.1.  log-sum-exp and log-softmax as defined in
 * "从原始Softmax到在线Softmax" (section deriving the stable form); the
 * cross-entropy of a labelled row, -log p_label, and its batch mean from the
 * same page's cross-entropy section.
 *
 * Conventions shared by all entry points
 *  - Layout: x and y are row-major; element (i, j) sits at base + i*ld + j
 *    (ld in elements, ld >= N).  Statistics are fp32.
 *  - dtype: OS_F32 (x, y are float) or OS_BF16 (x, y are bfloat16 bit
 *    patterns, 2 bytes each; arithmetic is fp32, y is rounded to nearest
 *    even).  y always has the dtype of x.
 *  - Asynchrony: every call enqueues work on `stream` and returns; outputs
 *    are valid once the stream reaches that point.  Multi-kernel paths are
 *    ordered by the stream alone (no host sync, no atomics).  Calls of more
 *    than 2^22 rows are enqueued as launches over consecutive runs of at
 *    most 2^22 rows (a launch counts its threads in 32 bits), with the same
 *    results per row as one launch would give.
 *  - Validation happens on the host; an invalid call enqueues nothing.
 *    Arguments are checked first, before any HIP call (M == 0 is a valid
 *    no-op).  Then the current device is read (hipGetDevice; its
 *    compute-unit count and architecture are cached per device on first
 *    use, thread-safely): OS_ERR_DEVICE unless it is a gfx950.  Last come
 *    the checks that depend on the device's plan (the workspace size).
 *    The stream must belong to the current device, as for any launch.
 *  - Plans: the path AUTO takes, the grids and the workspace size are pure
 *    functions of the shape and the device's CU count (os_softmax_plan);
 *    MI355X has 256 CUs, a partitioned device fewer.
 *  - HIP errors: a failed launch returns OS_ERR_HIP (from hipGetLastError,
 *    which may also report an earlier, unrelated error left on the thread).
 *  - Alignment is never an error: 16-byte vector memory operations are used
 *    when both bases and both row pitches are 16-byte aligned, element
 *    operations otherwise.
 *  - Aliasing: y == x with ld_y == ld_x (in place) is allowed; any other
 *    overlap between inputs and outputs is undefined.
 *  - Determinism: the work partition is a pure function of (M, N, dtype,
 *    path, alignment class, CU count) and no atomics are used, so repeated calls give
 *    bit-identical results.  Different paths round differently (within the
 *    documented accuracy).
 *  - Special values: an element -inf has weight 0; a row of only -inf gives
 *    m = -inf, d = 0, lse = -inf, y = NaN.  A NaN element makes d, lse and
 *    the row of y NaN (m is the max of the other elements); a +inf element
 *    gives m = +inf and a NaN row.
 */
#ifndef OS_SOFTMAX_H
#define OS_SOFTMAX_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

/* In C++ the enums below take int, the type of a C enum's values, as their
 * fixed underlying type: then every int a C caller passes is a value of the
 * enum type, which the library checks and rejects with a status when it is
 * not one of the enumerators (without a fixed type, C++ leaves values
 * outside the enumerators' bit range undefined). */
#ifdef __cplusplus
#define OS_ENUM_BASE : int
#else
#define OS_ENUM_BASE
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum OS_ENUM_BASE {
    OS_OK = 0,
    OS_ERR_NULL = 1,        /* a required pointer is NULL */
    OS_ERR_SHAPE = 2,       /* M < 0 or M > 2^31-1, N < 1 or N > 2^30, K < 1 */
    OS_ERR_STRIDE = 3,      /* ld < N (or ld_in < K), inc_out < 1 */
    OS_ERR_DTYPE = 4,       /* unknown dtype */
    OS_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
    OS_ERR_PATH = 6,        /* unknown path value */
    OS_ERR_UNSUPPORTED = 7, /* forced path cannot take this shape */
    OS_ERR_HIP = 8,         /* a HIP launch reported an error */
    OS_ERR_DEVICE = 9       /* no current device, or it is not a gfx950 (the
                               only architecture the kernels are built for);
                               os_softmax_plan: cu_count < 1 */
} os_status;

typedef enum OS_ENUM_BASE { OS_F32 = 0, OS_BF16 = 1 } os_dtype;

/* Execution paths.
 *  RESIDENT: each row is loaded once into registers, reduced, and
 *            normalised from registers (one read + one write of x).  Rows of
 *            up to 32768 elements.  ("5.2 CUDA Online Softmax 实现优化" §6,
 *            register-cached one-read version.)  For statistics and
 *            cross-entropy: the same kernel without pass 2.
 *  STREAM:   one workgroup per row; pass 1 streams the row folding (m, d),
 *            pass 2 re-reads it and writes y (two reads + one write).  Any N.
 *            For statistics and cross-entropy: pass 1 only (one read).
 *  SPLIT:    several workgroups per row: a partial-state kernel, then a
 *            normalise kernel whose workgroups first merge their row's
 *            partial states (for statistics and cross-entropy, the
 *            state-merge kernel instead); §7.1 of the same page names this
 *            two-stage scheme for few, very long rows.
 *  AUTO:     choose by shape: os_softmax_select_path for the softmax and
 *            log-softmax entry points, os_softmax_stats_select_path for
 *            the statistics and cross-entropy ones. */
typedef enum OS_ENUM_BASE {
    OS_PATH_AUTO = 0,
    OS_PATH_RESIDENT = 1,
    OS_PATH_STREAM = 2,
    OS_PATH_SPLIT = 3
} os_path;

/* Softmax forward: both passes of "5.2 CUDA Online Softmax 实现优化" §2.2
 * (pass 1 folds each row into its running state (m, d) by the recurrence of
 * §2.1, partial states combining by the merge of §4.1; pass 2 writes
 * y = e^(x - m) / d), on the path os_softmax_select_path picks.
 *  x        [M, ld_x] input, dtype dt (read only).
 *  y        [M, ld_y] output, dtype dt.
 *  m_out, d_out, lse_out  nullable fp32 [M]: the row's (m, d) as defined
 *           above (m is exactly the row max) and m + log d.
 *  ws       device workspace of at least os_softmax_workspace_bytes(M, N,
 *           dt, OS_PATH_AUTO) bytes, 256-byte aligned; may be NULL when that
 *           size is 0.  The library only uses it during the enqueued work.
 *  Returns OS_OK or the first validation error (nothing is enqueued then). */
os_status os_softmax_fwd(const void *x, int64_t ld_x, void *y, int64_t ld_y,
                         int64_t M, int64_t N, os_dtype dt,
                         float *m_out, float *d_out, float *lse_out,
                         void *ws, size_t ws_bytes, hipStream_t stream);

/* os_softmax_fwd on a caller-chosen path (AUTO behaves as os_softmax_fwd).
 * OS_ERR_UNSUPPORTED if the path cannot take the shape (RESIDENT with
 * N > 32768).  The workspace must cover os_softmax_workspace_bytes(M, N, dt,
 * path). */
os_status os_softmax_fwd_path(const void *x, int64_t ld_x, void *y,
                              int64_t ld_y, int64_t M, int64_t N,
                              os_dtype dt, float *m_out, float *d_out,
                              float *lse_out, void *ws, size_t ws_bytes,
                              os_path path, hipStream_t stream);

/* os_softmax_fwd_path for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid
 * allocation): the split path's workspace (partial and row states) is a
 * fixed 256 KiB array in device memory that the library holds, one copy
 * per device, from the first call on that device until the process ends;
 * there is no ws argument and nothing is allocated.
 *  - A plan that needs more than 256 KiB returns OS_ERR_WORKSPACE and
 *    enqueues nothing.  AUTO never does at 256 CUs (its largest split
 *    workspace, fewer than 512 rows, is under 25 KiB); forcing SPLIT on
 *    many rows can (about 16 bytes per row and chunk).
 *  - The array keeps the last call's contents; nothing in it has to start
 *    at any value (every partial state is written before it is read).
 *  - Every call on one device shares that device's array: calls that
 *    overlap on one device (other streams, other host threads) race and
 *    give wrong results.  Order them on one stream or with events.
 *  - The device address of the array is read once per device, on the first
 *    call with that device current (hipGetSymbolAddress); OS_ERR_HIP if it
 *    cannot be read.
 * Everything else (arguments, paths, results, errors) as
 * os_softmax_fwd_path; results are bit-identical to os_softmax_fwd_path
 * with a caller workspace. */
os_status os_softmax_fwd_noalloc(const void *x, int64_t ld_x, void *y,
                                 int64_t ld_y, int64_t M, int64_t N,
                                 os_dtype dt, float *m_out, float *d_out,
                                 float *lse_out, os_path path,
                                 hipStream_t stream);

/* Pass 1 only: the (m, d) state of each row, written to m_out[i*inc_out]
 * and d_out[i*inc_out] (both required, fp32), and optionally
 * lse_out[i*inc_out].  Called on a column window (x advanced by a column
 * offset, N the window width) it gives that window's partial state, which
 * os_state_merge combines with other windows' states ("Softmax 数值稳定性与
 * IO-Aware Attention" §4.1: chunk a row, take each chunk's state, merge). */
os_status os_softmax_stats(const void *x, int64_t ld_x, int64_t M, int64_t N,
                           os_dtype dt, float *m_out, float *d_out,
                           int64_t inc_out, float *lse_out, void *ws,
                           size_t ws_bytes, hipStream_t stream);

/* os_softmax_stats on a chosen path: RESIDENT (the register-resident row
 * kernel without pass 2; N <= 32768, else OS_ERR_UNSUPPORTED), STREAM (one
 * workgroup per row) or SPLIT (several per row, then the merge kernel). */
os_status os_softmax_stats_path(const void *x, int64_t ld_x, int64_t M,
                                int64_t N, os_dtype dt, float *m_out,
                                float *d_out, int64_t inc_out, float *lse_out,
                                void *ws, size_t ws_bytes, os_path path,
                                hipStream_t stream);

/* Log-softmax forward: y_ij = x_ij - lse_i, written as (x_ij - m_i) - log d_i
 * ("从原始Softmax到在线Softmax", stable-form section).  Arguments, paths,
 * workspace, layout and errors as os_softmax_fwd / os_softmax_fwd_path;
 * y has the dtype of x. */
os_status os_log_softmax_fwd(const void *x, int64_t ld_x, void *y,
                             int64_t ld_y, int64_t M, int64_t N, os_dtype dt,
                             float *m_out, float *d_out, float *lse_out,
                             void *ws, size_t ws_bytes, hipStream_t stream);

os_status os_log_softmax_fwd_path(const void *x, int64_t ld_x, void *y,
                                  int64_t ld_y, int64_t M, int64_t N,
                                  os_dtype dt, float *m_out, float *d_out,
                                  float *lse_out, void *ws, size_t ws_bytes,
                                  os_path path, hipStream_t stream);

/* Softmax / log-softmax over masked rows: row i takes part only through its
 * first n_i columns, n_i = N lowered to row_len[i] (clipped at 0) when
 * row_len (int32 [M] device array, nullable) is given, and to
 * i + causal_offset + 1 when causal_offset >= 0 (a causal mask; a negative
 * value means no causal mask).  Masked columns are not read; they behave as
 * -inf elements: y = 0 (softmax) or -inf (log-softmax) there, and a row with
 * n_i = 0 is all NaN with m = -inf, d = 0, lse = -inf.  ("Softmax 数值稳定性与
 * IO-Aware Attention" §9.2 lists mask boundaries among the edge cases.)
 * Everything else as os_softmax_fwd_path / os_log_softmax_fwd_path. */
os_status os_softmax_fwd_masked(const void *x, int64_t ld_x, void *y,
                                int64_t ld_y, int64_t M, int64_t N,
                                os_dtype dt, const int32_t *row_len,
                                int64_t causal_offset, float *m_out,
                                float *d_out, float *lse_out, void *ws,
                                size_t ws_bytes, os_path path,
                                hipStream_t stream);

os_status os_log_softmax_fwd_masked(const void *x, int64_t ld_x, void *y,
                                    int64_t ld_y, int64_t M, int64_t N,
                                    os_dtype dt, const int32_t *row_len,
                                    int64_t causal_offset, float *m_out,
                                    float *d_out, float *lse_out, void *ws,
                                    size_t ws_bytes, os_path path,
                                    hipStream_t stream);

/* Cross-entropy forward from logits ("从原始Softmax到在线Softmax",
 * cross-entropy section): one read of x.
 *  labels    int64 [M] device array, required.  A negative label marks a row
 *            to ignore: its loss is -0.0 (equal to 0 in any comparison; the
 *            sign marks the row as left out of the mean, and no computed
 *            loss is -0.0) and it is left out of the mean.  A label >= N
 *            gives a NaN loss (and so a NaN mean).
 *  loss_out  fp32 [M], required: lse_i - x_{i,label_i}.
 *  lse_out   fp32 [M], nullable.
 *  mean_out  fp32 scalar, nullable: the mean loss over rows whose label is
 *            not negative (NaN when there are none; computed by one more
 *            single-workgroup kernel in a fixed order, so deterministic).
 * Paths, workspace and errors as os_softmax_stats(_path). */
os_status os_cross_entropy_fwd(const void *x, int64_t ld_x, int64_t M,
                               int64_t N, os_dtype dt, const int64_t *labels,
                               float *loss_out, float *lse_out,
                               float *mean_out, void *ws, size_t ws_bytes,
                               hipStream_t stream);

os_status os_cross_entropy_fwd_path(const void *x, int64_t ld_x, int64_t M,
                                    int64_t N, os_dtype dt,
                                    const int64_t *labels, float *loss_out,
                                    float *lse_out, float *mean_out, void *ws,
                                    size_t ws_bytes, os_path path,
                                    hipStream_t stream);

/* Streaming statistics: fold the state of this column window into a
 * running per-row state, in place.  m_io[i*inc], d_io[i*inc] (fp32,
 * required) hold the running (m, d) of the columns seen so far -- start from
 * the identity (-inf, 0) -- and receive the merge of it with this window's
 * state ("Softmax 数值稳定性与 IO-Aware Attention" §4.1: chunk the row, take
 * each chunk's state, merge repeatedly; "从原始Softmax到在线Softmax": the state
 * is updated block by block).  lse_out (nullable) receives the LSE of the
 * merged state.  Calls on the same stream apply in order.  Paths, workspace
 * and errors as os_softmax_stats_path. */
os_status os_softmax_stats_update(const void *x, int64_t ld_x, int64_t M,
                                  int64_t N, os_dtype dt, float *m_io,
                                  float *d_io, int64_t inc, float *lse_out,
                                  void *ws, size_t ws_bytes, os_path path,
                                  hipStream_t stream);

/* Pass 2 alone, for a row state the caller already holds: for i < M,
 * j < N,
 *   os_softmax_normalize:      y[i*ld_y + j] = e^(x[i*ld_x + j] - m_i) / d_i
 *   os_log_softmax_normalize:  y[i*ld_y + j] = (x[i*ld_x + j] - m_i) - log d_i
 * with m_i = m_in[i*inc], d_i = d_in[i*inc] (fp32, device, read only).  The
 * outputs of a column window need only its row's final state, however that
 * state was reached: os_softmax_stats over the whole row, the statistics of
 * several windows merged by os_softmax_stats_update or os_state_merge, or
 * states gathered from other devices ("5.2 CUDA Online Softmax 实现优化"
 * §7.1, the second stage of a split row; "Softmax 数值稳定性与 IO-Aware
 * Attention：从在线归一化到FlashAttention" §4.1, the merged state).  So x
 * may be a window of a longer row: the call then writes that window of the
 * row's softmax.
 *  x, y     device, M rows of N elements, row pitches ld_x, ld_y >= N; y
 *           has x's dtype; y == x with ld_y == ld_x (in place) is allowed.
 *  m_in, d_in  the row states; the state must cover the elements of x
 *           (m_i at least their max, d_i their sum of e^(x - m_i) together
 *           with any other columns of the row), as the functions above
 *           produce.  The identity (-inf, 0) gives a NaN row, like a row of
 *           only -inf.
 *  inc      stride between the states of consecutive rows, >= 1.
 * One read of x and one write of y, on `stream`; no workspace.  Errors:
 * OS_ERR_SHAPE, OS_ERR_DTYPE, OS_ERR_STRIDE (a pitch < N or inc < 1),
 * OS_ERR_NULL (x, y, m_in or d_in NULL with M > 0), OS_ERR_HIP. */
os_status os_softmax_normalize(const void *x, int64_t ld_x, void *y,
                               int64_t ld_y, int64_t M, int64_t N,
                               os_dtype dt, const float *m_in,
                               const float *d_in, int64_t inc,
                               hipStream_t stream);
os_status os_log_softmax_normalize(const void *x, int64_t ld_x, void *y,
                                   int64_t ld_y, int64_t M, int64_t N,
                                   os_dtype dt, const float *m_in,
                                   const float *d_in, int64_t inc,
                                   hipStream_t stream);

/* Merge K partial states per row ("5.2 CUDA Online Softmax 实现优化" §4.1):
 * row i's states are (m_in[i*ld_in + k], d_in[i*ld_in + k]), k < K, fp32.
 * (-inf, 0) is an exact identity.  Writes m_out[i], d_out[i] (required) and
 * lse_out[i] (nullable).  Outputs must not overlap the inputs. */
os_status os_state_merge(const float *m_in, const float *d_in, int64_t ld_in,
                         int64_t M, int64_t K, float *m_out, float *d_out,
                         float *lse_out, hipStream_t stream);

/* The launch plan of a row-wise call, as os_softmax_plan describes it. */
typedef struct {
    os_path path;            /* the path taken (AUTO resolved) */
    int32_t chunks_per_row;  /* SPLIT: workgroups per row (P); else 1 */
    int64_t chunk_len;       /* SPLIT: elements per chunk (C, the last
                                chunk of a row shorter); else N */
    size_t workspace_bytes;  /* workspace the call needs (0 unless SPLIT) */
} os_plan;

/* The plan of a row-wise call of shape (M, N, dt) on `path` for a device
 * with cu_count compute units.  read_only != 0: the statistics and
 * cross-entropy entry points (their AUTO rule streams rows longer than
 * 16384 elements when rows are many), else softmax / log-softmax.
 * A pure host function (no HIP call), for sizing buffers ahead of time and
 * for checking the plans on a machine without a GPU.  The rules, scaled by
 * cu_count (MI355X: 256):
 *   AUTO     RESIDENT when N <= 32768 and (M >= 2 cu_count or N <= 4096),
 *            except read-only calls with N > 16384 and M >= 2 cu_count,
 *            which STREAM; otherwise STREAM when M >= 2 cu_count, else
 *            SPLIT.
 *   SPLIT    rows cut into chunks of a multiple of 4096 elements, about
 *            8 cu_count workgroups in all ("5.2 CUDA Online Softmax 实现
 *            优化" §7.1, several blocks per long row and a second stage);
 *            workspace: two tables of M P floats and two of M floats, each
 *            rounded up to 256 bytes.
 * Errors: OS_ERR_DTYPE, OS_ERR_SHAPE, OS_ERR_PATH, OS_ERR_NULL (out),
 * OS_ERR_DEVICE (cu_count < 1), OS_ERR_UNSUPPORTED (RESIDENT with
 * N > 32768). */
os_status os_softmax_plan(int64_t M, int64_t N, os_dtype dt, os_path path,
                          int read_only, int cu_count, os_plan *out);

/* Workspace bytes that every row-wise entry point (softmax, log-softmax,
 * statistics, cross-entropy) needs for this shape and path on the current
 * device (0 unless the split path is taken): os_softmax_plan for the
 * device's CU count.  Returns 0 for invalid arguments, and when no gfx950
 * device is current (a call would then fail with OS_ERR_DEVICE). */
size_t os_softmax_workspace_bytes(int64_t M, int64_t N, os_dtype dt,
                                  os_path path);

/* The path AUTO resolves to at this shape on the current device for the
 * softmax and log-softmax entry points, masked or not.  OS_PATH_AUTO for
 * an invalid shape or dtype, or when no gfx950 device is current. */
os_path os_softmax_select_path(int64_t M, int64_t N, os_dtype dt);

/* The path AUTO resolves to for the read-only entry points
 * (os_softmax_stats*, os_softmax_stats_update, os_cross_entropy_fwd*):
 * that of os_softmax_select_path, except that with 2 rows per CU or more,
 * rows longer than 16384 elements take STREAM rather than RESIDENT (nothing
 * is kept for a pass 2).  The workspace size is the same either way
 * (OS_PATH_AUTO for an invalid shape or dtype, or no gfx950 device). */
os_path os_softmax_stats_select_path(int64_t M, int64_t N, os_dtype dt);

/* Static description of a status code (never NULL). */
const char *os_status_string(os_status s);

#ifdef __cplusplus
}
#endif
#endif /* OS_SOFTMAX_H */
