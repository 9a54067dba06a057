// C ABI of the row-wise online softmax library: argument validation (on the
// host, before any HIP call), path selection and launches.
#include <mutex>
#include <stdint.h>

#include "../../include/os_softmax.h"
#include "chunks.hpp"
#include "launch.hpp"

namespace {

constexpr int64_t kMaxN = int64_t(1) << 30;  // keeps in-row int indexing exact
constexpr int64_t kMaxM = (int64_t(1) << 31) - 1;

int esize(os_dtype dt) { return dt == OS_BF16 ? 2 : 4; }

bool aligned16(const void *p, int64_t ld, os_dtype dt) {
    return (reinterpret_cast<uintptr_t>(p) % 16 == 0) &&
           ((ld * esize(dt)) % 16 == 0);
}

os_status check_shape(int64_t M, int64_t N, os_dtype dt) {
    if (dt != OS_F32 && dt != OS_BF16) return OS_ERR_DTYPE;
    if (M < 0 || M > kMaxM || N < 1 || N > kMaxN) return OS_ERR_SHAPE;
    return OS_OK;
}

bool valid_path(os_path p) { return p >= OS_PATH_AUTO && p <= OS_PATH_SPLIT; }

// The current device, if it is one the kernels run on.
const os::Device *usable_device() {
    const os::Device *dev = os::current_device();
    return (dev != nullptr && dev->gfx950) ? dev : nullptr;
}

// Validation shared by every row-wise entry point once the pointers that
// the mode requires are known to be present.  What does not depend on the
// device is checked first, before any HIP call: the forced path's shape
// limit, and a split path forced without a workspace.  Then the current
// device (OS_ERR_DEVICE unless it is a gfx950), AUTO resolved for its CU
// count, and the workspace size of that plan.
os_status resolve(int64_t M, int64_t N, os_path path, void *ws,
                  size_t ws_bytes, os_path *out, int *cus,
                  bool read_only = false) {
    if (path == OS_PATH_RESIDENT && N > os::kResidentMaxN) return OS_ERR_UNSUPPORTED;
    if (path == OS_PATH_SPLIT && ws == nullptr) return OS_ERR_WORKSPACE;
    const os::Device *dev = usable_device();
    if (dev == nullptr) return OS_ERR_DEVICE;
    const os_path p = (path == OS_PATH_AUTO)
                          ? os::select_path(M, N, read_only, dev->cus)
                          : path;
    const size_t need = os::workspace_for(M, N, p, dev->cus);
    if (need > 0 && (ws == nullptr || ws_bytes < need)) return OS_ERR_WORKSPACE;
    *out = p;
    *cus = dev->cus;
    return OS_OK;
}

// Rows [r0, r0 + n) of a call as a call of its own: every per-row pointer
// moves to row r0, and a causal offset is taken relative to the new row 0.
os::FwdArgs rows_of(const os::FwdArgs &a, int64_t r0, int64_t n) {
    const int64_t es = a.dt == os::Dt::F32 ? 4 : 2;
    os::FwdArgs c = a;
    c.M = n;
    c.x = static_cast<const char *>(a.x) + r0 * a.ldx * es;
    if (a.y) c.y = static_cast<char *>(a.y) + r0 * a.ldy * es;
    if (a.m_out) c.m_out = a.m_out + r0 * a.inc_out;
    if (a.d_out) c.d_out = a.d_out + r0 * a.inc_out;
    if (a.lse_out) c.lse_out = a.lse_out + r0 * a.inc_out;
    if (a.labels) c.labels = a.labels + r0;
    if (a.loss) c.loss = a.loss + r0;
    if (a.row_len) c.row_len = a.row_len + r0;
    if (a.causal >= 0) c.causal = a.causal + r0;
    return c;
}

// One launch per part of at most 2^22 rows (the grid of a launch counts
// work-items in 32 bits); the parts run in stream order and share the
// workspace, which each part's plan fits in.
os_status launch(const os::FwdArgs &a, os_path p, void *ws) {
    const os::RowChunks rc = os::row_chunks(a.M);
    for (int64_t c = 0; c < rc.count; ++c) {
        const int64_t r0 = c * rc.rows;
        const int64_t n = a.M - r0 < rc.rows ? a.M - r0 : rc.rows;
        const os::FwdArgs part = rc.count == 1 ? a : rows_of(a, r0, n);
        switch (p) {
            case OS_PATH_RESIDENT: os::launch_resident(part); break;
            case OS_PATH_STREAM: os::launch_stream(part); break;
            default: os::launch_split(part, ws); break;
        }
        if (hipGetLastError() != hipSuccess) return OS_ERR_HIP;
    }
    return OS_OK;
}

os::FwdArgs make_args(const void *x, int64_t ld_x, void *y, int64_t ld_y,
                      int64_t M, int64_t N, os_dtype dt, os::Mode mode,
                      int cus, hipStream_t stream) {
    os::FwdArgs a{};
    a.x = x;
    a.ldx = ld_x;
    a.y = y;
    a.ldy = ld_y;
    a.M = M;
    a.N = static_cast<int>(N);
    a.mode = mode;
    a.inc_out = 1;
    a.causal = -1;
    a.dt = dt == OS_F32 ? os::Dt::F32 : os::Dt::BF16;
    a.vec = aligned16(x, ld_x, dt) && (y == nullptr || aligned16(y, ld_y, dt));
    a.cus = cus;
    a.stream = stream;
    return a;
}

// softmax and log-softmax forward (masked when row_len or causal >= 0)
os_status fwd(os::Mode mode, const void *x, int64_t ld_x, void *y,
              int64_t ld_y, int64_t M, int64_t N, os_dtype dt, float *m_out,
              float *d_out, float *lse_out, void *ws, size_t ws_bytes,
              os_path path, hipStream_t stream,
              const int32_t *row_len = nullptr, int64_t causal = -1) {
    os_status s = check_shape(M, N, dt);
    if (s != OS_OK) return s;
    if (!valid_path(path)) return OS_ERR_PATH;
    if (ld_x < N || ld_y < N) return OS_ERR_STRIDE;
    if (M == 0) return OS_OK;
    if (x == nullptr || y == nullptr) return OS_ERR_NULL;
    os_path p;
    int cus;
    if ((s = resolve(M, N, path, ws, ws_bytes, &p, &cus)) != OS_OK) return s;
    os::FwdArgs a = make_args(x, ld_x, y, ld_y, M, N, dt, mode, cus, stream);
    a.m_out = m_out;
    a.d_out = d_out;
    a.lse_out = lse_out;
    a.row_len = row_len;
    // an offset of N - 1 or more admits every column of every row; larger
    // ones are clamped to N so that row + offset stays far inside int64
    a.causal = causal < 0 ? -1 : (causal > N ? N : causal);
    return launch(a, p, ws);
}

}  // namespace

// ---------------------------------------------------------------------------
// Workspace without allocation, for callers that cannot allocate device
// memory: a fixed array in device memory that os_softmax_fwd_noalloc uses
// in place of a caller workspace.  Each device holds its own copy, from
// the library's first use on it until the process ends.  In host code the
// array's name is a host-side handle, not a device address: the device
// address is read once per device with hipGetSymbolAddress (with that
// device current) and only that address is passed to kernels.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(256) << 10;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;

struct ScratchEntry {
    std::once_flag once;
    void *ptr;
};

ScratchEntry g_scratch[kMaxScratchDevices];

// The current device's copy of the scratch array, or nullptr if its
// address cannot be read.
void *scratch_of_current_device() {
    int id = -1;
    if (hipGetDevice(&id) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (id < 0 || id >= kMaxScratchDevices) return nullptr;
    ScratchEntry &e = g_scratch[id];
    std::call_once(e.once, [&e] {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            p = nullptr;
        }
        e.ptr = p;
    });
    return e.ptr;
}

}  // namespace

extern "C" {

os_status os_softmax_fwd_noalloc(const void *x, int64_t ld_x, void *y,
                                 int64_t ld_y, int64_t M, int64_t N,
                                 os_dtype dt, float *m_out, float *d_out,
                                 float *lse_out, os_path path,
                                 hipStream_t stream) {
    // the arguments first, before any HIP call
    os_status s = check_shape(M, N, dt);
    if (s != OS_OK) return s;
    if (!valid_path(path)) return OS_ERR_PATH;
    if (ld_x < N || ld_y < N) return OS_ERR_STRIDE;
    if (M == 0) return OS_OK;
    if (x == nullptr || y == nullptr) return OS_ERR_NULL;
    if (path == OS_PATH_RESIDENT && N > os::kResidentMaxN) return OS_ERR_UNSUPPORTED;
    if (usable_device() == nullptr) return OS_ERR_DEVICE;
    void *ws = scratch_of_current_device();
    if (ws == nullptr) return OS_ERR_HIP;
    // a plan that needs more than the array fails with OS_ERR_WORKSPACE
    return fwd(os::Mode::Prob, x, ld_x, y, ld_y, M, N, dt, m_out, d_out,
               lse_out, ws, kScratchBytes, path, stream);
}

os_status os_softmax_plan(int64_t M, int64_t N, os_dtype dt, os_path path,
                          int read_only, int cu_count, os_plan *out) {
    os_status s = check_shape(M, N, dt);
    if (s != OS_OK) return s;
    if (!valid_path(path)) return OS_ERR_PATH;
    if (out == nullptr) return OS_ERR_NULL;
    if (cu_count < 1) return OS_ERR_DEVICE;
    if (path == OS_PATH_RESIDENT && N > os::kResidentMaxN) return OS_ERR_UNSUPPORTED;
    const os_path p = (path == OS_PATH_AUTO)
                          ? os::select_path(M, N, read_only != 0, cu_count)
                          : path;
    out->path = p;
    out->chunks_per_row = 1;
    out->chunk_len = N;
    if (p == OS_PATH_SPLIT) {
        const os::SplitPlan sp = os::split_plan(M, N, cu_count);
        out->chunks_per_row = sp.P;
        out->chunk_len = sp.C;
    }
    out->workspace_bytes = os::workspace_for(M, N, p, cu_count);
    return OS_OK;
}

os_path os_softmax_select_path(int64_t M, int64_t N, os_dtype dt) {
    if (check_shape(M, N, dt) != OS_OK) return OS_PATH_AUTO;
    const os::Device *dev = usable_device();
    if (dev == nullptr) return OS_PATH_AUTO;
    return os::select_path(M, N, false, dev->cus);
}

os_path os_softmax_stats_select_path(int64_t M, int64_t N, os_dtype dt) {
    if (check_shape(M, N, dt) != OS_OK) return OS_PATH_AUTO;
    const os::Device *dev = usable_device();
    if (dev == nullptr) return OS_PATH_AUTO;
    return os::select_path(M, N, true, dev->cus);
}

size_t os_softmax_workspace_bytes(int64_t M, int64_t N, os_dtype dt,
                                  os_path path) {
    if (check_shape(M, N, dt) != OS_OK || !valid_path(path)) return 0;
    if (path == OS_PATH_RESIDENT) return 0;
    const os::Device *dev = usable_device();
    if (dev == nullptr) return 0;
    const os_path p = path == OS_PATH_AUTO
                          ? os::select_path(M, N, false, dev->cus)
                          : path;
    return os::workspace_for(M, N, p, dev->cus);
}

os_status os_softmax_fwd_path(const void *x, int64_t ld_x, void *y,
                              int64_t ld_y, int64_t M, int64_t N,
                              os_dtype dt, float *m_out, float *d_out,
                              float *lse_out, void *ws, size_t ws_bytes,
                              os_path path, hipStream_t stream) {
    return fwd(os::Mode::Prob, x, ld_x, y, ld_y, M, N, dt, m_out, d_out,
               lse_out, ws, ws_bytes, path, stream);
}

os_status os_softmax_fwd(const void *x, int64_t ld_x, void *y, int64_t ld_y,
                         int64_t M, int64_t N, os_dtype dt, float *m_out,
                         float *d_out, float *lse_out, void *ws,
                         size_t ws_bytes, hipStream_t stream) {
    return fwd(os::Mode::Prob, x, ld_x, y, ld_y, M, N, dt, m_out, d_out,
               lse_out, ws, ws_bytes, OS_PATH_AUTO, stream);
}

os_status os_log_softmax_fwd_path(const void *x, int64_t ld_x, void *y,
                                  int64_t ld_y, int64_t M, int64_t N,
                                  os_dtype dt, float *m_out, float *d_out,
                                  float *lse_out, void *ws, size_t ws_bytes,
                                  os_path path, hipStream_t stream) {
    return fwd(os::Mode::LogProb, x, ld_x, y, ld_y, M, N, dt, m_out, d_out,
               lse_out, ws, ws_bytes, path, stream);
}

os_status os_log_softmax_fwd(const void *x, int64_t ld_x, void *y,
                             int64_t ld_y, int64_t M, int64_t N, os_dtype dt,
                             float *m_out, float *d_out, float *lse_out,
                             void *ws, size_t ws_bytes, hipStream_t stream) {
    return fwd(os::Mode::LogProb, x, ld_x, y, ld_y, M, N, dt, m_out, d_out,
               lse_out, ws, ws_bytes, OS_PATH_AUTO, stream);
}

os_status os_softmax_fwd_masked(const void *x, int64_t ld_x, void *y,
                                int64_t ld_y, int64_t M, int64_t N,
                                os_dtype dt, const int32_t *row_len,
                                int64_t causal_offset, float *m_out,
                                float *d_out, float *lse_out, void *ws,
                                size_t ws_bytes, os_path path,
                                hipStream_t stream) {
    return fwd(os::Mode::Prob, x, ld_x, y, ld_y, M, N, dt, m_out, d_out,
               lse_out, ws, ws_bytes, path, stream, row_len, causal_offset);
}

os_status os_log_softmax_fwd_masked(const void *x, int64_t ld_x, void *y,
                                    int64_t ld_y, int64_t M, int64_t N,
                                    os_dtype dt, const int32_t *row_len,
                                    int64_t causal_offset, float *m_out,
                                    float *d_out, float *lse_out, void *ws,
                                    size_t ws_bytes, os_path path,
                                    hipStream_t stream) {
    return fwd(os::Mode::LogProb, x, ld_x, y, ld_y, M, N, dt, m_out, d_out,
               lse_out, ws, ws_bytes, path, stream, row_len, causal_offset);
}

namespace {

// softmax / log-softmax of rows (or column windows of rows) for a row state
// the caller holds: pass 2 alone
os_status normalize(os::Mode mode, const void *x, int64_t ld_x, void *y,
                    int64_t ld_y, int64_t M, int64_t N, os_dtype dt,
                    const float *m_in, const float *d_in, int64_t inc,
                    hipStream_t stream) {
    os_status s = check_shape(M, N, dt);
    if (s != OS_OK) return s;
    if (ld_x < N || ld_y < N || inc < 1) return OS_ERR_STRIDE;
    if (M == 0) return OS_OK;
    if (x == nullptr || y == nullptr || m_in == nullptr || d_in == nullptr)
        return OS_ERR_NULL;
    const os::Device *dev = usable_device();
    if (dev == nullptr) return OS_ERR_DEVICE;
    const os::FwdArgs a = make_args(x, ld_x, y, ld_y, M, N, dt, mode, dev->cus,
                                    stream);
    const os::RowChunks rc = os::row_chunks(M);
    for (int64_t c = 0; c < rc.count; ++c) {
        const int64_t r0 = c * rc.rows;
        const int64_t n = M - r0 < rc.rows ? M - r0 : rc.rows;
        os::launch_state_normalize(rc.count == 1 ? a : rows_of(a, r0, n),
                                   m_in + r0 * inc, d_in + r0 * inc, inc);
        if (hipGetLastError() != hipSuccess) return OS_ERR_HIP;
    }
    return OS_OK;
}

}  // namespace

os_status os_softmax_normalize(const void *x, int64_t ld_x, void *y,
                               int64_t ld_y, int64_t M, int64_t N,
                               os_dtype dt, const float *m_in,
                               const float *d_in, int64_t inc,
                               hipStream_t stream) {
    return normalize(os::Mode::Prob, x, ld_x, y, ld_y, M, N, dt, m_in, d_in,
                     inc, stream);
}

os_status os_log_softmax_normalize(const void *x, int64_t ld_x, void *y,
                                   int64_t ld_y, int64_t M, int64_t N,
                                   os_dtype dt, const float *m_in,
                                   const float *d_in, int64_t inc,
                                   hipStream_t stream) {
    return normalize(os::Mode::LogProb, x, ld_x, y, ld_y, M, N, dt, m_in, d_in,
                     inc, stream);
}

namespace {

os_status stats(const void *x, int64_t ld_x, int64_t M, int64_t N,
                os_dtype dt, float *m_out, float *d_out, int64_t inc_out,
                float *lse_out, void *ws, size_t ws_bytes, os_path path,
                hipStream_t stream, bool accumulate) {
    os_status s = check_shape(M, N, dt);
    if (s != OS_OK) return s;
    if (!valid_path(path)) return OS_ERR_PATH;
    if (ld_x < N || inc_out < 1) return OS_ERR_STRIDE;
    if (M == 0) return OS_OK;
    if (x == nullptr || m_out == nullptr || d_out == nullptr) return OS_ERR_NULL;
    os_path p;
    int cus;
    if ((s = resolve(M, N, path, ws, ws_bytes, &p, &cus, true)) != OS_OK) return s;
    os::FwdArgs a = make_args(x, ld_x, nullptr, 0, M, N, dt, os::Mode::Stats,
                              cus, stream);
    a.m_out = m_out;
    a.d_out = d_out;
    a.lse_out = lse_out;
    a.inc_out = inc_out;
    a.accumulate = accumulate;
    return launch(a, p, ws);
}

}  // namespace

os_status os_softmax_stats_path(const void *x, int64_t ld_x, int64_t M,
                                int64_t N, os_dtype dt, float *m_out,
                                float *d_out, int64_t inc_out, float *lse_out,
                                void *ws, size_t ws_bytes, os_path path,
                                hipStream_t stream) {
    return stats(x, ld_x, M, N, dt, m_out, d_out, inc_out, lse_out, ws,
                 ws_bytes, path, stream, false);
}

os_status os_softmax_stats_update(const void *x, int64_t ld_x, int64_t M,
                                  int64_t N, os_dtype dt, float *m_io,
                                  float *d_io, int64_t inc, float *lse_out,
                                  void *ws, size_t ws_bytes, os_path path,
                                  hipStream_t stream) {
    return stats(x, ld_x, M, N, dt, m_io, d_io, inc, lse_out, ws, ws_bytes,
                 path, stream, true);
}

os_status os_softmax_stats(const void *x, int64_t ld_x, int64_t M, int64_t N,
                           os_dtype dt, float *m_out, float *d_out,
                           int64_t inc_out, float *lse_out, void *ws,
                           size_t ws_bytes, hipStream_t stream) {
    return os_softmax_stats_path(x, ld_x, M, N, dt, m_out, d_out, inc_out,
                                 lse_out, ws, ws_bytes, OS_PATH_AUTO, stream);
}

os_status os_cross_entropy_fwd_path(const void *x, int64_t ld_x, int64_t M,
                                    int64_t N, os_dtype dt,
                                    const int64_t *labels, float *loss_out,
                                    float *lse_out, float *mean_out, void *ws,
                                    size_t ws_bytes, os_path path,
                                    hipStream_t stream) {
    os_status s = check_shape(M, N, dt);
    if (s != OS_OK) return s;
    if (!valid_path(path)) return OS_ERR_PATH;
    if (ld_x < N) return OS_ERR_STRIDE;
    if (M == 0) {
        // no rows: the mean of nothing is NaN, and it is still an output
        if (mean_out == nullptr) return OS_OK;
        if (usable_device() == nullptr) return OS_ERR_DEVICE;
        os::launch_ce_mean(nullptr, 0, mean_out, stream);
        return hipGetLastError() == hipSuccess ? OS_OK : OS_ERR_HIP;
    }
    if (x == nullptr || labels == nullptr || loss_out == nullptr)
        return OS_ERR_NULL;
    os_path p;
    int cus;
    if ((s = resolve(M, N, path, ws, ws_bytes, &p, &cus, true)) != OS_OK) return s;
    os::FwdArgs a = make_args(x, ld_x, nullptr, 0, M, N, dt, os::Mode::Stats,
                              cus, stream);
    a.lse_out = lse_out;
    a.labels = labels;
    a.loss = loss_out;
    if ((s = launch(a, p, ws)) != OS_OK) return s;
    if (mean_out != nullptr) {
        os::launch_ce_mean(loss_out, M, mean_out, stream);
        if (hipGetLastError() != hipSuccess) return OS_ERR_HIP;
    }
    return OS_OK;
}

os_status os_cross_entropy_fwd(const void *x, int64_t ld_x, int64_t M,
                               int64_t N, os_dtype dt, const int64_t *labels,
                               float *loss_out, float *lse_out,
                               float *mean_out, void *ws, size_t ws_bytes,
                               hipStream_t stream) {
    return os_cross_entropy_fwd_path(x, ld_x, M, N, dt, labels, loss_out,
                                     lse_out, mean_out, ws, ws_bytes,
                                     OS_PATH_AUTO, stream);
}

os_status os_state_merge(const float *m_in, const float *d_in, int64_t ld_in,
                         int64_t M, int64_t K, float *m_out, float *d_out,
                         float *lse_out, hipStream_t stream) {
    if (M < 0 || M > kMaxM || K < 1 || K > kMaxN) return OS_ERR_SHAPE;
    if (ld_in < K) return OS_ERR_STRIDE;
    if (M == 0) return OS_OK;
    if (m_in == nullptr || d_in == nullptr || m_out == nullptr ||
        d_out == nullptr)
        return OS_ERR_NULL;
    if (usable_device() == nullptr) return OS_ERR_DEVICE;
    const os::RowChunks rc = os::row_chunks(M);
    for (int64_t c = 0; c < rc.count; ++c) {
        const int64_t r0 = c * rc.rows;
        const int64_t n = M - r0 < rc.rows ? M - r0 : rc.rows;
        os::launch_state_merge(m_in + r0 * ld_in, d_in + r0 * ld_in, ld_in, n,
                               static_cast<int>(K), m_out + r0, d_out + r0,
                               lse_out ? lse_out + r0 : nullptr, 1, stream);
        if (hipGetLastError() != hipSuccess) return OS_ERR_HIP;
    }
    return OS_OK;
}

const char *os_status_string(os_status s) {
    switch (s) {
        case OS_OK: return "OS_OK: success";
        case OS_ERR_NULL: return "OS_ERR_NULL: a required pointer is NULL";
        case OS_ERR_SHAPE: return "OS_ERR_SHAPE: M, N or K out of range";
        case OS_ERR_STRIDE: return "OS_ERR_STRIDE: row stride smaller than the row, or inc_out < 1";
        case OS_ERR_DTYPE: return "OS_ERR_DTYPE: unknown dtype";
        case OS_ERR_WORKSPACE: return "OS_ERR_WORKSPACE: workspace missing or too small";
        case OS_ERR_PATH: return "OS_ERR_PATH: unknown path";
        case OS_ERR_UNSUPPORTED: return "OS_ERR_UNSUPPORTED: the forced path cannot take this shape";
        case OS_ERR_HIP: return "OS_ERR_HIP: a HIP launch failed";
        case OS_ERR_DEVICE: return "OS_ERR_DEVICE: no current device, or it is not a gfx950 (or the cu_count given is < 1)";
    }
    return "unknown os_status";
}

}  // extern "C"
