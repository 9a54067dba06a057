// Internal (C++) launch interface between the C ABI and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "plan.hpp"

namespace os {

// The properties of a device that the plans and the kernels depend on,
// read once per device (thread-safe) and kept for the life of the process.
struct Device {
    int cus;      // compute units
    bool gfx950;  // the architecture these kernels are built for
};

// The current device's properties, or nullptr when no device is current or
// its properties cannot be read.
const Device *current_device();

enum class Dt { F32, BF16 };
enum class Mode { Prob, LogProb, Stats };

struct FwdArgs {
    const void *x;
    int64_t ldx;
    void *y;          // NULL for Mode::Stats
    int64_t ldy;
    int64_t M;
    int N;
    Mode mode;
    // row statistics (all nullable); m / d / lse at row * inc_out
    float *m_out;
    float *d_out;
    float *lse_out;
    int64_t inc_out;
    bool accumulate;  // m_out / d_out hold a running state to merge into
    // cross-entropy (Mode::Stats only): loss[row] against labels[row]
    const int64_t *labels;
    float *loss;
    // masked rows (Mode::Prob / LogProb only): valid lengths (nullable) and
    // a causal offset (< 0: none)
    const int32_t *row_len;
    int64_t causal;
    Dt dt;
    bool vec;         // 16-byte vector access is legal for x (and y)
    int cus;          // compute units of the device (sizes the grids)
    hipStream_t stream;

    bool masked() const { return row_len != nullptr || causal >= 0; }
};

// Resident single-read path (rows of up to kResidentMaxN elements).
void launch_resident(const FwdArgs &a);

// Streaming path, one workgroup per row.
void launch_stream(const FwdArgs &a);

// Split path: partial states into ws; then, for statistics alone (and the
// cross-entropy), the state-merge kernel, and for softmax / log-softmax the
// normalise kernel, which merges the row's partial states itself.
void launch_split(const FwdArgs &a, void *ws);

// Pass 2 alone (Mode::Prob or Mode::LogProb) with the caller's row state
// (m, d) at row * inc; long rows are cut into chunks of whole multiples of
// 4096 elements.
void launch_state_normalize(const FwdArgs &a, const float *sm, const float *sd,
                            int64_t inc);

// Second-level state merge of K fp32 states per row (no cross-entropy):
// m, d and lse (nullable) at row * inc.
void launch_state_merge(const float *m_in, const float *d_in, int64_t ld,
                        int64_t M, int K, float *m_out, float *d_out,
                        float *lse_out, int64_t inc, hipStream_t stream);

// Mean of loss[i] over the rows not marked ignored (loss -0.0; one
// workgroup).
void launch_ce_mean(const float *loss, int64_t M, float *mean,
                    hipStream_t stream);

}  // namespace os
