// Internal (C++) launch interface between the C ABI and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace os {

enum class Dt { F32, BF16 };

struct FwdArgs {
    const void *x;
    int64_t ldx;
    void *y;          // NULL for statistics only
    int64_t ldy;
    int64_t M;
    int N;
    float *m_out;
    float *d_out;
    int64_t inc_out;  // stride of m_out / d_out / lse_out (1 for softmax)
    float *lse_out;
    Dt dt;
    bool vec;         // 16-byte vector access is legal for x (and y)
    hipStream_t stream;
};

// Resident single-read path: rows of up to kResidentMaxN elements.
constexpr int kResidentMaxN = 32768;
void launch_resident(const FwdArgs &a);

// Streaming path, one workgroup per row (softmax if a.y, else stats only).
void launch_stream(const FwdArgs &a);

// Split-row plan: P chunks of C elements per row.
struct SplitPlan {
    int P;
    int C;
};
SplitPlan split_plan(int64_t M, int64_t N);
size_t split_workspace_bytes(int64_t M, int64_t N);

// Split path: partial states into ws, state merge, then (if a.y) normalise.
void launch_split(const FwdArgs &a, void *ws);

// Second-level state merge.  Row states go to (m_a, d_a) at row * inc_a
// and to (m_b, d_b, lse_b) at row * inc_b; every pointer is nullable.
void launch_state_merge(const float *m_in, const float *d_in, int64_t ld,
                        int64_t M, int K, float *m_a, float *d_a,
                        int64_t inc_a, float *m_b, float *d_b, float *lse_b,
                        int64_t inc_b, hipStream_t stream);

}  // namespace os
