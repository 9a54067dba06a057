// Launch plans of the row-wise entry points as pure functions of the shape
// and the device's compute-unit count (host only, no HIP calls), so that the
// workspace size a caller queries, the path AUTO takes and the grids the
// launchers use always agree for one device.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/os_softmax.h"

namespace os {

// Resident single-read path: rows of up to kResidentMaxN elements.
constexpr int kResidentMaxN = 32768;

// Per-CU sizing (MI355X: 256 CUs in 8 XCDs):
//  - AUTO keeps rows resident (one workgroup per row) when there are at
//    least 2 rows per CU, i.e. 2 of the 512-thread workgroups per CU;
//  - the split path aims at 8 workgroups per CU;
//  - pass 2 alone cuts rows into chunks until there are 64 workgroups per
//    CU (no pass 1 shares its chunks, so shorter chunks keep more loads in
//    flight);
//  - the persistent resident kernel runs 2 workgroups per CU.
constexpr int64_t kManyRowsPerCu = 2;
constexpr int64_t kSplitWgsPerCu = 8;
constexpr int64_t kNormalizeWgsPerCu = 64;
constexpr int64_t kPersistentWgsPerCu = 2;

// AUTO thresholds that do not depend on the device.
constexpr int64_t kShortRow = 4096;             // resident whatever M
constexpr int64_t kReadOnlyResidentMax = 16384; // read-only ops stream longer rows

constexpr int64_t kChunkAlign = 4096;  // chunk length granularity (elements)

struct SplitPlan {
    int P;  // chunks (workgroups) per row
    int C;  // elements per chunk (the last chunk of a row may be shorter)
};

inline int64_t cu_or_one(int cus) { return cus < 1 ? 1 : cus; }

// Rows cut into chunks of whole multiples of kChunkAlign elements until
// there are about target workgroups (one chunk per row at the least).
inline SplitPlan chunk_plan(int64_t M, int64_t N, int64_t target) {
    if (M < 1) M = 1;  // no rows: the plan of one (nothing is launched)
    int64_t P = (target + M - 1) / M;
    if (P < 1) P = 1;
    int64_t C = (N + P - 1) / P;
    C = (C + kChunkAlign - 1) / kChunkAlign * kChunkAlign;
    P = (N + C - 1) / C;
    return SplitPlan{static_cast<int>(P), static_cast<int>(C)};
}

inline SplitPlan split_plan(int64_t M, int64_t N, int cus) {
    return chunk_plan(M, N, kSplitWgsPerCu * cu_or_one(cus));
}

inline SplitPlan normalize_plan(int64_t M, int64_t N, int cus) {
    return chunk_plan(M, N, kNormalizeWgsPerCu * cu_or_one(cus));
}

inline size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// The split path's workspace: the partial states (m and d tables of M x P
// floats) and the merged row states (two tables of M floats), each table
// 256-byte aligned.
inline size_t split_workspace_bytes(int64_t M, int64_t N, int cus) {
    const SplitPlan plan = split_plan(M, N, cus);
    return 2 * align256(sizeof(float) * static_cast<size_t>(M) * plan.P) +
           2 * align256(sizeof(float) * static_cast<size_t>(M));
}

inline int64_t persistent_grid(int64_t M, int cus) {
    const int64_t g = kPersistentWgsPerCu * cu_or_one(cus);
    return M < g ? M : g;
}

// AUTO: rows that fit in registers go resident, unless they are long and
// so few that one workgroup per row would leave most CUs idle; longer rows
// with many rows stream, one workgroup per row; few long rows are split
// across workgroups.  The read-only passes (statistics, cross-entropy)
// follow the same rule, except that with many rows they stream rows longer
// than 16384 elements: they keep nothing for a pass 2, and the streaming
// fold has more loads in flight than the resident kernel sized for one
// (MI355X, fp32 1024 x 32768 statistics: 23.1 us streamed against 26.9 us
// resident).
inline os_path select_path(int64_t M, int64_t N, bool read_only, int cus) {
    const int64_t many = kManyRowsPerCu * cu_or_one(cus);
    if (N <= kResidentMaxN && (M >= many || N <= kShortRow)) {
        if (read_only && N > kReadOnlyResidentMax && M >= many)
            return OS_PATH_STREAM;
        return OS_PATH_RESIDENT;
    }
    if (M >= many) return OS_PATH_STREAM;
    return OS_PATH_SPLIT;
}

inline size_t workspace_for(int64_t M, int64_t N, os_path resolved, int cus) {
    return (resolved == OS_PATH_SPLIT && M > 0) ? split_workspace_bytes(M, N, cus)
                                                : 0;
}

}  // namespace os
