// Host-side launch chunking (plain C++, no HIP).  A dispatch counts its grid
// in work-items in 32 bits, so a call whose grid would pass 2^32 work-items
// is issued as several launches over disjoint parts of the problem, in
// stream order.  The limits below keep every launch under 2^31 work-items.
#pragma once

#include <stdint.h>

namespace os {

// Row kernels use at most 512 threads per row (the split path 512 per chunk
// of a row, P > 1 chunks only when rows are fewer than 2 per CU), so 2^22
// rows per launch keep a launch within 2^31 work-items.
constexpr int64_t kMaxRowsPerLaunch = int64_t(1) << 22;

// Attention workgroups have 512 threads: at most 2^22 per launch.
constexpr int64_t kMaxAttnBlocksPerLaunch = int64_t(1) << 22;

// Rows [0, M) as `count` launches of `rows` rows each (the last one takes
// the rest).  The parts are balanced, so none is much shorter than the
// others: rows >= ceil(M / count) - 1 and, when count > 1, rows > max / 2.
struct RowChunks {
    int64_t count;
    int64_t rows;
};

inline RowChunks row_chunks(int64_t M, int64_t max_rows = kMaxRowsPerLaunch) {
    if (M <= max_rows) return RowChunks{1, M};
    const int64_t count = (M + max_rows - 1) / max_rows;
    return RowChunks{count, (M + count - 1) / count};
}

// Attention: B x H heads of `per_head` workgroups each.  A launch covers
// either whole batches (all H heads of each) or a run of heads of one batch.
struct HeadChunk {
    int64_t b0, nb;  // batches [b0, b0 + nb)
    int64_t h0, nh;  // heads [h0, h0 + nh) of each of them (nh = H for whole batches)
};

// Calls f(HeadChunk) for each launch in order; every (b, h) is covered once
// and no launch exceeds max_blocks workgroups.  per_head must be in
// [1, max_blocks].
template <class F>
void for_each_head_chunk(int64_t B, int64_t H, int64_t per_head, F &&f,
                         int64_t max_blocks = kMaxAttnBlocksPerLaunch) {
    const int64_t heads = max_blocks / per_head;  // heads per launch, >= 1
    if (heads >= H) {
        const int64_t batches = heads / H;
        for (int64_t b0 = 0; b0 < B; b0 += batches)
            f(HeadChunk{b0, B - b0 < batches ? B - b0 : batches, 0, H});
        return;
    }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h0 = 0; h0 < H; h0 += heads)
            f(HeadChunk{b, 1, h0, H - h0 < heads ? H - h0 : heads});
}

}  // namespace os
