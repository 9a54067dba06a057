// gfx950 kernels of the row-wise online softmax.
//
// Pass 1 produces each row's state (m, d); pass 2 writes
// y = e^(x - m) * (1/d) ("5.2 CUDA Online Softmax 实现优化" §2.2: two passes;
// the reciprocal-then-multiply form of its kernels).
//
// Memory layout: a row is a sequence of slots (16-byte vectors, or single
// elements when the row is not 16-byte aligned).  Within a row the slot
// order is lane-fastest: slot = k * (64 * WAVES) + wave * 64 + lane, so
// every memory instruction of a wavefront touches 64 consecutive slots
// (1 KiB contiguous for vectors) and a workgroup sweeps the row front to back.
#pragma once

#include "merge.hpp"

namespace os {

// ---------------------------------------------------------------------------
// Resident single-read path ("5.2 CUDA Online Softmax 实现优化" §6: keep the
// row on chip after pass 1 and normalise from registers; x is read once).
// WAVES wavefronts share a row; with WAVES == 1 a workgroup runs ROWS
// independent rows (one per wavefront, no barrier).  Each lane keeps
// EPL = SPL * W elements in VGPRs; the row must have N <= SPL*W*64*WAVES.
// ---------------------------------------------------------------------------
template <class Tr, bool VEC, int WAVES, int ROWS, int SPL, bool NT = false>
__global__ __launch_bounds__(kWave *WAVES *ROWS) void resident_kernel(
    const typename Tr::elem_t *x, int64_t ldx, typename Tr::elem_t *y,
    int64_t ldy, int64_t M, int N, float *m_out, float *d_out,
    float *lse_out) {
    static_assert(WAVES == 1 || ROWS == 1, "rows share a workgroup only "
                                           "when each row has one wave");
    using S = Slot<Tr, VEC, NT>;
    constexpr int W = S::W;
    constexpr int EPL = SPL * W;
    constexpr int STRIDE = kWave * WAVES;  // slots between a lane's slots
    __shared__ float2 lds[WAVES];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    int64_t row;
    int wr;  // wave index within the row
    if constexpr (ROWS > 1) {
        row = static_cast<int64_t>(blockIdx.x) * ROWS + wave;
        wr = 0;
        if (row >= M) return;  // whole wavefront leaves; no barrier follows
    } else {
        row = blockIdx.x;
        wr = wave;
    }
    const typename Tr::elem_t *xr = x + row * ldx;
    typename Tr::elem_t *yr = y + row * ldy;
    const int base = wr * kWave + lane;
    const bool full = (N == SPL * W * STRIDE);

    float v[EPL];
    if (full) {
#pragma unroll
        for (int k = 0; k < SPL; ++k) S::load_full(xr, k * STRIDE + base, &v[k * W]);
    } else {
#pragma unroll
        for (int k = 0; k < SPL; ++k) S::load(xr, k * STRIDE + base, N, &v[k * W]);
    }

    // pass 1: lane fold -> wavefront merge -> cross-wave merge.  The lane's
    // state is that of its EPL resident values: m_l = their max and
    // d_l = sum_i e^(v_i - m_l).  The terms e^(v_i - m_l) stay in registers.
    const float ml = tree_max<EPL>(v);
    const float rl = safe_ref(ml);
#pragma unroll
    for (int i = 0; i < EPL; ++i) v[i] = (v[i] - rl) * kLog2e;
    exp2_inplace<Tr::kExactTiny, EPL>(v);
    State st = wave_merge(ml, tree_sum<EPL>(v));
    st = block_merge<WAVES>(st, wr, lane, lds);

    // pass 2 from registers: e^(x - m) / d = e^(x - m_l) * (e^(m_l - m) / d)
    const float scale = exp_shifted(ml - safe_ref(st.m)) * (1.0f / st.d);
#pragma unroll
    for (int i = 0; i < EPL; ++i) v[i] *= scale;
    if (full) {
#pragma unroll
        for (int k = 0; k < SPL; ++k) S::store_full(yr, k * STRIDE + base, &v[k * W]);
    } else {
#pragma unroll
        for (int k = 0; k < SPL; ++k) S::store(yr, k * STRIDE + base, N, &v[k * W]);
    }

    if (wr == 0 && lane == 0) {
        if (m_out) m_out[row] = st.m;
        if (d_out) d_out[row] = st.d;
        if (lse_out) lse_out[row] = st.m + __builtin_logf(st.d);
    }
}

// ---------------------------------------------------------------------------
// Persistent variant of the resident path ("5.2 CUDA Online Softmax 实现优化"
// §7: a fixed grid walks the rows with a grid stride, here combined with the
// register-resident row of §6).  While row r is reduced and written, the
// loads of the wavefront's next row r + stride are already in flight, so
// the memory pipe never drains between rows.  WAVES wavefronts share a row;
// with WAVES == 1 each of the ROWS wavefronts of a workgroup walks its own
// rows.  The cross-wave LDS cells are double-buffered by iteration parity:
// the barrier of iteration i+1 orders the reads of cells (i & 1) before any
// wave writes them again in iteration i+2.
// ---------------------------------------------------------------------------
template <class Tr, bool VEC, int WAVES, int ROWS, int SPL, bool NT>
__global__ __launch_bounds__(kWave *WAVES *ROWS) void resident_persistent_kernel(
    const typename Tr::elem_t *x, int64_t ldx, typename Tr::elem_t *y,
    int64_t ldy, int64_t M, int N, float *m_out, float *d_out,
    float *lse_out) {
    static_assert(WAVES == 1 || ROWS == 1, "rows share a workgroup only "
                                           "when each row has one wave");
    using S = Slot<Tr, VEC, NT>;
    constexpr int W = S::W;
    constexpr int EPL = SPL * W;
    constexpr int STRIDE = kWave * WAVES;
    __shared__ float2 lds[2][WAVES];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int wr = (ROWS > 1) ? 0 : wave;
    const int64_t first = (ROWS > 1) ? static_cast<int64_t>(blockIdx.x) * ROWS + wave
                                     : static_cast<int64_t>(blockIdx.x);
    const int64_t step = static_cast<int64_t>(gridDim.x) * ROWS;
    const int base = wr * kWave + lane;
    const bool full = (N == SPL * W * STRIDE);

    auto load_row = [&](int64_t row, float *v) {
        const typename Tr::elem_t *xr = x + row * ldx;
        if (full) {
#pragma unroll
            for (int k = 0; k < SPL; ++k) S::load_full(xr, k * STRIDE + base, &v[k * W]);
        } else {
#pragma unroll
            for (int k = 0; k < SPL; ++k) S::load(xr, k * STRIDE + base, N, &v[k * W]);
        }
    };

    if (first >= M) return;  // (ROWS > 1 only: a whole wavefront without rows)
    float cur[EPL], nxt[EPL];
    load_row(first, cur);
    int it = 0;
    for (int64_t row = first; row < M; row += step, ++it) {
        const int64_t rn = row + step;
        if (rn < M) load_row(rn, nxt);

        const float ml = tree_max<EPL>(cur);
        const float rl = safe_ref(ml);
#pragma unroll
        for (int i = 0; i < EPL; ++i) cur[i] = (cur[i] - rl) * kLog2e;
        exp2_inplace<Tr::kExactTiny, EPL>(cur);
        State st = wave_merge(ml, tree_sum<EPL>(cur));
        st = block_merge<WAVES>(st, wr, lane, lds[it & 1]);

        const float scale = exp_shifted(ml - safe_ref(st.m)) * (1.0f / st.d);
#pragma unroll
        for (int i = 0; i < EPL; ++i) cur[i] *= scale;
        typename Tr::elem_t *yr = y + row * ldy;
        if (full) {
#pragma unroll
            for (int k = 0; k < SPL; ++k) S::store_full(yr, k * STRIDE + base, &cur[k * W]);
        } else {
#pragma unroll
            for (int k = 0; k < SPL; ++k) S::store(yr, k * STRIDE + base, N, &cur[k * W]);
        }
        if (wr == 0 && lane == 0) {
            if (m_out) m_out[row] = st.m;
            if (d_out) d_out[row] = st.d;
            if (lse_out) lse_out[row] = st.m + __builtin_logf(st.d);
        }
#pragma unroll
        for (int i = 0; i < EPL; ++i) cur[i] = nxt[i];
    }
}

// ---------------------------------------------------------------------------
// Streaming building blocks: a workgroup of WAVES wavefronts walks a range
// of n elements in tiles of U slots per lane.  The next tile's loads are
// issued before the current tile is consumed (two tiles of registers).
// ---------------------------------------------------------------------------
template <class Tr, bool VEC, int WAVES, int U, bool NTL = false,
          bool NTS = NTL>
struct Tiles {
    using S = Slot<Tr, VEC, NTL, NTS>;
    using elem_t = typename Tr::elem_t;
    static constexpr int W = S::W;
    static constexpr int K = U * W;               // elements per lane per tile
    static constexpr int STRIDE = kWave * WAVES;  // slots between u and u+1
    static constexpr int TILE = U * STRIDE;       // slots per tile

    __device__ __forceinline__ static void load_tile(const elem_t *p, int t,
                                                     int base, int n, bool full,
                                                     float *v) {
        if (full) {
#pragma unroll
            for (int u = 0; u < U; ++u) S::load_full(p, t * TILE + u * STRIDE + base, &v[u * W]);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) S::load(p, t * TILE + u * STRIDE + base, n, &v[u * W]);
        }
    }

    __device__ __forceinline__ static void store_tile(elem_t *p, int t,
                                                      int base, int n, bool full,
                                                      const float *v) {
        if (full) {
#pragma unroll
            for (int u = 0; u < U; ++u) S::store_full(p, t * TILE + u * STRIDE + base, &v[u * W]);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) S::store(p, t * TILE + u * STRIDE + base, n, &v[u * W]);
        }
    }

    __device__ __forceinline__ static int num_tiles(int n) {
        const int slots = (n + W - 1) / W;
        return (slots + TILE - 1) / TILE;
    }
    __device__ __forceinline__ static bool tile_full(int t, int n) {
        return (t + 1) * TILE * W <= n;
    }

    // Pass 1 over [0, n): fold every element into the lane state (m, d).
    __device__ __forceinline__ static void fold(const elem_t *p, int n,
                                                int base, float &m, float &d) {
        const int nt = num_tiles(n);
        float cur[K], nxt[K];
        load_tile(p, 0, base, n, tile_full(0, n), cur);
        for (int t = 0; t < nt; ++t) {
            if (t + 1 < nt) load_tile(p, t + 1, base, n, tile_full(t + 1, n), nxt);
            fold_chunk<K>(m, d, cur);
#pragma unroll
            for (int i = 0; i < K; ++i) cur[i] = nxt[i];
        }
    }

    // Pass 2 over [0, n): y = e^(x - r) * inv.  Tile t+1 is read before tile
    // t is written, which is safe in place (they are different elements).
    // REV walks the tiles last to first: after a pass 1 that went first to
    // last, the most recently read lines come first, while they are most
    // likely still in the Infinity Cache.
    template <bool REV = false>
    __device__ __forceinline__ static void normalize(const elem_t *p, elem_t *q,
                                                     int n, int base, float r,
                                                     float inv) {
        const int nt = num_tiles(n);
        float cur[K], nxt[K];
        const int t0 = REV ? nt - 1 : 0;
        load_tile(p, t0, base, n, tile_full(t0, n), cur);
        for (int i = 0; i < nt; ++i) {
            const int t = REV ? nt - 1 - i : i;
            const int tn = REV ? t - 1 : t + 1;
            if (i + 1 < nt) load_tile(p, tn, base, n, tile_full(tn, n), nxt);
#pragma unroll
            for (int k = 0; k < K; ++k) cur[k] = (cur[k] - r) * kLog2e;
            exp2_inplace<Tr::kExactTiny, K>(cur);
#pragma unroll
            for (int k = 0; k < K; ++k) cur[k] *= inv;
            store_tile(q, t, base, n, tile_full(t, n), cur);
#pragma unroll
            for (int k = 0; k < K; ++k) cur[k] = nxt[k];
        }
    }
};

// ---------------------------------------------------------------------------
// Cache policy of the two-read paths: non-temporal pass-1 loads, pass-2
// loads and pass-2 stores, and the pass-2 tile order (REV: last tile first).
// ---------------------------------------------------------------------------
template <bool NT1, bool NT2, bool NTS, bool REV>
struct TwoPass {
    static constexpr bool nt1 = NT1, nt2 = NT2, nts = NTS, rev = REV;
};
using StreamingNT = TwoPass<true, true, true, false>;

// ---------------------------------------------------------------------------
// Streaming two-read path: one workgroup per row.  With WRITE_Y false it is
// the pass-1-only statistics kernel (states written with stride inc_out).
// ---------------------------------------------------------------------------
template <class Tr, bool VEC, int WAVES, int U, bool WRITE_Y,
          class Pol = StreamingNT>
__global__ __launch_bounds__(kWave *WAVES) void stream_kernel(
    const typename Tr::elem_t *x, int64_t ldx, typename Tr::elem_t *y,
    int64_t ldy, int64_t M, int N, float *m_out, float *d_out,
    int64_t inc_out, float *lse_out) {
    using T = Tiles<Tr, VEC, WAVES, U, Pol::nt1>;
    using T2 = Tiles<Tr, VEC, WAVES, U, Pol::nt2, Pol::nts>;
    __shared__ float2 lds[WAVES];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t row = blockIdx.x;
    const int base = wave * kWave + lane;
    const typename Tr::elem_t *xr = x + row * ldx;

    float m = kNegInf, d = 0.0f;
    T::fold(xr, N, base, m, d);
    State st = wave_merge(m, d);
    st = block_merge<WAVES>(st, wave, lane, lds);

    if constexpr (WRITE_Y) {
        T2::template normalize<Pol::rev>(xr, y + row * ldy, N, base,
                                         safe_ref(st.m), 1.0f / st.d);
    }
    if (threadIdx.x == 0) {
        const int64_t o = row * inc_out;
        if (m_out) m_out[o] = st.m;
        if (d_out) d_out[o] = st.d;
        if (lse_out) lse_out[o] = st.m + __builtin_logf(st.d);
    }
}

// ---------------------------------------------------------------------------
// Split-row path ("5.2 CUDA Online Softmax 实现优化" §7.1: when rows are few
// and long, several workgroups share a row and a second stage combines their
// partial results).  Row i is cut into P chunks of C elements (the last one
// shorter); workgroup b handles row b / P, chunk b % P.
// ---------------------------------------------------------------------------
template <class Tr, bool VEC, int WAVES, int U, class Pol = StreamingNT>
__global__ __launch_bounds__(kWave *WAVES) void split_partial_kernel(
    const typename Tr::elem_t *x, int64_t ldx, int N, int P, int C,
    float *ws_m, float *ws_d) {
    using T = Tiles<Tr, VEC, WAVES, U, Pol::nt1>;
    __shared__ float2 lds[WAVES];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t b = blockIdx.x;
    const int64_t row = b / P;
    const int p = static_cast<int>(b - row * P);
    const int c0 = p * C;
    const int n = min(C, N - c0);

    float m = kNegInf, d = 0.0f;
    T::fold(x + row * ldx + c0, n, wave * kWave + lane, m, d);
    State st = wave_merge(m, d);
    st = block_merge<WAVES>(st, wave, lane, lds);
    if (threadIdx.x == 0) {
        ws_m[b] = st.m;
        ws_d[b] = st.d;
    }
}

template <class Tr, bool VEC, int WAVES, int U, class Pol = StreamingNT>
__global__ __launch_bounds__(kWave *WAVES) void split_normalize_kernel(
    const typename Tr::elem_t *x, int64_t ldx, typename Tr::elem_t *y,
    int64_t ldy, int N, int P, int C, const float *row_m,
    const float *row_d, int64_t inc) {
    using T = Tiles<Tr, VEC, WAVES, U, Pol::nt2, Pol::nts>;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t b = blockIdx.x;
    const int64_t row = b / P;
    const int p = static_cast<int>(b - row * P);
    const int c0 = p * C;
    const int n = min(C, N - c0);
    const float m = row_m[row * inc];
    const float d = row_d[row * inc];
    T::template normalize<Pol::rev>(x + row * ldx + c0, y + row * ldy + c0,
                                    n, wave * kWave + lane, safe_ref(m),
                                    1.0f / d);
}

// ---------------------------------------------------------------------------
// Second-level state merge ("5.2 CUDA Online Softmax 实现优化" §4.1): one
// wavefront per row, ROWS rows per workgroup.  Each lane folds states
// k = lane, lane + 64, ... with the pairwise merge; the wavefront merge
// combines the 64 lane states.
// ---------------------------------------------------------------------------
template <int ROWS>
__global__ __launch_bounds__(kWave *ROWS) void state_merge_kernel(
    const float *m_in, const float *d_in, int64_t ld, int64_t M, int K,
    float *m_a, float *d_a, int64_t inc_a, float *m_b, float *d_b,
    float *lse_b, int64_t inc_b) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row = static_cast<int64_t>(blockIdx.x) * ROWS + threadIdx.x / kWave;
    if (row >= M) return;
    const float *mr = m_in + row * ld;
    const float *dr = d_in + row * ld;
    float m = kNegInf, d = 0.0f;
    for (int k = lane; k < K; k += kWave) merge_into(m, d, mr[k], dr[k]);
    const State st = wave_merge(m, d);
    if (lane == 0) {
        // two optional destinations: (m_a, d_a) at stride inc_a, and
        // (m_b, d_b, lse_b) at stride inc_b
        if (m_a) m_a[row * inc_a] = st.m;
        if (d_a) d_a[row * inc_a] = st.d;
        const int64_t o = row * inc_b;
        if (m_b) m_b[o] = st.m;
        if (d_b) d_b[o] = st.d;
        if (lse_b) lse_b[o] = st.m + __builtin_logf(st.d);
    }
}

}  // namespace os
