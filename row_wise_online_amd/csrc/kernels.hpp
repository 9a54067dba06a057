// gfx950 kernels of the row-wise online softmax.
//
// Pass 1 produces each row's state (m, d); pass 2 writes
// y = e^(x - m) * (1/d) ("5.2 CUDA Online Softmax 实现优化" §2.2: two passes;
// the reciprocal-then-multiply form of its kernels), or the log-softmax
// y = x - LSE ("从原始Softmax到在线Softmax", stable-form section), or nothing
// (statistics only, optionally with the cross-entropy of a labelled row,
// LSE - x_label, from the same page's cross-entropy section).
//
// Memory layout: a row is a sequence of slots (16-byte vectors, or single
// elements when the row is not 16-byte aligned).  Within a row the slot
// order is lane-fastest: slot = k * (64 * WAVES) + wave * 64 + lane, so
// every memory instruction of a wavefront touches 64 consecutive slots
// (1 KiB contiguous for vectors) and a workgroup sweeps the row front to back.
#pragma once

#include <type_traits>

#include "merge.hpp"

namespace os {

// What pass 2 writes.
enum class Out { Prob, LogProb, None };

// Per-row outputs of pass 1.  m, d and lse are nullable and written at
// row * inc.  In the cross-entropy kernels (CE = true) labels and loss are
// required and loss[row] is the cross-entropy of the row against
// labels[row]: -0.0 for a negative (ignored) label, NaN for a label >= N,
// else LSE - x_label.  A computed loss, (m - x_c) + log d with both terms
// >= +0, is never -0.0, so the sign of zero tells the batch mean which rows
// to leave out without reading the labels again.
struct StatsOut {
    float *m;
    float *d;
    float *lse;
    int64_t inc;
    const int64_t *labels;
    float *loss;
    // accumulate: m and d already hold a running state (the identity is
    // (-inf, 0)); the row's state is merged into it in place and lse is that
    // of the merged state
    bool accumulate;
};

// Masked rows (kernels instantiated with MASKED = true): row i takes part
// only through its first n_i columns, n_i = N lowered to len[i] (clipped at
// 0) when len is given and to i + causal + 1 when causal >= 0.  The other
// columns are never read: they load as -inf, so pass 2 writes 0 (softmax)
// or -inf (log-softmax) there, and a row with n_i = 0 is all NaN like a row
// of only -inf.
struct Mask {
    const int32_t *len;
    int64_t causal;
};

template <bool MASKED>
__device__ __forceinline__ int valid_cols(const Mask &mk, int64_t row, int N) {
    if constexpr (!MASKED) {
        return N;
    } else {
        int n = N;
        if (mk.len) {
            const int l = mk.len[row];
            n = min(n, l < 0 ? 0 : l);
        }
        if (mk.causal >= 0 && row + mk.causal + 1 < n)
            n = static_cast<int>(row + mk.causal + 1);
        return n;
    }
}

// The cross-entropy target of a row (kernels instantiated with CE = true).
// It is fetched before the row's own loads are issued: the label, then the
// element at the label clamped into the row (no branch, so nothing waits
// for it), widened only when the loss is written.  Its two dependent loads
// are then in flight together with the row instead of following the
// reduction.  Both addresses are wavefront-uniform.
template <class Tr>
struct Target {
    int64_t c;                   // the label
    typename Tr::elem_t raw;     // x[row, clamp(c, 0, N - 1)] as stored
};

template <class Tr, bool CE>
__device__ __forceinline__ Target<Tr> fetch_target(const StatsOut &o,
                                                   int64_t row,
                                                   const typename Tr::elem_t *xr,
                                                   int N) {
    Target<Tr> t{-1, typename Tr::elem_t(0)};
    if constexpr (CE) {
        t.c = o.labels[row];
        const int64_t cc = t.c < 0 ? 0 : (t.c >= N ? N - 1 : t.c);
        t.raw = xr[cc];
    }
    return t;
}

// Written by one thread of the row once the row state is final.  The
// cross-entropy is formed as (m - x_c) + log d rather than (m + log d) - x_c,
// so that the large common part m cancels before rounding.
template <class Tr, bool CE>
__device__ __forceinline__ void write_row_stats(const StatsOut &o, int64_t row,
                                                State st, const Target<Tr> &t,
                                                int N) {
    const int64_t k = row * o.inc;
    if (o.accumulate) merge_into(st.m, st.d, o.m[k], o.d[k]);
    const float logd = __builtin_logf(st.d);
    if (o.m) o.m[k] = st.m;
    if (o.d) o.d[k] = st.d;
    if (o.lse) o.lse[k] = st.m + logd;
    if constexpr (CE) {
        float l;
        if (t.c < 0) {
            l = -0.0f;
        } else if (t.c >= N) {
            l = __builtin_nanf("");
        } else {
            l = (safe_ref(st.m) - Tr::to_f32(t.raw)) + logd;
        }
        o.loss[row] = l;
    }
}

// The same for a state in r form (r = d - 1): log d is log1p(r), so the
// log-sum-exp and a cross-entropy near 0 keep full relative precision where
// d rounds to 1; d is written as 1 + r.  A running state held in m / d
// (accumulate) enters the merge as r = d - 1.
template <class Tr, bool CE>
__device__ __forceinline__ void write_row_stats(const StatsOut &o, int64_t row,
                                                StateR st, const Target<Tr> &t,
                                                int N) {
    const int64_t k = row * o.inc;
    if (o.accumulate) merge_into_r(st.m, st.r, o.m[k], o.d[k] - 1.0f);
    const float logd = log1pf(st.r);
    if (o.m) o.m[k] = st.m;
    if (o.d) o.d[k] = 1.0f + st.r;
    if (o.lse) o.lse[k] = st.m + logd;
    if constexpr (CE) {
        float l;
        if (t.c < 0) {
            l = -0.0f;
        } else if (t.c >= N) {
            l = __builtin_nanf("");
        } else {
            l = (safe_ref(st.m) - Tr::to_f32(t.raw)) + logd;
        }
        o.loss[row] = l;
    }
}

// 1/d and log d of a row state in either form.
__device__ __forceinline__ float inv_d(const State &s) { return 1.0f / s.d; }
__device__ __forceinline__ float log_d(const State &s) { return __builtin_logf(s.d); }
__device__ __forceinline__ float inv_d(const StateR &s) { return 1.0f / (1.0f + s.r); }
__device__ __forceinline__ float log_d(const StateR &s) { return log1pf(s.r); }

// The state form of a pass: log-softmax keeps r = d - 1, whose log1p keeps
// the log-probabilities near 0; softmax and the read-only passes keep d
// (softmax divides by d; the statistics and the cross-entropy, fp32 outputs
// whose bar is absolute, take log d within fp32 rounding of 1, and the
// extra compare and select per element of the r form would cost them
// 20-50 % on the short rows, where their VALU work is near the memory time).
template <Out OUT>
using StateOf = typename std::conditional<OUT == Out::LogProb, StateR, State>::type;

// ---------------------------------------------------------------------------
// Resident single-read path ("5.2 CUDA Online Softmax 实现优化" §6: keep the
// row on chip after pass 1 and normalise from registers; x is read once).
// One workgroup of WAVES wavefronts per row; each lane keeps EPL = SPL * W
// elements in VGPRs; the row must have N <= SPL * W * 64 * WAVES.
//
// Prob: the lane's state is that of its EPL values, m_l = their max and
// d_l = sum_i e^(v_i - m_l); the terms e^(v_i - m_l) stay in registers and
// pass 2 scales them by e^(m_l - m) / d (one exponential per element).
// LogProb / None: the registers keep x; pass 2 (LogProb) writes
// (x - m) - log d.
// ---------------------------------------------------------------------------
template <class Tr, bool VEC, int WAVES, int SPL, bool NT, Out OUT>
struct ResidentRow {
    using S = Slot<Tr, VEC, NT>;
    using elem_t = typename Tr::elem_t;
    static constexpr int W = S::W;
    static constexpr int EPL = SPL * W;
    static constexpr int STRIDE = kWave * WAVES;  // slots between a lane's slots
    static constexpr int CAPACITY = EPL * STRIDE;

    __device__ __forceinline__ static void load(const elem_t *xr, int N,
                                                int base, float *v) {
        if (N == CAPACITY) {
#pragma unroll
            for (int k = 0; k < SPL; ++k) S::load_full(xr, k * STRIDE + base, &v[k * W]);
        } else {
#pragma unroll
            for (int k = 0; k < SPL; ++k) S::load(xr, k * STRIDE + base, N, &v[k * W]);
        }
    }

    // Pass 1 to the row state; v is left as pass 2 needs it.  Softmax: the
    // lane's terms e^(v - m_lane) replace v and the state is (m, d);
    // otherwise v keeps x and the state is (m, r).
    __device__ __forceinline__ static StateOf<OUT> reduce(float *v, int wr,
                                                          int lane, float2 *lds,
                                                          float &ml) {
        ml = tree_max<EPL>(v);
        const float rl = safe_ref(ml);
        if constexpr (OUT == Out::Prob) {
#pragma unroll
            for (int i = 0; i < EPL; ++i) v[i] = (v[i] - rl) * kLog2e;
            exp2_inplace<Tr::kExactTiny, EPL>(v);
            const float dl = tree_sum<EPL>(v);
            State st = wave_merge(ml, dl);
            return block_merge<WAVES>(st, wr, lane, lds);
        } else if constexpr (OUT == Out::LogProb) {
            const StateR st = wave_merge_r(ml, lane_r<EPL>(v, ml));
            return block_merge_r<WAVES>(st, wr, lane, lds);
        } else {
            const float dl = tree_sum_exp<EPL>(v, rl);
            State st = wave_merge(ml, dl);
            return block_merge<WAVES>(st, wr, lane, lds);
        }
    }

    __device__ __forceinline__ static void write(elem_t *yr, int N, int base,
                                                 const StateOf<OUT> &st,
                                                 float ml, float *v) {
        if constexpr (OUT == Out::Prob) {
            const float scale = exp_shifted(ml - safe_ref(st.m)) * (1.0f / st.d);
#pragma unroll
            for (int i = 0; i < EPL; ++i) v[i] *= scale;
        } else if constexpr (OUT == Out::LogProb) {
            const float r = safe_ref(st.m);
            const float logd = log_d(st);
#pragma unroll
            for (int i = 0; i < EPL; ++i) v[i] = (v[i] - r) - logd;
        }
        if constexpr (OUT != Out::None) {
            if (N == CAPACITY) {
#pragma unroll
                for (int k = 0; k < SPL; ++k) S::store_full(yr, k * STRIDE + base, &v[k * W]);
            } else {
#pragma unroll
                for (int k = 0; k < SPL; ++k) S::store(yr, k * STRIDE + base, N, &v[k * W]);
            }
        }
    }
};

template <class Tr, bool VEC, int WAVES, int SPL, bool NT, Out OUT,
          bool CE = false, bool MASKED = false>
__global__ __launch_bounds__(kWave *WAVES) void resident_kernel(
    const typename Tr::elem_t *x, int64_t ldx, typename Tr::elem_t *y,
    int64_t ldy, int N, StatsOut so, Mask mk) {
    using R = ResidentRow<Tr, VEC, WAVES, SPL, NT, OUT>;
    __shared__ float2 lds[WAVES];
    const int lane = threadIdx.x & (kWave - 1);
    const int wr = threadIdx.x / kWave;
    const int64_t row = blockIdx.x;
    const typename Tr::elem_t *xr = x + row * ldx;
    const int base = wr * kWave + lane;

    const Target<Tr> tg = fetch_target<Tr, CE>(so, row, xr, N);
    float v[R::EPL];
    R::load(xr, valid_cols<MASKED>(mk, row, N), base, v);
    float ml;
    const auto st = R::reduce(v, wr, lane, lds, ml);
    R::write(y + row * ldy, N, base, st, ml, v);
    if (threadIdx.x == 0) write_row_stats<Tr, CE>(so, row, st, tg, N);
}

// ---------------------------------------------------------------------------
// Persistent variant of the resident path ("5.2 CUDA Online Softmax 实现优化"
// §7: a fixed grid walks the rows with a grid stride, here combined with the
// register-resident row of §6).  While row r is reduced and written, the
// loads of the workgroup's next row r + gridDim.x are already in flight, so
// the memory pipe never drains between rows.  The cross-wave LDS cells are
// double-buffered by iteration parity: the barrier of iteration i+1 orders
// the reads of cells (i & 1) before any wave writes them again in i+2.
// ---------------------------------------------------------------------------
template <class Tr, bool VEC, int WAVES, int SPL, bool NT, Out OUT,
          bool CE = false, bool MASKED = false>
__global__ __launch_bounds__(kWave *WAVES) void resident_persistent_kernel(
    const typename Tr::elem_t *x, int64_t ldx, typename Tr::elem_t *y,
    int64_t ldy, int64_t M, int N, StatsOut so, Mask mk) {
    using R = ResidentRow<Tr, VEC, WAVES, SPL, NT, OUT>;
    __shared__ float2 lds[2][WAVES];
    const int lane = threadIdx.x & (kWave - 1);
    const int wr = threadIdx.x / kWave;
    const int64_t step = gridDim.x;
    const int base = wr * kWave + lane;

    float cur[R::EPL], nxt[R::EPL];
    R::load(x + static_cast<int64_t>(blockIdx.x) * ldx,
            valid_cols<MASKED>(mk, blockIdx.x, N), base, cur);
    int it = 0;
    for (int64_t row = blockIdx.x; row < M; row += step, ++it) {
        const int64_t rn = row + step;
        const Target<Tr> tg = fetch_target<Tr, CE>(so, row, x + row * ldx, N);
        if (rn < M) R::load(x + rn * ldx, valid_cols<MASKED>(mk, rn, N), base, nxt);
        float ml;
        const auto st = R::reduce(cur, wr, lane, lds[it & 1], ml);
        R::write(y + row * ldy, N, base, st, ml, cur);
        if (threadIdx.x == 0) write_row_stats<Tr, CE>(so, row, st, tg, N);
#pragma unroll
        for (int i = 0; i < R::EPL; ++i) cur[i] = nxt[i];
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

    // Pass 1 over [0, n) in r form: fold every element into (m, r).
    __device__ __forceinline__ static void fold_r(const elem_t *p, int n,
                                                  int base, float &m, float &r) {
        const int nt = num_tiles(n);
        float cur[K], nxt[K];
        load_tile(p, 0, base, n, tile_full(0, n), cur);
        for (int t = 0; t < nt; ++t) {
            if (t + 1 < nt) load_tile(p, t + 1, base, n, tile_full(t + 1, n), nxt);
            fold_chunk_r<K>(m, r, cur);
#pragma unroll
            for (int i = 0; i < K; ++i) cur[i] = nxt[i];
        }
    }

    // Pass 2 over [0, n) for the row state st: Prob writes e^(x - m) / d,
    // LogProb writes (x - m) - log d.  Only [0, nl) is read (nl <= n; the
    // rest loads as -inf: masked columns).  Tile t+1 is read before tile t
    // is written, which is safe in place (they are different elements).
    // REV walks the tiles last to first: after a pass 1 that went first to
    // last, the most recently read lines come first, while they are most
    // likely still in the Infinity Cache.
    template <Out OUT, bool REV, class St>
    __device__ __forceinline__ static void normalize(const elem_t *p, elem_t *q,
                                                     int nl, int n, int base,
                                                     const St &st) {
        static_assert(OUT != Out::None, "pass 2 writes something");
        const float r = safe_ref(st.m);
        const float inv = inv_d(st);
        const float logd = log_d(st);
        const int nt = num_tiles(n);
        float cur[K], nxt[K];
        const int t0 = REV ? nt - 1 : 0;
        load_tile(p, t0, base, nl, tile_full(t0, nl), cur);
        for (int i = 0; i < nt; ++i) {
            const int t = REV ? nt - 1 - i : i;
            const int tn = REV ? t - 1 : t + 1;
            if (i + 1 < nt) load_tile(p, tn, base, nl, tile_full(tn, nl), nxt);
            if constexpr (OUT == Out::Prob) {
#pragma unroll
                for (int k = 0; k < K; ++k) cur[k] = (cur[k] - r) * kLog2e;
                exp2_inplace<Tr::kExactTiny, K>(cur);
#pragma unroll
                for (int k = 0; k < K; ++k) cur[k] *= inv;
            } else {
#pragma unroll
                for (int k = 0; k < K; ++k) cur[k] = (cur[k] - r) - logd;
            }
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
// Streaming two-read path: one workgroup per row.  With OUT == None it is a
// pass-1-only statistics kernel (one read of x).
// ---------------------------------------------------------------------------
template <class Tr, bool VEC, int WAVES, int U, Out OUT, class Pol = StreamingNT,
          bool CE = false, bool MASKED = false>
__global__ __launch_bounds__(kWave *WAVES) void stream_kernel(
    const typename Tr::elem_t *x, int64_t ldx, typename Tr::elem_t *y,
    int64_t ldy, int N, StatsOut so, Mask mk) {
    using T = Tiles<Tr, VEC, WAVES, U, Pol::nt1>;
    using T2 = Tiles<Tr, VEC, WAVES, U, Pol::nt2, Pol::nts>;
    __shared__ float2 lds[WAVES];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t row = blockIdx.x;
    const int base = wave * kWave + lane;
    const typename Tr::elem_t *xr = x + row * ldx;

    const Target<Tr> tg = fetch_target<Tr, CE>(so, row, xr, N);
    const int nv = valid_cols<MASKED>(mk, row, N);
    StateOf<OUT> st;
    if constexpr (OUT == Out::LogProb) {
        float m = kNegInf, r = -1.0f;
        T::fold_r(xr, nv, base, m, r);
        st = block_merge_r<WAVES>(wave_merge_r(m, r), wave, lane, lds);
    } else {
        float m = kNegInf, d = 0.0f;
        T::fold(xr, nv, base, m, d);
        st = block_merge<WAVES>(wave_merge(m, d), wave, lane, lds);
    }

    if constexpr (OUT != Out::None) {
        T2::template normalize<OUT, Pol::rev>(xr, y + row * ldy, nv, N, base, st);
    }
    if (threadIdx.x == 0) write_row_stats<Tr, CE>(so, row, st, tg, N);
}

// ---------------------------------------------------------------------------
// Split-row path ("5.2 CUDA Online Softmax 实现优化" §7.1: when rows are few
// and long, several workgroups share a row and a second stage combines their
// partial results).  Row i is cut into P chunks of C elements (the last one
// shorter); workgroup b handles row b / P, chunk b % P.
// ---------------------------------------------------------------------------
// RF: the partial states are written in r form, (m, d - 1), for the pass
// that keeps r (log-softmax); else (m, d).
template <class Tr, bool VEC, int WAVES, int U, class Pol = StreamingNT,
          bool MASKED = false, bool RF = false>
__global__ __launch_bounds__(kWave *WAVES) void split_partial_kernel(
    const typename Tr::elem_t *x, int64_t ldx, int N, int P, int C,
    float *ws_m, float *ws_d, Mask mk) {
    using T = Tiles<Tr, VEC, WAVES, U, Pol::nt1>;
    __shared__ float2 lds[WAVES];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t b = blockIdx.x;
    const int64_t row = b / P;
    const int p = static_cast<int>(b - row * P);
    const int c0 = p * C;
    // may be <= 0 for a chunk past a masked row's end: nothing is read and
    // the chunk's state is the identity
    const int n = min(C, valid_cols<MASKED>(mk, row, N) - c0);

    float m = kNegInf;
    float second;
    if constexpr (RF) {
        float r = -1.0f;
        T::fold_r(x + row * ldx + c0, n, wave * kWave + lane, m, r);
        const StateR st = block_merge_r<WAVES>(wave_merge_r(m, r), wave, lane, lds);
        m = st.m;
        second = st.r;
    } else {
        float d = 0.0f;
        T::fold(x + row * ldx + c0, n, wave * kWave + lane, m, d);
        const State st = block_merge<WAVES>(wave_merge(m, d), wave, lane, lds);
        m = st.m;
        second = st.d;
    }
    if (threadIdx.x == 0) {
        ws_m[b] = m;
        ws_d[b] = second;
    }
}

// The normalise pass of the split path, with the second-level merge folded
// in: every wavefront first merges the row's P partial states (lane k
// folds states k, k + 64, ... with the pairwise merge, then the wavefront
// merge), the same order state_merge_kernel uses, so every workgroup of the
// row gets the same state bit for bit.  P is at most a few hundred, so the
// merge is a few loads per lane; it saves the merge launch.  The row's first
// workgroup writes the requested row statistics.
template <class Tr, bool VEC, int WAVES, int U, Out OUT, class Pol = StreamingNT,
          bool MASKED = false>
__global__ __launch_bounds__(kWave *WAVES) void split_normalize_kernel(
    const typename Tr::elem_t *x, int64_t ldx, typename Tr::elem_t *y,
    int64_t ldy, int N, int P, int C, const float *part_m,
    const float *part_d, StatsOut so, Mask mk) {
    using T = Tiles<Tr, VEC, WAVES, U, Pol::nt2, Pol::nts>;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t b = blockIdx.x;
    const int64_t row = b / P;
    const int p = static_cast<int>(b - row * P);
    const int c0 = p * C;
    const int n = min(C, N - c0);
    const int nl = min(n, valid_cols<MASKED>(mk, row, N) - c0);
    StateOf<OUT> st;
    if constexpr (OUT == Out::LogProb) {
        float m = kNegInf, r = -1.0f;
        for (int k = lane; k < P; k += kWave) merge_into_r(m, r, part_m[row * P + k], part_d[row * P + k]);
        st = wave_merge_r(m, r);
    } else {
        float m = kNegInf, d = 0.0f;
        for (int k = lane; k < P; k += kWave) merge_into(m, d, part_m[row * P + k], part_d[row * P + k]);
        st = wave_merge(m, d);
    }
    if (p == 0 && threadIdx.x == 0)
        write_row_stats<Tr, false>(so, row, st, Target<Tr>{-1, typename Tr::elem_t(0)}, N);
    T::template normalize<OUT, Pol::rev>(x + row * ldx + c0, y + row * ldy + c0,
                                         nl, n, wave * kWave + lane, st);
}

// ---------------------------------------------------------------------------
// Pass 2 alone, with a row state the caller holds: the outputs of a column
// window need only the final (m, d) of its row, however that state was
// reached (the statistics of several windows merged, as the split path's
// second stage does for its chunks, "5.2 CUDA Online Softmax 实现优化" §7.1).
// Rows are cut into P chunks of C columns; workgroup b normalises chunk
// b % P of row b / P with (m[row * inc], d[row * inc]).
// One read and one write per element, both non-temporal.
// ---------------------------------------------------------------------------
template <class Tr, bool VEC, int WAVES, int U, Out OUT>
__global__ __launch_bounds__(kWave *WAVES) void state_normalize_kernel(
    const typename Tr::elem_t *x, int64_t ldx, typename Tr::elem_t *y,
    int64_t ldy, int N, int P, int C, const float *sm, const float *sd,
    int64_t inc) {
    using T = Tiles<Tr, VEC, WAVES, U, true, true>;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t b = blockIdx.x;
    const int64_t row = b / P;
    const int p = static_cast<int>(b - row * P);
    const int c0 = p * C;
    const int n = min(C, N - c0);
    const State st{sm[row * inc], sd[row * inc]};
    T::template normalize<OUT, false>(x + row * ldx + c0, y + row * ldy + c0, n,
                                      n, wave * kWave + lane, st);
}

// ---------------------------------------------------------------------------
// Second-level state merge ("5.2 CUDA Online Softmax 实现优化" §4.1): one
// wavefront per row, ROWS rows per workgroup.  Each lane folds states
// k = lane, lane + 64, ... with the pairwise merge; the wavefront merge
// combines the 64 lane states.  The row state goes to (m_a, d_a) at stride
// inc_a and to the StatsOut b; with CE, b's cross-entropy reads
// x[row, label] from x (element type Tr; unused otherwise).
// ---------------------------------------------------------------------------
template <int ROWS, class Tr = F32, bool CE = false>
__global__ __launch_bounds__(kWave *ROWS) void state_merge_kernel(
    const float *m_in, const float *d_in, int64_t ld, int64_t M, int K,
    float *m_a, float *d_a, int64_t inc_a, StatsOut b,
    const typename Tr::elem_t *x, int64_t ldx, int N) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row = static_cast<int64_t>(blockIdx.x) * ROWS + threadIdx.x / kWave;
    if (row >= M) return;
    const float *mr = m_in + row * ld;
    const float *dr = d_in + row * ld;
    const Target<Tr> tg = fetch_target<Tr, CE>(b, row, x + row * ldx, N);
    float m = kNegInf, d = 0.0f;
    for (int k = lane; k < K; k += kWave) merge_into(m, d, mr[k], dr[k]);
    const State st = wave_merge(m, d);
    if (lane == 0) {
        if (m_a) m_a[row * inc_a] = st.m;
        if (d_a) d_a[row * inc_a] = st.d;
        write_row_stats<Tr, CE>(b, row, st, tg, N);
    }
}

// ---------------------------------------------------------------------------
// Batch mean of the cross-entropy ("从原始Softmax到在线Softmax", cross-entropy
// section: the mean over the batch), over the rows whose label is not
// negative: those whose loss is not -0.0, the mark the row kernels leave on
// ignored rows.  One workgroup of THREADS lanes, so the result needs no
// atomics and is deterministic.  Only the losses are read (4 B per row).
// With a 16-byte aligned loss vector a lane takes groups of 4 consecutive
// rows and keeps as many groups in flight as the rows need, up to 8, so a
// batch of up to THREADS * 32 rows costs one memory round trip; the last
// M mod 4 rows (and every row when unaligned) go one per lane.  Each lane
// sums in a fixed order with compensation, then a fixed butterfly / LDS
// order combines the lanes.  NaN when no row counts.
// ---------------------------------------------------------------------------
// Adds a row's loss to the lane's compensated sum (s, e: Kahan's running
// error term, so a lane's many rows keep an fp32 sum within a few units of
// rounding however long the batch) unless the row is marked ignored.
__device__ __forceinline__ void ce_count(float l, float &s, float &e, float &c) {
    if (__float_as_uint(l) != 0x80000000u) {
        const float y = l - e;
        const float t = s + y;
        e = (t - s) - y;
        s = t;
        c += 1.0f;
    }
}

// Rows [0, 4 M4) in groups of 4, G groups per lane in flight.
template <int THREADS, int G>
__device__ __forceinline__ void ce_sum_groups(const float4 *l4, int64_t M4,
                                              float &s, float &e, float &c) {
    for (int64_t g0 = threadIdx.x; g0 < M4; g0 += int64_t(THREADS) * G) {
        // groups past the end load the last group again (no branch, so all
        // G loads issue back to back) and are not counted
        float4 lv[G];
#pragma unroll
        for (int k = 0; k < G; ++k) {
            const int64_t g = g0 + int64_t(k) * THREADS;
            lv[k] = l4[g < M4 ? g : M4 - 1];
        }
#pragma unroll
        for (int k = 0; k < G; ++k) {
            if (g0 + int64_t(k) * THREADS < M4) {
                ce_count(lv[k].x, s, e, c);
                ce_count(lv[k].y, s, e, c);
                ce_count(lv[k].z, s, e, c);
                ce_count(lv[k].w, s, e, c);
            }
        }
    }
}

template <int THREADS>
__global__ __launch_bounds__(THREADS) void ce_mean_kernel(const float *loss,
                                                          int64_t M,
                                                          float *mean) {
    constexpr int WAVES = THREADS / kWave;
    __shared__ float2 lds[WAVES];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    float s = 0.0f, e = 0.0f, c = 0.0f;
    int64_t done = 0;
    if (reinterpret_cast<uintptr_t>(loss) % 16 == 0) {
        const int64_t M4 = M / 4;
        const float4 *l4 = reinterpret_cast<const float4 *>(loss);
        if (M4 <= THREADS) ce_sum_groups<THREADS, 1>(l4, M4, s, e, c);
        else if (M4 <= 2 * THREADS) ce_sum_groups<THREADS, 2>(l4, M4, s, e, c);
        else if (M4 <= 4 * THREADS) ce_sum_groups<THREADS, 4>(l4, M4, s, e, c);
        else ce_sum_groups<THREADS, 8>(l4, M4, s, e, c);
        done = M4 * 4;
    }
    for (int64_t i = done + threadIdx.x; i < M; i += THREADS) ce_count(loss[i], s, e, c);
    s -= e;
    s = wave_allreduce(s, OpAdd{});
    c = wave_allreduce(c, OpAdd{});
    if (lane == 0) lds[wave] = make_float2(s, c);
    __syncthreads();
    if (threadIdx.x == 0) {
        float ts = 0.0f, tc = 0.0f;
        for (int w = 0; w < WAVES; ++w) {
            ts += lds[w].x;
            tc += lds[w].y;
        }
        *mean = (tc > 0.0f) ? ts / tc : __builtin_nanf("");
    }
}

}  // namespace os
