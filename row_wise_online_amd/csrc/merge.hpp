// The (m, d) state, the lane fold, the 64-lane wavefront merge and the
// cross-wave merge through LDS.
//
// The state and its merge follow "5.2 CUDA Online Softmax 实现优化"
// (AIInfraGuide) §2.1 (running max m and normaliser d, corrected by
// e^(m_old - m_new) when the max grows) and §4.1 (merge of two partial
// states; associative, so any reduction tree gives the same value in exact
// arithmetic).  The hierarchy lane -> wavefront -> workgroup mirrors the
// per-thread / shuffle / shared-memory levels of "Softmax 数值稳定性与
// IO-Aware Attention：从在线归一化到 FlashAttention" §4.2, re-cut for 64-lane
// CDNA wavefronts.
//
// gfx950 choices:
//  * A lane's register-resident slice is folded as one chunk: the chunk max
//    first, then one exponential per element relative to max(m, chunk max),
//    and one correction exponential for the old d.  This is the recurrence
//    applied to a block of elements, with one exp per element instead of two.
//  * The wavefront merge is the n-ary form of the merge: an all-reduce of the
//    maxima, one correction exponential per lane, then an all-reduce of the
//    corrected d.  Both all-reduces are butterflies over DPP
//    (quad_perm, row_half_mirror, row_mirror), one ds_swizzle (lanes 16
//    apart) and two v_readlane (the two 32-lane halves).  max and + are
//    commutative, so both partners of every butterfly step compute the same
//    bits and every lane ends with the identical wave state -- no broadcast.
#pragma once

#include "common.hpp"

namespace os {

struct State {
    float m;
    float d;
};

// ---- cross-lane moves -----------------------------------------------------
// DPP controls (gfx9 encoding).
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm:[1,0,3,2]  lane ^ 1
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm:[2,3,0,1]  lane ^ 2
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7 - i within 8 lanes
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15 - i within 16 lanes
// ds_swizzle bit-mask mode: and_mask 0x1f, or_mask 0, xor_mask 0x10:
// lane i reads lane i ^ 16 inside each 32-lane half.
constexpr int kSwizzleXor16 = 0x401F;

template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    const int i = __float_as_int(v);
    return __int_as_float(
        __builtin_amdgcn_update_dpp(i, i, CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float swizzle_xor16(float v) {
    return __int_as_float(
        __builtin_amdgcn_ds_swizzle(__float_as_int(v), kSwizzleXor16));
}

__device__ __forceinline__ float read_lane(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

struct OpMax {
    __device__ __forceinline__ float operator()(float a, float b) const {
        return fmaxf(a, b);
    }
};
struct OpAdd {
    __device__ __forceinline__ float operator()(float a, float b) const {
        return a + b;
    }
};

// All-reduce over the 64 lanes of a wavefront; every lane returns the same
// value.  Must be called with all 64 lanes active.
template <class Op>
__device__ __forceinline__ float wave_allreduce(float v, Op op) {
    v = op(v, dpp_move<kDppQuadXor1>(v));
    v = op(v, dpp_move<kDppQuadXor2>(v));
    v = op(v, dpp_move<kDppRowHalfMirror>(v));
    v = op(v, dpp_move<kDppRowMirror>(v));
    v = op(v, swizzle_xor16(v));
    return op(read_lane(v, 0), read_lane(v, 32));
}

// ---- in-register helpers ----------------------------------------------------
template <int K>
__device__ __forceinline__ float tree_max(const float *v) {
    if constexpr (K == 1) {
        return v[0];
    } else {
        constexpr int H = K / 2;
        return fmaxf(tree_max<H>(v), tree_max<K - H>(v + H));
    }
}

template <int K>
__device__ __forceinline__ float tree_sum(const float *v) {
    if constexpr (K == 1) {
        return v[0];
    } else {
        constexpr int H = K / 2;
        return tree_sum<H>(v) + tree_sum<K - H>(v + H);
    }
}

// Sum of e^(v[k] - r), pairwise (depth log2 K) for accuracy and ILP.  The
// terms may flush below 2^-126: next to the term of the max (1) they are
// far below the sum's rounding.
template <int K>
__device__ __forceinline__ float tree_sum_exp(const float *v, float r) {
    if constexpr (K == 1) {
        return exp2_fast((v[0] - r) * kLog2e);
    } else {
        constexpr int H = K / 2;
        return tree_sum_exp<H>(v, r) + tree_sum_exp<K - H>(v + H, r);
    }
}

// t[k] <- 2^t[k] in place.  With EXACT_TINY a wavefront whose arguments
// reach below -126 takes the subnormal-exact exponential (a uniform
// branch); otherwise the bare v_exp_f32.
template <bool EXACT_TINY, int K>
__device__ __forceinline__ void exp2_inplace(float *t) {
    if constexpr (EXACT_TINY) {
        if (wave_any(lane_may_underflow<K>(t))) {
#pragma unroll
            for (int k = 0; k < K; ++k) t[k] = exp2_full(t[k]);
            return;
        }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) t[k] = exp2_fast(t[k]);
}

// ---- the lane fold ----------------------------------------------------------
// Fold K register values into the lane state (m, d):
//   m' = max(m, v_0..v_{K-1}),  d = d e^(m - m') + sum_k e^(v_k - m').
// Starting from the identity (-inf, 0) this is the state of the chunk alone.
template <int K>
__device__ __forceinline__ void fold_chunk(float &m, float &d, const float *v) {
    const float mn = fmaxf(m, tree_max<K>(v));
    const float r = safe_ref(mn);
    const float s = tree_sum_exp<K>(v, r);
    d = d * exp2_fast((m - r) * kLog2e) + s;
    m = mn;
}

// Merge one more state (mk, dk) into the lane state (pairwise merge).
__device__ __forceinline__ void merge_into(float &m, float &d, float mk,
                                           float dk) {
    const float mn = fmaxf(m, mk);
    const float r = safe_ref(mn);
    d = d * exp_shifted(m - r) + dk * exp_shifted(mk - r);
    m = mn;
}

// ---- the wavefront merge ----------------------------------------------------
// n-ary merge of the 64 lane states: m = max_l m_l, d = sum_l d_l e^(m_l - m).
__device__ __forceinline__ State wave_merge(float m, float d) {
    const float mw = wave_allreduce(m, OpMax{});
    const float r = safe_ref(mw);
    const float dl = d * exp_shifted(m - r);
    const float dw = wave_allreduce(dl, OpAdd{});
    return {mw, dw};
}

// ---- the cross-wave merge through LDS -------------------------------------
// W wave states of one row -> LDS -> one barrier.  Then lane w < W of every
// wave holds state w (the rest hold the identity) and the n-ary merge runs
// across those lanes: a max over the first W lanes, one correction
// exponential per lane, a sum over the first W lanes (log2 W DPP butterfly
// steps each), and a v_readlane of lane 0 makes the row state wave-uniform.
// Every wave computes the same bits, so all lanes of the workgroup hold the
// identical row state.
template <int W, class Op>
__device__ __forceinline__ float first_lanes_allreduce(float v, Op op) {
    static_assert(W == 2 || W == 4 || W == 8 || W == 16, "2..16 waves");
    v = op(v, dpp_move<kDppQuadXor1>(v));
    if constexpr (W >= 4) v = op(v, dpp_move<kDppQuadXor2>(v));
    if constexpr (W >= 8) v = op(v, dpp_move<kDppRowHalfMirror>(v));
    if constexpr (W >= 16) v = op(v, dpp_move<kDppRowMirror>(v));
    return read_lane(v, 0);
}

template <int W>
__device__ __forceinline__ State block_merge(State s, int wave, int lane,
                                             float2 *lds) {
    if constexpr (W == 1) {
        return s;
    } else {
        if (lane == 0) lds[wave] = make_float2(s.m, s.d);
        __syncthreads();
        const float2 mine = (lane < W) ? lds[lane] : make_float2(kNegInf, 0.0f);
        const float m = first_lanes_allreduce<W>(mine.x, OpMax{});
        const float r = safe_ref(m);
        const float e = mine.y * exp_shifted(mine.x - r);
        const float d = first_lanes_allreduce<W>(e, OpAdd{});
        return {m, d};
    }
}

}  // namespace os
