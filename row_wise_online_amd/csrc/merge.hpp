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

// ---- the state with r = d - 1 ------------------------------------------------
// For the outputs that take a logarithm of the normaliser (log-softmax, the
// log-sum-exp, the cross-entropy) the state carries r = d - 1 in place of d:
// the row's terms other than one instance of its max, summed apart from
// that term's 1.  When every other term is below 2^-24 of the max, d rounds
// to 1 in fp32 and log d to 0, while r keeps the small sum to full relative
// precision and log1p(r) gives log d to full relative precision.  Then the
// max element's log-probability, -log1p(r), and a confident row's
// cross-entropy are exact to fp32 rounding rather than 0.  The identity is
// (-inf, -1).  Elements equal to the max add exactly 1 each, except the
// one instance the 1 of d stands for.
struct StateR {
    float m;
    float r;
};

constexpr float kPosInf = __builtin_huge_valf();

// The sum of e^(v_k - ref) over the v_k other than mn, and the count c of
// the v_k equal to mn.  Summed in groups of at most 8 (pairwise inside a
// group, then over the groups), so that few terms are live at once.
template <int K>
__device__ __forceinline__ float sum_apart(const float *v, float mn, float ref,
                                           int &c) {
    constexpr int G = K < 8 ? K : 8;
    static_assert(K % G == 0, "whole groups");
    float part[K / G];
    c = 0;
#pragma unroll
    for (int g = 0; g < K / G; ++g) {
        float t[G];
#pragma unroll
        for (int k = 0; k < G; ++k) {
            const float x = v[g * G + k];
            const bool eq = x == mn;
            t[k] = eq ? 0.0f : exp2_fast((x - ref) * kLog2e);
            c += eq ? 1 : 0;
        }
        part[g] = tree_sum<G>(t);
    }
    return tree_sum<K / G>(part);
}

// r of a lane's K values alone (a fresh lane state, max ml): the values
// equal to ml are one max and c - 1 further terms of exactly 1.  A lane of
// only -inf is the identity; a max of +inf makes r NaN (the row is NaN, as
// a NaN element makes it).
template <int K>
__device__ __forceinline__ float lane_r(const float *v, float ml) {
    int c;
    const float s = sum_apart<K>(v, ml, safe_ref(ml), c);
    float r = s + static_cast<float>(c - 1);
    if (ml == kNegInf) r = -1.0f;
    if (ml == kPosInf) r = __builtin_nanf("");
    return r;
}

// Fold K register values into the lane state (m, r): with mn the new max,
//   m == mn:  r += sum_k e^(v_k - m), each v_k == m adding exactly 1;
//   m <  mn:  r = (1 + r) e^(m - mn) + sum_{v_k != mn} e^(v_k - mn) + (c - 1)
// where c counts the v_k equal to mn (c >= 1: one of them is the new max).
// Only -inf so far leaves the identity; a max of +inf makes r NaN.
template <int K>
__device__ __forceinline__ void fold_chunk_r(float &m, float &r, const float *v) {
    const float mn = fmaxf(m, tree_max<K>(v));
    const float ref = safe_ref(mn);
    int c;
    const float s = sum_apart<K>(v, mn, ref, c);
    float rn = (m == mn) ? (r + s) + static_cast<float>(c)
                         : fmaf(1.0f + r, exp2_fast((m - ref) * kLog2e),
                                s + static_cast<float>(c - 1));
    if (mn == kNegInf) rn = r;
    if (mn == kPosInf) rn = __builtin_nanf("");
    m = mn;
    r = rn;
}

// A state's share of a merged r: its own r if its max is the merged max m
// (then `first` chooses whether its 1 is the implicit one of the merged d),
// else all of its d, (1 + r) e^(m_k - m).
__device__ __forceinline__ float share_r(float mk, float rk, float m, float ref,
                                         bool first) {
    if (mk == m && m != kNegInf) return first ? rk : rk + 1.0f;
    return (1.0f + rk) * exp_shifted(mk - ref);
}

// Merge one more state (mk, rk) into the lane state (m, r).
__device__ __forceinline__ void merge_into_r(float &m, float &r, float mk,
                                             float rk) {
    const float mn = fmaxf(m, mk);
    const float ref = safe_ref(mn);
    const float a = share_r(m, r, mn, ref, true);
    const float b = share_r(mk, rk, mn, ref, !(m == mn));
    r = (mn == kNegInf) ? -1.0f : (mn == kPosInf ? __builtin_nanf("") : a + b);
    m = mn;
}

// n-ary merge of the 64 lane states in r form.  The lowest lane holding the
// merged max contributes its r, every other lane its share; a wavefront of
// identities stays the identity.
__device__ __forceinline__ StateR wave_merge_r(float m, float r) {
    const float mw = wave_allreduce(m, OpMax{});
    const uint64_t at_max = __builtin_amdgcn_ballot_w64(m == mw && mw != kNegInf);
    const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const bool first = at_max != 0 && lane == __builtin_ctzll(at_max);
    const float c = share_r(m, r, mw, safe_ref(mw), first);
    const float rw = wave_allreduce(c, OpAdd{});
    return {mw, mw == kNegInf ? -1.0f : (mw == kPosInf ? __builtin_nanf("") : rw)};
}

// The cross-wave merge of block_merge in r form.
template <int W>
__device__ __forceinline__ StateR block_merge_r(StateR s, int wave, int lane,
                                                float2 *lds) {
    if constexpr (W == 1) {
        return s;
    } else {
        if (lane == 0) lds[wave] = make_float2(s.m, s.r);
        __syncthreads();
        const float2 mine = (lane < W) ? lds[lane] : make_float2(kNegInf, -1.0f);
        const float m = first_lanes_allreduce<W>(mine.x, OpMax{});
        const uint64_t at_max =
            __builtin_amdgcn_ballot_w64(lane < W && mine.x == m && m != kNegInf);
        const bool first = at_max != 0 && lane == __builtin_ctzll(at_max);
        const float c = share_r(mine.x, mine.y, m, safe_ref(m), first);
        const float r = first_lanes_allreduce<W>(c, OpAdd{});
        return {m, m == kNegInf ? -1.0f : (m == kPosInf ? __builtin_nanf("") : r)};
    }
}

}  // namespace os
