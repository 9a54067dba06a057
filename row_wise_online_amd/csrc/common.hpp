// Element types, 16-byte vector memory access and the exp helper shared by
// the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace os {

constexpr int kWave = 64;                    // CDNA wavefront width
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

// Exponentials are evaluated as 2^(t * log2 e) with t = x - m formed first
// (exact when x is near m) and then scaled; folding -m * log2 e into an fma
// would lose the low bits of large maxima.
//
// exp2_fast is the bare v_exp_f32: results below 2^-126 come out as zero.
// That loses nothing in a sum that already holds a term of 1 (the max), and
// stays within the fp32 output tolerance, but a bf16 output can still
// represent values down to 2^-133, so bf16 outputs use exp2_full whenever
// an argument falls below -126 (see any_may_underflow).
__device__ __forceinline__ float exp2_fast(float t) {
    return __builtin_amdgcn_exp2f(t);
}
// exp2_full: __builtin_exp2f lowers to v_exp_f32 plus a range fix-up that
// keeps results in the fp32 subnormal range accurate.
__device__ __forceinline__ float exp2_full(float t) {
    return __builtin_exp2f(t);
}
// Accurate e^t, used for the per-lane and per-row correction factors.
__device__ __forceinline__ float exp_shifted(float t) {
    return exp2_full(t * kLog2e);
}

// True if some t[k] lies in (-inf, -126), where exp2_fast would flush a
// subnormal result.  On the bit patterns: t in (-inf, -126) exactly when
// bits(t) - bits(-126) - 1 < bits(-inf) - bits(-126) - 1 as unsigned
// integers (NaN, -inf, zero and t >= -126 all land above the bound), so one
// subtract and a running unsigned min per value decide it.
template <int K>
__device__ __forceinline__ bool lane_may_underflow(const float *t) {
    constexpr uint32_t kLo = 0xC2FC0001u;            // just below -126.0f
    constexpr uint32_t kSpan = 0xFF800000u - kLo;    // up to -inf, exclusive
    uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
    for (int k = 0; k < K; ++k) mn = min(mn, __float_as_uint(t[k]) - kLo);
    return mn < kSpan;
}

// Wavefront-uniform OR of a per-lane predicate (a scalar result).
__device__ __forceinline__ bool wave_any(bool p) {
    return __builtin_amdgcn_ballot_w64(p) != 0;
}

// The reference point used for exponents: the max itself, or 0 when the
// max is -inf (a state holding only -inf / padding).  With it, padding and
// -inf elements give e^(-inf) = 0, the identity state (-inf, 0) merges to
// itself, and a NaN folded into d stays NaN.
__device__ __forceinline__ float safe_ref(float m) {
    return (m == kNegInf) ? 0.0f : m;
}

// ---- element types --------------------------------------------------------
// Traits give: the stored type, E = elements per 16-byte vector, and the
// conversions between a 16-byte vector and E fp32 values.

struct F32 {
    using elem_t = float;
    static constexpr int E = 4;
    static constexpr bool kExactTiny = false;  // fp32 y below 2^-126 may be 0
    __device__ __forceinline__ static float to_f32(float v) { return v; }
    __device__ __forceinline__ static float from_f32(float v) { return v; }
    __device__ __forceinline__ static void unpack(const uint4 &u, float *f) {
        f[0] = __uint_as_float(u.x);
        f[1] = __uint_as_float(u.y);
        f[2] = __uint_as_float(u.z);
        f[3] = __uint_as_float(u.w);
    }
    __device__ __forceinline__ static uint4 pack(const float *f) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                          __float_as_uint(f[2]), __float_as_uint(f[3]));
    }
};

// bf16 stored as its 16-bit pattern.  Widening is exact (the pattern is the
// top half of the fp32 with the same value); narrowing rounds to nearest
// even (v_cvt_pk_bf16_f32 on gfx950).
struct BF16 {
    using elem_t = uint16_t;
    static constexpr int E = 8;
    static constexpr bool kExactTiny = true;   // keep bf16 subnormal outputs
    __device__ __forceinline__ static float to_f32(uint16_t b) {
        return __uint_as_float(static_cast<uint32_t>(b) << 16);
    }
    __device__ __forceinline__ static uint16_t from_f32(float v) {
        return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
    }
    __device__ __forceinline__ static uint32_t pack2(float lo, float hi) {
        typedef float f2 __attribute__((ext_vector_type(2)));
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        f2 v = {lo, hi};
        b2 r = __builtin_convertvector(v, b2);
        return __builtin_bit_cast(uint32_t, r);
    }
    __device__ __forceinline__ static void unpack(const uint4 &u, float *f) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    __device__ __forceinline__ static uint4 pack(const float *f) {
        return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]),
                          pack2(f[4], f[5]), pack2(f[6], f[7]));
    }
};

// ---- memory access --------------------------------------------------------
// A "slot" is the unit one lane moves per memory instruction: a 16-byte
// vector (VEC = true, E elements) or one element (VEC = false).  Slots of a
// row are numbered 0, 1, ...; slot s covers elements [s*W, s*W + W) with
// W = E or 1.  A slot that runs past N is loaded element by element with
// -inf fill, and stored element by element.
//
// NTL / NTS mark the vector loads / stores non-temporal (the "nt" cache
// policy on gfx950): where every byte is touched once, there is nothing to
// gain from keeping the lines in L2 / Infinity Cache.

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ uint4 vload(const void *p) {
    const u32x4 *q = static_cast<const u32x4 *>(p);
    u32x4 r;
    if constexpr (NT) r = __builtin_nontemporal_load(q); else r = *q;
    return make_uint4(r.x, r.y, r.z, r.w);
}

template <bool NT>
__device__ __forceinline__ void vstore(void *p, const uint4 &v) {
    u32x4 *q = static_cast<u32x4 *>(p);
    const u32x4 w = {v.x, v.y, v.z, v.w};
    if constexpr (NT) __builtin_nontemporal_store(w, q); else *q = w;
}

template <class Tr, bool VEC, bool NTL = false, bool NTS = NTL>
struct Slot {
    static constexpr int W = VEC ? Tr::E : 1;
    using elem_t = typename Tr::elem_t;

    // Load slot s of a row into f[0..W), -inf beyond column N.
    __device__ __forceinline__ static void load(const elem_t *row, int s,
                                                int N, float *f) {
        const int j0 = s * W;
        if constexpr (VEC) {
            if (j0 + W <= N) {
                Tr::unpack(vload<NTL>(row + j0), f);
            } else {
#pragma unroll
                for (int e = 0; e < W; ++e)
                    f[e] = (j0 + e < N) ? Tr::to_f32(row[j0 + e]) : kNegInf;
            }
        } else {
            f[0] = (j0 < N) ? Tr::to_f32(row[j0]) : kNegInf;
        }
    }

    // Load a slot known to lie entirely inside the row.
    __device__ __forceinline__ static void load_full(const elem_t *row, int s,
                                                     float *f) {
        const int j0 = s * W;
        if constexpr (VEC) {
            Tr::unpack(vload<NTL>(row + j0), f);
        } else {
            f[0] = Tr::to_f32(row[j0]);
        }
    }

    __device__ __forceinline__ static void store(elem_t *row, int s, int N,
                                                 const float *f) {
        const int j0 = s * W;
        if constexpr (VEC) {
            if (j0 + W <= N) {
                vstore<NTS>(row + j0, Tr::pack(f));
            } else {
#pragma unroll
                for (int e = 0; e < W; ++e)
                    if (j0 + e < N) row[j0 + e] = Tr::from_f32(f[e]);
            }
        } else {
            if (j0 < N) row[j0] = Tr::from_f32(f[0]);
        }
    }

    __device__ __forceinline__ static void store_full(elem_t *row, int s,
                                                      const float *f) {
        const int j0 = s * W;
        if constexpr (VEC) {
            vstore<NTS>(row + j0, Tr::pack(f));
        } else {
            row[j0] = Tr::from_f32(f[0]);
        }
    }
};

}  // namespace os
