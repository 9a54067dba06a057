// Attention forward on gfx950 matrix cores with the online softmax carried
// across key tiles: the FlashAttention consumer of the running (m, d) state
// ("5.2 CUDA Online Softmax 实现优化" §8.2; "从原始Softmax到在线Softmax",
// FlashAttention section: m, l and the unnormalised output are rescaled by
// e^(m_old - m_new) whenever a key block raises the max; "Softmax 数值稳定性
// 与 IO-Aware Attention" §7: the loop over K/V tiles).
//
// Work split.  One workgroup = 4 waves = 128 query rows of one (batch,
// head); each wave owns 32 rows.  K and V tiles of 64 keys are staged in LDS
// (double-buffered, one barrier per tile; the next tile's global loads are
// issued before the current tile's math).
//
// Products on v_mfma_f32_32x32x16_bf16 (lane l: operand row/column l % 32,
// k = 8 (l / 32) + j for j < 8; result register r: row 8 (r / 4) +
// 4 (l / 32) + r % 4, column l % 32):
//   S^T = K Q^T : A = a 32-key x 16-d slice of K from LDS, B = the wave's Q
//                 fragment held in registers.  Each lane then holds the
//                 scores of ONE query row (column l % 32) for 16 keys of a
//                 32-key block, so the row max needs one exchange between
//                 the two wave halves (v_permlane32_swap) and the row sum
//                 none until the end.
//   O^T += V^T P^T : B = the probabilities straight from the S accumulator
//                 registers (converted to bf16): register r of a 32-key
//                 block is key 8 (r / 4) + 4 (l / 32) + r % 4, so k-slot
//                 8 (l / 32) + j of the 16-key step s holds key
//                 16 s + 8 (j / 4) + 4 (l / 32) + j % 4.  A = the matching
//                 V^T slice, gathered from the row-major V tile by two
//                 ds_read_b64_tr_b16 (LDS transpose reads) per operand.
//
// The softmax runs in base 2: t = s * c with c = scale * log2(e), the
// running max m2 is kept in the same units, p = 2^(s c - m2), and
// lse = (m2 + log2 l) ln 2.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/os_attention.h"
#include "common.hpp"

namespace os {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kBlockM = kWaves * kRowsPerWave;   // query rows per workgroup
constexpr int kBlockN = 64;                      // keys per tile
constexpr int kThreads = kWaves * kWave;
constexpr float kLn2 = 0.69314718055994531f;

// LDS tile geometry (elements).  Row pitches are padded so that the MFMA
// operand reads spread over all banks: K rows by 32 bytes (a 32-row
// ds_read_b128 touches 8 distinct 32-byte bank groups), V rows by 64 bytes
// (the 8 rows of a transpose read fall on 4 distinct 64-byte groups).
template <int D>
struct Geo {
    static constexpr int KP = D + 16;
    static constexpr int VP = D + 32;
    static constexpr int KT = kBlockN * KP;
    static constexpr int VT = kBlockN * VP;
    static constexpr int kChunksPerRow = D / 8;                      // 16 B each
    static constexpr int kChunks = kBlockN * kChunksPerRow / kThreads;  // per thread
    static constexpr int kLdsElems = 2 * (KT + VT);
};

struct Params {
    const uint16_t *q, *k, *v;
    void *o;
    float *lse;
    int64_t qs[3], ks[3], vs[3], os[3];
    int H, BH, Sq, Sk, nqb;
    int causal;      // < 0: no mask; else key j admitted for query i if j <= i + causal
    float c;         // scale * log2(e)
};

__device__ __forceinline__ float swap_halves_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                              __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float swap_halves_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                              __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &u) {
    return __builtin_bit_cast(bf16x8, u);
}

template <int D>
struct Tile {
    uint4 k[Geo<D>::kChunks], v[Geo<D>::kChunks];

    // Global -> registers for keys [k0, k0 + 64): rows past Sk read as zero
    // (never from memory), so they add nothing to P.V.
    __device__ __forceinline__ void load(const uint16_t *kh, int64_t kss,
                                         const uint16_t *vh, int64_t vss,
                                         int k0, int Sk, int tid) {
#pragma unroll
        for (int i = 0; i < Geo<D>::kChunks; ++i) {
            const int ch = tid + i * kThreads;
            const int row = ch / Geo<D>::kChunksPerRow;
            const int col = (ch % Geo<D>::kChunksPerRow) * 8;
            const int key = k0 + row;
            if (key < Sk) {
                k[i] = *reinterpret_cast<const uint4 *>(kh + key * kss + col);
                v[i] = *reinterpret_cast<const uint4 *>(vh + key * vss + col);
            } else {
                k[i] = make_uint4(0, 0, 0, 0);
                v[i] = make_uint4(0, 0, 0, 0);
            }
        }
    }

    __device__ __forceinline__ void store(uint16_t *ks, uint16_t *vs,
                                          int tid) const {
#pragma unroll
        for (int i = 0; i < Geo<D>::kChunks; ++i) {
            const int ch = tid + i * kThreads;
            const int row = ch / Geo<D>::kChunksPerRow;
            const int col = (ch % Geo<D>::kChunksPerRow) * 8;
            *reinterpret_cast<uint4 *>(ks + row * Geo<D>::KP + col) = k[i];
            *reinterpret_cast<uint4 *>(vs + row * Geo<D>::VP + col) = v[i];
        }
    }
};

template <int D, bool CAUSAL, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(Params p) {
    using G = Geo<D>;
    constexpr int NT = D / 16;      // 16-wide d steps of q.k
    constexpr int NDB = D / 32;     // 32-wide d blocks of the output
    __shared__ __attribute__((aligned(16))) uint16_t smem[G::kLdsElems];
    uint16_t *k_lds = smem;                  // [2][64][KP]
    uint16_t *v_lds = smem + 2 * G::KT;      // [2][64][VP]

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int half = lane >> 5;              // which 8-wide k slice of an operand
    const int l32 = lane & 31;               // operand row / column
    const int g16 = lane & 15;               // lane within a 16-lane group
    const int grp = (lane >> 4) & 1;         // 16-row half of a 32-row V^T slice

    // the longest causal query blocks first; heads fastest
    const int bh = blockIdx.x % p.BH;
    const int qb = p.nqb - 1 - blockIdx.x / p.BH;
    const int b = bh / p.H, h = bh % p.H;
    const int q0 = qb * kBlockM;
    const int wrow0 = q0 + w * kRowsPerWave;   // the wave's first query row
    const int qrow = wrow0 + l32;               // this lane's query row

    const uint16_t *qh = p.q + b * p.qs[0] + h * p.qs[1];
    const uint16_t *kh = p.k + b * p.ks[0] + h * p.ks[1];
    const uint16_t *vh = p.v + b * p.vs[0] + h * p.vs[1];

    // the wave's Q fragment: row qrow, d = 16 t + 8 half + (0..7)
    bf16x8 qf[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (qrow < p.Sq)
            u = *reinterpret_cast<const uint4 *>(qh + qrow * p.qs[2] + 16 * t +
                                                 8 * half);
        qf[t] = as_bf16x8(u);
    }

    // keys this workgroup needs: all, or up to the causal limit of its last row
    int kend = p.Sk;
    if (CAUSAL) {
        const int64_t lim = int64_t(q0) + kBlockM + p.causal;
        kend = lim < p.Sk ? int(lim) : p.Sk;
    }
    const int nkt = (kend + kBlockN - 1) / kBlockN;
    // a wave whose rows are all past Sq, or (causal) past which a tile lies,
    // skips the math but still loads its share of every tile
    const bool wave_live = wrow0 < p.Sq;
    const int64_t wave_last_key = int64_t(wrow0) + kRowsPerWave - 1 + p.causal;

    float m2 = kNegInf;   // running max of s * c
    float l = 0.0f;       // this lane's share of the running sum (its 32 keys per tile)
    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

    Tile<D> tile;
    tile.load(kh, p.ks[2], vh, p.vs[2], 0, p.Sk, tid);
    tile.store(k_lds, v_lds, tid);
    __syncthreads();

    for (int kt = 0; kt < nkt; ++kt) {
        const int buf = kt & 1;
        const int k0 = kt * kBlockN;
        if (kt + 1 < nkt)
            tile.load(kh, p.ks[2], vh, p.vs[2], k0 + kBlockN, p.Sk, tid);

        const bool live = wave_live && (!CAUSAL || int64_t(k0) <= wave_last_key);
        if (live) {
            const uint16_t *kt_lds = k_lds + buf * G::KT;
            const uint16_t *vt_lds = v_lds + buf * G::VT;
            // ---- S^T = K Q^T for two 32-key blocks ----
            f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int t = 0; t < NT; ++t) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(
                        kt_lds + (32 * kb + l32) * G::KP + 16 * t + 8 * half);
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t],
                                                                     s[kb], 0, 0, 0);
                }
            }
            // ---- mask keys past Sk and (causal) past the row's limit ----
            const bool tail = k0 + kBlockN > p.Sk;
            const bool diag = CAUSAL && int64_t(k0) + kBlockN - 1 > int64_t(wrow0) + p.causal;
            if (tail || diag) {
                const int64_t row_last = int64_t(qrow) + p.causal;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
                        bool out = key >= p.Sk;
                        if (CAUSAL) out = out || key > row_last;
                        if (out) s[kb][r] = kNegInf;
                    }
            }
            // ---- online softmax update of this row ----
            float mx = kNegInf;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            mx = swap_halves_max(mx);
            const float m2n = fmaxf(m2, mx * p.c);
            const float alpha = exp2_fast(m2 - m2n);   // 0 on the first tile
            float rs = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float e = exp2_fast(fmaf(s[kb][r], p.c, -m2n));
                    s[kb][r] = e;
                    rs += e;
                }
            l = l * alpha + rs;
            m2 = m2n;
            if (wave_any(alpha != 1.0f)) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
            }
            // ---- probabilities as the bf16 B operand, one per 16-key step ----
            bf16x8 pf[4];
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int kb = st >> 1, r0 = 8 * (st & 1);
                f32x8 x = {s[kb][r0 + 0], s[kb][r0 + 1], s[kb][r0 + 2], s[kb][r0 + 3],
                           s[kb][r0 + 4], s[kb][r0 + 5], s[kb][r0 + 6], s[kb][r0 + 7]};
                pf[st] = __builtin_convertvector(x, bf16x8);
            }
            // ---- O^T += V^T P^T ----
            // transpose read: lane x of a 16-lane group supplies the address
            // of row (base + x / 4), columns 4 (x % 4) .. + 3; lane i then
            // receives column i of those 4 rows.
            const lds_char *vb = (const lds_char *)(vt_lds);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const int row = 16 * st + 4 * half + (g16 >> 2);
                    const int col = 32 * db + 16 * grp + 4 * (g16 & 3);
                    const lds_char *a0 = vb + 2 * (row * G::VP + col);
                    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (lds_bf16x4 *)a0);
                    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (lds_bf16x4 *)(a0 + 2 * 8 * G::VP));
                    const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3,
                                                              4, 5, 6, 7);
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[st],
                                                                       acc[db], 0, 0, 0);
                }
            }
        }
        if (kt + 1 < nkt)
            tile.store(k_lds + (buf ^ 1) * G::KT, v_lds + (buf ^ 1) * G::VT, tid);
        __syncthreads();
    }

    // ---- epilogue: o = o~ / l, lse = (m2 + log2 l) ln 2 ----
    const float lt = swap_halves_sum(l);
    if (qrow < p.Sq) {
        const float inv = 1.0f / lt;
        const int64_t obase = b * p.os[0] + h * p.os[1] + int64_t(qrow) * p.os[2];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int d = 32 * db + 8 * rg + 4 * half;
                f32x4 x = {acc[db][4 * rg + 0] * inv, acc[db][4 * rg + 1] * inv,
                           acc[db][4 * rg + 2] * inv, acc[db][4 * rg + 3] * inv};
                if (OUT_BF16) {
                    bf16x4 y = __builtin_convertvector(x, bf16x4);
                    *reinterpret_cast<bf16x4 *>(static_cast<uint16_t *>(p.o) + obase + d) = y;
                } else {
                    *reinterpret_cast<f32x4 *>(static_cast<float *>(p.o) + obase + d) = x;
                }
            }
        if (p.lse != nullptr && half == 0)
            p.lse[int64_t(bh) * p.Sq + qrow] = (m2 + __builtin_amdgcn_logf(lt)) * kLn2;
    }
}

template <int D, bool CAUSAL, bool OUT_BF16>
void launch_d(const Params &p, int64_t blocks, hipStream_t stream) {
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, OUT_BF16>), dim3(unsigned(blocks)),
                       dim3(kThreads), 0, stream, p);
}

template <int D>
void launch(const Params &p, bool causal, bool out_bf16, int64_t blocks,
            hipStream_t stream) {
    if (causal) {
        if (out_bf16) launch_d<D, true, true>(p, blocks, stream);
        else launch_d<D, true, false>(p, blocks, stream);
    } else {
        if (out_bf16) launch_d<D, false, true>(p, blocks, stream);
        else launch_d<D, false, false>(p, blocks, stream);
    }
}

bool aligned16(const void *ptr) { return reinterpret_cast<uintptr_t>(ptr) % 16 == 0; }

}  // namespace attn
}  // namespace os

extern "C" os_status os_attention_fwd(
    const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
    int64_t H, int64_t Sq, int64_t Sk, int64_t D, const int64_t *q_strides,
    const int64_t *k_strides, const int64_t *v_strides, const int64_t *o_strides,
    os_dtype o_dtype, float scale, int64_t causal_offset, hipStream_t stream) {
    using namespace os::attn;
    constexpr int64_t kMax = (int64_t(1) << 31) - 1;
    if (o_dtype != OS_F32 && o_dtype != OS_BF16) return OS_ERR_DTYPE;
    if (B < 0 || H < 0 || Sq < 0 || Sk < 1 || Sq > kMax || Sk > kMax)
        return OS_ERR_SHAPE;
    if (D != 64 && D != 128) return OS_ERR_UNSUPPORTED;
    if (!(scale > 0.0f) || !(scale <= 3.4028234663852886e38f)) return OS_ERR_UNSUPPORTED;
    if (!q_strides || !k_strides || !v_strides || !o_strides) return OS_ERR_NULL;
    const int64_t nqb = (Sq + kBlockM - 1) / kBlockM;
    if (B > 0 && H > 0 && (B * H > kMax || nqb * B * H > kMax)) return OS_ERR_SHAPE;
    const int64_t *st[4] = {q_strides, k_strides, v_strides, o_strides};
    const int es[4] = {2, 2, 2, o_dtype == OS_BF16 ? 2 : 4};
    for (int t = 0; t < 4; ++t) {
        for (int j = 0; j < 3; ++j) {
            if (st[t][j] < 0 || (st[t][j] * es[t]) % 16 != 0) return OS_ERR_STRIDE;
        }
        if (st[t][2] < D) return OS_ERR_STRIDE;
    }
    if (B == 0 || H == 0 || Sq == 0) return OS_OK;
    if (!q || !k || !v || !o) return OS_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return OS_ERR_STRIDE;

    Params p{};
    p.q = static_cast<const uint16_t *>(q);
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.o = o;
    p.lse = lse;
    for (int j = 0; j < 3; ++j) {
        p.qs[j] = q_strides[j];
        p.ks[j] = k_strides[j];
        p.vs[j] = v_strides[j];
        p.os[j] = o_strides[j];
    }
    p.H = int(H);
    p.BH = int(B * H);
    p.Sq = int(Sq);
    p.Sk = int(Sk);
    p.nqb = int(nqb);
    // an offset that admits every key of every row is no mask
    const bool causal = causal_offset >= 0 && causal_offset < Sk - 1;
    p.causal = causal ? int(causal_offset) : 0;
    p.c = float(double(scale) * 1.4426950408889634);
    const int64_t blocks = nqb * B * H;
    if (D == 64) launch<64>(p, causal, o_dtype == OS_BF16, blocks, stream);
    else launch<128>(p, causal, o_dtype == OS_BF16, blocks, stream);
    return hipGetLastError() == hipSuccess ? OS_OK : OS_ERR_HIP;
}
