// Attention forward on gfx950 matrix cores with the online softmax carried
// across key tiles: the FlashAttention consumer of the running (m, d) state
// ("5.2 CUDA Online Softmax 实现优化" §8.2; "从原始Softmax到在线Softmax",
// FlashAttention section: m, l and the unnormalised output are rescaled by
// e^(m_old - m_new) whenever a key block raises the max; "Softmax 数值稳定性
// 与 IO-Aware Attention" §7: the loop over K/V tiles).
//
// Work split.  One workgroup = 8 waves = 256 query rows of one (batch,
// head) (under a causal mask, two such blocks in turn: the pair {n - 1 - i,
// i} of the n query blocks, so every workgroup has the same work); each
// wave owns 32 rows, and each K/V tile in LDS feeds all 8.  At up to ~240
// VGPRs two waves fit per SIMD, i.e. one workgroup per CU.  K and V tiles of
// 64 keys (128 at d = 32) stream through LDS rings (three tiles each at
// d = 128, two at d = 64 and 32: 96 or 32 KiB), filled by direct-to-LDS
// buffer loads (buffer_load_dwordx4 ... lds): no VGPR
// staging, and lanes past the last key read as zero because each tile's
// buffer descriptor covers only the keys that exist.
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
// Ping-pong.  Each tile is worked in two halves: a VALU half (the
// probabilities p = 2^(s c - m2), their row sum, their bf16 copies) and a
// matrix half (O^T += V^T P^T for the tile, then the scores of the next
// tile).  The two waves that share a SIMD (waves w and w + 4 of the
// workgroup) run half a tile apart, so one wave's exponentials overlap the
// other wave's MFMAs; where each group of four waves puts its barriers (both
// execute the same number) keeps them apart.  The schedule, in barrier
// intervals: in interval 2j group 0 does tile j's VALU half and group 1 tile
// j - 1's matrix half; in interval 2j + 1 group 0 does tile j's matrix half
// and group 1 tile j's VALU half.  The loads for tile t's matrix half (V of
// tile t, K of tile t + 1) are waited for before the barrier that opens
// interval 2t + 1; each load instruction holds its wave for tens of cycles,
// so they go into the shorter half of an interval.
//   d = 128 (the matrix half is the longer one): rings of three tiles; each
//     group issues its share with its VALU half of tile t - 1, group 0 in
//     interval 2t - 2 and group 1 in interval 2t - 1.  The slot of tile t
//     was last read (by tile t - 3) in interval 2t - 4.
//   d = 64 and 32 (the VALU half is the longer one): rings of two tiles;
//     group 0 issues both groups' shares at the start of its matrix half of
//     tile t - 1, in interval 2t - 1.  The slot was last read in interval
//     2t - 2.
//
// Online state in base 2: t = s c with c = scale log2(e).  Each row starts
// its reference point m2 at the max of its first tile; later it moves only
// when some lane's sum of p exceeds 2^8 (the sum bounds every p of the
// lane): then the exact row max is taken, o~ and l are rescaled by
// 2^(m2_old - m2_new) and the tile's p recomputed.  Every p stays below 2^8,
// and the result does not depend on which reference point is used, since o
// and l are both taken relative to it; lse = (m2 + log2 l) ln 2.
//
// LDS layouts (rows of 2D bytes, no padding): 16-byte chunk c of row r of a
// K tile sits in slot c ^ fk(r), of a V tile in slot c ^ fv(r).  LDS serves
// 256 bytes per clock: a 128-bit read 16 lanes at a time, a 64-bit read 32
// lanes at a time.  The swizzles give the 16 K rows of each 16-lane group of
// an operand read, and the 4 V rows of each 32-lane group of a transpose
// read, disjoint banks, so neither read conflicts (rocprofv3 counts zero
// SQ_LDS_BANK_CONFLICT cycles for this kernel).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/os_attention.h"
#include "chunks.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace os {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWaves = 8;
constexpr int kRowsPerWave = 32;
constexpr int kBlockM = kWaves * kRowsPerWave;   // query rows per workgroup
constexpr int kThreads = kWaves * kWave;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kOver = 256.0f;                  // a row sum above this moves m2
constexpr int kKAhead = 3;                       // K operand reads issued ahead
// Buffer descriptor word 3 for raw (unswizzled, stride 0) dword buffers.
constexpr int kRsrcWord3 = 0x00020000;
// Row strides (elements) below this keep a tile's byte offsets in 32 bits.
constexpr int64_t kMaxRowStride = int64_t(1) << 23;

template <int D>
struct Geo {
    // keys per tile: 64, or 128 at d = 32, whose tiles would otherwise be
    // too short to pay for their barriers
    static constexpr int BN = D == 32 ? 128 : 64;
    static constexpr int KB = BN / 32;                  // 32-key score blocks
    static constexpr int NST = BN / 16;                 // 16-key P.V steps
    static constexpr int RB = 2 * D;                    // bytes per row
    static constexpr int TILE = BN * RB;                // bytes per K or V tile
    static constexpr int CPR = D / 8;                   // 16-byte chunks per row
    static constexpr int RPB = 1024 / RB;               // rows per 1 KB wave load
    static constexpr int NDMA = TILE / 1024 / kWaves;   // wave loads per tile
    static_assert(NDMA >= 1 && NDMA * kWaves * 1024 == TILE,
                  "the waves' 1 KiB loads must cover a tile exactly");
    static constexpr int NSLOT = D == 128 ? 3 : 2;      // tiles per ring
    static constexpr int kLdsBytes = 2 * NSLOT * TILE;  // V ring, then K ring
    static constexpr int VRING = 0, KRING = NSLOT * TILE;
    // a row is 16 (d = 128), 8 (d = 64) or 4 (d = 32) chunks; a 16-lane
    // group of a K operand read covers 16 consecutive rows, a 32-lane group
    // of a V transpose read 4 consecutive rows of 64 bytes
    __device__ static int fk(int r) {
        return D == 128 ? (r & 15) : D == 64 ? ((r >> 1) & 7) : ((r >> 2) & 3);
    }
    __device__ static int fv(int r) {
        return D == 128 ? 4 * (r & 3) : D == 64 ? 4 * ((r >> 1) & 1) : 0;
    }
};

struct Params {
    const uint16_t *q, *k, *v;
    void *o;
    float *lse;
    int64_t qs[3], ks[3], vs[3], os[3];
    int H, BH, Sq, Sk, nqb;
    int causal;      // key j admitted for query i if j <= i + causal (CAUSAL only)
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

// Direct-to-LDS load of one key tile (K or V) of one head: wave w writes
// 1 KB blocks w, w + kWaves, ...; lane l's 16 bytes land at block + 16 l.
// Block i of the wave holds rows kWaves i RPB (>= 16) further down than
// block 0, and the swizzle of a row depends only on its low four bits,
// which that step leaves alone, so one per-lane offset (row and chunk
// within block 0) plus a uniform offset per block addresses every load.
// Keys at or past Sk lie outside the descriptor and arrive as zeros.
template <int D>
__device__ __forceinline__ void load_tile(const uint16_t *head, int64_t row_bytes,
                                          int k0, int Sk, lds_char *dst,
                                          uint32_t off, int w) {
    using G = Geo<D>;
    int rows = Sk - k0;
    rows = rows < 0 ? 0 : (rows > G::BN ? G::BN : rows);
    // every field of the descriptor is wave-uniform; say so, so that it is
    // built in scalar registers
    const uint64_t a = reinterpret_cast<uint64_t>(head) + uint64_t(int64_t(k0) * row_bytes);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
    const int nrec = __builtin_amdgcn_readfirstlane(int(rows * row_bytes));
    char *base = reinterpret_cast<char *>((uint64_t(hi) << 32) | lo);
    __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(base, 0, nrec, kRsrcWord3);
    const int step = int(kWaves * G::RPB * row_bytes);
#pragma unroll
    for (int i = 0; i < G::NDMA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (lds_void *)(dst + (i * kWaves + w) * 1024), 16, off, i * step, 0, 0);
}

__device__ __forceinline__ void wait_loads() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int D, bool CAUSAL, bool OUT_BF16>
struct Kernel {
    using G = Geo<D>;
    static constexpr int NT = D / 16;      // 16-wide d steps of q.k
    static constexpr int NDB = D / 32;     // 32-wide d blocks of the output

    lds_char *lds;
    const Params &p;
    int w, lane, half, l32;
    int wrow0, qrow, Sk;
    const uint16_t *kh, *vh;
    int64_t krb, vrb;                 // row strides in bytes
    uint32_t dk, dv;                  // per-lane DMA source offsets (block 0)
    uint32_t koff[NT];                // per-lane K operand offsets
    uint32_t voff[NDB];               // per-lane V^T transpose-read offsets
    bf16x8 qf[NT];
    f32x16 acc[NDB];
    f32x16 sc[G::KB];                 // scores of the tile in hand
    bf16x8 pf[G::NST];                // its probabilities as the P.V operand
    float m2, l;

    __device__ __forceinline__ Kernel(lds_char *lds_, const Params &p_) : lds(lds_), p(p_) {}

    __device__ __forceinline__ bool needs_mask(int kt) const {
        const int k0 = kt * G::BN;
        bool m = k0 + G::BN > Sk;
        if (CAUSAL) m = m || int64_t(k0) + G::BN - 1 > int64_t(wrow0) + p.causal;
        return m;
    }

    __device__ __forceinline__ void mask(f32x16 (&s)[G::KB], int kt) const {
        const int k0 = kt * G::BN;
        int64_t lim = Sk;
        if (CAUSAL) {
            const int64_t c = int64_t(qrow) + p.causal + 1;
            lim = c < lim ? c : lim;
        }
        const int64_t rem = lim - k0 - 4 * half;
#pragma unroll
        for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (32 * kb + 8 * (r >> 2) + (r & 3) >= rem) s[kb][r] = kNegInf;
    }

    __device__ __forceinline__ float rowmax(const f32x16 (&s)[G::KB]) const {
        float mx[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
        for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx[r & 3] = fmaxf(mx[r & 3], s[kb][r]);
        return swap_halves_max(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3])));
    }

    // S^T = K Q^T for the tile in K-ring slot KBUF.  The K operands are read
    // by inline asm PF operands ahead of their product, with explicit
    // lgkmcnt waits (as for the V reads below).  koff holds KRING, which
    // keeps the immediate offset below 64 KiB.
    template <int KBUF, int I>
    __device__ __forceinline__ void k_issue(u32x4 *kf, uint32_t base) const {
        constexpr int t = I / G::KB, kb = I % G::KB;
        constexpr int off = KBUF * G::TILE + kb * 32 * G::RB;
        asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(kf[I]) : "v"(base + koff[t]), "n"(off));
    }

    template <int KBUF, int N, int PF, int I>
    __device__ __forceinline__ void qk_rec(f32x16 (&s)[G::KB], u32x4 *kf, uint32_t base) const {
        if constexpr (I < N) {
            constexpr int t = I / G::KB, kb = I % G::KB;
            if constexpr (I + PF < N) k_issue<KBUF, I + PF>(kf, base);
            constexpr int later = (N - 1 - I) < PF ? (N - 1 - I) : PF;
            asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(kf[I]) : "n"(later));
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[I]),
                                                             qf[t], s[kb], 0, 0, 0);
            qk_rec<KBUF, N, PF, I + 1>(s, kf, base);
        }
    }

    template <int KBUF, int PF, int I>
    __device__ __forceinline__ void k_prologue(u32x4 *kf, uint32_t base) const {
        if constexpr (I < PF) {
            k_issue<KBUF, I>(kf, base);
            k_prologue<KBUF, PF, I + 1>(kf, base);
        }
    }

    template <int KBUF>
    __device__ __forceinline__ void qk(f32x16 (&s)[G::KB]) const {
        constexpr int N = NT * G::KB;
        constexpr int PF = kKAhead < N ? kKAhead : N;
        const uint32_t base = uint32_t(reinterpret_cast<uintptr_t>(lds));
#pragma unroll
        for (int kb = 0; kb < G::KB; ++kb) s[kb] = f32x16{};
        u32x4 kf[N];
        k_prologue<KBUF, PF, 0>(kf, base);
        qk_rec<KBUF, N, PF, 0>(s, kf, base);
    }

    // O^T += V^T P^T for 16-key steps ST0..ST1 of the tile in V-ring slot
    // VBUF.  The transpose reads are issued as inline asm, two operands
    // ahead of the product that uses them, with explicit lgkmcnt waits: the
    // compiler would otherwise precede the first of them with a wait for
    // every direct-to-LDS load in flight (it cannot tell that they touch
    // other LDS), i.e. for the next tiles' loads issued at the top of the
    // step.  LDS operations complete in order, so waiting until at most
    // 2 n remain, with n operands issued after this one, is enough; any
    // LDS operation the compiler adds only makes its own waits stricter.
    template <int VBUF, int ST0, int I>
    __device__ __forceinline__ void tr_issue(u32x2 *lo, u32x2 *hi, uint32_t base) const {
        constexpr int st = ST0 + I / NDB, db = I % NDB;
        constexpr int off = G::VRING + VBUF * G::TILE + 16 * st * G::RB;
        const uint32_t a = base + voff[db];
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo[I]) : "v"(a), "n"(off));
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                     : "=v"(hi[I]) : "v"(a), "n"(off + 8 * G::RB));
    }

    template <int VBUF, int ST0, int N, int I>
    __device__ __forceinline__ void pv_rec(const bf16x8 (&pf)[G::NST], u32x2 *lo, u32x2 *hi,
                                           uint32_t base) {
        if constexpr (I < N) {
            constexpr int st = ST0 + I / NDB, db = I % NDB;
            if constexpr (I + 2 < N) tr_issue<VBUF, ST0, I + 2>(lo, hi, base);
            constexpr int later = (N - 1 - I) < 2 ? (N - 1 - I) : 2;  // operands issued after I
            asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(lo[I]), "+v"(hi[I]) : "n"(2 * later));
            const u32x4 u = {lo[I][0], lo[I][1], hi[I][0], hi[I][1]};
            const bf16x8 vf = __builtin_bit_cast(bf16x8, u);
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[st], acc[db], 0, 0, 0);
            pv_rec<VBUF, ST0, N, I + 1>(pf, lo, hi, base);
        }
    }

    template <int VBUF, int ST0, int ST1>
    __device__ __forceinline__ void pv(const bf16x8 (&pf)[G::NST]) {
        constexpr int N = (ST1 - ST0 + 1) * NDB;     // operands (MFMAs) in this call
        const uint32_t base = uint32_t(reinterpret_cast<uintptr_t>(lds));
        u32x2 lo[N], hi[N];
        tr_issue<VBUF, ST0, 0>(lo, hi, base);
        if constexpr (N > 1) tr_issue<VBUF, ST0, 1>(lo, hi, base);
        pv_rec<VBUF, ST0, N, 0>(pf, lo, hi, base);
    }

    // p = 2^(s c - m2) for the tile in sc, their sum (returned), and their
    // bf16 copies in pf (8 keys each)
    __device__ __forceinline__ float probs() {
        float rs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                f32x8 e;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    e[r] = exp2_fast(fmaf(sc[kb][8 * hh + r], p.c, -m2));
                    rs[r & 3] += e[r];
                }
                pf[2 * kb + hh] = __builtin_convertvector(e, bf16x8);
            }
        return (rs[0] + rs[1]) + (rs[2] + rs[3]);
    }

    // VALU half of tile j: its probabilities and row sum.  The reference
    // point m2 moves only when some lane's sum exceeds kOver, which bounds
    // every p of that lane: then the exact row max is taken, o~ and l are
    // rescaled and the probabilities recomputed (rare once a row's max has
    // been seen; a NaN sum keeps its NaN, as the row is NaN anyway).
    __device__ __forceinline__ void h1(int j) {
        if (j > 0 && needs_mask(j)) mask(sc, j);
        float rs = probs();
        if (wave_any(rs > kOver)) {
            const float m2n = fmaxf(m2, rowmax(sc) * p.c);
            const float alpha = exp2_fast(m2 - m2n);
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
            l *= alpha;
            m2 = m2n;
            rs = probs();
        }
        l += rs;
    }

    // matrix half of tile j (PAR = j mod NSLOT): O^T += V^T P^T from V slot
    // PAR, then the scores of tile j + 1 from the next K slot
    template <int PAR>
    __device__ __forceinline__ void h2() {
        pv<PAR, 0, G::NST - 1>(pf);
        qk<(PAR + 1) % G::NSLOT>(sc);
    }

    // the loads for tile t's matrix half: V of tile t (slot t mod NSLOT)
    // and K of tile t + 1 (slot (t + 1) mod NSLOT)
    // the same loads for wave w and its partner w + kWaves / 2 (issued by
    // group 0 alone at d = 64 and 32).  The partner's rows lie kWaves / 2 RPB
    // (a multiple of 16) rows further down, which leaves the swizzle alone,
    // so its per-lane offsets are this wave's plus that many rows.
    static constexpr bool kGroup0Loads = D != 128;
    __device__ __forceinline__ void dma_pair(int t) {
        constexpr int hw = kWaves / 2;
        lds_char *vdst = lds + G::VRING + (t % G::NSLOT) * G::TILE;
        lds_char *kdst = lds + G::KRING + ((t + 1) % G::NSLOT) * G::TILE;
        load_tile<D>(vh, vrb, t * G::BN, Sk, vdst, dv, w);
        load_tile<D>(vh, vrb, t * G::BN, Sk, vdst, dv + uint32_t(hw * G::RPB * vrb), w + hw);
        load_tile<D>(kh, krb, (t + 1) * G::BN, Sk, kdst, dk, w);
        load_tile<D>(kh, krb, (t + 1) * G::BN, Sk, kdst, dk + uint32_t(hw * G::RPB * krb),
                     w + hw);
    }

    __device__ __forceinline__ void dma(int t) {
        load_tile<D>(vh, vrb, t * G::BN, Sk, lds + G::VRING + (t % G::NSLOT) * G::TILE, dv, w);
        load_tile<D>(kh, krb, (t + 1) * G::BN, Sk,
                     lds + G::KRING + ((t + 1) % G::NSLOT) * G::TILE, dk, w);
    }

    __device__ __forceinline__ void bar() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    }

    // The two waves of each SIMD (waves w and w + 4) run half a tile apart:
    // group 0 does tile j's VALU half while group 1 does tile j - 1's matrix
    // half, and the other way round, held in step by where each group puts
    // its barriers (both execute the same number).  The loads of tile j + 1
    // (V of tile j + 1, K of tile j + 2) go with each group's VALU half of
    // tile j at d = 128, with group 0's matrix half of tile j at d = 64 and
    // 32 (both groups' shares); every wave has waited for its own before the
    // barrier that opens interval 2j + 3.
    template <int GROUP, int PAR>
    __device__ __forceinline__ void tile(int j) {
        if (GROUP == 0 && G::NSLOT == 3) {
            dma(j + 1);
            h1(j);
            // tile j's loads (issued an interval earlier) have landed; tile
            // j + 1's may still be in flight
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * G::NDMA) : "memory");
            bar();
            h2<PAR>();
            bar();
        } else if (GROUP == 0) {
            h1(j);
            wait_loads();
            bar();
            if (kGroup0Loads) dma_pair(j + 1);
            else dma(j + 1);
            h2<PAR>();
            bar();
        } else {
            if (!kGroup0Loads) dma(j + 1);
            h1(j);
            bar();
            h2<PAR>();
            wait_loads();
            bar();
        }
    }

    template <int GROUP>
    __device__ __forceinline__ void tiles(int nkt) {
        if (GROUP == 1) bar();
        int j = 0;
        if constexpr (G::NSLOT == 3) {
            for (; j + 2 < nkt; j += 3) {
                tile<GROUP, 0>(j);
                tile<GROUP, 1>(j + 1);
                tile<GROUP, 2>(j + 2);
            }
            if (j < nkt) tile<GROUP, 0>(j);
            if (j + 1 < nkt) tile<GROUP, 1>(j + 1);
        } else {
            for (; j + 1 < nkt; j += 2) {
                tile<GROUP, 0>(j);
                tile<GROUP, 1>(j + 1);
            }
            if (j < nkt) tile<GROUP, 0>(j);
        }
        if (GROUP == 0) bar();
    }

    __device__ __forceinline__ void run() {
        const int tid = threadIdx.x;
        lane = tid & (kWave - 1);
        w = __builtin_amdgcn_readfirstlane(tid / kWave);
        half = lane >> 5;
        l32 = lane & 31;
        const int g16 = lane & 15;
        const int grp = (lane >> 4) & 1;

        // heads fastest.  Under a causal mask query block i needs about i
        // key tiles, so a workgroup takes the pair {n - 1 - i, i} (all pairs
        // then cost the same and fit in one round of residency).
        const int bh = blockIdx.x % p.BH;
        const int i = blockIdx.x / p.BH;
        const int b = bh / p.H, h = bh % p.H;
        Sk = p.Sk;
        kh = p.k + b * p.ks[0] + h * p.ks[1];
        vh = p.v + b * p.vs[0] + h * p.vs[1];
        krb = p.ks[2] * 2;
        vrb = p.vs[2] * 2;

        // per-lane offsets: DMA sources, K operand reads, V^T transpose reads
        {
            const int r = w * G::RPB + lane / G::CPR;
            const int slot = lane % G::CPR;
            dk = uint32_t(r * krb + 16 * (slot ^ G::fk(r)));
            dv = uint32_t(r * vrb + 16 * (slot ^ G::fv(r)));
        }
        // chunk 2 t + half of row 32 kb + l32 sits in slot (2 t + half) ^ fk(l32)
#pragma unroll
        for (int t = 0; t < NT; ++t)
            koff[t] = uint32_t(G::KRING + l32 * G::RB + 16 * ((2 * t + half) ^ G::fk(l32)));
        const int vrow = 4 * half + (g16 >> 2);
        const int x = 2 * grp + ((g16 & 3) >> 1);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            voff[db] = uint32_t(vrow * G::RB + 16 * ((4 * db + x) ^ G::fv(vrow)) +
                                8 * (g16 & 1));

        const uint16_t *qh = p.q + b * p.qs[0] + h * p.qs[1];
        if (CAUSAL) {
            const int qa = p.nqb - 1 - i;
            block(qa, bh, qh, b, h);
            if (i != qa) {
                __syncthreads();       // every wave is done with the LDS rings
                block(i, bh, qh, b, h);
            }
        } else {
            block(p.nqb - 1 - i, bh, qh, b, h);
        }
    }

    // one block of kBlockM query rows against all the keys it admits
    __device__ __forceinline__ void block(int qb, int bh, const uint16_t *qh, int b, int h) {
        const int q0 = qb * kBlockM;
        wrow0 = q0 + w * kRowsPerWave;
        qrow = wrow0 + l32;

        // the wave's Q fragment: row qrow, d = 16 t + 8 half + (0..7)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (qrow < p.Sq)
                u = *reinterpret_cast<const uint4 *>(qh + qrow * p.qs[2] + 16 * t +
                                                     8 * half);
            qf[t] = as_bf16x8(u);
        }

        // keys this workgroup needs: all, or up to the causal limit of its last row
        int kend = Sk;
        if (CAUSAL) {
            const int64_t lim = int64_t(q0) + kBlockM + p.causal;
            kend = lim < Sk ? int(lim) : Sk;
        }
        const int nkt = (kend + G::BN - 1) / G::BN;

        m2 = kNegInf;
        l = 0.0f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

        // prologue: K of tile 0 (slot 0), then tile 0's loads (V 0, K 1);
        // every wave forms the scores of tile 0 and starts its reference
        // point at their row max
        load_tile<D>(kh, krb, 0, Sk, lds + G::KRING, dk, w);
        dma(0);
        wait_loads();
        bar();
        qk<0>(sc);
        if (needs_mask(0)) mask(sc, 0);
        m2 = rowmax(sc) * p.c;

        if (w < kWaves / 2) tiles<0>(nkt);
        else tiles<1>(nkt);
        wait_loads();

        // epilogue: o = o~ / l, lse = (m2 + log2 l) ln 2
        const float lt = swap_halves_sum(l);
        if (qrow < p.Sq) {
            const float inv = 1.0f / lt;
            const int64_t obase = b * p.os[0] + h * p.os[1] + int64_t(qrow) * p.os[2];
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int d = 32 * db + 8 * rg + 4 * half;
                    f32x4 xo = {acc[db][4 * rg + 0] * inv, acc[db][4 * rg + 1] * inv,
                                acc[db][4 * rg + 2] * inv, acc[db][4 * rg + 3] * inv};
                    if (OUT_BF16) {
                        bf16x4 y = __builtin_convertvector(xo, bf16x4);
                        *reinterpret_cast<bf16x4 *>(static_cast<uint16_t *>(p.o) + obase + d) = y;
                    } else {
                        *reinterpret_cast<f32x4 *>(static_cast<float *>(p.o) + obase + d) = xo;
                    }
                }
            if (p.lse != nullptr && half == 0)
                p.lse[int64_t(bh) * p.Sq + qrow] = (m2 + __builtin_amdgcn_logf(lt)) * kLn2;
        }
    }
};

template <int D, bool CAUSAL, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(Params p) {
    __shared__ __attribute__((aligned(1024))) char smem[Geo<D>::kLdsBytes];
    Kernel<D, CAUSAL, OUT_BF16> k((lds_char *)smem, p);
    k.run();
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
    // sequence lengths up to 2^30 keep every row and tile index (including
    // the look-ahead tiles past the end) inside int
    constexpr int64_t kMaxSeq = int64_t(1) << 30;
    if (o_dtype != OS_F32 && o_dtype != OS_BF16) return OS_ERR_DTYPE;
    if (B < 0 || H < 0 || Sq < 0 || Sk < 1 || Sq > kMaxSeq || Sk > kMaxSeq)
        return OS_ERR_SHAPE;
    if (D != 32 && D != 64 && D != 128) return OS_ERR_UNSUPPORTED;
    if (!(scale > 0.0f) || !(scale <= 3.4028234663852886e38f)) return OS_ERR_UNSUPPORTED;
    if (!q_strides || !k_strides || !v_strides || !o_strides) return OS_ERR_NULL;
    const int64_t nqb = (Sq + kBlockM - 1) / kBlockM;
    if (B > 0 && H > 0 && (B > kMax / H || nqb * B * H > kMax)) return OS_ERR_SHAPE;
    const int64_t *st[4] = {q_strides, k_strides, v_strides, o_strides};
    const int es[4] = {2, 2, 2, o_dtype == OS_BF16 ? 2 : 4};
    for (int t = 0; t < 4; ++t) {
        for (int j = 0; j < 3; ++j) {
            if (st[t][j] < 0 || (st[t][j] * es[t]) % 16 != 0) return OS_ERR_STRIDE;
        }
        if (st[t][2] < D) return OS_ERR_STRIDE;
    }
    if (k_strides[2] >= kMaxRowStride || v_strides[2] >= kMaxRowStride)
        return OS_ERR_UNSUPPORTED;
    if (B == 0 || H == 0 || Sq == 0) return OS_OK;
    if (!q || !k || !v || !o) return OS_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return OS_ERR_STRIDE;
    const os::Device *dev = os::current_device();
    if (dev == nullptr || !dev->gfx950) return OS_ERR_DEVICE;

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
    // causal: one workgroup per pair of query blocks {nqb - 1 - i, i}
    const int64_t per_head = causal ? (nqb + 1) / 2 : nqb;
    // A launch's grid counts work-items in 32 bits: beyond 2^22 workgroups
    // the heads are launched in parts (whole batches, or runs of heads of
    // one batch), each a call of its own on the heads it covers.
    const int oes = o_dtype == OS_BF16 ? 2 : 4;
    bool ok = true;
    os::for_each_head_chunk(B, H, per_head, [&](const os::HeadChunk &c) {
        if (!ok) return;
        Params pc = p;
        pc.q = p.q + c.b0 * p.qs[0] + c.h0 * p.qs[1];
        pc.k = p.k + c.b0 * p.ks[0] + c.h0 * p.ks[1];
        pc.v = p.v + c.b0 * p.vs[0] + c.h0 * p.vs[1];
        pc.o = static_cast<char *>(o) + (c.b0 * p.os[0] + c.h0 * p.os[1]) * oes;
        if (lse) pc.lse = lse + (c.b0 * H + c.h0) * Sq;
        pc.H = int(c.nh);
        pc.BH = int(c.nb * c.nh);
        const int64_t blocks = per_head * c.nb * c.nh;
        if (D == 32) launch<32>(pc, causal, o_dtype == OS_BF16, blocks, stream);
        else if (D == 64) launch<64>(pc, causal, o_dtype == OS_BF16, blocks, stream);
        else launch<128>(pc, causal, o_dtype == OS_BF16, blocks, stream);
        ok = ok && hipGetLastError() == hipSuccess;
    });
    return ok ? OS_OK : OS_ERR_HIP;
}
