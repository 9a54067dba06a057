// Split-row path (partial states -> state merge, alone for statistics or
// folded into the normalise kernel), the normalise pass for a given row
// state, the public state-merge launcher and the cross-entropy mean.
#include "kernels.hpp"
#include "launch.hpp"

namespace os {
namespace {

// 8 waves per chunk workgroup (a 128 KiB fp32 chunk is two 64 KiB tiles):
// fp32 16 x 4194304 softmax 119.0 us and statistics 43.7 us, against 123.1
// and 44.6 us with 4 waves (MI355X, 8 rotating buffer sets); a plan of 4x
// the workgroups, or tiles of a whole chunk, were slower.  Chunks shorter
// than one such tile (rows of a few thousand elements on a forced split
// path) take 4 waves or 1, so that a tile is not mostly past the chunk's end.
constexpr int kSplitWaves = 8;
constexpr int kMergeRows = 4;          // rows (wavefronts) per merge workgroup

// Temporal pass-1 loads leave x in the Infinity Cache for the normalise
// pass (non-temporal); on fp32 16 x 4194304 this is 126 us against 142 us
// with non-temporal loads in both passes.  Statistics alone read x once,
// non-temporally.
using SplitPolicy = TwoPass<false, true, true, false>;
using StatsPolicy = TwoPass<true, true, true, false>;

template <class Tr, bool VEC>
constexpr int tile_slots() {
    return VEC ? 32 / Tr::E : 16;
}

struct WsLayout {
    float *part_m, *part_d, *row_m, *row_d;
};

WsLayout layout(void *ws, int64_t M, int P) {
    char *p = static_cast<char *>(ws);
    const size_t part = align256(sizeof(float) * static_cast<size_t>(M) * P);
    const size_t rows = align256(sizeof(float) * static_cast<size_t>(M));
    WsLayout l;
    l.part_m = reinterpret_cast<float *>(p);
    l.part_d = reinterpret_cast<float *>(p + part);
    l.row_m = reinterpret_cast<float *>(p + 2 * part);
    l.row_d = reinterpret_cast<float *>(p + 2 * part + rows);
    return l;
}

template <class Tr, bool VEC, class Pol, bool MK, int WAVES>
void run(const FwdArgs &a, void *ws, const SplitPlan &plan) {
    using E = typename Tr::elem_t;
    constexpr int U = tile_slots<Tr, VEC>();
    const WsLayout l = layout(ws, a.M, plan.P);
    const dim3 grid(static_cast<unsigned>(a.M * plan.P));
    const dim3 block(kWave * WAVES);
    const E *x = static_cast<const E *>(a.x);

    const Mask mk{a.row_len, a.causal};
    // log-softmax keeps r = d - 1; softmax, statistics and cross-entropy d
    if (a.mode != Mode::LogProb) {
        split_partial_kernel<Tr, VEC, WAVES, U, Pol, MK, false>
            <<<grid, block, 0, a.stream>>>(x, a.ldx, a.N, plan.P, plan.C,
                                           l.part_m, l.part_d, mk);
    } else {
        split_partial_kernel<Tr, VEC, WAVES, U, Pol, MK, true>
            <<<grid, block, 0, a.stream>>>(x, a.ldx, a.N, plan.P, plan.C,
                                           l.part_m, l.part_d, mk);
    }

    const StatsOut so{a.m_out, a.d_out, a.lse_out, a.inc_out, a.labels, a.loss,
                      a.accumulate};
    if (a.mode == Mode::Stats) {
        // statistics alone: the row states go to whichever of the caller's
        // m / d / lse / cross-entropy are asked for, in one merge launch
        const dim3 mgrid(static_cast<unsigned>((a.M + kMergeRows - 1) / kMergeRows));
        const dim3 mblock(kWave * kMergeRows);
        if (a.labels) {
            state_merge_kernel<kMergeRows, Tr, true><<<mgrid, mblock, 0, a.stream>>>(
                l.part_m, l.part_d, plan.P, a.M, plan.P, l.row_m, l.row_d, 1, so,
                x, a.ldx, a.N);
        } else {
            state_merge_kernel<kMergeRows, Tr, false><<<mgrid, mblock, 0, a.stream>>>(
                l.part_m, l.part_d, plan.P, a.M, plan.P, l.row_m, l.row_d, 1, so,
                x, a.ldx, a.N);
        }
        return;
    }

    // softmax / log-softmax: the normalise kernel merges the partial states
    // itself and writes the requested statistics
    E *y = static_cast<E *>(a.y);
    if (a.mode == Mode::Prob) {
        split_normalize_kernel<Tr, VEC, WAVES, U, Out::Prob, Pol, MK>
            <<<grid, block, 0, a.stream>>>(x, a.ldx, y, a.ldy, a.N, plan.P, plan.C,
                                           l.part_m, l.part_d, so, mk);
    } else {
        split_normalize_kernel<Tr, VEC, WAVES, U, Out::LogProb, Pol, MK>
            <<<grid, block, 0, a.stream>>>(x, a.ldx, y, a.ldy, a.N, plan.P, plan.C,
                                           l.part_m, l.part_d, so, mk);
    }
}

// Waves per chunk workgroup: kSplitWaves, unless the chunk (at most the
// row) is shorter than such a workgroup's tile of 64 lanes x U slots per
// wave.
template <class Tr, bool VEC, class Pol, bool MK>
void by_waves(const FwdArgs &a, void *ws) {
    const SplitPlan plan = split_plan(a.M, a.N, a.cus);
    const int64_t len = plan.C < a.N ? plan.C : a.N;
    const int64_t tile = int64_t(kWave) * tile_slots<Tr, VEC>() * (VEC ? Tr::E : 1);
    if (len >= kSplitWaves * tile) run<Tr, VEC, Pol, MK, kSplitWaves>(a, ws, plan);
    else if (len >= 4 * tile) run<Tr, VEC, Pol, MK, 4>(a, ws, plan);
    else run<Tr, VEC, Pol, MK, 1>(a, ws, plan);
}

template <class Tr, bool VEC>
void by_mode(const FwdArgs &a, void *ws) {
    if (a.mode == Mode::Stats) by_waves<Tr, VEC, StatsPolicy, false>(a, ws);
    else if (a.masked()) by_waves<Tr, VEC, SplitPolicy, true>(a, ws);
    else by_waves<Tr, VEC, SplitPolicy, false>(a, ws);
}

}  // namespace

void launch_split(const FwdArgs &a, void *ws) {
    if (a.dt == Dt::F32) {
        if (a.vec) by_mode<F32, true>(a, ws); else by_mode<F32, false>(a, ws);
    } else {
        if (a.vec) by_mode<BF16, true>(a, ws); else by_mode<BF16, false>(a, ws);
    }
}

namespace {

template <class Tr, bool VEC, int WAVES, int U>
void state_normalize(const FwdArgs &a, const SplitPlan &plan, const float *sm,
                     const float *sd, int64_t inc) {
    using E = typename Tr::elem_t;
    const dim3 grid(static_cast<unsigned>(a.M * plan.P));
    const dim3 block(kWave * WAVES);
    const E *x = static_cast<const E *>(a.x);
    E *y = static_cast<E *>(a.y);
    if (a.mode == Mode::Prob) {
        state_normalize_kernel<Tr, VEC, WAVES, U, Out::Prob>
            <<<grid, block, 0, a.stream>>>(x, a.ldx, y, a.ldy, a.N, plan.P,
                                           plan.C, sm, sd, inc);
    } else {
        state_normalize_kernel<Tr, VEC, WAVES, U, Out::LogProb>
            <<<grid, block, 0, a.stream>>>(x, a.ldx, y, a.ldy, a.N, plan.P,
                                           plan.C, sm, sd, inc);
    }
}

// Chunks for pass 2 alone (normalize_plan): rows are cut at multiples of
// kChunkAlign elements until there are about 64 workgroups per CU.  With no
// pass 1 to share a chunk with, more and shorter chunks keep more loads in
// flight: on fp32 16 x 4194304 83.7 us against 92.0 us with the split
// path's 8 per CU, on fp32 1024 x 32768 43.0 us against 46.2 us (MI355X).

// Workgroup shape by the bytes one workgroup covers (a row, or a chunk of
// one): with 16-byte slots the tile is the whole row up to 32 KiB, as on
// the resident path (one wavefront up to 4 KiB, then 4 or 8), and longer
// rows loop over tiles of 8 slots per lane.
template <class Tr, bool VEC>
void run_state_normalize(const FwdArgs &a, const float *sm, const float *sd,
                         int64_t inc) {
    const SplitPlan plan = normalize_plan(a.M, a.N, a.cus);
    const int64_t len = plan.C < a.N ? plan.C : a.N;
    const int64_t bytes = len * static_cast<int64_t>(sizeof(typename Tr::elem_t));
    if (bytes <= 1024) state_normalize<Tr, VEC, 1, 1>(a, plan, sm, sd, inc);
    else if (bytes <= 2048) state_normalize<Tr, VEC, 1, 2>(a, plan, sm, sd, inc);
    else if (bytes <= 4096) state_normalize<Tr, VEC, 1, 4>(a, plan, sm, sd, inc);
    else if (bytes <= 8192) state_normalize<Tr, VEC, 4, 2>(a, plan, sm, sd, inc);
    else if (bytes <= 16384) state_normalize<Tr, VEC, 8, 2>(a, plan, sm, sd, inc);
    else if (bytes <= 32768) state_normalize<Tr, VEC, 8, 4>(a, plan, sm, sd, inc);
    else state_normalize<Tr, VEC, 8, 8>(a, plan, sm, sd, inc);
}

}  // namespace

void launch_state_normalize(const FwdArgs &a, const float *sm, const float *sd,
                            int64_t inc) {
    if (a.dt == Dt::F32) {
        if (a.vec) run_state_normalize<F32, true>(a, sm, sd, inc);
        else run_state_normalize<F32, false>(a, sm, sd, inc);
    } else {
        if (a.vec) run_state_normalize<BF16, true>(a, sm, sd, inc);
        else run_state_normalize<BF16, false>(a, sm, sd, inc);
    }
}

void launch_state_merge(const float *m_in, const float *d_in, int64_t ld,
                        int64_t M, int K, float *m_out, float *d_out,
                        float *lse_out, int64_t inc, hipStream_t stream) {
    const StatsOut so{nullptr, nullptr, lse_out, inc, nullptr, nullptr, false};
    state_merge_kernel<kMergeRows, F32, false>
        <<<dim3(static_cast<unsigned>((M + kMergeRows - 1) / kMergeRows)),
           dim3(kWave * kMergeRows), 0, stream>>>(m_in, d_in, ld, M, K, m_out,
                                                  d_out, inc, so, nullptr, 0, 0);
}

void launch_ce_mean(const float *loss, int64_t M, float *mean,
                    hipStream_t stream) {
    ce_mean_kernel<1024><<<dim3(1), dim3(1024), 0, stream>>>(loss, M, mean);
}

}  // namespace os
