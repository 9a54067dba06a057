// Launchers of the resident single-read path (and of the register-resident
// statistics pass, which is the same kernel without pass 2).
#include "kernels.hpp"
#include "launch.hpp"

namespace os {
namespace {

// Persistent form for the longest rows: a grid of at most two 512-thread
// workgroups per CU (persistent_grid) walks the rows, prefetching each
// workgroup's next row while it finishes the current one.

StatsOut stats_of(const FwdArgs &a) {
    return StatsOut{a.m_out, a.d_out, a.lse_out, a.inc_out, a.labels, a.loss,
                    a.accumulate};
}

template <class Tr, bool VEC, int WAVES, int EPL, Out OUT, bool CE, bool MK>
void run(const FwdArgs &a) {
    constexpr int W = VEC ? Tr::E : 1;
    static_assert(EPL % W == 0, "a lane holds whole slots");
    constexpr int SPL = EPL / W;
    using E = typename Tr::elem_t;
    resident_kernel<Tr, VEC, WAVES, SPL, true, OUT, CE, MK>
        <<<dim3(static_cast<unsigned>(a.M)), dim3(kWave * WAVES), 0, a.stream>>>(
            static_cast<const E *>(a.x), a.ldx, static_cast<E *>(a.y), a.ldy,
            a.N, stats_of(a), Mask{a.row_len, a.causal});
}

template <class Tr, bool VEC, int WAVES, int EPL, Out OUT, bool CE, bool MK>
void run_persistent(const FwdArgs &a) {
    constexpr int W = VEC ? Tr::E : 1;
    static_assert(EPL % W == 0, "a lane holds whole slots");
    constexpr int SPL = EPL / W;
    const int64_t g = persistent_grid(a.M, a.cus);
    using E = typename Tr::elem_t;
    resident_persistent_kernel<Tr, VEC, WAVES, SPL, true, OUT, CE, MK>
        <<<dim3(static_cast<unsigned>(g)), dim3(kWave * WAVES), 0, a.stream>>>(
            static_cast<const E *>(a.x), a.ldx, static_cast<E *>(a.y), a.ldy,
            a.M, a.N, stats_of(a), Mask{a.row_len, a.causal});
}

// Variant ladder by row length (elements), measured on MI355X (interleaved
// medians on cold buffers): one 64-thread workgroup per row up to 1024
// columns (bf16 32768 x 1024: 5.87 TB/s); 8 waves x 8 values per lane for
// 4096 columns (fp32: 5.9 TB/s, ahead of 4 x 16 and 2 x 32), except for
// the read-only passes, which write nothing per element and take 2 x 32
// (fp32 4096 x 4096 statistics 11.8 us against 12.1 us, cross-entropy
// 14.1 against 14.5 us; 4 x 16 11.9 and 14.1-14.2 us); 8 waves x 64
// values per lane, persistent, for 32768 columns (fp32: 6.07 TB/s).  Shapes
// with more waves and fewer values per lane were slower for log-softmax
// too (fp32 4096 columns: 16 x 4 32.5 us, 4 x 16 24.1 us against 23.9 us;
// bf16 1024 columns: 2 x 8 30.5 us against 23.6 us), except the longest
// rows (below).
template <class Tr, bool VEC, Out OUT, bool CE = false, bool MK = false>
void dispatch(const FwdArgs &a) {
    const int N = a.N;
    constexpr bool kSmallOk = !VEC || Tr::E <= 4;  // EPL 4 holds whole slots
    if (kSmallOk && N <= 256) {
        if constexpr (kSmallOk) run<Tr, VEC, 1, 4, OUT, CE, MK>(a);
    } else if (N <= 512) {
        run<Tr, VEC, 1, 8, OUT, CE, MK>(a);
    } else if (N <= 1024) {
        run<Tr, VEC, 1, 16, OUT, CE, MK>(a);
    } else if (N <= 2048) {
        run<Tr, VEC, 4, 8, OUT, CE, MK>(a);
    } else if (N <= 4096) {
        if constexpr (OUT == Out::None) run<Tr, VEC, 2, 32, OUT, CE, MK>(a);
        else run<Tr, VEC, 8, 8, OUT, CE, MK>(a);
    } else if (N <= 8192) {
        run<Tr, VEC, 8, 16, OUT, CE, MK>(a);
    } else if (N <= 16384) {
        run<Tr, VEC, 8, 32, OUT, CE, MK>(a);
    } else if constexpr (OUT == Out::LogProb) {
        // the r-form fold keeps x and more temporaries live: 16 waves of 32
        // values per lane (fp32 1024 x 32768 log-softmax 44.2 us against
        // 46.1 us with 8 waves of 64; softmax is 2 us slower this way)
        run_persistent<Tr, VEC, 16, 32, OUT, CE, MK>(a);
    } else {
        run_persistent<Tr, VEC, 8, 64, OUT, CE, MK>(a);
    }
}

template <class Tr, bool VEC>
void by_mode(const FwdArgs &a) {
    const bool mk = a.masked();
    switch (a.mode) {
        case Mode::Prob:
            if (mk) dispatch<Tr, VEC, Out::Prob, false, true>(a);
            else dispatch<Tr, VEC, Out::Prob>(a);
            break;
        case Mode::LogProb:
            if (mk) dispatch<Tr, VEC, Out::LogProb, false, true>(a);
            else dispatch<Tr, VEC, Out::LogProb>(a);
            break;
        default:
            if (a.labels) dispatch<Tr, VEC, Out::None, true>(a);
            else dispatch<Tr, VEC, Out::None>(a);
            break;
    }
}

}  // namespace

void launch_resident(const FwdArgs &a) {
    if (a.dt == Dt::F32) {
        if (a.vec) by_mode<F32, true>(a); else by_mode<F32, false>(a);
    } else {
        if (a.vec) by_mode<BF16, true>(a); else by_mode<BF16, false>(a);
    }
}

}  // namespace os
