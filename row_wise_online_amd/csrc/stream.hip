// Launchers of the streaming path (one workgroup per row): two reads of x
// for softmax / log-softmax, one read for statistics and cross-entropy.
#include "kernels.hpp"
#include "launch.hpp"

namespace os {
namespace {

// Waves per workgroup: 4 for the two-read passes; 8 for the one-read
// statistics and cross-entropy pass, which keeps twice the loads in flight
// per row (fp32 1024 x 32768 statistics 22.1 us against 23.1 us with 4).
constexpr int kStreamWaves = 4;
constexpr int kStatsWaves = 8;

// Pass 1 loads are temporal so that the row stays in the Infinity Cache;
// pass 2 walks the row last tile first (the most recently read lines
// first) with non-temporal loads and stores.  Measured on fp32 1024 x 32768:
// 52 us against 68 us with non-temporal pass-1 loads.  A statistics-only
// pass has no second read and loads non-temporally.
using StreamPolicy = TwoPass<false, true, true, true>;
using StatsPolicy = TwoPass<true, true, true, false>;

// Slots per lane per tile: 32 values per lane for vectors, 16 elements per
// lane for element access.
template <class Tr, bool VEC>
constexpr int tile_slots() {
    return VEC ? 32 / Tr::E : 16;
}

template <class Tr, bool VEC, Out OUT, class Pol, bool CE, bool MK, int WAVES>
void launch_waves(const FwdArgs &a) {
    using E = typename Tr::elem_t;
    constexpr int U = tile_slots<Tr, VEC>();
    const StatsOut so{a.m_out, a.d_out, a.lse_out, a.inc_out, a.labels, a.loss,
                      a.accumulate};
    stream_kernel<Tr, VEC, WAVES, U, OUT, Pol, CE, MK>
        <<<dim3(static_cast<unsigned>(a.M)), dim3(kWave * WAVES), 0, a.stream>>>(
            static_cast<const E *>(a.x), a.ldx, static_cast<E *>(a.y), a.ldy,
            a.N, so, Mask{a.row_len, a.causal});
}

// Rows shorter than one tile of the full workgroup (only on a stream path
// forced onto short rows; AUTO streams rows of more than 16384 elements)
// take a single wavefront, so that a tile is not mostly past the row's end.
template <class Tr, bool VEC, Out OUT, class Pol, bool CE = false,
          bool MK = false>
void run(const FwdArgs &a) {
    constexpr int WAVES = OUT == Out::None ? kStatsWaves : kStreamWaves;
    constexpr int64_t kTile = int64_t(kWave) * WAVES * tile_slots<Tr, VEC>() * (VEC ? Tr::E : 1);
    if (a.N >= kTile) launch_waves<Tr, VEC, OUT, Pol, CE, MK, WAVES>(a);
    else launch_waves<Tr, VEC, OUT, Pol, CE, MK, 1>(a);
}

template <class Tr, bool VEC>
void by_mode(const FwdArgs &a) {
    const bool mk = a.masked();
    switch (a.mode) {
        case Mode::Prob:
            if (mk) run<Tr, VEC, Out::Prob, StreamPolicy, false, true>(a);
            else run<Tr, VEC, Out::Prob, StreamPolicy>(a);
            break;
        case Mode::LogProb:
            if (mk) run<Tr, VEC, Out::LogProb, StreamPolicy, false, true>(a);
            else run<Tr, VEC, Out::LogProb, StreamPolicy>(a);
            break;
        default:
            if (a.labels) run<Tr, VEC, Out::None, StatsPolicy, true>(a);
            else run<Tr, VEC, Out::None, StatsPolicy>(a);
            break;
    }
}

}  // namespace

void launch_stream(const FwdArgs &a) {
    if (a.dt == Dt::F32) {
        if (a.vec) by_mode<F32, true>(a); else by_mode<F32, false>(a);
    } else {
        if (a.vec) by_mode<BF16, true>(a); else by_mode<BF16, false>(a);
    }
}

}  // namespace os
