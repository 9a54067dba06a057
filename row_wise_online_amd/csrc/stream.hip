// Launchers of the streaming path (one workgroup per row) and of the
// statistics-only kernel.
#include "kernels.hpp"
#include "launch.hpp"

namespace os {
namespace {

constexpr int kStreamWaves = 4;

// Pass 1 loads are temporal so that the row stays in the Infinity Cache;
// pass 2 walks the row last tile first (the most recently read lines
// first) with non-temporal loads and stores.  Measured on fp32 1024 x 32768:
// 52 us against 68 us with non-temporal pass-1 loads.
using StreamPolicy = TwoPass<false, true, true, true>;

// Slots per lane per tile: 32 values per lane for vectors, 16 elements per
// lane for element access.
template <class Tr, bool VEC>
constexpr int tile_slots() {
    return VEC ? 32 / Tr::E : 16;
}

template <class Tr, bool VEC>
void run(const FwdArgs &a) {
    using E = typename Tr::elem_t;
    constexpr int U = tile_slots<Tr, VEC>();
    const dim3 grid(static_cast<unsigned>(a.M));
    const dim3 block(kWave * kStreamWaves);
    const E *x = static_cast<const E *>(a.x);
    if (a.y) {
        stream_kernel<Tr, VEC, kStreamWaves, U, true, StreamPolicy><<<grid, block, 0, a.stream>>>(
            x, a.ldx, static_cast<E *>(a.y), a.ldy, a.M, a.N, a.m_out, a.d_out,
            a.inc_out, a.lse_out);
    } else {
        stream_kernel<Tr, VEC, kStreamWaves, U, false, StreamPolicy><<<grid, block, 0, a.stream>>>(
            x, a.ldx, nullptr, 0, a.M, a.N, a.m_out, a.d_out, a.inc_out,
            a.lse_out);
    }
}

}  // namespace

void launch_stream(const FwdArgs &a) {
    if (a.dt == Dt::F32) {
        if (a.vec) run<F32, true>(a); else run<F32, false>(a);
    } else {
        if (a.vec) run<BF16, true>(a); else run<BF16, false>(a);
    }
}

}  // namespace os
