// Launchers of the resident single-read path.
#include "kernels.hpp"
#include "launch.hpp"

namespace os {
namespace {

template <class Tr, bool VEC, int WAVES, int EPL>
void run(const FwdArgs &a) {
    constexpr int W = VEC ? Tr::E : 1;
    static_assert(EPL % W == 0, "a lane holds whole slots");
    constexpr int SPL = EPL / W;
    const dim3 grid(static_cast<unsigned>(a.M));
    const dim3 block(kWave * WAVES);
    using E = typename Tr::elem_t;
    resident_kernel<Tr, VEC, WAVES, 1, SPL, true><<<grid, block, 0, a.stream>>>(
        static_cast<const E *>(a.x), a.ldx, static_cast<E *>(a.y), a.ldy, a.M,
        a.N, a.m_out, a.d_out, a.lse_out);
}

// Variant ladder by row length (elements): one workgroup per row, sized so
// that each lane holds at most 64 values; rows of up to 1024 elements get a
// single wavefront (64-thread workgroups, no barrier).  Measured on MI355X:
// one-wave workgroups beat four independent rows per 256-thread workgroup,
// and 8 waves x 64 values beat 16 waves x 32 values for 32K-wide rows.
template <class Tr, bool VEC>
void dispatch(const FwdArgs &a) {
    const int N = a.N;
    constexpr bool kSmallOk = !VEC || Tr::E <= 4;  // EPL 4 holds whole slots
    if (kSmallOk && N <= 256) {
        if constexpr (kSmallOk) run<Tr, VEC, 1, 4>(a);
    } else if (N <= 512) {
        run<Tr, VEC, 1, 8>(a);
    } else if (N <= 1024) {
        run<Tr, VEC, 1, 16>(a);
    } else if (N <= 2048) {
        run<Tr, VEC, 2, 16>(a);
    } else if (N <= 4096) {
        run<Tr, VEC, 4, 16>(a);
    } else if (N <= 8192) {
        run<Tr, VEC, 8, 16>(a);
    } else if (N <= 16384) {
        run<Tr, VEC, 8, 32>(a);
    } else {
        run<Tr, VEC, 8, 64>(a);
    }
}

}  // namespace

void launch_resident(const FwdArgs &a) {
    if (a.dt == Dt::F32) {
        if (a.vec) dispatch<F32, true>(a); else dispatch<F32, false>(a);
    } else {
        if (a.vec) dispatch<BF16, true>(a); else dispatch<BF16, false>(a);
    }
}

}  // namespace os
