// Launchers of the resident single-read path.
#include "kernels.hpp"
#include "launch.hpp"

namespace os {
namespace {

template <class Tr, bool VEC, int WAVES, int ROWS, int EPL>
void run(const FwdArgs &a) {
    constexpr int W = VEC ? Tr::E : 1;
    static_assert(EPL % W == 0, "a lane holds whole slots");
    constexpr int SPL = EPL / W;
    const dim3 grid(static_cast<unsigned>((a.M + ROWS - 1) / ROWS));
    const dim3 block(kWave * WAVES * ROWS);
    using E = typename Tr::elem_t;
    resident_kernel<Tr, VEC, WAVES, ROWS, SPL><<<grid, block, 0, a.stream>>>(
        static_cast<const E *>(a.x), a.ldx, static_cast<E *>(a.y), a.ldy, a.M,
        a.N, a.m_out, a.d_out, a.lse_out);
}

// Variant ladder by row length: elements per lane (EPL) and wavefronts per
// row are chosen so that a row fits in registers with at most 32 values per
// lane; short rows get one wavefront each, four rows per workgroup.
template <class Tr, bool VEC>
void dispatch(const FwdArgs &a) {
    const int N = a.N;
    constexpr bool kSmallOk = !VEC || Tr::E <= 4;  // EPL 4 holds whole slots
    if (kSmallOk && N <= 256) {
        if constexpr (kSmallOk) run<Tr, VEC, 1, 4, 4>(a);
    } else if (N <= 512) {
        run<Tr, VEC, 1, 4, 8>(a);
    } else if (N <= 1024) {
        run<Tr, VEC, 1, 4, 16>(a);
    } else if (N <= 2048) {
        run<Tr, VEC, 4, 1, 8>(a);
    } else if (N <= 4096) {
        run<Tr, VEC, 4, 1, 16>(a);
    } else if (N <= 8192) {
        run<Tr, VEC, 8, 1, 16>(a);
    } else if (N <= 16384) {
        run<Tr, VEC, 16, 1, 16>(a);
    } else {
        run<Tr, VEC, 16, 1, 32>(a);
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
