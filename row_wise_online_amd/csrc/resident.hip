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

// Persistent form for the longest rows: a grid of at most kPersistentWgs
// workgroups (two 512-thread workgroups per CU on 256 CUs) walks the rows,
// prefetching each wavefront's next row while it normalises the current one.
constexpr int64_t kPersistentWgs = 512;

template <class Tr, bool VEC, int WAVES, int EPL>
void run_persistent(const FwdArgs &a) {
    constexpr int W = VEC ? Tr::E : 1;
    static_assert(EPL % W == 0, "a lane holds whole slots");
    constexpr int SPL = EPL / W;
    const int64_t g = a.M < kPersistentWgs ? a.M : kPersistentWgs;
    using E = typename Tr::elem_t;
    resident_persistent_kernel<Tr, VEC, WAVES, 1, SPL, true>
        <<<dim3(static_cast<unsigned>(g)), dim3(kWave * WAVES), 0, a.stream>>>(
            static_cast<const E *>(a.x), a.ldx, static_cast<E *>(a.y), a.ldy,
            a.M, a.N, a.m_out, a.d_out, a.lse_out);
}

// Variant ladder by row length (elements), measured on MI355X (interleaved
// medians on cold buffers): one 64-thread workgroup per row up to 1024
// columns (bf16 32768 x 1024: 5.87 TB/s); 8 waves x 8 values per lane for
// 4096 columns (fp32: 5.88 TB/s, ahead of 4 x 16 and 2 x 32); 8 waves x 64
// values per lane, persistent, for 32768 columns (fp32: 6.06 TB/s).
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
        run<Tr, VEC, 4, 8>(a);
    } else if (N <= 4096) {
        run<Tr, VEC, 8, 8>(a);
    } else if (N <= 8192) {
        run<Tr, VEC, 8, 16>(a);
    } else if (N <= 16384) {
        run<Tr, VEC, 8, 32>(a);
    } else {
        run_persistent<Tr, VEC, 8, 64>(a);
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
