// Bandwidth and launch ceilings for the benchmark (not part of the softmax
// library or its ABI).  Each kernel moves the same bytes as a softmax launch
// in the same launch shape -- one workgroup of 64 * WAVES lanes per row,
// each lane SPL 16-byte vectors spaced 64 * WAVES vectors apart, loads and
// stores non-temporal -- but does no arithmetic:
//   ceil_copy   reads a row and writes it back elsewhere (the softmax's
//               traffic without its reduction: the bound a one-read,
//               one-write pass of this shape can reach on this device);
//   ceil_read   reads only (a store that depends on every load, and almost
//               never happens, keeps the loads);
//   ceil_write  writes only;
//   ceil_empty  a kernel that touches no memory, launched back to back, for
//               the fixed cost of one launch on a stream;
//   ceil_memcpy hipMemcpyAsync device to device, the runtime's own copy.
// Rows must be exactly 64 * WAVES * SPL vectors long and every base and
// pitch 16-byte aligned; the host checks both, so every access is in bounds.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int WAVES, int SPL>
__global__ __launch_bounds__(64 * WAVES) void copy_rows(const u32x4 *src,
                                                        u32x4 *dst,
                                                        int64_t pitch) {
    const u32x4 *s = src + static_cast<int64_t>(blockIdx.x) * pitch + threadIdx.x;
    u32x4 *d = dst + static_cast<int64_t>(blockIdx.x) * pitch + threadIdx.x;
    u32x4 v[SPL];
#pragma unroll
    for (int k = 0; k < SPL; ++k) v[k] = __builtin_nontemporal_load(s + k * 64 * WAVES);
#pragma unroll
    for (int k = 0; k < SPL; ++k) __builtin_nontemporal_store(v[k], d + k * 64 * WAVES);
}

template <int WAVES, int SPL>
__global__ __launch_bounds__(64 * WAVES) void read_rows(const u32x4 *src,
                                                        float *sink,
                                                        int64_t pitch) {
    const u32x4 *s = src + static_cast<int64_t>(blockIdx.x) * pitch + threadIdx.x;
    u32x4 v[SPL];
#pragma unroll
    for (int k = 0; k < SPL; ++k) v[k] = __builtin_nontemporal_load(s + k * 64 * WAVES);
    uint32_t acc = 0;
#pragma unroll
    for (int k = 0; k < SPL; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    // a store that depends on every load keeps them; it almost never
    // happens, so the kernel writes (next to) nothing
    if (acc == 0x9e3779b9u) sink[blockIdx.x] = 1.0f;
}

template <int WAVES, int SPL>
__global__ __launch_bounds__(64 * WAVES) void write_rows(u32x4 *dst,
                                                         int64_t pitch) {
    u32x4 *d = dst + static_cast<int64_t>(blockIdx.x) * pitch + threadIdx.x;
    const u32x4 v = {blockIdx.x, threadIdx.x, 0u, 0x3f800000u};
#pragma unroll
    for (int k = 0; k < SPL; ++k) __builtin_nontemporal_store(v, d + k * 64 * WAVES);
}

__global__ void empty_kernel() {}

enum Op { kCopy, kRead, kWrite };

template <int WAVES, int SPL>
void launch(Op op, const void *src, void *dst, int64_t rows, int64_t pitch,
            hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(rows)), block(64 * WAVES);
    if (op == kCopy)
        copy_rows<WAVES, SPL><<<grid, block, 0, s>>>(
            static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), pitch);
    else if (op == kRead)
        read_rows<WAVES, SPL><<<grid, block, 0, s>>>(
            static_cast<const u32x4 *>(src), static_cast<float *>(dst), pitch);
    else
        write_rows<WAVES, SPL><<<grid, block, 0, s>>>(static_cast<u32x4 *>(dst),
                                                      pitch);
}

template <int WAVES>
bool by_spl(Op op, int spl, const void *src, void *dst, int64_t rows,
            int64_t pitch, hipStream_t s) {
    switch (spl) {
        case 1: launch<WAVES, 1>(op, src, dst, rows, pitch, s); return true;
        case 2: launch<WAVES, 2>(op, src, dst, rows, pitch, s); return true;
        case 4: launch<WAVES, 4>(op, src, dst, rows, pitch, s); return true;
        case 8: launch<WAVES, 8>(op, src, dst, rows, pitch, s); return true;
        case 16: launch<WAVES, 16>(op, src, dst, rows, pitch, s); return true;
    }
    return false;
}

bool aligned16(const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// 0: enqueued; 1: a shape or alignment the kernels do not take (nothing is
// enqueued); 2: the launch failed.
int run(Op op, const void *src, void *dst, int64_t rows, int64_t row_bytes,
        int64_t pitch_bytes, int waves, int spl, hipStream_t s) {
    if (rows < 1 || rows > (int64_t(1) << 22)) return 1;
    if (row_bytes != int64_t(16) * 64 * waves * spl) return 1;
    if (pitch_bytes < row_bytes || pitch_bytes % 16 != 0) return 1;
    if ((op != kWrite && !aligned16(src)) || !aligned16(dst)) return 1;
    const int64_t pitch = pitch_bytes / 16;
    bool ok;
    switch (waves) {
        case 1: ok = by_spl<1>(op, spl, src, dst, rows, pitch, s); break;
        case 2: ok = by_spl<2>(op, spl, src, dst, rows, pitch, s); break;
        case 4: ok = by_spl<4>(op, spl, src, dst, rows, pitch, s); break;
        case 8: ok = by_spl<8>(op, spl, src, dst, rows, pitch, s); break;
        default: ok = false;
    }
    if (!ok) return 1;
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // namespace

extern "C" {

// src and dst: rows x pitch_bytes, row_bytes = 16 * 64 * waves * spl of
// each row moved; waves in {1, 2, 4, 8}, spl in {1, 2, 4, 8, 16}.
int ceil_copy(const void *src, void *dst, int64_t rows, int64_t row_bytes,
              int64_t pitch_bytes, int waves, int spl, hipStream_t s) {
    return run(kCopy, src, dst, rows, row_bytes, pitch_bytes, waves, spl, s);
}

// sink: rows floats.
int ceil_read(const void *src, float *sink, int64_t rows, int64_t row_bytes,
              int64_t pitch_bytes, int waves, int spl, hipStream_t s) {
    if (sink == nullptr) return 1;
    return run(kRead, src, sink, rows, row_bytes, pitch_bytes, waves, spl, s);
}

int ceil_write(void *dst, int64_t rows, int64_t row_bytes, int64_t pitch_bytes,
               int waves, int spl, hipStream_t s) {
    return run(kWrite, nullptr, dst, rows, row_bytes, pitch_bytes, waves, spl, s);
}

// An empty kernel of `grid` workgroups of `threads` lanes.
int ceil_empty(int64_t grid, int threads, hipStream_t s) {
    if (grid < 1 || grid > (int64_t(1) << 22) || threads < 1 || threads > 1024)
        return 1;
    empty_kernel<<<dim3(static_cast<unsigned>(grid)), dim3(threads), 0, s>>>();
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int ceil_memcpy(void *dst, const void *src, size_t bytes, hipStream_t s) {
    if (dst == nullptr || src == nullptr) return 1;
    return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s) == hipSuccess
               ? 0
               : 2;
}

}  // extern "C"
