// Streaming-read probe for gfx950: the HBM read rate a plain kernel reaches
// on this device, the ceiling the memory-bound decode kernels are compared
// with.  Every thread reads 16-byte pieces with U loads in flight and folds
// them into one word that is stored (to one 4-byte sink) only if it equals
// a constant the probe's inputs never fold to, so the loads stay live and
// nothing is written.
//
// Two layouts: contiguous (workgroup w streams its own range of the buffer,
// the shape of the decode kernel's shares) and grid-stride (all workgroups
// sweep the buffer together, piece i of round r at r * grid * threads + i).
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr unsigned kNever = 0x9E3779B9u;

template <int U, bool GRID>
__global__ __launch_bounds__(1024) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                           int64_t per_wg, unsigned* __restrict__ sink) {
    const int64_t nthreads = blockDim.x;
    int64_t lo, hi, step;
    if (GRID) {
        lo = (int64_t)blockIdx.x * nthreads + threadIdx.x;
        hi = n16;
        step = (int64_t)gridDim.x * nthreads;
    } else {
        lo = (int64_t)blockIdx.x * per_wg + threadIdx.x;
        hi = min<int64_t>((int64_t)(blockIdx.x + 1) * per_wg, n16);
        step = nthreads;
    }
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t i = lo; i < hi; i += step * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = i + u * step;
            v[u] = j < hi ? src[j] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    const unsigned x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (x == kNever) sink[0] = x;
}

template <bool GRID>
const void* probe_of(int unroll) {
    return unroll == 1 ? reinterpret_cast<const void*>(&stream_read_kernel<1, GRID>)
         : unroll == 2 ? reinterpret_cast<const void*>(&stream_read_kernel<2, GRID>)
         : unroll == 4 ? reinterpret_cast<const void*>(&stream_read_kernel<4, GRID>)
         : unroll == 8 ? reinterpret_cast<const void*>(&stream_read_kernel<8, GRID>)
                       : reinterpret_cast<const void*>(&stream_read_kernel<16, GRID>);
}

}  // namespace
}  // namespace pa

extern "C" int paged_attn_probe_stream_read(const void* src, int64_t bytes, int32_t workgroups, int32_t threads,
                                            int32_t unroll, int32_t grid_stride, void* sink, void* stream) {
    using namespace pa;
    if (!src || !sink) return fail(PA_ERR_NULL, "probe: NULL buffer");
    if (bytes < 16 || bytes % 16 || (uintptr_t)src % 16)
        return fail(PA_ERR_ARG, "probe: the buffer must be 16-byte aligned, a positive multiple of 16 bytes");
    if (workgroups < 1 || workgroups > (1 << 20) || threads < 64 || threads > 1024 || threads % 64)
        return fail(PA_ERR_ARG, "probe: workgroups in [1, 2^20], threads a multiple of 64 in [64, 1024]");
    if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8 && unroll != 16)
        return fail(PA_ERR_ARG, "probe: unroll must be 1, 2, 4, 8 or 16");
    const int64_t n16 = bytes / 16;
    int64_t per_wg = (n16 + workgroups - 1) / workgroups;
    const u32x4* s = static_cast<const u32x4*>(src);
    unsigned* k = static_cast<unsigned*>(sink);
    const void* fn = grid_stride ? probe_of<true>(unroll) : probe_of<false>(unroll);
    void* args[] = {&s, const_cast<int64_t*>(&n16), &per_wg, &k};
    if (hipLaunchKernel(fn, dim3((unsigned)workgroups), dim3((unsigned)threads), args, 0,
                        static_cast<hipStream_t>(stream)) != hipSuccess)
        return fail(PA_ERR_HIP, "probe launch failed: %s", hipGetErrorString(hipGetLastError()));
    return PA_OK;
}
