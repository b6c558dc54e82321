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
// A gather variant reads whole cache blocks named by a list, the paged
// pattern itself.
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

// Gather probe: the whole cache blocks named by a list (every kv head of
// each, as a decode call that covers all heads reads them), from up to four
// arrays with their own block strides (K, V and, for an fp8 cache, the two
// scale arrays), `piece` = 16 bytes.  Workgroup w reads blocks [w*n/G,
// (w+1)*n/G) of the list; their ids go through LDS first (kGatherIds at a
// time) so that no load waits for an index load.
constexpr int kGatherIds = 1024;
struct GatherArgs {
    const char* base[4];
    int64_t stride[4];      // bytes between consecutive blocks of the array
    int32_t pieces[4];      // 16-byte pieces of one block read from the array (0: unused)
    const int32_t* ids;     // block ids (clamped into [0, nb))
    int32_t n, nb;
    unsigned* sink;
};

template <int U>
__global__ __launch_bounds__(1024) void gather_read_kernel(GatherArgs a) {
    __shared__ int s_id[kGatherIds];
    const int T = blockDim.x;
    const int b0 = (int)((int64_t)blockIdx.x * a.n / gridDim.x), b1 = (int)((int64_t)(blockIdx.x + 1) * a.n / gridDim.x);
    const int per = a.pieces[0] + a.pieces[1] + a.pieces[2] + a.pieces[3];
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int c0 = b0; c0 < b1; c0 += kGatherIds) {
        const int cn = min(kGatherIds, b1 - c0);
        __syncthreads();
        for (int i = threadIdx.x; i < cn; i += T) s_id[i] = min(max(a.ids[c0 + i], 0), a.nb - 1);
        __syncthreads();
        const int total = cn * per;
        for (int p = threadIdx.x; p < total; p += T * U) {
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int q = p + u * T;
                v[u] = u32x4{0u, 0u, 0u, 0u};
                if (q < total) {
                    const int blk = q / per;
                    int r = q - blk * per, j = 0;
                    if (r >= a.pieces[0]) {
                        r -= a.pieces[0]; j = 1;
                        if (r >= a.pieces[1]) { r -= a.pieces[1]; j = 2; if (r >= a.pieces[2]) { r -= a.pieces[2]; j = 3; } }
                    }
                    v[u] = *reinterpret_cast<const u32x4*>(a.base[j] + (int64_t)s_id[blk] * a.stride[j] + 16 * r);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) acc ^= v[u];
        }
    }
    const unsigned x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (x == kNever) a.sink[0] = x;
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

extern "C" int paged_attn_probe_gather_read(const void* const* arrays, const int64_t* block_strides,
                                            const int32_t* block_bytes, const int32_t* block_ids, int32_t n,
                                            int32_t num_blocks, int32_t workgroups, int32_t threads, int32_t unroll,
                                            void* sink, void* stream) {
    using namespace pa;
    if (!arrays || !block_strides || !block_bytes || !block_ids || !sink) return fail(PA_ERR_NULL, "probe: NULL argument");
    if (n < 1 || num_blocks < 1 || workgroups < 1 || workgroups > (1 << 20) || threads < 64 || threads > 1024 ||
        threads % 64 || (unroll != 4 && unroll != 8 && unroll != 16))
        return fail(PA_ERR_ARG, "probe: invalid sizes");
    GatherArgs a;
    int64_t per = 0;
    for (int j = 0; j < 4; ++j) {
        a.base[j] = static_cast<const char*>(arrays[j]);
        a.stride[j] = block_strides[j];
        if (block_bytes[j] < 0 || block_bytes[j] % 16 || (block_bytes[j] > 0 && (!arrays[j] || (uintptr_t)arrays[j] % 16 ||
                                                                                  block_strides[j] < block_bytes[j] ||
                                                                                  block_strides[j] % 16)))
            return fail(PA_ERR_ARG, "probe: array %d: block bytes a multiple of 16 within the stride, 16-byte aligned", j);
        a.pieces[j] = block_bytes[j] / 16;
        per += a.pieces[j];
    }
    if (per < 1 || per * (int64_t)kGatherIds >= (int64_t(1) << 31)) return fail(PA_ERR_ARG, "probe: block size");
    a.ids = block_ids;
    a.n = n;
    a.nb = num_blocks;
    a.sink = static_cast<unsigned*>(sink);
    void* args[] = {&a};
    const void* fn = unroll == 4 ? reinterpret_cast<const void*>(&gather_read_kernel<4>)
                   : unroll == 8 ? reinterpret_cast<const void*>(&gather_read_kernel<8>)
                                 : reinterpret_cast<const void*>(&gather_read_kernel<16>);
    if (hipLaunchKernel(fn, dim3((unsigned)workgroups), dim3((unsigned)threads), args, 0,
                        static_cast<hipStream_t>(stream)) != hipSuccess)
        return fail(PA_ERR_HIP, "probe launch failed: %s", hipGetErrorString(hipGetLastError()));
    return PA_OK;
}
