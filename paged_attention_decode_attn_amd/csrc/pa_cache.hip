// Paged KV-cache write for gfx950: the new tokens' K and V rows go to the
// cache slots a slot mapping names, copied as bf16 or quantised per token to
// OCP fp8 e4m3fn with one fp32 scale per (token, kv head).
//
// The operation: ATOM model operations guide, "KV cache operations" (the
// standard write for a bf16 cache and the fp8 write with per-token
// quantisation) and its slot-mapping file ("which KV slot a token is written
// to"); the ROCm blog "Optimizing ATOM and vLLM-ATOM for High-Interactivity
// Inference", "Attention Input Fusion" (fp8 scales calculated as K/V are
// written into the paged cache).  Scale rule: the row's absolute maximum
// divided by 448, the largest finite e4m3fn value (1 for an all-zero row);
// every element is divided by that stored scale (the correctly rounded
// float32 quotient, so a code is the rounding of exactly the quotient that
// dequantisation multiplies back) and the codes round to nearest, ties to
// even.
//
// A thread takes 8 consecutive elements (16 bytes of bf16) of one (token,
// kv head) row of both K and V for a bf16 cache, 16 for fp8, so a wave
// reads and writes whole contiguous token rows (a tuning override gives each
// thread several such pieces, one grid apart, all loads issued before the
// stores).  The threads of a row sit in one aligned lane group of the wave
// and reduce the row's maximum with cross-lane exchanges.
#include <hip/hip_runtime.h>

#include <cmath>

#include "pa_internal.h"

namespace pa {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kFp8Max = 448.0f;
constexpr int kWriteThreads = 256;

struct WriteArgs {
    const char* k_new; const char* v_new; int64_t n_st, n_sh, vn_st, vn_sh;   // bytes
    const int32_t* slots; int64_t slot_s;                                     // elements
    char* kc; char* vc; int64_t k_sblk, k_stok, k_sh, v_sblk, v_stok, v_sh;   // bytes
    float* ks; float* vs; int64_t ks_sblk, ks_sh, vs_sblk, vs_sh;             // floats
    int64_t T, slots_total;
    int32_t Hkv, D;
    uint32_t bs;                                                              // tokens per block
    int32_t bs_shift;                                                         // log2(bs), or -1
    int32_t small;                                                            // every piece index < 2^31
};

__device__ __forceinline__ float bf16_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Quotients x / s whose e4m3fn code equals that of the correctly rounded
// float32 quotient, from r = RN(1 / s): q = RN(x r), the residual
// e = RN(x - s q) (one fused multiply-add) and RN(q + e r) (another) give
// RN(x / s) (Markstein's correction of a quotient by a correctly rounded
// reciprocal; an exact-arithmetic emulation of these three roundings
// matched the correctly rounded quotient for every pair of bf16 mantissas
// of x and of the row maximum, at every ratio of their magnitudes that
// leaves the quotient between 2^-12 and 448).  Below 2^-12 a quotient's
// code is a signed zero whatever its low bits, and RN(x / s) always has
// the sign of x, so the codes take x's sign bit afterwards (the corrected
// quotient of a tiny x can lose its sign when it rounds to zero).  For rows
// with s below 2^-80 the reciprocal or the residual could leave the normal
// range, and a wave holding such a row divides instead.
constexpr float kSmallScale = 0x1p-80f;

template <bool DIVIDE>
__device__ __forceinline__ float quot(float x, float s, float r) {
    if (DIVIDE && s < kSmallScale) return __fdiv_rn(x, s);
    const float q = x * r;
    const float e = __builtin_fmaf(-q, s, x);
    return __builtin_fmaf(e, r, q);
}

// x / s clamped to +-448 for the two bf16 values of one dword
template <bool DIVIDE>
__device__ __forceinline__ float q_lo(unsigned w, float s, float r) {
    return fminf(fmaxf(quot<DIVIDE>(bf16_lo(w), s, r), -kFp8Max), kFp8Max);
}
template <bool DIVIDE>
__device__ __forceinline__ float q_hi(unsigned w, float s, float r) {
    return fminf(fmaxf(quot<DIVIDE>(bf16_hi(w), s, r), -kFp8Max), kFp8Max);
}

// The sign bits of the four bf16 values of dwords a (values 0, 1) and b
// (values 2, 3) at the sign bits of four packed bytes.
__device__ __forceinline__ unsigned signs4(unsigned a, unsigned b) {
    return __builtin_amdgcn_perm(b, a, 0x07050301u) & 0x80808080u;
}

// 8 bf16 values -> 8 e4m3fn bytes of x / s (r = RN(1 / s)): each
// conversion packs two codes into the low or the high half of a dword.
template <bool DIVIDE>
__device__ __forceinline__ u32x2 encode8_with(const u32x4& x, float s, float r) {
    u32x2 out;
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q_lo<DIVIDE>(x[0], s, r), q_hi<DIVIDE>(x[0], s, r), 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q_lo<DIVIDE>(x[1], s, r), q_hi<DIVIDE>(x[1], s, r), w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q_lo<DIVIDE>(x[2], s, r), q_hi<DIVIDE>(x[2], s, r), 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q_lo<DIVIDE>(x[3], s, r), q_hi<DIVIDE>(x[3], s, r), w1, true);
    out[0] = (unsigned)w0 | signs4(x[0], x[1]);
    out[1] = (unsigned)w1 | signs4(x[2], x[3]);
    return out;
}
__device__ __forceinline__ u32x2 encode8(const u32x4& x, float s, float r) {
    if (__any(s < kSmallScale)) return encode8_with<true>(x, s, r);
    return encode8_with<false>(x, s, r);
}

__device__ __forceinline__ float absmax8(const u32x4& x) {
    float m = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) m = fmaxf(m, fmaxf(fabsf(bf16_lo(x[w])), fabsf(bf16_hi(x[w]))));
    return m;
}

// Thread piece `item` of the row grid: token t, kv head h, piece r of the
// row (8 elements for a bf16 cache, 16 for fp8).
struct Piece {
    int64_t t;
    int h, r;
};

template <int RP>
__device__ __forceinline__ Piece piece_of(const WriteArgs& a, int64_t item) {
    if (a.small) {
        // 32-bit division (a few instructions instead of a 64-bit sequence)
        const uint32_t per_token = (uint32_t)a.Hkv * RP;
        const uint32_t t = (uint32_t)item / per_token;
        const int rem = (int)((uint32_t)item - t * per_token);
        return Piece{(int64_t)t, rem / RP, rem % RP};
    }
    const int64_t per_token = (int64_t)a.Hkv * RP;
    const int64_t t = item / per_token;
    const int rem = (int)(item - t * per_token);
    return Piece{t, rem / RP, rem - (rem / RP) * RP};
}

// The stored scale RN(m / 448) of a row maximum m > 0, by the same
// correction with the correctly rounded constant 1 / 448 (checked against
// the correctly rounded quotient for every positive finite bf16 m with
// exact arithmetic); 1 for an all-zero row.
constexpr float kInv448 = 1.0f / kFp8Max;
__device__ __forceinline__ float scale_of(float m) {
    if (!(m > 0.f)) return 1.f;
    const float q = m * kInv448;
    const float e = __builtin_fmaf(-q, kFp8Max, m);
    return __builtin_fmaf(e, kInv448, q);
}

// A 16-byte piece of a new row.  The bf16 write is a plain copy and streams
// its rows with non-temporal loads and stores (1.3 % faster on 65536-token
// writes); the fp8 write, which does arithmetic between them, was 3-7 %
// slower that way and keeps plain ones.
template <bool FP8>
__device__ __forceinline__ u32x4 load_row(const char* p) {
    if constexpr (FP8) return *reinterpret_cast<const u32x4*>(p);
    else return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// A thread takes NV 16-byte vectors (8 bf16 each) of one row of K and of V:
// one for a bf16 cache (a plain copy), two for fp8, so that the row's
// scale work (the maximum's cross-lane reduction, the scale and its
// reciprocal, the slot's addresses) is shared by 16 elements per lane and
// every code store is 16 bytes.  RP = D / (8 NV) lanes hold a row, an
// aligned lane group.  U pieces per thread, item = gid + k * (threads
// launched), k < U: every load of the thread goes out before its first store.
template <bool FP8, int RP, int U>
__global__ __launch_bounds__(kWriteThreads) void cache_write_kernel(WriteArgs a) {
    constexpr int NV = FP8 ? 2 : 1;
    const int64_t gid = (int64_t)blockIdx.x * kWriteThreads + threadIdx.x;
    const int64_t nthreads = (int64_t)gridDim.x * kWriteThreads;
    u32x4 k[U][NV], v[U][NV];
    int64_t slot[U];
    bool live[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        // every lane of a row group takes part in the reductions below, so
        // the group is either wholly in range or wholly out (RP divides 64,
        // and the stride between a thread's pieces is a multiple of 64)
        const Piece pc = piece_of<RP>(a, gid + u * nthreads);
        const bool live_token = pc.t < a.T;
        slot[u] = live_token ? (int64_t)a.slots[pc.t * a.slot_s] : -1;
        live[u] = slot[u] >= 0 && slot[u] < a.slots_total;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            k[u][i] = u32x4{0u, 0u, 0u, 0u};
            v[u][i] = u32x4{0u, 0u, 0u, 0u};
            if (live[u]) {
                k[u][i] = load_row<FP8>(a.k_new + pc.t * a.n_st + pc.h * a.n_sh + 16 * (NV * pc.r + i));
                v[u][i] = load_row<FP8>(a.v_new + pc.t * a.vn_st + pc.h * a.vn_sh + 16 * (NV * pc.r + i));
            }
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const Piece pc = piece_of<RP>(a, gid + u * nthreads);
        const int h = pc.h, r = pc.r;
        // slots are below 2^31, so the block / position split is 32-bit
        const uint32_t us = (uint32_t)max<int64_t>(slot[u], 0);
        const uint32_t ublk = a.bs_shift >= 0 ? us >> a.bs_shift : us / a.bs;
        const int64_t blk = ublk, pos = us - ublk * a.bs;
        if constexpr (!FP8) {
            if (live[u]) {
                __builtin_nontemporal_store(k[u][0], reinterpret_cast<u32x4*>(a.kc + blk * a.k_sblk + pos * a.k_stok +
                                                                              h * a.k_sh + 16 * r));
                __builtin_nontemporal_store(v[u][0], reinterpret_cast<u32x4*>(a.vc + blk * a.v_sblk + pos * a.v_stok +
                                                                              h * a.v_sh + 16 * r));
            }
        } else {
            float mk = fmaxf(absmax8(k[u][0]), absmax8(k[u][1]));
            float mv = fmaxf(absmax8(v[u][0]), absmax8(v[u][1]));
#pragma unroll
            for (int o = 1; o < RP; o <<= 1) {
                mk = fmaxf(mk, __shfl_xor(mk, o));
                mv = fmaxf(mv, __shfl_xor(mv, o));
            }
            // scale = absmax / 448 (stored); every element divided by it
            const float sk = scale_of(mk);
            const float sv = scale_of(mv);
            const float rk = __fdiv_rn(1.f, sk), rv = __fdiv_rn(1.f, sv);
            if (live[u]) {
                const u32x2 k0 = encode8(k[u][0], sk, rk), k1 = encode8(k[u][1], sk, rk);
                const u32x2 v0 = encode8(v[u][0], sv, rv), v1 = encode8(v[u][1], sv, rv);
                *reinterpret_cast<u32x4*>(a.kc + blk * a.k_sblk + pos * a.k_stok + h * a.k_sh + 16 * r) =
                    u32x4{k0[0], k0[1], k1[0], k1[1]};
                *reinterpret_cast<u32x4*>(a.vc + blk * a.v_sblk + pos * a.v_stok + h * a.v_sh + 16 * r) =
                    u32x4{v0[0], v0[1], v1[0], v1[1]};
                if (r == 0) {
                    a.ks[blk * a.ks_sblk + h * a.ks_sh + pos] = sk;
                    a.vs[blk * a.vs_sblk + h * a.vs_sh + pos] = sv;
                }
            }
        }
    }
}

template <bool FP8, int U>
const void* write_kernel_of(int D) {
    // lanes per row: D / 8 for bf16 (8 elements each), D / 16 for fp8 (16)
    constexpr int S = FP8 ? 16 : 8;
    return D == 256 ? reinterpret_cast<const void*>(&cache_write_kernel<FP8, 256 / S, U>)
         : D == 128 ? reinterpret_cast<const void*>(&cache_write_kernel<FP8, 128 / S, U>)
                    : reinterpret_cast<const void*>(&cache_write_kernel<FP8, 64 / S, U>);
}

}  // namespace
}  // namespace pa

extern "C" int paged_attn_reshape_and_cache(const pa_tensor* k_new, const pa_tensor* v_new,
                                            const pa_tensor* slot_mapping, pa_tensor* k_cache,
                                            pa_tensor* v_cache, pa_tensor* k_scale, pa_tensor* v_scale,
                                            void* stream) {
    using namespace pa;
    WriteProblem p;
    int st = validate_write(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, &p);
    if (st) return st;
    if (p.T == 0) return PA_OK;
    WriteArgs a;
    a.k_new = static_cast<const char*>(p.k_new); a.n_st = p.kn_st; a.n_sh = p.kn_sh;
    a.v_new = static_cast<const char*>(p.v_new); a.vn_st = p.vn_st; a.vn_sh = p.vn_sh;
    a.slots = p.slots; a.slot_s = p.slot_s;
    a.kc = static_cast<char*>(p.kc); a.k_sblk = p.k_sblk; a.k_stok = p.k_stok; a.k_sh = p.k_sh;
    a.vc = static_cast<char*>(p.vc); a.v_sblk = p.v_sblk; a.v_stok = p.v_stok; a.v_sh = p.v_sh;
    a.ks = p.ks; a.ks_sblk = p.ks_sblk; a.ks_sh = p.ks_sh;
    a.vs = p.vs; a.vs_sblk = p.vs_sblk; a.vs_sh = p.vs_sh;
    a.T = p.T; a.slots_total = p.NB * p.BS;
    a.Hkv = (int32_t)p.Hkv; a.D = (int32_t)p.D; a.bs = (uint32_t)p.BS;
    a.bs_shift = (p.BS & (p.BS - 1)) == 0 ? __builtin_ctzll((unsigned long long)p.BS) : -1;
    // pieces of 8 (bf16) or 16 (fp8) elements, one per thread unless the
    // tuning override asks for more (2 or 4 pieces per thread measured no
    // faster on bulk writes)
    const int64_t pieces = p.T * p.Hkv * (p.D / (p.fp8 ? 16 : 8));
    const int upt = g_write_pieces.load() > 0 ? g_write_pieces.load() : 1;
    const int64_t threads = (pieces + upt - 1) / upt;
    const int64_t groups = (threads + kWriteThreads - 1) / kWriteThreads;
    // the largest piece index the grid forms is below groups * 256 * upt
    a.small = groups * kWriteThreads * upt < (int64_t(1) << 31);
    const void* fn = upt == 4 ? (p.fp8 ? write_kernel_of<true, 4>((int)p.D) : write_kernel_of<false, 4>((int)p.D))
                   : upt == 2 ? (p.fp8 ? write_kernel_of<true, 2>((int)p.D) : write_kernel_of<false, 2>((int)p.D))
                              : (p.fp8 ? write_kernel_of<true, 1>((int)p.D) : write_kernel_of<false, 1>((int)p.D));
    void* args[] = {&a};
    if (hipLaunchKernel(fn, dim3((unsigned)groups), dim3(kWriteThreads), args, 0,
                        static_cast<hipStream_t>(stream)) != hipSuccess)
        return fail(PA_ERR_HIP, "cache write launch failed: %s", hipGetErrorString(hipGetLastError()));
    return PA_OK;
}
