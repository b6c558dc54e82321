// Paged prefill attention for gfx950: packed variable-length query chunks
// (sequence b owns rows cu[b] .. cu[b+1]-1, the last n_b of its L_b cached
// tokens) attend causally to their sequence's keys through the block table.
//
// The operation: ATOM model operations guide, "Attention operations"
// (prefill always runs a variable-length flash-attention call; the kernel
// table also lists a unified paged prefill kernel) and "Backend
// abstraction" (block tables and cumulative sequence lengths prepared for
// every prefill step); its source-file list places a ragged prefill chunk's
// tokens in their own sequences.
//
// Workgroup = W waves on one (sequence, kv head, block of W*P positions);
// W = 8 waves of 32 rows, or 4 waves of 64 rows when q_heads / kv_heads >
// 32 (prefill_shape).  Wave w owns positions p0 + wP .. p0 + wP + P - 1 of
// the chunk for all G query heads of the kv head (row r = position r / G,
// head r % G), the N side of 16x16 MFMA tiles as in the decode kernel.  The
// workgroup walks the keys in 32-token tiles, T at a time: all threads load
// the next T tiles' K and V rows (16-byte buffer loads, sub-block addressing
// through a per-wave block-table window) into one group of padded LDS
// buffers while the waves compute on the other, so every K/V byte read from
// L2 serves every row of the workgroup.  Per tile and wave: S^T = K Q^T and
// O^T += V^T P^T with v_mfma_f32_16x16x32_bf16 (the V^T operand by
// transposing LDS reads), online softmax in base 2 with a lazy rescale, row
// sums by the matrix unit.  Waves of 32 rows at head_dim 64 and 128 run the
// same schedule on v_mfma_f32_32x32x16_bf16 (prefill_kernel32: a wave's 32
// rows are one 32-wide N side).  A wave skips the tiles past its last position; tiles that reach
// past its first position's causal limit take the masked step.  Keys past
// L_b are zero-filled in LDS, so unwritten cache slots never reach the
// output.  Workgroups are ordered longest first (work_order), which also
// keeps the workgroups running together on the same sequences' keys, so
// that they share the L2.
//
// The call's host-side validation (validate_prefill, paged_attn_check_prefill*)
// is plain C++ in pa_prefill_host.cpp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <type_traits>
#include <cmath>

#include "pa_prefill_internal.h"

namespace pa {


namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRsrcWord3 = 0x00020000;     // raw buffer resource, 32-bit data format
constexpr float kRescaleLog2 = 8.0f;       // lazy rescale threshold (log2 units)
constexpr int kTile = 32;                  // keys per tile (two 16-token sub-blocks)
constexpr unsigned kOnes = 0x3F803F80u;    // two bf16 ones

typedef __amdgpu_buffer_rsrc_t Rsrc;

struct PrefillArgs {
    const char* q;   int64_t q_st, q_sh;              // bytes
    char* out;       int64_t o_st, o_sh;              // bytes
    const char* k;   int64_t k_stok, k_sh;            // bytes
    const char* v;   int64_t v_stok, v_sh;
    uint32_t k_sblk, v_sblk, k_ssub, v_ssub;          // block / 16-token sub-block strides, bytes
    const int32_t* bt; int64_t bt_sb;
    const int32_t* ctx; int64_t ctx_s;
    const int32_t* cu;  int64_t cu_s;
    float scale_log2;                                 // |scale| * log2(e)
    int32_t q_neg;                                    // scale < 0: negate q
    int32_t k_span, v_span;                           // bytes of one (sub-block, head) slice
    int32_t B, Hkv, G, P, qblocks, bsub, wsub, NB, T;
    int32_t window;                                   // sliding window in tokens, 0 = none
    const float* sinks; int64_t sinks_s;              // per query head, may be null
    // fp8 cache: per (token, kv head) scales, logical [NB, BS, Hkv] with the
    // slot dimension contiguous; block and head strides in bytes
    const char* ks; const char* vs;
    uint32_t ks_sblk, vs_sblk, ks_sh, vs_sh;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ unsigned pack_bf16_rne(float a, float b) {
    f32x2 f = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

// Row maxima over the four lanes l, l^16, l^32, l^48 (one query row's
// partial results) with the cross-row swaps: v_permlane16_swap_b32 (and
// v_permlane32_swap_b32) on a value and a copy of it leaves each lane with
// its own value in one register and its partner's (lane l^16, l^32) in the
// other, so combining the two gives the pair's result on every lane.  The
// swap is written as one instruction: the compiler's builtin for it folds a
// combination of its two results into the first.
__device__ __forceinline__ void swap_pair(float x, bool rows32, float& r0, float& r1) {
    r0 = x;
    r1 = x;
    if (rows32) asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(r0), "+v"(r1));
    else asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(r0), "+v"(r1));
}
__device__ __forceinline__ float pair_max(float x, bool rows32) {
    float a, b;
    swap_pair(x, rows32, a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float row_max(float x) { return pair_max(pair_max(x, false), true); }

__device__ __forceinline__ Rsrc make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

// LDS row stride of a K or V tile: a pad per row spreads the rows that 16
// lanes read at one column over the banks (32 bytes measured best of 16, 32
// and 48).
constexpr int kRowPad = 32;
template <int D> constexpr int kRowBytes = 2 * D + kRowPad;
template <int D> constexpr int kTileBytes = kTile * kRowBytes<D>;
// The V tile of the 32-row kernel: its transposing reads take four key rows
// at two 16-column spans per half wave, so rows 16 dwords apart (mod the 64
// banks) keep the half wave's 32 lanes on distinct banks
template <int D, bool R32> constexpr int kRowBytesV = R32 ? 2 * D + 64 : kRowBytes<D>;
template <int D, bool R32> constexpr int kTileBytesV = kTile * kRowBytesV<D, R32>;
// The K tile of the 32-row kernel: 16 consecutive rows on distinct banks
// (a 16-byte pad: rows 4 dwords apart mod 64)
template <int D, bool R32> constexpr int kRowBytesK = R32 ? 2 * D + 16 : kRowBytes<D>;
template <int D, bool R32> constexpr int kTileBytesK = kTile * kRowBytesK<D, R32>;
// 16-byte pieces of one row, and per thread of a tile
template <int D> constexpr int kPieces = D / 8;
// (rounded up: with head_dim 64 and 8 waves half the threads load nothing)
template <int D, int W> constexpr int kPerThread = (kTile * kPieces<D> + 64 * W - 1) / (64 * W);
// fp8: 8-byte pieces (8 elements, 16 bytes once in bf16) of one row, per
// thread of a tile
template <int D> constexpr int kPieces8 = D / 8;
template <int D, int W> constexpr int kPerThread8 = (kTile * kPieces8<D> + 64 * W - 1) / (64 * W);
// one LDS buffer: K tile, V tile, and with fp8 the tile's 32 K scales
template <int D, bool FP8, bool R32 = false>
constexpr int kBufBytes = kTileBytesK<D, R32> + kTileBytesV<D, R32> + (FP8 ? 4 * kTile : 0);
// 32-key tiles staged per barrier (two LDS groups of this many buffers).
// Two: between barriers the two waves of a SIMD drift apart, so one's
// softmax overlaps the other's matrix work (measured on MI355X with the
// 16-row kernel: 2k-row chunks +4-6 %, 8k prompts +2 %, head_dim 256 +3 %;
// four tiles were no better).  One at head_dim 64 (its windowed prefill
// measured 2 % faster) and for 64-row waves (a second tile's staging
// registers spill there).
template <int D, int NT> constexpr int kTilesPerBarrier = D == 64 || NT == 4 ? 1 : 2;

// The block-table window: lane l holds sub-block 2*t0 + l of sequence b.
struct BlockRef {
    int blk, sub;
};

__device__ __forceinline__ BlockRef load_window(const PrefillArgs& a, int b, int t0, int lane) {
    const int idx = min(2 * t0 + lane, a.wsub - 1);
    const int e = a.bsub > 1 ? idx / a.bsub : idx;
    const int v = a.bt[(int64_t)b * a.bt_sb + e];
    return BlockRef{min(max(v, 0), a.NB - 1), idx - e * a.bsub};
}

// Global K/V pieces of tile `tile` for this thread: piece i is token
// u / kPieces of the tile, column u % kPieces (u = tid + 64 W i), 16 bytes
// of bf16 or 8 bytes of fp8 (the same 8 elements), plus with fp8 the
// token's K and V scales; every piece of one load instruction lies in one
// sub-block per wave, so its block id is a wave-uniform readlane of the
// window.
template <int D, int W, bool FP8>
struct Pieces {
    typedef typename std::conditional<FP8, u32x2, u32x4>::type PT;
    PT k[kPerThread<D, W>], v[kPerThread<D, W>];
    float ks[FP8 ? kPerThread<D, W> : 1], vs[FP8 ? kPerThread<D, W> : 1];
};

// head-h slices of the scale arrays (fp8)
struct ScaleBase {
    const char* k; const char* v;
};

template <int D, int W, bool FP8>
__device__ __forceinline__ void load_tile(Pieces<D, W, FP8>& pc, const PrefillArgs& a, const char* kh,
                                          const char* vh, const ScaleBase& sc, const BlockRef& br, int tile,
                                          int wbase, int L, int tid) {
    constexpr unsigned EB = FP8 ? 8u : 16u;                        // bytes of a piece in the cache
#pragma unroll
    for (int i = 0; i < kPerThread<D, W>; ++i) {
        const int piece = tid + 64 * W * i;
        if (kTile * kPieces<D> % (64 * W) != 0 && piece >= kTile * kPieces<D>) break;   // wave-uniform
        const int tok = piece / kPieces<D>, col = piece % kPieces<D>;
        const int sb = __builtin_amdgcn_readfirstlane(tok >> 4);   // uniform per wave
        const int rel = 2 * tile + sb - wbase;                     // window lane of the sub-block
        const uint32_t blk = (uint32_t)__builtin_amdgcn_readlane(br.blk, rel);
        const uint32_t sub = (uint32_t)__builtin_amdgcn_readlane(br.sub, rel);
        const int tok0 = kTile * tile + 16 * sb;                   // first token of the sub-block
        const bool live = tok0 < L;
        const Rsrc rk = make_rsrc(kh + (uint64_t)blk * a.k_sblk + sub * a.k_ssub, live ? a.k_span : 0);
        const Rsrc rv = make_rsrc(vh + (uint64_t)blk * a.v_sblk + sub * a.v_ssub, live ? a.v_span : 0);
        const unsigned ko = (unsigned)((tok & 15) * a.k_stok) + EB * col;
        const unsigned vo = (unsigned)((tok & 15) * a.v_stok) + EB * col;
        if constexpr (FP8) {
            pc.k[i] = __builtin_amdgcn_raw_buffer_load_b64(rk, ko, 0, 0);
            pc.v[i] = __builtin_amdgcn_raw_buffer_load_b64(rv, vo, 0, 0);
            // the 16 slots' scales of the sub-block: 64 contiguous bytes
            const Rsrc rks = make_rsrc(sc.k + (uint64_t)blk * a.ks_sblk + 64u * sub, live ? 64 : 0);
            const Rsrc rvs = make_rsrc(sc.v + (uint64_t)blk * a.vs_sblk + 64u * sub, live ? 64 : 0);
            pc.ks[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rks, 4u * (tok & 15), 0, 0));
            pc.vs[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rvs, 4u * (tok & 15), 0, 0));
        } else {
            pc.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, ko, 0, 0);
            pc.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, vo, 0, 0);
        }
    }
}

// Two e4m3fn bytes (bytes 0-1, or 2-3 with HI, of w) -> a bf16 pair, exact:
// every e4m3fn value, subnormals included, is a bf16 value.
template <bool HI>
__device__ __forceinline__ unsigned fp8x2_bf16x2(unsigned w) {
    return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// Two e4m3fn bytes times a scale -> a bf16 pair (round to nearest even).
template <bool HI>
__device__ __forceinline__ unsigned fp8x2_scaled_bf16x2(unsigned w, float s) {
    const f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
    return pack_bf16_rne(f[0] * s, f[1] * s);
}

// Store the pieces into an LDS tile buffer; keys at or past L, and with a
// sliding window keys below vlo (outside every row's window: their blocks
// may have been freed), become zeros (their slots may hold anything).  fp8:
// K becomes bf16 exactly and its scales go to lds_ks (applied to the
// scores, so K stays exact); V is scaled and rounded to bf16 (one rounding,
// as a bf16 cache has).
template <int D, int W, bool FP8, bool R32 = false>
__device__ __forceinline__ void store_tile(char* lds_k, char* lds_v, float* lds_ks, const Pieces<D, W, FP8>& pc,
                                           int tile, int L, int vlo, int tid) {
#pragma unroll
    for (int i = 0; i < kPerThread<D, W>; ++i) {
        const int piece = tid + 64 * W * i;
        if (kTile * kPieces<D> % (64 * W) != 0 && piece >= kTile * kPieces<D>) break;   // wave-uniform
        const int tok = piece / kPieces<D>, col = piece % kPieces<D>;
        const bool keep = kTile * tile + tok < L && kTile * tile + tok >= vlo;
        const u32x4 z = {0u, 0u, 0u, 0u};
        u32x4 k, v;
        if constexpr (FP8) {
            k = u32x4{fp8x2_bf16x2<false>(pc.k[i][0]), fp8x2_bf16x2<true>(pc.k[i][0]),
                      fp8x2_bf16x2<false>(pc.k[i][1]), fp8x2_bf16x2<true>(pc.k[i][1])};
            const float s = pc.vs[i];
            v = u32x4{fp8x2_scaled_bf16x2<false>(pc.v[i][0], s), fp8x2_scaled_bf16x2<true>(pc.v[i][0], s),
                      fp8x2_scaled_bf16x2<false>(pc.v[i][1], s), fp8x2_scaled_bf16x2<true>(pc.v[i][1], s)};
            if (col == 0) lds_ks[tok] = keep ? pc.ks[i] : 0.f;
        } else {
            k = pc.k[i];
            v = pc.v[i];
        }
        *reinterpret_cast<u32x4*>(lds_k + tok * kRowBytesK<D, R32> + 16 * col) = keep ? k : z;
        *reinterpret_cast<u32x4*>(lds_v + tok * kRowBytesV<D, R32> + 16 * col) = keep ? v : z;
    }
}

template <int D, int NT>
struct Acc {
    float m[NT];
    float nm[NT <= 2 ? NT : 1];  // -m, or 0 while m is -inf (32-row waves)
    f32x4 l[NT];                 // row sums: every element holds the lane's row's sum
    float t[NT];                 // score above which m must rise: (m + kRescaleLog2) / c
    f32x4 o[NT][D / 16];
};

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16
// lanes, lane i receives element i % 4 of the 8-byte pieces that lanes
// i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4 of the group address.  With
// lane s of the group at head_dim 4 (s % 4) .. + 3 of key row s / 4, lane i
// gets head_dim i of those four keys: a column of V, the V^T operand.
__device__ __forceinline__ u32x2 read_vt(const char* p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
}

// Wave priority over the phases of a tile (s_setprio).  The two waves of a
// SIMD run the same phases at about the same time (they meet at every tile's
// barrier); raising a wave's priority while it reads K/V fragments and issues
// matrix instructions, and lowering it for the softmax arithmetic, lets the
// other wave's softmax fill the matrix unit's gaps instead of competing with
// its issue.  Which phases pay depends on the shape (measured on MI355X,
// 8k-token prompts and 2k-row chunks): head_dim 128 bf16 fragments + score
// product and value product, 9 % faster; with an fp8 cache the whole tile,
// 4 %, leaving the conversion work around the next tile's stores at the base
// priority; head_dim 256 fragments + score product, 10 % (fp8 2 %), the value
// product included slower; head_dim 64 bf16 the value product, 1.5 %; fp8
// head_dim 64 and the 64-row waves none (every variant slower).
enum TilePrio { kPrioNone, kPrioScores, kPrioMatrix, kPrioTile, kPrioValue };
template <int D, int NT, bool FP8>
constexpr TilePrio kTilePrio = NT == 4 ? kPrioNone
                             : D == 256 ? kPrioScores
                             : D == 128 ? (FP8 ? kPrioTile : kPrioMatrix)
                             : (FP8 ? kPrioNone : kPrioValue);

// One 32-key tile of one wave: K fragments (A operand, token = lane % 16,
// head_dim 8 * (lane / 16) ... of each 32-wide step) and V^T fragments
// (A operand, head_dim 16 j + lane % 16, the eight keys 4 (lane / 16) + i
// and 16 + 4 (lane / 16) + i of the lane's score fragments, by transposing
// reads of the key-major V tile) read from LDS, then the decode kernel's step: S^T = K Q^T, base-2 online
// softmax with a lazy rescale, O^T += V^T P^T.  masked (wave-uniform): some
// key of the tile lies past some row's causal limit.  One copy of the step
// serves both cases: two inlined copies would not fit the register file.
// fp8 (lds_ks non-null): the scores of key k are multiplied by its K scale.
template <int D, int NT, bool FP8>
__device__ __forceinline__ void tile_step(Acc<D, NT>& s, const u32x4 (&qf)[NT][D / 32], const char* lds_k,
                                          const char* lds_v, const float* lds_ks, const int (&lim)[NT],
                                          const int (&low)[NT], int kbase, float c, int lane, bool masked,
                                          bf16x8 ones) {
    constexpr int J = D / 16;
    constexpr TilePrio P = kTilePrio<D, NT, FP8>;
    const int n16 = lane & 15, grp = lane >> 4;
    if constexpr (P == kPrioScores || P == kPrioMatrix || P == kPrioTile) __builtin_amdgcn_s_setprio(1);
    bf16x8 kf[2][D / 32];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
            kf[mt][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(
                lds_k + (16 * mt + n16) * kRowBytes<D> + 2 * (32 * kk + 8 * grp)));
    // lane (n16, grp) addresses key 4 grp + n16 / 4 (and 16 more), head_dim
    // 16 j + 4 (n16 % 4)
    const char* vrow = lds_v + (4 * grp + (n16 >> 2)) * kRowBytes<D> + 8 * (n16 & 3);
    u32x4 vt[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const u32x2 lo = read_vt(vrow + 32 * j);
        const u32x2 hi = read_vt(vrow + 16 * kRowBytes<D> + 32 * j);
        vt[j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    // fp8: the K scales of the lane's keys 4 grp + i and 16 + 4 grp + i
    f32x4 ksc0 = {1.f, 1.f, 1.f, 1.f}, ksc1 = {1.f, 1.f, 1.f, 1.f};
    if constexpr (FP8) {
        ksc0 = *reinterpret_cast<const f32x4*>(lds_ks + 4 * grp);
        ksc1 = *reinterpret_cast<const f32x4*>(lds_ks + 16 + 4 * grp);
    }

#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        // four tiles: one at a time (interleaving their score and softmax
        // work would not fit the register file next to the accumulators and
        // query fragments); two tiles interleave freely
        if (NT > 2 && nt > 0) __builtin_amdgcn_sched_barrier(0);
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            const bf16x8 qb = as_bf16x8(qf[nt][kk]);
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][kk], qb, s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][kk], qb, s1, 0, 0, 0);
        }
        if constexpr (P == kPrioScores || P == kPrioMatrix) __builtin_amdgcn_s_setprio(0);
        float y[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            y[i] = FP8 ? s0[i] * ksc0[i] : s0[i];
            y[4 + i] = FP8 ? s1[i] * ksc1[i] : s1[i];
        }
        if (masked) {
            // keys past the row's causal limit or below its window: -inf,
            // whose exponent below is 0 (c > 0, so c * -inf stays -inf)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int tok = kbase + 16 * (i >> 2) + 4 * grp + (i & 3);
                y[i] = (tok > lim[nt] || tok < low[nt]) ? -__builtin_inff() : y[i];
            }
        }
        // the running max m (log2 units) only has to rise when some score
        // exceeds it by more than kRescaleLog2: a compare per score against
        // the row's threshold, the row max itself only when it does
        bool over = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) over |= y[i] > s.t[nt];
        if (__any(over)) {
            float mx = fmaxf(fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3])), fmaxf(fmaxf(y[4], y[5]), fmaxf(y[6], y[7])));
            mx = row_max(mx);
            const float m_new = fmaxf(s.m[nt], c * mx);
            const float alpha = m_new == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(s.m[nt] - m_new);
            s.l[nt] *= alpha;               // (all four elements)
#pragma unroll
            for (int j = 0; j < J; ++j) s.o[nt][j] *= alpha;
            s.m[nt] = m_new;
            if constexpr (NT <= 2) s.nm[nt] = m_new == -__builtin_inff() ? 0.f : -m_new;
            s.t[nt] = (m_new + kRescaleLog2) / c;
        }
        // 32-row waves keep -m as state (set at a rescale); 64-row waves
        // recompute it (no registers to spare)
        float neg_m;
        if constexpr (NT <= 2) neg_m = s.nm[nt];
        else neg_m = s.m[nt] == -__builtin_inff() ? 0.f : -s.m[nt];
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(y[i], c, neg_m));
        u32x4 pw;
#pragma unroll
        for (int w = 0; w < 4; ++w) pw[w] = pack_bf16_rne(p[2 * w], p[2 * w + 1]);
        const bf16x8 pb = as_bf16x8(pw);
        if constexpr (P == kPrioMatrix || P == kPrioValue) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int j = 0; j < J; ++j)
            s.o[nt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vt[j]), pb, s.o[nt][j], 0, 0, 0);
        // row sums by the matrix unit: an all-ones A operand sums the 32 keys
        // of P for every row, already across the lanes holding the row, and
        // from the same bf16 P as the accumulators
        if constexpr (NT <= 2)
            s.l[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb, s.l[nt], 0, 0, 0);
        else
            s.l[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u32x4{kOnes, kOnes, kOnes, kOnes}), pb,
                                                             s.l[nt], 0, 0, 0);
        if constexpr (P == kPrioMatrix || P == kPrioValue) __builtin_amdgcn_s_setprio(0);
    }
    if constexpr (P == kPrioTile) __builtin_amdgcn_s_setprio(0);
}

// 32-row waves on the 32x32x16 matrix instruction (head_dim 64 and 128): per
// 32-key tile 8 or 16 matrix instructions instead of 18 or 34 of the
// 16x16x32 shape, one cross-lane step for a row's max instead of two, row
// sums by the vector unit; measured on MI355X 26-28 % faster on windowed
// head_dim-64 prompts and 6.5-7 % with an fp8 cache at head_dim 128, level
// (within 2 %) with a bf16 cache at head_dim 128.
// Operand layouts of v_mfma_f32_32x32x16_bf16 (lane l, n = l % 32, h = l / 32):
// A lane l holds A[n][8h .. 8h+7], B lane l holds B[8h .. 8h+7][n], and
// element i of the f32x16 result is D[8 (i / 4) + 4h + i % 4][n].
//  * S^T = K Q^T: keys are M (the tile's 32), the wave's 32 query rows N, head_dim
//    the reduction in steps of 16: element i of the scores is key
//    8 (i / 4) + 4h + i % 4 of row n, so a lane holds 16 scores of one row and
//    the row's other 16 sit in lane l ^ 32.
//  * O^T += V^T P^T: head_dim blocks of 32 are M, the 32 keys the reduction in
//    two steps of 16.  Step ks takes the lane's probabilities 8 ks .. 8 ks + 7
//    as its B operand as they stand (keys 16 ks + 8 (j / 4) + 4h + j % 4), so
//    the V^T operand of lane l holds those keys at head_dim 32 mb + n: two
//    transposing LDS reads of four keys each.
//  * Row sums: v_dot2 of the bf16 probabilities with ones, per lane (its 16
//    keys), combined with lane l ^ 32 in the epilogue.
template <int D>
struct Acc32 {
    float m, nm, t;          // running max (log2 units), -m (0 while m is -inf), rescale threshold
    float l;                 // this lane's part of the row sum
    f32x16 o[D / 32];        // element i: head_dim 32 mb + 8 (i / 4) + 4h + i % 4 of row n
};

template <int D, bool FP8>
__device__ __forceinline__ void tile_step32(Acc32<D>& s, const u32x4 (&qf)[D / 16], const char* lds_k,
                                            const char* lds_v, const float* lds_ks, int lim, int low, int kbase,
                                            float c, int lane, bool masked) {
    const int n = lane & 31, h = lane >> 5;
    f32x16 sc = {};
    const char* krow = lds_k + n * kRowBytesK<D, true> + 16 * h;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(krow + 32 * kk)),
                                                     as_bf16x8(qf[kk]), sc, 0, 0, 0);
    // V^T operands: lane (g = lane / 16, s = lane % 16) reads key 4h + s / 4 (+ 16 ks,
    // + 8), head_dim 32 mb + 16 (g % 2) + 4 (s % 4)
    constexpr int RV = kRowBytesV<D, true>;
    const char* vbase = lds_v + (4 * h + ((lane & 15) >> 2)) * RV + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    u32x4 vt[2][D / 32];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) {
            const u32x2 lo = read_vt(vbase + 16 * ks * RV + 64 * mb);
            const u32x2 hi = read_vt(vbase + (16 * ks + 8) * RV + 64 * mb);
            vt[ks][mb] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
    float y[16];
    if constexpr (FP8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 kq = *reinterpret_cast<const f32x4*>(lds_ks + 8 * q + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) y[4 * q + e] = sc[4 * q + e] * kq[e];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] = sc[i];
    }
    if (masked) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int tok = kbase + 8 * (i >> 2) + 4 * h + (i & 3);
            y[i] = (tok > lim || tok < low) ? -__builtin_inff() : y[i];
        }
    }
    bool over = false;
#pragma unroll
    for (int i = 0; i < 16; ++i) over |= y[i] > s.t;
    if (__any(over)) {
        float mx = y[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, y[i]);
        mx = pair_max(mx, true);
        const float m_new = fmaxf(s.m, c * mx);
        const float alpha = m_new == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(s.m - m_new);
        s.l *= alpha;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) s.o[mb] *= alpha;
        s.m = m_new;
        s.nm = m_new == -__builtin_inff() ? 0.f : -m_new;
        s.t = (m_new + kRescaleLog2) / c;
    }
    // the packed probabilities as separate words (the row-sum dot products
    // read them one by one; taken as elements of a vector, the compiler fed
    // the first element to all four)
    unsigned pk[8];
#pragma unroll
    for (int w = 0; w < 8; ++w)
        pk[w] = pack_bf16_rne(__builtin_amdgcn_exp2f(__builtin_fmaf(y[2 * w], c, s.nm)),
                              __builtin_amdgcn_exp2f(__builtin_fmaf(y[2 * w + 1], c, s.nm)));
    const u32x4 pw[2] = {u32x4{pk[0], pk[1], pk[2], pk[3]}, u32x4{pk[4], pk[5], pk[6], pk[7]}};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
            s.o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vt[ks][mb]), as_bf16x8(pw[ks]), s.o[mb], 0, 0, 0);
    const bf16x2 one2 = __builtin_bit_cast(bf16x2, kOnes);
#pragma unroll
    for (int w = 0; w < 8; ++w) s.l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[w]), one2, s.l, false);
}

// Longest work first.  Workgroup (b, qb, g) reads the keys below
// K(b, qb) = (L_b - n_b) + min((qb + 1) WP, n_b) (WP positions per
// workgroup), so its work grows with K; launched in order of decreasing K
// (ties: lower b first; the kv heads of one (b, qb) consecutive), the
// longest workgroups start first and the short ones fill the tail, whatever
// the mix of prefix and chunk lengths.  Rank r = blockIdx.x maps to its item
// by a binary search over K: lane b of the wave holds sequence b (B <= 64)
// and counts its items with K >= x in closed form.  Every wave computes the
// same answer; false: the rank is past the last item.
struct SeqWork {
    int A, n, nb;        // prefix length L - n, chunk rows, position blocks
};
__device__ __forceinline__ int count_ge(const SeqWork& s, int x, int WP, double inv_wp) {
    // items qb < nb with A + min((qb + 1) WP, n) >= x: nb - (ceil(y / WP) - 1)
    // for y = x - A in (0, n].  The quotient in double: z / WP for z < 2^32
    // is within 2^-20 of the exact value, and a non-integer quotient is at
    // least 1 / WP >= 2^-8 above its floor, so adding 2^-12 and truncating
    // is exact.
    const int y = x - s.A;
    if (y <= 0) return s.nb;
    if (y > s.n) return 0;
    const int q = (int)__builtin_fma((double)y + (double)(WP - 1), inv_wp, 0x1p-12);
    return s.nb - (q - 1);
}
// Sum (max) over the wave: inclusive scans within each row of 16 lanes by
// DPP row shifts (lanes shifted in from outside the row contribute 0), then
// the four rows' last lanes.
__device__ __forceinline__ int wave_sum(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);      // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);      // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);      // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);      // row_shr:8
    return __builtin_amdgcn_readlane(v, 15) + __builtin_amdgcn_readlane(v, 31) + __builtin_amdgcn_readlane(v, 47) +
           __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int wave_max_nonneg(int v) {
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false));
    return max(max(__builtin_amdgcn_readlane(v, 15), __builtin_amdgcn_readlane(v, 31)),
               max(__builtin_amdgcn_readlane(v, 47), __builtin_amdgcn_readlane(v, 63)));
}
__device__ __forceinline__ bool work_order(const PrefillArgs& a, int rank, int lane, int WP, int& b, int& qb,
                                           int& g) {
    SeqWork s = {0, 0, 0};
    int Lmax = 0;
    if (lane < a.B) {
        const int c0 = min(max(a.cu[(int64_t)lane * a.cu_s], 0), a.T);
        const int L = min(a.ctx[(int64_t)lane * a.ctx_s], 16 * a.wsub);
        const int n = min(min(a.cu[(int64_t)(lane + 1) * a.cu_s], a.T) - c0, L);
        if (n > 0) {
            s.A = L - n;
            s.n = n;
            s.nb = (n + WP - 1) / WP;
            Lmax = L;
        }
    }
    const int item = rank / a.Hkv;
    g = rank - item * a.Hkv;
    if (item >= wave_sum(s.nb)) return false;
    Lmax = wave_max_nonneg(Lmax);
    const double inv_wp = 1.0 / (double)WP;
    // the largest x with more than `item` items of key >= x: the item's key
    int lo = 1, hi = Lmax + 1;                       // count(lo) > item >= count(hi)
    while (hi - lo > 1) {
        const int mid = lo + (hi - lo) / 2;
        if (wave_sum(count_ge(s, mid, WP, inv_wp)) > item) lo = mid;
        else hi = mid;
    }
    // among the sequences with an item of key lo, the j-th (by b)
    const int j = item - wave_sum(count_ge(s, lo + 1, WP, inv_wp));
    const bool has = count_ge(s, lo, WP, inv_wp) > count_ge(s, lo + 1, WP, inv_wp);
    uint64_t m = __ballot(has);
    for (int k = 0; k < j; ++k) m &= m - 1;
    b = __builtin_amdgcn_readfirstlane(__builtin_ctzll(m));
    // the item of key lo is sequence b's lowest position block with key >= lo
    qb = __builtin_amdgcn_readfirstlane(__shfl(s.nb - count_ge(s, lo, WP, inv_wp), b));
    return true;
}

// NT: 16-row tiles per wave (rows = 16 NT = positions P x query heads G);
// W: waves per workgroup.
template <int D, int NT, int W, bool FP8>
__global__ __launch_bounds__(64 * W) void prefill_kernel(PrefillArgs a) {
    constexpr int J = D / 16;
    extern __shared__ __align__(16) char lds[];            // [2 buffers][K tile, V tile (, K scales)]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, grp = lane >> 4;
    int b, qb, g;
    if (a.B > 1 && a.B <= 64 && a.window <= 0) {
        if (!work_order(a, (int)blockIdx.x, lane, W * a.P, b, qb, g)) return;
    } else {
        // one sequence (the same order), many, or a sliding window (every
        // workgroup then has about the same work): the highest position
        // blocks of every (sequence, kv head) first
        const int pairs = a.B * a.Hkv;
        qb = a.qblocks - 1 - (int)(blockIdx.x / pairs);
        const int pr = blockIdx.x % pairs;
        b = pr / a.Hkv;
        g = pr - b * a.Hkv;
    }
    // the chunk's rows, clamped to the packed rows and to the sequence
    const int c0 = min(max(a.cu[(int64_t)b * a.cu_s], 0), a.T);
    const int L = min(a.ctx[(int64_t)b * a.ctx_s], 16 * a.wsub);
    const int n = min(min(a.cu[(int64_t)(b + 1) * a.cu_s], a.T) - c0, L);
    const int p0 = qb * W * a.P;                      // first position (in the chunk) of the workgroup
    if (n <= 0 || p0 >= n) return;
    const int pw = p0 + wave * a.P;                        // first position of this wave
    // keys the workgroup needs: below L - n + min(p0 + W P, n); this wave's
    // rows need keys below L - n + min(pw + P, n) (none if pw >= n).  With
    // a sliding window w the row at position a sees keys a - w + 1 .. a, so
    // the workgroup starts at its first row's window (jstart, keys below
    // vlo are outside every row's window) and a wave at its own (wstart).
    const int w = a.window;
    const int kend = L - n + min(p0 + W * a.P, n);
    const int wend = pw < n ? L - n + min(pw + a.P, n) : 0;
    const int ntiles = (kend + kTile - 1) / kTile;
    const int wtiles = (wend + kTile - 1) / kTile;
    const int vlo = w > 0 ? max(0, L - n + p0 - w + 1) : 0;
    const int jstart = vlo / kTile;
    const int wstart = w > 0 && pw < n ? max(0, L - n + pw - w + 1) / kTile : 0;
    // tiles wholly at or below every row's causal limit (the first row's
    // limit is L - n + pw) and, with a window, wholly at or above every
    // row's lower limit (the last row's is L - n + min(pw + P, n) - w) take
    // the step without masks
    const int wclean = pw < n ? (L - n + pw + 1) / kTile : 0;
    const int wlow = w > 0 && pw < n ? L - n + min(pw + a.P, n) - w : 0;

    // query fragments and per-row causal limits (and lower limits)
    u32x4 qf[NT][D / 32];
    int lim[NT], low[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int row = 16 * nt + n16;
        const int t = row / a.G, hl = row - t * a.G;
        const int pos = pw + t;
        const bool live = t < a.P && pos < n;
        lim[nt] = live ? L - n + pos : L - 1;
        low[nt] = w > 0 && live ? L - n + pos - w + 1 : INT_MIN;
        const char* qrow = a.q + (int64_t)(c0 + (live ? pos : 0)) * a.q_st + (int64_t)(g * a.G + hl) * a.q_sh;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            u32x4 x = live ? *reinterpret_cast<const u32x4*>(qrow + 2 * (32 * kk + 8 * grp)) : u32x4{0u, 0u, 0u, 0u};
            qf[nt][kk] = a.q_neg ? x ^ 0x80008000u : x;
        }
    }

    const char* kh = a.k + (int64_t)g * a.k_sh;
    const char* vh = a.v + (int64_t)g * a.v_sh;
    // buffer i at lds + i * BB: K tile, V tile at + TB, with fp8 the K scales
    // at + 2 TB (plain arithmetic on the shared array keeps the accesses in
    // LDS instructions)
    constexpr int TB = kTileBytes<D>, BB = kBufBytes<D, FP8>;
    ScaleBase sc = {nullptr, nullptr};
    if constexpr (FP8) sc = ScaleBase{a.ks + (int64_t)g * a.ks_sh, a.vs + (int64_t)g * a.vs_sh};

    Acc<D, NT> s;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        s.m[nt] = -__builtin_inff();
        if constexpr (NT <= 2) s.nm[nt] = 0.f;
        s.t[nt] = -__builtin_inff();
        s.l[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < J; ++j) s.o[nt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float c = a.scale_log2;
    // the all-ones operand of the row-sum MFMA, held in registers for the
    // whole loop with 32-row waves (rebuilt per tile it costs three moves;
    // 64-row waves have no registers to spare for it)
    bf16x8 ones = as_bf16x8(u32x4{kOnes, kOnes, kOnes, kOnes});
    if constexpr (NT <= 2) asm volatile("" : "+v"(ones));

    constexpr int T = kTilesPerBarrier<D, NT>;
    if constexpr (T == 1) {
        // tile jstart into its buffer (tile j lives in buffer j & 1)
        BlockRef br = load_window(a, b, jstart, lane);
        int wbase = 2 * jstart;                                // first sub-block of the block-table window
        Pieces<D, W, FP8> pc;
        load_tile<D, W, FP8>(pc, a, kh, vh, sc, br, jstart, wbase, L, tid);
        {
            const int first = (jstart & 1) * BB;
            store_tile<D, W, FP8>(lds + first, lds + first + TB, reinterpret_cast<float*>(lds + first + 2 * TB), pc,
                                  jstart, L, vlo, tid);
        }
        __syncthreads();
        for (int j = jstart; j < ntiles; ++j) {
            const bool more = j + 1 < ntiles;
            if (more) {
                // a block-table window holds 64 sub-blocks = 32 tiles
                if (((j + 1 - jstart) & 31) == 0) {
                    br = load_window(a, b, j + 1, lane);
                    wbase = 2 * (j + 1);
                }
                load_tile<D, W, FP8>(pc, a, kh, vh, sc, br, j + 1, wbase, L, tid);
            }
            const int cur = (j & 1) * BB, nxt = BB - cur;
            if (j >= wstart && j < wtiles)
                tile_step<D, NT, FP8>(s, qf, lds + cur, lds + cur + TB, reinterpret_cast<const float*>(lds + cur + 2 * TB),
                                      lim, low, kTile * j, c, lane, j >= wclean || kTile * j < wlow, ones);
            if (more)
                store_tile<D, W, FP8>(lds + nxt, lds + nxt + TB, reinterpret_cast<float*>(lds + nxt + 2 * TB), pc, j + 1,
                                      L, vlo, tid);
            __syncthreads();
        }
    } else {
        // T tiles per barrier: the group of tiles jstart + T i ... lives in
        // buffers T (i & 1) ... T (i & 1) + T - 1, and the global loads of the
        // next group are in flight while this one is computed
        BlockRef br = load_window(a, b, jstart, lane);
        int wbase = 2 * jstart;                                // first sub-block of the block-table window
        Pieces<D, W, FP8> pc[T];
    #pragma unroll
        for (int h = 0; h < T; ++h)
            if (jstart + h < ntiles) load_tile<D, W, FP8>(pc[h], a, kh, vh, sc, br, jstart + h, wbase, L, tid);
    #pragma unroll
        for (int h = 0; h < T; ++h)
            if (jstart + h < ntiles)
                store_tile<D, W, FP8>(lds + h * BB, lds + h * BB + TB, reinterpret_cast<float*>(lds + h * BB + 2 * TB), pc[h],
                                      jstart + h, L, vlo, tid);
        __syncthreads();
        for (int j = jstart, it = 0; j < ntiles; j += T, ++it) {
            const bool more = j + T < ntiles;
            if (more) {
                // a block-table window holds 64 sub-blocks = 32 tiles (T divides 32,
                // so a group never straddles two)
                if (((j + T - jstart) & 31) == 0) {
                    br = load_window(a, b, j + T, lane);
                    wbase = 2 * (j + T);
                }
    #pragma unroll
                for (int h = 0; h < T; ++h)
                    if (j + T + h < ntiles) load_tile<D, W, FP8>(pc[h], a, kh, vh, sc, br, j + T + h, wbase, L, tid);
            }
            const int cur = (it & 1) * T * BB, nxt = T * BB - cur;
    #pragma unroll
            for (int h = 0; h < T; ++h) {
                const int jj = j + h;
                const int base = cur + h * BB;
                if (jj >= wstart && jj < wtiles)
                    tile_step<D, NT, FP8>(s, qf, lds + base, lds + base + TB,
                                          reinterpret_cast<const float*>(lds + base + 2 * TB), lim, low, kTile * jj, c,
                                          lane, jj >= wclean || kTile * jj < wlow, ones);
            }
            if (more) {
    #pragma unroll
                for (int h = 0; h < T; ++h)
                    if (j + T + h < ntiles)
                        store_tile<D, W, FP8>(lds + nxt + h * BB, lds + nxt + h * BB + TB,
                                              reinterpret_cast<float*>(lds + nxt + h * BB + 2 * TB), pc[h], j + T + h, L, vlo,
                                              tid);
            }
            __syncthreads();
        }
    }

    // epilogue: lane holds d = 16 j + 4 grp + i of row 16 nt + n16
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        float lt = s.l[nt][0];
        const int row = 16 * nt + n16;
        const int t = row / a.G, hl = row - t * a.G;
        const int pos = pw + t;
        if (!(t < a.P && pos < n)) continue;
        const int h = g * a.G + hl;
        if (a.sinks) {
            // the sink logit joins the normaliser: l += 2^(sink log2(e) - m)
            const float sk = a.sinks[(int64_t)h * a.sinks_s] * kLog2e;
            if (sk > -__builtin_inff()) lt += __builtin_amdgcn_exp2f(sk - s.m[nt]);
        }
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        char* orow = a.out + (int64_t)(c0 + pos) * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const u32x2 wv = {pack_bf16_rne(s.o[nt][j][0] * inv, s.o[nt][j][1] * inv),
                              pack_bf16_rne(s.o[nt][j][2] * inv, s.o[nt][j][3] * inv)};
            *reinterpret_cast<u32x2*>(orow + 2 * (16 * j + 4 * grp)) = wv;
        }
    }
}

// NT: 16-row tiles per wave (rows = 16 NT = positions P x query heads G);
// W: waves per workgroup.
template <int D, int W, bool FP8>
__global__ __launch_bounds__(64 * W) void prefill_kernel32(PrefillArgs a) {
    constexpr int NT = 2;
    constexpr int J = D / 16;
    extern __shared__ __align__(16) char lds[];            // [2 buffers][K tile, V tile (, K scales)]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, grp = lane >> 4;
    int b, qb, g;
    if (a.B > 1 && a.B <= 64 && a.window <= 0) {
        if (!work_order(a, (int)blockIdx.x, lane, W * a.P, b, qb, g)) return;
    } else {
        // one sequence (the same order), many, or a sliding window (every
        // workgroup then has about the same work): the highest position
        // blocks of every (sequence, kv head) first
        const int pairs = a.B * a.Hkv;
        qb = a.qblocks - 1 - (int)(blockIdx.x / pairs);
        const int pr = blockIdx.x % pairs;
        b = pr / a.Hkv;
        g = pr - b * a.Hkv;
    }
    // the chunk's rows, clamped to the packed rows and to the sequence
    const int c0 = min(max(a.cu[(int64_t)b * a.cu_s], 0), a.T);
    const int L = min(a.ctx[(int64_t)b * a.ctx_s], 16 * a.wsub);
    const int n = min(min(a.cu[(int64_t)(b + 1) * a.cu_s], a.T) - c0, L);
    const int p0 = qb * W * a.P;                      // first position (in the chunk) of the workgroup
    if (n <= 0 || p0 >= n) return;
    const int pw = p0 + wave * a.P;                        // first position of this wave
    // keys the workgroup needs: below L - n + min(p0 + W P, n); this wave's
    // rows need keys below L - n + min(pw + P, n) (none if pw >= n).  With
    // a sliding window w the row at position a sees keys a - w + 1 .. a, so
    // the workgroup starts at its first row's window (jstart, keys below
    // vlo are outside every row's window) and a wave at its own (wstart).
    const int w = a.window;
    const int kend = L - n + min(p0 + W * a.P, n);
    const int wend = pw < n ? L - n + min(pw + a.P, n) : 0;
    const int ntiles = (kend + kTile - 1) / kTile;
    const int wtiles = (wend + kTile - 1) / kTile;
    const int vlo = w > 0 ? max(0, L - n + p0 - w + 1) : 0;
    const int jstart = vlo / kTile;
    const int wstart = w > 0 && pw < n ? max(0, L - n + pw - w + 1) / kTile : 0;
    // tiles wholly at or below every row's causal limit (the first row's
    // limit is L - n + pw) and, with a window, wholly at or above every
    // row's lower limit (the last row's is L - n + min(pw + P, n) - w) take
    // the step without masks
    const int wclean = pw < n ? (L - n + pw + 1) / kTile : 0;
    const int wlow = w > 0 && pw < n ? L - n + min(pw + a.P, n) - w : 0;

    // query fragments (B operand: row n, head_dim 16 kk + 8h ..) and the row's
    // causal limit (and lower limit)
    u32x4 qf[D / 16];
    int lim, low;
    {
        const int row = lane & 31, hh = lane >> 5;
        const int t = row / a.G, hl = row - t * a.G;
        const int pos = pw + t;
        const bool live = t < a.P && pos < n;
        lim = live ? L - n + pos : L - 1;
        low = w > 0 && live ? L - n + pos - w + 1 : INT_MIN;
        const char* qrow = a.q + (int64_t)(c0 + (live ? pos : 0)) * a.q_st + (int64_t)(g * a.G + hl) * a.q_sh;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            u32x4 x = live ? *reinterpret_cast<const u32x4*>(qrow + 2 * (16 * kk + 8 * hh)) : u32x4{0u, 0u, 0u, 0u};
            qf[kk] = a.q_neg ? x ^ 0x80008000u : x;
        }
    }

    const char* kh = a.k + (int64_t)g * a.k_sh;
    const char* vh = a.v + (int64_t)g * a.v_sh;
    // buffer i at lds + i * BB: K tile, V tile at + TB, with fp8 the K scales
    // at + 2 TB (plain arithmetic on the shared array keeps the accesses in
    // LDS instructions)
    constexpr int TB = kTileBytesK<D, true>, TBV = kTileBytesV<D, true>, BB = kBufBytes<D, FP8, true>;
    ScaleBase sc = {nullptr, nullptr};
    if constexpr (FP8) sc = ScaleBase{a.ks + (int64_t)g * a.ks_sh, a.vs + (int64_t)g * a.vs_sh};

    Acc32<D> s;
    s.m = -__builtin_inff();
    s.nm = 0.f;
    s.t = -__builtin_inff();
    s.l = 0.f;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) s.o[mb] = f32x16{};
    const float c = a.scale_log2;

    // T tiles per barrier: the group of tiles jstart + T i ... lives in
    // buffers T (i & 1) ... T (i & 1) + T - 1, and the global loads of the
    // next group are in flight while this one is computed
    constexpr int T = kTilesPerBarrier<D, NT>;
    BlockRef br = load_window(a, b, jstart, lane);
    int wbase = 2 * jstart;                                // first sub-block of the block-table window
    Pieces<D, W, FP8> pc[T];
#pragma unroll
    for (int h = 0; h < T; ++h)
        if (jstart + h < ntiles) load_tile<D, W, FP8>(pc[h], a, kh, vh, sc, br, jstart + h, wbase, L, tid);
#pragma unroll
    for (int h = 0; h < T; ++h)
        if (jstart + h < ntiles)
            store_tile<D, W, FP8, true>(lds + h * BB, lds + h * BB + TB, reinterpret_cast<float*>(lds + h * BB + TB + TBV), pc[h],
                                  jstart + h, L, vlo, tid);
    __syncthreads();
    for (int j = jstart, it = 0; j < ntiles; j += T, ++it) {
        const bool more = j + T < ntiles;
        if (more) {
            // a block-table window holds 64 sub-blocks = 32 tiles (T divides 32,
            // so a group never straddles two)
            if (((j + T - jstart) & 31) == 0) {
                br = load_window(a, b, j + T, lane);
                wbase = 2 * (j + T);
            }
#pragma unroll
            for (int h = 0; h < T; ++h)
                if (j + T + h < ntiles) load_tile<D, W, FP8>(pc[h], a, kh, vh, sc, br, j + T + h, wbase, L, tid);
        }
        const int cur = (it & 1) * T * BB, nxt = T * BB - cur;
#pragma unroll
        for (int h = 0; h < T; ++h) {
            const int jj = j + h;
            const int base = cur + h * BB;
            if (jj >= wstart && jj < wtiles)
                tile_step32<D, FP8>(s, qf, lds + base, lds + base + TB,
                                    reinterpret_cast<const float*>(lds + base + TB + TBV), lim, low, kTile * jj, c, lane,
                                    jj >= wclean || kTile * jj < wlow);
        }
        if (more) {
#pragma unroll
            for (int h = 0; h < T; ++h)
                if (j + T + h < ntiles)
                    store_tile<D, W, FP8, true>(lds + nxt + h * BB, lds + nxt + h * BB + TB,
                                          reinterpret_cast<float*>(lds + nxt + h * BB + TB + TBV), pc[h], j + T + h, L, vlo,
                                          tid);
        }
        __syncthreads();
    }

    // epilogue: lane holds head_dim 32 mb + 8 q + 4h + e of row n (e < 4)
    {
        float a0, a1;
        swap_pair(s.l, true, a0, a1);
        float lt = a0 + a1;
        const int row = lane & 31, hh = lane >> 5;
        const int t = row / a.G, hl = row - t * a.G;
        const int pos = pw + t;
        if (t < a.P && pos < n) {
            const int h = g * a.G + hl;
            if (a.sinks) {
                const float sk = a.sinks[(int64_t)h * a.sinks_s] * kLog2e;
                if (sk > -__builtin_inff()) lt += __builtin_amdgcn_exp2f(sk - s.m);
            }
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
            char* orow = a.out + (int64_t)(c0 + pos) * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x2 wv = {pack_bf16_rne(s.o[mb][4 * q] * inv, s.o[mb][4 * q + 1] * inv),
                                      pack_bf16_rne(s.o[mb][4 * q + 2] * inv, s.o[mb][4 * q + 3] * inv)};
                    *reinterpret_cast<u32x2*>(orow + 2 * (32 * mb + 8 * q + 4 * hh)) = wv;
                }
        }
    }
}


struct PrefillShape {
    int nt, waves;
};

// 32 rows per wave in 8-wave workgroups (under 256 registers: two waves per
// SIMD, so one wave's softmax arithmetic can overlap the other's matrix
// work; 64 rows in 4-wave workgroups measured 1.4x slower, one wave per
// SIMD with its accumulators in AGPRs).  Ratios G > 32 need 64-row waves.
PrefillShape prefill_shape(int D, int G) {
    // head_dim 256: one 16-row tile per wave (a 256-wide step's fragments
    // and accumulators leave no room for a second), G <= 16
    if (D == 256) return {1, 8};
    if (G > 32) return {4, 4};
    return {2, 8};
}

template <int D, bool FP8>
const void* prefill_kernel_of_d(PrefillShape sh) {
    if (sh.nt == 4) return reinterpret_cast<const void*>(&prefill_kernel<D, 4, 4, FP8>);
    return reinterpret_cast<const void*>(&prefill_kernel32<D, 8, FP8>);
}

template <bool FP8>
const void* prefill_kernel_of_f(int D, PrefillShape sh) {
    if (D == 256) return reinterpret_cast<const void*>(&prefill_kernel<256, 1, 8, FP8>);
    return D == 128 ? prefill_kernel_of_d<128, FP8>(sh) : prefill_kernel_of_d<64, FP8>(sh);
}

const void* prefill_kernel_of(int D, bool fp8, PrefillShape sh) {
    return fp8 ? prefill_kernel_of_f<true>(D, sh) : prefill_kernel_of_f<false>(D, sh);
}

}  // namespace
}  // namespace pa

extern "C" {

int paged_attn_prefill_ext(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                           const pa_tensor* block_tables, const pa_tensor* context_lens,
                           const pa_tensor* cu_seqlens_q, int32_t max_query_len, float scale,
                           const pa_tensor* k_scale, const pa_tensor* v_scale, int32_t sliding_window,
                           const pa_tensor* sinks, pa_tensor* out, void* stream) {
    using namespace pa;
    PrefillProblem p;
    int st = validate_prefill(q, k_cache, v_cache, block_tables, context_lens, cu_seqlens_q, max_query_len, scale,
                              k_scale, v_scale, sliding_window, sinks, out, &p);
    if (st) return st;
    if (p.B == 0 || p.T == 0 || max_query_len == 0) return PA_OK;
    PrefillArgs a;
    a.q = static_cast<const char*>(p.q); a.q_st = p.q_st; a.q_sh = p.q_sh;
    a.out = static_cast<char*>(p.out); a.o_st = p.o_st; a.o_sh = p.o_sh;
    a.k = static_cast<const char*>(p.k); a.k_stok = p.k_stok; a.k_sh = p.k_sh;
    a.v = static_cast<const char*>(p.v); a.v_stok = p.v_stok; a.v_sh = p.v_sh;
    a.k_sblk = (uint32_t)p.k_sblk; a.v_sblk = (uint32_t)p.v_sblk;
    a.k_ssub = (uint32_t)(PA_BLOCK_SIZE * p.k_stok); a.v_ssub = (uint32_t)(PA_BLOCK_SIZE * p.v_stok);
    a.bt = p.bt; a.bt_sb = p.bt_sb;
    a.ctx = p.ctx; a.ctx_s = p.ctx_s;
    a.cu = p.cu; a.cu_s = p.cu_s;
    // kept positive so that a masked score's -inf times it stays -inf (a zero
    // scale becomes a negligible one: every score then weighs the same)
    a.scale_log2 = std::max(std::fabs(p.scale) * kLog2e, 1e-30f);
    a.q_neg = p.scale < 0.f;
    const int64_t eb = p.fp8 ? 1 : 2;                 // bytes per cache element
    a.k_span = (int32_t)(15 * p.k_stok + eb * p.D);
    a.v_span = (int32_t)(15 * p.v_stok + eb * p.D);
    a.ks = reinterpret_cast<const char*>(p.ks);
    a.vs = reinterpret_cast<const char*>(p.vs);
    a.ks_sblk = (uint32_t)(4 * p.ks_sblk); a.vs_sblk = (uint32_t)(4 * p.vs_sblk);
    a.ks_sh = (uint32_t)(4 * p.ks_sh); a.vs_sh = (uint32_t)(4 * p.vs_sh);
    a.B = (int32_t)p.B; a.Hkv = (int32_t)p.Hkv; a.G = (int32_t)p.G;
    // rows per wave and waves per workgroup (see prefill_shape)
    const PrefillShape sh = prefill_shape((int)p.D, (int)p.G);
    a.P = (int32_t)(16 * sh.nt / p.G);
    a.qblocks = (int32_t)((max_query_len + sh.waves * a.P - 1) / (sh.waves * a.P));
    a.bsub = (int32_t)(p.BS / PA_BLOCK_SIZE);
    a.wsub = (int32_t)(p.W * a.bsub);
    a.NB = (int32_t)std::min<int64_t>(p.NB, INT32_MAX);
    a.T = (int32_t)p.T;
    a.window = p.window;
    a.sinks = p.sinks; a.sinks_s = p.sinks_s;
    const int64_t grid = (int64_t)a.qblocks * p.B * p.Hkv;
    if (grid >= (int64_t(1) << 31)) return fail(PA_ERR_UNSUPPORTED, "prefill: grid too large");
    const void* fn = prefill_kernel_of((int)p.D, p.fp8, sh);
    // LDS: two groups of T tile buffers (the 32-row kernel's buffers are laid
    // out for its own reads)
    const bool r32 = sh.nt == 2 && p.D <= 128;
    size_t buf, tpb;
    if (p.D == 256) {
        buf = p.fp8 ? kBufBytes<256, true> : kBufBytes<256, false>;
        tpb = kTilesPerBarrier<256, 1>;
    } else if (p.D == 128) {
        buf = r32 ? (p.fp8 ? kBufBytes<128, true, true> : kBufBytes<128, false, true>)
                  : (p.fp8 ? kBufBytes<128, true> : kBufBytes<128, false>);
        tpb = sh.nt == 4 ? kTilesPerBarrier<128, 4> : kTilesPerBarrier<128, 2>;
    } else {
        buf = r32 ? (p.fp8 ? kBufBytes<64, true, true> : kBufBytes<64, false, true>)
                  : (p.fp8 ? kBufBytes<64, true> : kBufBytes<64, false>);
        tpb = kTilesPerBarrier<64, 2>;
    }
    const size_t lds = 2 * tpb * buf;
    void* args[] = {&a};
    if (hipLaunchKernel(fn, dim3((unsigned)grid), dim3(64 * sh.waves), args, lds,
                        static_cast<hipStream_t>(stream)) != hipSuccess)
        return fail(PA_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(hipGetLastError()));
    return PA_OK;
}

int paged_attn_prefill(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                       const pa_tensor* block_tables, const pa_tensor* context_lens,
                       const pa_tensor* cu_seqlens_q, int32_t max_query_len, float scale,
                       const pa_tensor* k_scale, const pa_tensor* v_scale, pa_tensor* out, void* stream) {
    return paged_attn_prefill_ext(q, k_cache, v_cache, block_tables, context_lens, cu_seqlens_q, max_query_len,
                                  scale, k_scale, v_scale, 0, nullptr, out, stream);
}


}  // extern "C"
