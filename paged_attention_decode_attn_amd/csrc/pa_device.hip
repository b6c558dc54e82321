// HIP half of the library for gfx950 (CDNA4): the split-context partition
// kernel, the log-sum-exp merge kernel, the per-stream workspace and the
// paged_attn_decode entry point.
//
// Method (ROCm blog "Optimizing ATOM and vLLM-ATOM for High-Interactivity
// Inference", "Attention Decode: Split Memory Work to Fill the Device"):
// decode attention is a memory-bound, single-query operation, so the KV
// range of every (sequence, kv head) pair is split into partitions that run
// as separate workgroups; each keeps an online-softmax state and writes its
// partial output plus a float32 log-sum-exp, and a second kernel merges the
// partitions.  The partition size is chosen from shapes and the CU count
// (pa_host.cpp), never from device data.
//
// Partition kernel: a persistent grid of at most one workgroup per resident
// slot.  The chunks (32-token pieces) of every (sequence, kv-head group)
// segment are numbered sequence-major and split into even shares, one per
// workgroup, so every workgroup streams the same number of chunks to within
// one whatever the ragged context lengths; a share may start or end inside
// a segment.  A workgroup is HG waves, wave v serving kv head gg*HG + v of
// each segment it meets, so a CU reads adjacent head rows of the same
// tokens (at head_dim 256, P waves per kv head, one per 16-row tile).  A
// segment wholly inside one share writes its output rows; a split one
// leaves an fp32 partial and a base-2 log-sum-exp per row.
//  * All G*Qmax query rows that share kv head g form the N side of 16x16
//    MFMA tiles (rows r = t*G + h_local; tiles of 16 rows), so every K/V
//    byte is read from HBM once per kv head (at head_dim 256 with more than
//    16 rows, once per tile from the CU's caches).
//  * A wave walks its piece of a segment in 32-token steps (two 16-token
//    sub-blocks) through a ring of register buffers: raw buffer loads of
//    the next steps are in flight while the current one computes; loads
//    past the sequence or below a sliding window go through an empty
//    range, so the code between a load and its use is straight-line.
//  * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: sub-block mt of the step is
//    the M side (token slot = lane % 16), head_dim the reduction.  Each lane
//    then holds 8 scores of one query row.
//  * O^T += V^T P^T with the same MFMA: head_dim is the M side, the 32
//    tokens the reduction, P (bf16) the N side.  The lane's 8 probabilities
//    are already in B-operand order; V^T is formed in registers from 16-byte
//    row loads by lane permutes (bf16) or by the fp8->bf16 conversions,
//    which place the bytes as the operand needs them.  The output tile puts
//    a query row's accumulators in the same lanes as that row's softmax
//    state, so rescaling needs no cross-lane traffic.
//  * fp8 e4m3fn K/V are widened exactly to bf16 in registers; the
//    per-(token, kv head) scales fold into the score column (k) and the
//    probability (v) instead of multiplying every element.
//  * Row max uses two cross-lane exchanges per step; row sums stay
//    lane-partial until the epilogue.
//  * Positions >= L_b, causally hidden keys and keys below a sliding
//    window get score -inf by selection; V rows and scales past L_b or below
//    every row's window are zeroed, so NaN or garbage in unread cache slots
//    never reaches the output.
//  * A cache block of BS = 16m tokens is m contiguous 16-token sub-blocks;
//    the kernel addresses sub-blocks (block-table entry i / m, sub-block
//    i % m), so every block size runs the same 16-token code.
//  * A sliding window only narrows a sequence's chunk range and adds a
//    lower mask bound; attention sinks (one logit per query head) join the
//    softmax normaliser in the epilogue or the merge.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr unsigned kSelLo = 0x05040100u;   // v_perm: (src1.lo16, src0.lo16)
constexpr unsigned kSelHi = 0x07060302u;   // v_perm: (src1.hi16, src0.hi16)
constexpr unsigned kSelByte01 = 0x05010400u;  // v_perm: src1.b0, src0.b0, src1.b1, src0.b1
constexpr unsigned kSelByte23 = 0x07030602u;  // v_perm: src1.b2, src0.b2, src1.b3, src0.b3
constexpr int kRsrcWord3 = 0x00020000;        // raw buffer resource, 32-bit data format
constexpr float kRescaleLog2 = 8.0f;          // lazy rescale threshold (log2 units)
constexpr int kChunkTokens = 32;              // tokens per step (two 16-token blocks)
constexpr int kWindowChunks = 32;             // chunks per 64-entry block-table window
constexpr int kLockstep = 4;                  // steps between workgroup barriers (power of 2)

typedef __amdgpu_buffer_rsrc_t Rsrc;

struct PartArgs {
    const char* q;   int64_t q_sb, q_st, q_sh;        // bytes
    const char* k;   int64_t k_stok, k_sh;            // bytes
    const char* v;   int64_t v_stok, v_sh;            // bytes
    const float* ks; int64_t ks_sh;                   // floats
    const float* vs; int64_t vs_sh;
    uint32_t k_sblk, v_sblk, ks_sblk, vs_sblk;        // block strides, bytes (< 2^32)
    uint32_t k_ssub, v_ssub;                          // bytes between 16-token sub-blocks of a block
    const int32_t* bt; int64_t bt_sb;
    const int32_t* ctx; int64_t ctx_s;
    const int32_t* ql;  int64_t ql_s;
    const float* sinks; int64_t sinks_s;              // per query head, may be null
    char* out;       int64_t o_sb, o_st, o_sh;        // bytes
    float* ws_o;     float* ws_lse;                   // partial results: 2 slots per (workgroup, wave, row)
    int32_t* ws_pre;                                  // chunk prefix per sequence, for the merge (may be null)
    float scale_log2;                                 // |scale| * log2(e)
    int32_t q_neg;                                    // scale < 0: negate q
    int32_t k_span, v_span;                           // bytes of one (16-token sub-block, head) slice
    int32_t bsub;                                     // 16-token sub-blocks per cache block
    int32_t wsub;                                     // sub-blocks a table row reaches (W * bsub)
    int32_t window;                                   // sliding window in tokens, 0 = none
    int32_t B, Hq, Hkv, G, Qmax, NB, rows, HG, min_share;
    int32_t whole;                                    // 1: workgroup w runs segment w whole
    int32_t P;                                        // waves per kv head (16-row tiles; head_dim 256)
};

struct RedArgs {
    const float* ws_o; const float* ws_lse; const int32_t* ws_pre;
    const int32_t* ql;  int64_t ql_s;
    const float* sinks; int64_t sinks_s;              // per query head, may be null
    char* out;       int64_t o_sb, o_st, o_sh;        // bytes
    int32_t B, Hq, Hkv, G, Qmax, rows, HG, grid, min_share;
    int32_t red_rows, red_col4, red_lanes;            // merge workgroup shape (see reduce_kernel)
    int32_t spec;                                     // 1: one sequence, grid a multiple of the head groups
};

template <typename T>
__device__ __forceinline__ T ldg(const char* p) {
    return *reinterpret_cast<const T*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ unsigned pack_bf16_rne(float a, float b) {
    f32x2 f = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

// Per-step register tiles.  KL: 16-byte K loads per lane and block;
// V: one load of D/16 elements per lane and token slot.
template <int D, bool FP8> struct VLoad;
template <> struct VLoad<256, false> { typedef u32x8 T; };
template <> struct VLoad<256, true>  { typedef u32x4 T; };
template <> struct VLoad<128, false> { typedef u32x4 T; };
template <> struct VLoad<64, false>  { typedef u32x2 T; };
template <> struct VLoad<128, true>  { typedef u32x2 T; };
template <> struct VLoad<64, true>   { typedef unsigned T; };

// fp8 with head_dim 64: a lane's piece of a V row is only 4 bytes, so V and
// the scales travel in 16-byte loads shared by each quad of lanes and are
// spread over the quad in registers (unpack_quad): 5 load instructions per
// step instead of 14.
template <int D, bool FP8> constexpr bool kQuadV = FP8 && D == 64;

template <int D, bool FP8> struct Step {
    static constexpr int KL = FP8 ? D / 64 : D / 32;
    u32x4 k[2][KL];
    typename VLoad<D, FP8>::T v[8];
    f32x4 ksc[2], vsc[2];
    u32x4 vq[2];     // kQuadV: 16-byte V pieces of blocks 0 and 1
    u32x4 sq;        // kQuadV: one 16-byte piece of the step's scales
};

template <int D, bool FP8, int NT> struct State {
    float m[NT], l[NT];
    f32x4 acc[NT][D / 16];
};

// Buffer resource over one (block, kv head) slice: the base is wave-uniform
// and lives in SGPRs, the lane offsets are loop-invariant VGPRs, and the
// range check returns zeros (without a memory access) for offsets past
// `bytes`, so a block that lies past the sequence costs no traffic.
__device__ __forceinline__ Rsrc make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}
template <typename T> __device__ __forceinline__ T bload(Rsrc r, unsigned off);
template <> __device__ __forceinline__ u32x4 bload<u32x4>(Rsrc r, unsigned off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
template <> __device__ __forceinline__ u32x8 bload<u32x8>(Rsrc r, unsigned off) {
    const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16u, 0, 0);
    return u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
template <> __device__ __forceinline__ u32x2 bload<u32x2>(Rsrc r, unsigned off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
template <> __device__ __forceinline__ unsigned bload<unsigned>(Rsrc r, unsigned off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// Per-item bases: the kv head's slice of block 0 of each cache array.
struct HeadBase {
    const char* k; const char* v; const char* ks; const char* vs;
};

// A lane's block-table window entry: the cache block and the 16-token
// sub-block within it of sub-block 2*pc + lane of the sequence.
struct BlockRef {
    int blk, sub;
};

// GEN: the general variant (cache blocks of more than 16 tokens, a sliding
// window, attention sinks); without it blocks are 16 tokens, there is no
// window and no sink, and none of their code is emitted.
template <int D, bool FP8, bool GEN>
__device__ __forceinline__ void load_step(Step<D, FP8>& st, const PartArgs& a, const HeadBase& hb, BlockRef br,
                                          int step, int nsteps, int hi_key, int lo_key,
                                          const unsigned (&koff)[Step<D, FP8>::KL], const unsigned (&voff)[4],
                                          unsigned soff) {
    typedef typename VLoad<D, FP8>::T VT;
    constexpr int KL = Step<D, FP8>::KL;
    // hi_key: the keys of the sequence, counted from the piece's first token;
    // lo_key: with a sliding window, the first key that some row sees,
    // counted the same way.  For step < nsteps, sub-block 2*step holds keys
    // of the sequence and sub-block 2*step + 1 may lie past it; a sub-block
    // past the sequence, a whole step past the window (a prefetch beyond its
    // end) or a sub-block wholly below lo_key reads as zeros through an empty
    // range, which costs no memory traffic.
    const int last_blk = ((hi_key + 15) >> 4) - 1;
    const int lo_blk = lo_key >> 4;
    const bool in = step < nsteps;
    const bool has0 = in && (!GEN || 2 * step >= lo_blk);
    const bool has1 = in && 2 * step + 1 <= last_blk && (!GEN || 2 * step + 1 >= lo_blk);
    const int sc = min(step, nsteps - 1);
    const int l0 = 2 * sc, l1 = min(2 * sc + 1, last_blk);
    const uint32_t u0 = (uint32_t)__builtin_amdgcn_readlane(br.blk, l0);
    const uint32_t u1 = (uint32_t)__builtin_amdgcn_readlane(br.blk, l1);
    const uint32_t s0 = GEN ? (uint32_t)__builtin_amdgcn_readlane(br.sub, l0) : 0u;
    const uint32_t s1 = GEN ? (uint32_t)__builtin_amdgcn_readlane(br.sub, l1) : 0u;
    const Rsrc k0 = make_rsrc(hb.k + (uint64_t)u0 * a.k_sblk + s0 * a.k_ssub, has0 ? a.k_span : 0);
    const Rsrc k1 = make_rsrc(hb.k + (uint64_t)u1 * a.k_sblk + s1 * a.k_ssub, has1 ? a.k_span : 0);
    const Rsrc v0 = make_rsrc(hb.v + (uint64_t)u0 * a.v_sblk + s0 * a.v_ssub, has0 ? a.v_span : 0);
    const Rsrc v1 = make_rsrc(hb.v + (uint64_t)u1 * a.v_sblk + s1 * a.v_ssub, has1 ? a.v_span : 0);
    // In the step holding lo_key, the K and V rows of lanes whose token lies
    // below it are skipped too (an offset past every range reads zeros
    // without a memory access), so a window is read from its first token,
    // not from the start of its first sub-block.  Lane tokens: K 16*mt + n16;
    // V 16*(s/4) + 4*grp + s%4 (with quad-shared V, 16*mt + 4*grp + n16%4).
    unsigned ko[2][KL], vo[8];
#pragma unroll
    for (int c = 0; c < KL; ++c) ko[0][c] = ko[1][c] = koff[c];
#pragma unroll
    for (int i = 0; i < 8; ++i) vo[i] = voff[kQuadV<D, FP8> ? 0 : (i & 3)];
    if constexpr (GEN) {
        const int lo = lo_key - kChunkTokens * step;
        if (lo > 0) {
            const int n16 = __lane_id() & 15, grp = __lane_id() >> 4;
            constexpr unsigned kNoRead = 0x80000000u;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                if (16 * mt + n16 < lo) {
#pragma unroll
                    for (int c = 0; c < KL; ++c) ko[mt][c] = kNoRead;
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int tok = kQuadV<D, FP8> ? 16 * (i & 1) + 4 * grp + (n16 & 3) : 16 * (i >> 2) + 4 * grp + (i & 3);
                if (tok < lo) vo[i] = kNoRead;
            }
        }
    }
#pragma unroll
    for (int c = 0; c < KL; ++c) {
        st.k[0][c] = bload<u32x4>(k0, ko[0][c]);
        st.k[1][c] = bload<u32x4>(k1, ko[1][c]);
    }
    if constexpr (kQuadV<D, FP8>) {
        // lane (n16 = 4q + r, grp): bytes 16q..16q+15 of slot 4grp + r of
        // each block, and one scale piece: quad position r picks k scales of
        // block 0 or 1 or v scales of block 0 or 1, slots 4grp..4grp+3 (the
        // block ids are valid pool blocks, so the plain load stays in bounds;
        // scales of positions past L are zeroed before use)
        st.vq[0] = bload<u32x4>(v0, vo[0]);
        st.vq[1] = bload<u32x4>(v1, vo[1]);
        const int r = __lane_id() & 3;
        const char* base = (r & 2) ? hb.vs : hb.ks;
        const uint64_t sblk = (r & 2) ? a.vs_sblk : a.ks_sblk;
        // a sub-block's 16 slot scales are 64 contiguous bytes
        st.sq = *reinterpret_cast<const u32x4*>(base + (uint64_t)((r & 1) ? u1 : u0) * sblk +
                                                 64u * ((r & 1) ? s1 : s0) + soff);
        return;
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) st.v[s] = bload<VT>(s < 4 ? v0 : v1, vo[s]);
    if constexpr (FP8) {
        // one block's 16 slot scales of this kv head are contiguous (64 bytes)
        const Rsrc ks0 = make_rsrc(hb.ks + (uint64_t)u0 * a.ks_sblk + 64u * s0, has0 ? 64 : 0);
        const Rsrc ks1 = make_rsrc(hb.ks + (uint64_t)u1 * a.ks_sblk + 64u * s1, has1 ? 64 : 0);
        const Rsrc vs0 = make_rsrc(hb.vs + (uint64_t)u0 * a.vs_sblk + 64u * s0, has0 ? 64 : 0);
        const Rsrc vs1 = make_rsrc(hb.vs + (uint64_t)u1 * a.vs_sblk + 64u * s1, has1 ? 64 : 0);
        st.ksc[0] = __builtin_bit_cast(f32x4, bload<u32x4>(ks0, soff));
        st.ksc[1] = __builtin_bit_cast(f32x4, bload<u32x4>(ks1, soff));
        st.vsc[0] = __builtin_bit_cast(f32x4, bload<u32x4>(vs0, soff));
        st.vsc[1] = __builtin_bit_cast(f32x4, bload<u32x4>(vs1, soff));
    }
}

// DPP quad permutations (lane i of each quad reads lane sel[i]).
template <int CTRL>
__device__ __forceinline__ unsigned quad_perm(unsigned x) {
    return (unsigned)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, false);
}
constexpr int kQuadXor2 = 0x4E;      // [2, 3, 0, 1]
constexpr int kQuadXor1 = 0xB1;      // [1, 0, 3, 2]

// 4x4 transpose of dwords within each quad of lanes: dword k of quad lane r
// becomes dword r of quad lane k.  Two exchange rounds (partner r^2 swaps
// dword pairs, partner r^1 swaps single dwords).
__device__ __forceinline__ u32x4 quad_transpose(u32x4 m, int r) {
    const bool hi = r & 2, odd = r & 1;
    unsigned x0 = hi ? m[0] : m[2], x1 = hi ? m[1] : m[3];
    x0 = quad_perm<kQuadXor2>(x0);
    x1 = quad_perm<kQuadXor2>(x1);
    m[0] = hi ? x0 : m[0]; m[1] = hi ? x1 : m[1];
    m[2] = hi ? m[2] : x0; m[3] = hi ? m[3] : x1;
    x0 = odd ? m[0] : m[1];
    x1 = odd ? m[2] : m[3];
    x0 = quad_perm<kQuadXor1>(x0);
    x1 = quad_perm<kQuadXor1>(x1);
    m[0] = odd ? x0 : m[0]; m[2] = odd ? x1 : m[2];
    m[1] = odd ? m[1] : x0; m[3] = odd ? m[3] : x1;
    return m;
}

// kQuadV: spread the quad-shared loads into the per-lane layout of the other
// variants: v[i] = 4 bytes (d = 4*n16 ..) of this lane's token slot i, and
// the k/v scales of its 4 slots in each block.
template <int D, bool FP8>
__device__ __forceinline__ void unpack_quad(Step<D, FP8>& st, int lane) {
    const int r = lane & 3;
    const u32x4 t0 = quad_transpose(st.vq[0], r);
    const u32x4 t1 = quad_transpose(st.vq[1], r);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        st.v[i] = t0[i];
        st.v[4 + i] = t1[i];
        st.ksc[0][i] = __builtin_bit_cast(float, quad_perm<0x00>(st.sq[i]));
        st.ksc[1][i] = __builtin_bit_cast(float, quad_perm<0x55>(st.sq[i]));
        st.vsc[0][i] = __builtin_bit_cast(float, quad_perm<0xAA>(st.sq[i]));
        st.vsc[1][i] = __builtin_bit_cast(float, quad_perm<0xFF>(st.sq[i]));
    }
}

// Two e4m3fn bytes (bytes 0-1, or 2-3 with HI, of `w`) -> packed bf16 pair, exact:
// every e4m3fn value, subnormals included, is a bf16 value.
template <bool HI>
__device__ __forceinline__ unsigned fp8x2_to_bf16x2(unsigned w) {
    return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// V^T fragment of output tile j: element s = V[token slot s][d = (D/16)*m + j]
// for this lane's m = lane % 16, packed as bf16 pairs (s, s+1).  bf16: the
// pair is two half-words of the row loads, one v_perm each.
template <int D>
__device__ __forceinline__ bf16x8 vt_bf16(const typename VLoad<D, false>::T (&v)[8], int j) {
    u32x4 x;
#pragma unroll
    for (int p = 0; p < 4; ++p)
        x[p] = __builtin_amdgcn_perm(v[2 * p + 1][j / 2], v[2 * p][j / 2], (j & 1) ? kSelHi : kSelLo);
    return as_bf16x8(x);
}

// fp8: the same fragments for every tile at once.  A byte permute
// interleaves slots 2p and 2p+1 (bytes e of both words side by side), and
// each half of the result widens to the bf16 pair of d-index 4*dw + e.
template <int D>
__device__ __forceinline__ void vt_fp8(const typename VLoad<D, true>::T (&v)[8], u32x4 (&vt)[D / 16]) {
    constexpr int J = D / 16;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
#pragma unroll
        for (int dw = 0; dw < J / 4; ++dw) {
            unsigned w0, w1;
            if constexpr (J == 4) { w0 = v[2 * p]; w1 = v[2 * p + 1]; }
            else { w0 = v[2 * p][dw]; w1 = v[2 * p + 1][dw]; }
            const unsigned lo = __builtin_amdgcn_perm(w1, w0, kSelByte01);
            const unsigned hi = __builtin_amdgcn_perm(w1, w0, kSelByte23);
            vt[4 * dw + 0][p] = fp8x2_to_bf16x2<false>(lo);
            vt[4 * dw + 1][p] = fp8x2_to_bf16x2<true>(lo);
            vt[4 * dw + 2][p] = fp8x2_to_bf16x2<false>(hi);
            vt[4 * dw + 3][p] = fp8x2_to_bf16x2<true>(hi);
        }
    }
}

// fp8 K fragments (A operand of S^T) of block mt, widened to bf16 once for
// every row tile.  (A bf16 load is its own fragment and goes to the matrix
// unit as loaded: copying it into a fragment array first made the compiler
// keep part of the register ring in scratch memory for one variant.)
template <int D>
__device__ __forceinline__ void build_kf(const Step<D, true>& st, bf16x8 (&kf)[2][D / 32]) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        // load c holds bytes e = 0..15 of d = (D/4)*grp + 16c + e; MFMA
        // step kk = 2c + h takes bytes 8h .. 8h+7, i.e. the adjacent-d
        // pairs of two words
#pragma unroll
        for (int c = 0; c < D / 64; ++c) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                u32x4 x;
#pragma unroll
                for (int p2 = 0; p2 < 2; ++p2) {
                    const unsigned word = st.k[mt][c][2 * h + p2];
                    x[2 * p2] = fp8x2_to_bf16x2<false>(word);
                    x[2 * p2 + 1] = fp8x2_to_bf16x2<true>(word);
                }
                kf[mt][2 * c + h] = as_bf16x8(x);
            }
        }
    }
}

// One 32-token step of the online softmax for every row tile.  MASK: some
// key of the step is past L or causally hidden from some row (only the
// last steps of a partition); without it no mask code is emitted.
//
// Scores stay unscaled (y = q.k, times the fp8 k scale) until the
// exponent, p = exp2(c*y - m) with c = |scale|*log2(e) >= 0 (a negative
// scale flips the sign of q instead), so the row max of c*y is c times the
// max of y.  The running max m is raised only when a row's max exceeds it by
// more than kRescaleLog2 (any row of the wave: the branch is uniform);
// otherwise p <= 2^kRescaleLog2 and l and the accumulators keep their scale.
// The result is the same: m, l and O all refer to one m.
template <int D, bool FP8, int NT, bool MASK, bool GEN>
__device__ __forceinline__ void compute_step(Step<D, FP8>& st, State<D, FP8, NT>& s, const u32x4 (&qf)[NT][D / 32],
                                             const PartArgs& a, int cbase, int L, int nq, int vlo, int lane,
                                             int r0) {
    constexpr int J = D / 16;
    const int n16 = lane & 15, grp = lane >> 4;
    if constexpr (kQuadV<D, FP8>) unpack_quad<D, FP8>(st, lane);

    if constexpr (MASK) {
        // zero V rows (and scales) of positions >= L or below every row's
        // window (vlo) so that p = 0 never meets NaN or garbage from
        // unwritten or recycled slots
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int tok = cbase + 16 * (i >> 2) + 4 * grp + (i & 3);
            if (tok >= L || (GEN && tok < vlo)) {
                st.v[i] = typename VLoad<D, FP8>::T{};
                if constexpr (FP8) {
                    st.vsc[i >> 2][i & 3] = 0.f;
                    st.ksc[i >> 2][i & 3] = 0.f;
                }
            }
        }
    }

    bf16x8 kf[2][D / 32];
    if constexpr (FP8) build_kf<D>(st, kf);
    u32x4 vtf[FP8 ? J : 1];
    if constexpr (FP8) vt_fp8<D>(st.v, vtf);
    const float c = a.scale_log2;

#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            const bf16x8 qb = as_bf16x8(qf[nt][kk]);
            bf16x8 k0, k1;
            if constexpr (FP8) {
                k0 = kf[0][kk];
                k1 = kf[1][kk];
            } else {
                k0 = as_bf16x8(st.k[0][kk]);
                k1 = as_bf16x8(st.k[1][kk]);
            }
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qb, s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qb, s1, 0, 0, 0);
        }
        float y[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (FP8) {
                y[i] = s0[i] * st.ksc[0][i];
                y[4 + i] = s1[i] * st.ksc[1][i];
            } else {
                y[i] = s0[i];
                y[4 + i] = s1[i];
            }
        }
        bool hidden[8];
        if constexpr (MASK) {
            // row t sees keys lo .. lim: its causal limit and, with a
            // sliding window, the window's first position
            const int row = r0 + 16 * nt + n16;
            const int t = row / a.G;
            const int lim = (row < a.rows && t < nq) ? L - nq + t : L - 1;
            const int lo = GEN && a.window > 0 ? lim - a.window + 1 : 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int tok = cbase + 16 * (i >> 2) + 4 * grp + (i & 3);
                hidden[i] = tok > lim || (GEN && tok < lo);
                y[i] = hidden[i] ? -__builtin_inff() : y[i];
            }
        }
        float mx = fmaxf(fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3])), fmaxf(fmaxf(y[4], y[5]), fmaxf(y[6], y[7])));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        float mxs = c * mx;
        if constexpr (MASK) mxs = mx == -__builtin_inff() ? -__builtin_inff() : mxs;
        if (__any(mxs > s.m[nt] + kRescaleLog2)) {
            const float m_new = fmaxf(s.m[nt], mxs);
            const float alpha = m_new == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(s.m[nt] - m_new);
            s.l[nt] *= alpha;
#pragma unroll
            for (int j = 0; j < J; ++j) s.acc[nt][j] *= alpha;
            s.m[nt] = m_new;
        }
        const float neg_m = s.m[nt] == -__builtin_inff() ? 0.f : -s.m[nt];
        float p[8];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(y[i], c, neg_m));
            if constexpr (MASK) p[i] = hidden[i] ? 0.f : p[i];
            psum += p[i];
        }
        s.l[nt] += psum;
        if constexpr (FP8) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] *= st.vsc[0][i];
                p[4 + i] *= st.vsc[1][i];
            }
        }
        u32x4 pw;
#pragma unroll
        for (int w = 0; w < 4; ++w) pw[w] = pack_bf16_rne(p[2 * w], p[2 * w + 1]);
        const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
        for (int j = 0; j < J; ++j) {
            bf16x8 vt;
            if constexpr (FP8) vt = as_bf16x8(vtf[j]);
            else vt = vt_bf16<D>(st.v, j);
            s.acc[nt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pb, s.acc[nt][j], 0, 0, 0);
        }
    }
}

// Block-table window of a piece: sub-block 2*pc + lane of sequence b
// (clamped to the table's reach), its block id clamped into the pool.
template <bool GEN>
__device__ __forceinline__ BlockRef load_window(const PartArgs& a, int b, int pc, int lane) {
    const int idx = min(2 * pc + lane, a.wsub - 1);
    const int e = GEN && a.bsub > 1 ? idx / a.bsub : idx;
    const int v = a.bt[(int64_t)b * a.bt_sb + e];
    return BlockRef{min(max(v, 0), a.NB - 1), idx - e * (GEN ? a.bsub : 1)};
}

// First 32-token chunk of sequence b that a query row can see: 0, or with
// a sliding window the chunk of the earliest row's first key.
template <bool GEN>
__device__ __forceinline__ int first_chunk(const PartArgs& a, int L, int nq) {
    return GEN && a.window > 0 ? max(0, L - nq - a.window + 1) / kChunkTokens : 0;
}

// Query head h's sink logit in log2 units (log2(e) * sink), or -inf.
__device__ __forceinline__ float sink_log2(const float* sinks, int64_t stride, int h) {
    return sinks ? sinks[(int64_t)h * stride] * kLog2e : -__builtin_inff();
}

// One segment = chunks [c0, c1) of the cb chunks (32 tokens each) that
// sequence b's rows see, for kv head g, run by one wave of workgroup w
// (chunk c is the sequence's chunk first_chunk + c).  The segment's
// online-softmax state ends as the output row when the segment is the whole
// sequence, otherwise as a normalised fp32 partial output and its base-2
// log-sum-exp in the workgroup's partial slot `slot` (0: the first segment
// of its share, 1: the last) for the merge kernel.  Chunks are processed in
// pieces of up to 32 (one 64-entry block-table window per piece).
template <int D, bool FP8, int NT, bool GEN>
__device__ __forceinline__ void process_segment(const PartArgs& a, int b, int g, int wave, int c0, int c1, int cb,
                                                int w, int slot, int lane, int r0) {
    constexpr int J = D / 16;
    constexpr int KL = Step<D, FP8>::KL;
    constexpr int E = FP8 ? 1 : 2;
    // register buffers: loads of R-1 steps ahead in flight (head_dim 256:
    // one buffer, its bf16 step alone is 128 registers; the CU's other
    // waves keep the loads flowing)
    constexpr int R = (NT > 2 || D > 128) ? 1 : 2;
    const int n16 = lane & 15, grp = lane >> 4;

    // Start-up loads issued together: the first block-table window, the
    // query fragments and the lengths do not depend on each other, so the
    // first K/V loads wait for one round trip only (with a sliding window the
    // window's first chunk waits for the lengths).
    const bool direct = c0 == 0 && c1 == cb;
    if (GEN && a.window > 0) {
        const int L0 = min(a.ctx[(int64_t)b * a.ctx_s], 16 * a.wsub);
        const int nq0 = min(a.ql ? a.ql[(int64_t)b * a.ql_s] : a.Qmax, a.Qmax);
        const int cs = first_chunk<GEN>(a, L0, nq0);
        c0 += cs;
        c1 += cs;
    }
    BlockRef br = load_window<GEN>(a, b, c0, lane);
    // query fragments: row r = r0 + 16*nt + n16 -> (t, h_local) = (r / G,
    // r % G); rows t < Qmax are in bounds, rows past query_len are zeroed
    // below
    u32x4 qf[NT][D / 32];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int row = r0 + 16 * nt + n16;
        const int t = row / a.G, hl = row - t * a.G;
        const char* qrow = a.q + (int64_t)b * a.q_sb + (int64_t)t * a.q_st + (int64_t)(g * a.G + hl) * a.q_sh;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            const int d0 = FP8 ? (D / 4) * grp + 8 * kk : 32 * kk + 8 * grp;
            qf[nt][kk] = row < a.rows ? *reinterpret_cast<const u32x4*>(qrow + 2 * d0) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    const int L = min(a.ctx[(int64_t)b * a.ctx_s], 16 * a.wsub);
    const int nq = min(a.ql ? a.ql[(int64_t)b * a.ql_s] : a.Qmax, a.Qmax);
    // keys below vlo are outside every row's window
    const int vlo = GEN && a.window > 0 ? L - nq - a.window + 1 : 0;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int row = r0 + 16 * nt + n16;
        const bool live = row / a.G < nq;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
            qf[nt][kk] = live ? (a.q_neg ? qf[nt][kk] ^ 0x80008000u : qf[nt][kk]) : u32x4{0u, 0u, 0u, 0u};
    }

    HeadBase hb;
    hb.k = a.k + (int64_t)g * a.k_sh;
    hb.v = a.v + (int64_t)g * a.v_sh;
    hb.ks = reinterpret_cast<const char*>(a.ks + (int64_t)g * a.ks_sh);
    hb.vs = reinterpret_cast<const char*>(a.vs + (int64_t)g * a.vs_sh);
    unsigned koff[KL];
#pragma unroll
    for (int c = 0; c < KL; ++c)
        koff[c] = (unsigned)(n16 * a.k_stok) + (FP8 ? (unsigned)((D / 4) * grp + 16 * c) : (unsigned)((32 * c + 8 * grp) * 2));
    unsigned voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) voff[i] = (unsigned)((4 * grp + i) * a.v_stok) + (unsigned)((D / 16) * n16 * E);
    if constexpr (kQuadV<D, FP8>) voff[0] = (unsigned)((4 * grp + (n16 & 3)) * a.v_stok) + 16u * (unsigned)(n16 >> 2);
    const unsigned soff = 16u * (unsigned)grp;

    State<D, FP8, NT> s;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        s.m[nt] = -__builtin_inff();
        s.l[nt] = 0.f;
#pragma unroll
        for (int j = 0; j < J; ++j) s.acc[nt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int pc = c0; pc < c1; pc += kWindowChunks) {
        if (pc != c0) br = load_window<GEN>(a, b, pc, lane);
        const int tok0 = kChunkTokens * pc;
        const int nsteps = min(c1, pc + kWindowChunks) - pc;
        // steps [0, nclean) hold only keys below L that every query row
        // sees; with a sliding window every step takes the masked variant
        // (a window's range is short, and its first steps are masked anyway)
        const int nclean = GEN && a.window > 0 ? 0 : min(nsteps, max(0, L - nq + 1 - tok0) / kChunkTokens);
        // with a sliding window, the first key some row sees, counted from
        // the piece's first token
        const int lo_key = GEN && a.window > 0 ? vlo - tok0 : 0;
        // A ring of R register buffers: while a step computes, the loads of
        // the next R-1 steps are in flight.  Loads are issued on every path
        // (past the window they read nothing), so the code between a load
        // and its use is straight-line and the memory-counter waits exact;
        // the last steps of the piece take the masked variant.
        Step<D, FP8> buf[R];
#pragma unroll
        for (int i = 0; i + 1 < R; ++i) load_step<D, FP8, GEN>(buf[i], a, hb, br, i, nsteps, L - tok0, lo_key, koff, voff, soff);
        // Every kLockstep steps the workgroup's waves meet at a barrier.  Two
        // waves share each SIMD, and the older one otherwise wins the issue
        // and memory arbitration until it is done, leaving the younger to
        // finish alone; held within a few steps of each other, the waves
        // keep the CU's load pipeline full to the end of the share.  Every
        // wave of a workgroup runs the same chunks, so the barriers match.
        int st = 0;
        for (; st + R <= nclean; st += R) {
#pragma unroll
            for (int i = 0; i < R; ++i) {
                load_step<D, FP8, GEN>(buf[(i + R - 1) % R], a, hb, br, st + i + R - 1, nsteps, L - tok0, lo_key, koff, voff,
                                       soff);
                if (((st + i) & (kLockstep - 1)) == 0) __syncthreads();
                compute_step<D, FP8, NT, false, GEN>(buf[i], s, qf, a, tok0 + kChunkTokens * (st + i), L, nq, vlo, lane,
                                                     r0);
            }
        }
        for (; st < nsteps; st += R) {
#pragma unroll
            for (int i = 0; i < R; ++i) {
                load_step<D, FP8, GEN>(buf[(i + R - 1) % R], a, hb, br, st + i + R - 1, nsteps, L - tok0, lo_key, koff, voff,
                                       soff);
                if (st + i < nsteps)
                    compute_step<D, FP8, NT, true, GEN>(buf[i], s, qf, a, tok0 + kChunkTokens * (st + i), L, nq, vlo,
                                                        lane, r0);
            }
        }
    }

    // epilogue: lane holds d = (D/16)*(4*grp + i) + j, j < D/16, of row r0 + 16*nt + n16
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        float lt = s.l[nt];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        const int row = r0 + 16 * nt + n16;
        const int t = row / a.G, hl = row - t * a.G;
        if (!(row < a.rows && t < nq)) continue;
        const int h = g * a.G + hl;
        if (GEN && direct && a.sinks) {
            // the sink joins the normaliser: l += 2^(sink - m), m in log2 units
            const float sk = sink_log2(a.sinks, a.sinks_s, h);
            if (sk > -__builtin_inff()) lt += __builtin_amdgcn_exp2f(sk - s.m[nt]);
        }
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        if (direct) {
            char* orow = a.out + (int64_t)b * a.o_sb + (int64_t)t * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = J * (4 * grp + i);
                if constexpr (J >= 8) {
#pragma unroll
                    for (int h = 0; h < J / 8; ++h) {
                        u32x4 wv;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            wv[e] = pack_bf16_rne(s.acc[nt][8 * h + 2 * e][i] * inv,
                                                  s.acc[nt][8 * h + 2 * e + 1][i] * inv);
                        *reinterpret_cast<u32x4*>(orow + 2 * (d0 + 8 * h)) = wv;
                    }
                } else {
                    u32x2 wv;
#pragma unroll
                    for (int e = 0; e < 2; ++e)
                        wv[e] = pack_bf16_rne(s.acc[nt][2 * e][i] * inv, s.acc[nt][2 * e + 1][i] * inv);
                    *reinterpret_cast<u32x2*>(orow + 2 * d0) = wv;
                }
            }
        } else {
            const int64_t pid = ((int64_t)(2 * w + slot) * a.HG + wave) * a.rows + row;
            float* wo = a.ws_o + pid * D;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = J * (4 * grp + i);
#pragma unroll
                for (int e = 0; e < J / 4; ++e) {
                    f32x4 wv;
#pragma unroll
                    for (int k = 0; k < 4; ++k) wv[k] = s.acc[nt][4 * e + k][i] * inv;
                    *reinterpret_cast<f32x4*>(wo + d0 + 4 * e) = wv;
                }
            }
            if (grp == 0) a.ws_lse[pid] = lt > 0.f ? s.m[nt] + __log2f(lt) : -__builtin_inff();
        }
    }
}

// Even shares of the chunk space.  The chunks (32-token pieces) of every
// (sequence, kv-head group) segment, sequence-major, are numbered 0..C-1;
// workgroup w of n takes [w*C/n, (w+1)*C/n).  n is the launched grid,
// lowered so that every share holds at least min_share chunks.  The merge
// kernel recomputes the same numbers to find a row's partial results.
__device__ __forceinline__ int share_count(int grid, int64_t C, int min_share) {
    const int64_t cap = C / max(min_share, 1);
    return (int)max<int64_t>(1, min<int64_t>(grid, cap));
}
__device__ __forceinline__ int64_t share_begin(int w, int64_t C, int n) { return (int64_t)w * C / n; }
// the workgroup whose share holds chunk c (the largest w with share_begin(w) <= c)
__device__ __forceinline__ int share_owner(int64_t c, int64_t C, int n) {
    return (int)(((c + 1) * n + C - 1) / C) - 1;
}

// Partition kernel.  A workgroup is HG waves, wave v serving kv head
// gg*HG + v of the segments in its share (at head_dim 256 with more than 16
// rows, HG*P waves, P per kv head), so the waves of a CU read the adjacent
// head rows of the same tokens (whole contiguous token rows of the cache).  Every workgroup gets the same number of chunks to within one,
// whatever the ragged context lengths: a share may start and end inside a
// sequence and may hold several whole sequences.  The per-sequence chunk
// counts are scanned (workgroup 0 also stores the scan for the merge
// kernel): for up to 64 sequences by every wave in its own lanes, else by
// wave 0 into LDS; every wave finds a chunk's sequence with a 64-wide
// ballot over that prefix (a share's chunks only increase).
template <int D, bool FP8, int NT, bool GEN>
__global__ __launch_bounds__(NT == 1 && D <= 128 ? 512 : 256)
__attribute__((amdgpu_waves_per_eu(NT == 1 && D <= 128 ? (FP8 && D == 64 ? 3 : 2) : 1)))
void partition_kernel(PartArgs a) {
    extern __shared__ int s_pre[];               // inclusive prefix of chunks per sequence
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // At head_dim 256 a wave holds one 16-row tile; a kv head with more
    // rows gets P waves, wave hk*P + i taking rows 16i .. 16i+15.  They run
    // the same chunks in step, so the K/V rows they share come from the
    // CU's caches after the first of them has read them.
    const int hk = D == 256 ? wave / a.P : wave;         // kv head within the group
    const int r0 = D == 256 ? 16 * (wave - hk * a.P) : 0;
    if (GEN && a.whole) {
        // one workgroup per (sequence, kv-head group) segment, run whole:
        // no scan, no partials, no merge
        const int ngrp = a.Hkv / a.HG;
        const int b = blockIdx.x / ngrp, gg = blockIdx.x - b * ngrp;
        const int L = min(a.ctx[(int64_t)b * a.ctx_s], 16 * a.wsub);
        const int nq = min(a.ql ? a.ql[(int64_t)b * a.ql_s] : a.Qmax, a.Qmax);
        const int cb = (L > 0 && nq > 0) ? (L + kChunkTokens - 1) / kChunkTokens - first_chunk<GEN>(a, L, nq) : 0;
        if (cb > 0) process_segment<D, FP8, NT, GEN>(a, b, gg * a.HG + hk, hk, 0, cb, cb, blockIdx.x, 0, lane, r0);
        return;
    }
    const int ngrp = a.Hkv / a.HG;
    if (a.B <= 64) {
        // up to 64 sequences: every wave scans the chunk counts itself (lane
        // b: sequence b) and keeps the prefix in a register, so no wave
        // waits for an LDS round and a barrier before its first loads
        int nc = 0;
        if (lane < a.B) {
            const int L = min(a.ctx[(int64_t)lane * a.ctx_s], 16 * a.wsub);
            const int nq = min(a.ql ? a.ql[(int64_t)lane * a.ql_s] : a.Qmax, a.Qmax);
            nc = (L > 0 && nq > 0) ? (L + kChunkTokens - 1) / kChunkTokens - first_chunk<GEN>(a, L, nq) : 0;
        }
        int x = nc;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        if (blockIdx.x == 0 && wave == 0 && a.ws_pre && lane < a.B) a.ws_pre[lane] = x;
        const int64_t C = (int64_t)__builtin_amdgcn_readlane(x, a.B - 1) * ngrp;
        const int n = share_count((int)gridDim.x, C, a.min_share);
        const int w = blockIdx.x;
        if (w >= n) return;
        const int64_t lo = share_begin(w, C, n), hi = share_begin(w + 1, C, n);
        for (int64_t pos = lo; pos < hi;) {
            const int b = __popcll(__ballot(lane < a.B && (int64_t)x * ngrp <= pos));
            const int pre = b > 0 ? __builtin_amdgcn_readlane(x, b - 1) : 0;
            const int cb = __builtin_amdgcn_readlane(x, b) - pre;
            const int within = (int)(pos - (int64_t)pre * ngrp);
            const int gg = within / cb;
            const int c0 = within - gg * cb;
            const int c1 = (int)min<int64_t>(cb, c0 + (hi - pos));
            process_segment<D, FP8, NT, GEN>(a, b, gg * a.HG + hk, hk, c0, c1, cb, w, pos == lo ? 0 : 1, lane, r0);
            pos += c1 - c0;
        }
        return;
    }
    if (wave == 0) {
        int carry = 0;
        for (int b0 = 0; b0 < a.B; b0 += 64) {
            const int b = b0 + lane;
            int nc = 0;
            if (b < a.B) {
                const int L = min(a.ctx[(int64_t)b * a.ctx_s], 16 * a.wsub);
                const int nq = min(a.ql ? a.ql[(int64_t)b * a.ql_s] : a.Qmax, a.Qmax);
                nc = (L > 0 && nq > 0) ? (L + kChunkTokens - 1) / kChunkTokens - first_chunk<GEN>(a, L, nq) : 0;
            }
            int x = nc;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(x, o);
                if (lane >= o) x += y;
            }
            if (b < a.B) {
                s_pre[b] = carry + x;
                if (blockIdx.x == 0 && a.ws_pre) a.ws_pre[b] = carry + x;
            }
            carry += __shfl(x, 63);
        }
    }
    __syncthreads();
    const int64_t C = (int64_t)(a.B > 0 ? s_pre[a.B - 1] : 0) * ngrp;
    const int n = share_count((int)gridDim.x, C, a.min_share);
    const int w = blockIdx.x;
    if (w >= n) return;
    const int64_t lo = share_begin(w, C, n), hi = share_begin(w + 1, C, n);
    int bbase = 0;
    for (int64_t pos = lo; pos < hi;) {
        // sequence b = number of sequences whose segments end at or before pos
        int b;
        for (;;) {
            const int idx = bbase + lane;
            const bool le = idx < a.B && (int64_t)s_pre[idx] * ngrp <= pos;
            const int k = __popcll(__ballot(le));
            if (k < 64) { b = bbase + k; break; }
            bbase += 64;
        }
        bbase = b & ~63;
        const int pre = b > 0 ? s_pre[b - 1] : 0;
        const int cb = s_pre[b] - pre;
        const int within = (int)(pos - (int64_t)pre * ngrp);
        const int gg = within / cb;
        const int c0 = within - gg * cb;
        const int c1 = (int)min<int64_t>(cb, c0 + (hi - pos));
        process_segment<D, FP8, NT, GEN>(a, b, gg * a.HG + hk, hk, c0, c1, cb, w, pos == lo ? 0 : 1, lane, r0);
        pos += c1 - c0;
    }
}

// Merge of the partial results of query rows: log-sum-exp weights in base
// 2, float32 throughout, bf16 round-to-nearest-even at the end.  The rows
// of one (sequence b, query t, kv head g) share a segment, which spans the
// shares of workgroups first..last; each of those left one partial per row
// in its slot (slot 1 for the first workgroup when the segment is not the
// first of its share).  A merge workgroup takes RG of those rows and CB
// float4 columns; each (row, column) has PL partial lanes, each running an
// online merge over partials pl, pl + PL, ... with U loads in flight, and
// the lanes combine through LDS.  The host picks RG, CB and PL from the
// expected partials per row, so that short lists merge in one round of
// loads over many rows and long lists spread over many lanes.
template <int D>
__global__ __launch_bounds__(kRedThreads) void reduce_kernel(RedArgs a) {
    constexpr int U = kRedUnroll;
    const int tid = threadIdx.x;
    const int RG = a.red_rows, CB = a.red_col4, PL = a.red_lanes;
    const int ncb = (D / 4) / CB, nrg = a.G / RG;
    int64_t id = blockIdx.x;
    const int cbi = (int)(id % ncb); id /= ncb;
    const int rgi = (int)(id % nrg); id /= nrg;
    const int g = (int)(id % a.Hkv); id /= a.Hkv;
    const int t = (int)(id % a.Qmax);
    const int b = (int)(id / a.Qmax);
    // thread = (pl, rg, c): columns fastest, so a wave reads whole partial rows
    const int c = tid % CB, rg = (tid / CB) % RG, pl = tid / (CB * RG);
    const bool active = pl < PL;
    const int hl = rgi * RG + rg;                 // query head within the group
    const int r = t * a.G + hl;                   // row within the kv head's rows
    const int col = 4 * (cbi * CB + c);
    const int ngrp = a.Hkv / a.HG;
    const int gg = g / a.HG, wave = g - gg * a.HG;
    const float ninf = -__builtin_inff();
    float l[U];
    f32x4 o[U];
    // one round of partial loads: partials p0, p0 + PL, ... of the row's
    // list (shares first .. first + np - 1, slot0 for the first)
    auto load_round = [&](int first, int np, int slot0, int p0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = p0 + u * PL;
            if (active && p < np) {
                const int64_t pid = ((int64_t)(2 * (first + p) + (p == 0 ? slot0 : 0)) * a.HG + wave) * a.rows + r;
                l[u] = a.ws_lse[pid];
                o[u] = *reinterpret_cast<const f32x4*>(a.ws_o + pid * D + col);
            } else {
                l[u] = ninf;
                o[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    // Loads that do not depend on each other go out together: the query
    // length, the chunk prefix and, for one sequence whose shares split
    // evenly between the kv-head groups (spec), the row's first round of
    // partials, whose places then do not depend on the context length (the
    // shares of group gg are gg*grid/ngrp .. (gg+1)*grid/ngrp - 1, slot 0,
    // whenever the sequence has at least grid/ngrp chunks per group); the
    // guess is checked against the prefix and reloaded if it misses.
    // (every load is unconditional, its address or its value selected, so
    // that no branch separates them)
    const int32_t* qlp = a.ql ? a.ql + (int64_t)b * a.ql_s : a.ws_pre + b;
    const int nq_raw = *qlp;
    const int pre_raw = a.ws_pre[max(b - 1, 0)];
    const int end = a.ws_pre[b];
    const int tot = a.ws_pre[a.B - 1];
    const int kspec = a.grid / ngrp;
    if (a.spec) load_round(gg * kspec, kspec, 0, pl);
    const int nq = min(a.ql ? nq_raw : a.Qmax, a.Qmax);
    const int pre = b > 0 ? pre_raw : 0;
    if (t >= nq) return;
    const int cb = end - pre;
    if (cb <= 0) return;
    const int64_t C = (int64_t)tot * ngrp;
    const int n = share_count(a.grid, C, a.min_share);
    const int64_t S = (int64_t)pre * ngrp + (int64_t)gg * cb;
    const int first = share_owner(S, C, n), last = share_owner(S + cb - 1, C, n);
    if (first == last) return;                  // written by the partition kernel
    const int np = last - first + 1;
    const int slot0 = share_begin(first, C, n) == S ? 0 : 1;
    const bool hit = a.spec && first == gg * kspec && np == kspec && slot0 == 0;

    float m = ninf, wsum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (active) {
        for (int p0 = pl; p0 < np; p0 += PL * U) {
            if (!(hit && p0 == pl)) load_round(first, np, slot0, p0);
            float mn = m;
#pragma unroll
            for (int u = 0; u < U; ++u) mn = fmaxf(mn, l[u]);
            const float mu = mn == ninf ? 0.f : mn;
            const float sc = __builtin_amdgcn_exp2f(m - mu);
            wsum *= sc;
            acc *= sc;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float wt = __builtin_amdgcn_exp2f(l[u] - mu);
                wsum += wt;
                acc += wt * o[u];
            }
            m = mn;
        }
    }
    // The partial lanes of one (row, column) are `stride` threads apart:
    // those in one wave combine by lane exchanges first, so the LDS round
    // below takes one entry per wave instead of one per lane.
    const int stride = CB * RG;
    for (int o = stride; o < 64; o <<= 1) {
        const float m2 = __shfl_xor(m, o), w2 = __shfl_xor(wsum, o);
        f32x4 a2;
#pragma unroll
        for (int k = 0; k < 4; ++k) a2[k] = __shfl_xor(acc[k], o);
        const float mn = fmaxf(m, m2);
        const float mu = mn == ninf ? 0.f : mn;
        const float s1 = __builtin_amdgcn_exp2f(m - mu), s2 = __builtin_amdgcn_exp2f(m2 - mu);
        wsum = wsum * s1 + w2 * s2;
        acc = acc * s1 + a2 * s2;
        m = mn;
    }
    __shared__ float sm[kRedThreads], sw[kRedThreads];
    __shared__ f32x4 sacc[kRedThreads];
    sm[tid] = m;
    sw[tid] = wsum;
    sacc[tid] = acc;
    __syncthreads();
    if (active && pl == 0) {
        const int qstep = stride < 64 ? 64 / stride : 1;   // partial lanes per wave
        const int h = g * a.G + hl;
        // a sink is one more partial: log-sum-exp = the sink, output 0
        const float sk = sink_log2(a.sinks, a.sinks_s, h);
        float M = fmaxf(m, sk);
        for (int q = qstep; q < PL; q += qstep) M = fmaxf(M, sm[tid + q * stride]);
        const float Mu = M == ninf ? 0.f : M;
        f32x4 tot = {0.f, 0.f, 0.f, 0.f};
        float wt = sk > ninf ? __builtin_amdgcn_exp2f(sk - Mu) : 0.f;
        for (int q = 0; q < PL; q += qstep) {
            const float sc = __builtin_amdgcn_exp2f(sm[tid + q * stride] - Mu);
            tot += sc * sacc[tid + q * stride];
            wt += sc * sw[tid + q * stride];
        }
        const float inv = wt > 0.f ? 1.f / wt : 0.f;
        u32x2 wv;
        wv[0] = pack_bf16_rne(tot[0] * inv, tot[1] * inv);
        wv[1] = pack_bf16_rne(tot[2] * inv, tot[3] * inv);
        char* orow = a.out + (int64_t)b * a.o_sb + (int64_t)t * a.o_st + (int64_t)h * a.o_sh;
        *reinterpret_cast<u32x2*>(orow + 2 * col) = wv;
    }
}

// ---------------------------------------------------------------- host side

struct Workspace {
    void* ptr = nullptr;
    size_t bytes = 0;
    bool captured = false;           // a call used it while its stream was capturing
    std::vector<void*> retired;      // smaller buffers a captured graph may still use
};

std::mutex g_mu;
std::map<std::pair<int, void*>, Workspace> g_ws;
std::vector<int> g_cus;

// Scratch of the no-allocation entry point: one array per device, in the
// code object's own device memory (allocated when the runtime loads the
// library on a device, held until the process ends).  Host code never
// passes the array's name to a kernel (on the host it only stands for the
// symbol); it looks the device address up once per device and passes that.
constexpr size_t kScratchBytes = size_t(48) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];
std::vector<void*> g_scratch;        // per device: scratch's device address (null: not looked up)

struct Profile {
    bool active = false;
    int max_calls = 0, calls = 0;
    std::vector<hipEvent_t> ev;   // 3 per call: before, between, after
    std::vector<bool> has_reduce;
} g_prof;

int device_cus(int dev) {
    std::lock_guard<std::mutex> lk(g_mu);
    if ((int)g_cus.size() <= dev) g_cus.resize(dev + 1, 0);
    if (g_cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        g_cus[dev] = n;
    }
    return g_cus[dev];
}

// The stream's workspace, grown to `need` bytes when it is smaller.  A
// buffer that a call used during stream capture may be referenced by a
// graph that is replayed later, so growth retires it (kept allocated until
// the process ends) instead of freeing it; a buffer never captured is freed
// once the stream has passed the calls that used it.
int get_workspace(int dev, void* stream, size_t need, void** out) {
    std::lock_guard<std::mutex> lk(g_mu);
    Workspace& w = g_ws[{dev, stream}];
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cs) != hipSuccess)
        return fail(PA_ERR_HIP, "hipStreamIsCapturing failed");
    const bool capturing = cs != hipStreamCaptureStatusNone;
    if (w.bytes >= need) {
        w.captured = w.captured || capturing;
        *out = w.ptr;
        return PA_OK;
    }
    if (capturing)
        return fail(PA_ERR_CAPTURE, "workspace of %zu bytes needed (have %zu) while the stream is capturing",
                    need, w.bytes);
    if (w.ptr) {
        if (w.captured) {
            w.retired.push_back(w.ptr);
        } else {
            // earlier calls on this stream may still read it
            if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess)
                return fail(PA_ERR_HIP, "hipStreamSynchronize failed");
            (void)hipFree(w.ptr);
        }
        w.ptr = nullptr;
        w.bytes = 0;
        w.captured = false;
    }
    const size_t bytes = need + need / 4;   // headroom against creeping sizes
    if (hipMalloc(&w.ptr, bytes) != hipSuccess) {
        (void)hipGetLastError();
        w.ptr = nullptr;
        return fail(PA_ERR_NOMEM, "hipMalloc of %zu workspace bytes failed", bytes);
    }
    w.bytes = bytes;
    *out = w.ptr;
    return PA_OK;
}

// The device address of this device's scratch array, looked up on the
// device's first no-allocation call (the device is current).
int scratch_address(int dev, void** out) {
    std::lock_guard<std::mutex> lk(g_mu);
    if ((int)g_scratch.size() <= dev) g_scratch.resize(dev + 1, nullptr);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(PA_ERR_HIP, "hipGetSymbolAddress of the scratch array failed: %s", hipGetErrorString(e));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return PA_OK;
}

template <int D, bool FP8, bool GEN>
const void* kernel_of(int nt) {
    return nt == 1 ? reinterpret_cast<const void*>(&partition_kernel<D, FP8, 1, GEN>)
         : nt == 2 ? reinterpret_cast<const void*>(&partition_kernel<D, FP8, 2, GEN>)
         : nt == 3 ? reinterpret_cast<const void*>(&partition_kernel<D, FP8, 3, GEN>)
                   : reinterpret_cast<const void*>(&partition_kernel<D, FP8, 4, GEN>);
}

// gen: the general variant (blocks of more than 16 tokens, window, sinks)
template <int D>
const void* kernel_of(bool fp8, int nt, bool gen) {
    if (fp8) return gen ? kernel_of<D, true, true>(nt) : kernel_of<D, true, false>(nt);
    return gen ? kernel_of<D, false, true>(nt) : kernel_of<D, false, false>(nt);
}

// head_dim 256 runs one 16-row tile per wave (with two, the step, the query
// fragments and the accumulators no longer fit the register file); more
// rows take more waves per kv head
template <bool FP8, bool GEN>
const void* kernel256_of(int) {
    return reinterpret_cast<const void*>(&partition_kernel<256, FP8, 1, GEN>);
}

const void* partition_kernel_of(int D, bool fp8, int nt, bool gen) {
    if (D == 256) {
        if (fp8) return gen ? kernel256_of<true, true>(nt) : kernel256_of<true, false>(nt);
        return gen ? kernel256_of<false, true>(nt) : kernel256_of<false, false>(nt);
    }
    return D == 128 ? kernel_of<128>(fp8, nt, gen) : kernel_of<64>(fp8, nt, gen);
}

}  // namespace
}  // namespace pa

namespace pa {
namespace {

// Both decode entry points: validation, plan, workspace (the stream's own,
// or with `noalloc` the device's static scratch array), the partition
// launch and the merge launch.
int decode_call(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                const pa_tensor* block_tables, const pa_tensor* context_lens, const pa_tensor* query_lens,
                float scale, const pa_tensor* k_scale, const pa_tensor* v_scale, int32_t sliding_window,
                const pa_tensor* sinks, pa_tensor* out, void* stream, bool noalloc) {
    Problem pr;
    int st = validate(q, k_cache, v_cache, block_tables, context_lens, query_lens, scale, k_scale, v_scale,
                      sliding_window, sinks, out, &pr);
    if (st) return st;
    if (pr.B == 0) return PA_OK;

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice failed");
    pa_plan plan;
    const int64_t max_ctx = max_context_tokens(pr.BS, pr.W, pr.window, pr.Qmax);
    if ((st = make_plan(pr.B, pr.Hq, pr.Hkv, pr.D, pr.Qmax, max_ctx, pr.fp8, device_cus(dev), &plan))) return st;
    void* ws = nullptr;
    if (plan.workspace_bytes > 0) {
        if (noalloc) {
            if ((size_t)plan.workspace_bytes > kScratchBytes)
                return fail(PA_ERR_UNSUPPORTED,
                            "the call needs %lld workspace bytes; the no-allocation entry point's scratch "
                            "holds %zu", (long long)plan.workspace_bytes, kScratchBytes);
            if ((st = scratch_address(dev, &ws))) return st;
        } else if ((st = get_workspace(dev, stream, (size_t)plan.workspace_bytes, &ws))) {
            return st;
        }
    }

    const size_t lds = plan.whole_segments ? 0 : (size_t)pr.B * sizeof(int);
    const bool general = pr.BS > PA_BLOCK_SIZE || pr.window > 0 || pr.sinks != nullptr || plan.whole_segments;
    const void* fn = partition_kernel_of((int)pr.D, pr.fp8, plan.row_tiles, general);
    const int HG = plan.heads_per_group;
    const int64_t grid = plan.workgroups;
    const int64_t nslot = 2 * grid * HG * plan.rows;      // partial slots (see PartArgs)
    PartArgs a;
    a.q = static_cast<const char*>(pr.q); a.q_sb = pr.q_sb * 2; a.q_st = pr.q_st * 2; a.q_sh = pr.q_sh * 2;
    a.k = static_cast<const char*>(pr.k); a.k_stok = pr.k_stok; a.k_sh = pr.k_sh;
    a.v = static_cast<const char*>(pr.v); a.v_stok = pr.v_stok; a.v_sh = pr.v_sh;
    a.ks = pr.ks; a.ks_sh = pr.ks_sh;
    a.vs = pr.vs; a.vs_sh = pr.vs_sh;
    a.k_sblk = (uint32_t)pr.k_sblk; a.v_sblk = (uint32_t)pr.v_sblk;
    a.ks_sblk = (uint32_t)(pr.ks_sblk * 4); a.vs_sblk = (uint32_t)(pr.vs_sblk * 4);
    a.k_ssub = (uint32_t)(PA_BLOCK_SIZE * pr.k_stok); a.v_ssub = (uint32_t)(PA_BLOCK_SIZE * pr.v_stok);
    a.bt = pr.bt; a.bt_sb = pr.bt_sb;
    a.ctx = pr.ctx; a.ctx_s = pr.ctx_s;
    a.ql = pr.ql; a.ql_s = pr.ql_s;
    a.sinks = pr.sinks; a.sinks_s = pr.sinks_s;
    a.out = static_cast<char*>(pr.out); a.o_sb = pr.o_sb * 2; a.o_st = pr.o_st * 2; a.o_sh = pr.o_sh * 2;
    a.ws_o = static_cast<float*>(ws);
    a.ws_lse = ws ? a.ws_o + nslot * pr.D : nullptr;
    a.ws_pre = ws ? reinterpret_cast<int32_t*>(a.ws_lse + nslot) : nullptr;
    a.scale_log2 = std::fabs(pr.scale) * kLog2e;
    a.q_neg = pr.scale < 0.f;
    a.k_span = (int32_t)(15 * pr.k_stok + pr.D * (pr.fp8 ? 1 : 2));
    a.v_span = (int32_t)(15 * pr.v_stok + pr.D * (pr.fp8 ? 1 : 2));
    a.B = (int32_t)pr.B; a.Hq = (int32_t)pr.Hq; a.Hkv = (int32_t)pr.Hkv; a.G = (int32_t)pr.G; a.Qmax = (int32_t)pr.Qmax;
    a.bsub = (int32_t)(pr.BS / PA_BLOCK_SIZE);
    a.wsub = (int32_t)(pr.W * a.bsub);
    a.window = pr.window;
    a.whole = plan.whole_segments;
    a.NB = (int32_t)std::min<int64_t>(pr.NB, INT32_MAX);
    a.rows = plan.rows; a.HG = HG; a.min_share = plan.min_share_chunks;
    a.P = plan.row_waves;

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t e0 = nullptr, e1 = nullptr, e2 = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        if (g_prof.active && g_prof.calls < g_prof.max_calls) {
            const int c = g_prof.calls++;
            e0 = g_prof.ev[3 * c]; e1 = g_prof.ev[3 * c + 1]; e2 = g_prof.ev[3 * c + 2];
            g_prof.has_reduce[c] = plan.reduce_groups > 0;
        }
    }
    if (e0) (void)hipEventRecord(e0, s);
    {
        void* args[] = {&a};
        if (hipLaunchKernel(fn, dim3((unsigned)grid), dim3(64 * HG * a.P), args, lds, s) != hipSuccess)
            return fail(PA_ERR_HIP, "partition kernel launch failed: %s", hipGetErrorString(hipGetLastError()));
    }
    if (e1) (void)hipEventRecord(e1, s);
    if (plan.reduce_groups > 0) {
        RedArgs r;
        r.ws_o = a.ws_o; r.ws_lse = a.ws_lse; r.ws_pre = a.ws_pre;
        r.ql = a.ql; r.ql_s = a.ql_s;
        r.sinks = a.sinks; r.sinks_s = a.sinks_s;
        r.out = a.out; r.o_sb = a.o_sb; r.o_st = a.o_st; r.o_sh = a.o_sh;
        r.B = a.B; r.Hq = a.Hq; r.Hkv = a.Hkv; r.G = a.G; r.Qmax = a.Qmax; r.rows = a.rows; r.HG = HG;
        r.grid = (int32_t)grid; r.min_share = a.min_share;
        r.red_rows = plan.reduce_rows; r.red_col4 = plan.reduce_col4; r.red_lanes = plan.reduce_lanes;
        r.spec = pr.B == 1 && grid % (pr.Hkv / HG) == 0 && grid / (pr.Hkv / HG) <= (int64_t)plan.reduce_lanes * kRedUnroll;
        const dim3 rgrid((unsigned)plan.reduce_groups), rblock((unsigned)kRedThreads);
        if (pr.D == 256) hipLaunchKernelGGL(reduce_kernel<256>, rgrid, rblock, 0, s, r);
        else if (pr.D == 128) hipLaunchKernelGGL(reduce_kernel<128>, rgrid, rblock, 0, s, r);
        else hipLaunchKernelGGL(reduce_kernel<64>, rgrid, rblock, 0, s, r);
    }
    if (e2) (void)hipEventRecord(e2, s);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(PA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return PA_OK;
}

}  // namespace
}  // namespace pa

extern "C" {

int paged_attn_decode_ext(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                          const pa_tensor* block_tables, const pa_tensor* context_lens,
                          const pa_tensor* query_lens, float scale, const pa_tensor* k_scale,
                          const pa_tensor* v_scale, int32_t sliding_window, const pa_tensor* sinks,
                          pa_tensor* out, void* stream) {
    return pa::decode_call(q, k_cache, v_cache, block_tables, context_lens, query_lens, scale, k_scale, v_scale,
                           sliding_window, sinks, out, stream, false);
}

int paged_attn_decode(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                      const pa_tensor* block_tables, const pa_tensor* context_lens,
                      const pa_tensor* query_lens, float scale, const pa_tensor* k_scale,
                      const pa_tensor* v_scale, pa_tensor* out, void* stream) {
    return pa::decode_call(q, k_cache, v_cache, block_tables, context_lens, query_lens, scale, k_scale, v_scale,
                           0, nullptr, out, stream, false);
}

int paged_attn_decode_noalloc(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                              const pa_tensor* block_tables, const pa_tensor* context_lens,
                              const pa_tensor* query_lens, float scale, const pa_tensor* k_scale,
                              const pa_tensor* v_scale, pa_tensor* out, void* stream) {
    return pa::decode_call(q, k_cache, v_cache, block_tables, context_lens, query_lens, scale, k_scale, v_scale,
                           0, nullptr, out, stream, true);
}

int paged_attn_reserve(int64_t bytes, void* stream) {
    if (bytes < 0) return pa::fail(PA_ERR_ARG, "reserve: negative size");
    if (bytes == 0) return PA_OK;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return pa::fail(PA_ERR_HIP, "hipGetDevice failed");
    void* p = nullptr;
    return pa::get_workspace(dev, stream, (size_t)bytes, &p);
}

int paged_attn_profile_begin(int32_t max_calls) {
    using namespace pa;
    if (max_calls < 1) return fail(PA_ERR_ARG, "profile_begin: max_calls must be >= 1");
    std::lock_guard<std::mutex> lk(g_mu);
    for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
    g_prof.ev.assign(3 * (size_t)max_calls, nullptr);
    for (auto& e : g_prof.ev)
        if (hipEventCreate(&e) != hipSuccess) return fail(PA_ERR_HIP, "hipEventCreate failed");
    g_prof.has_reduce.assign(max_calls, false);
    g_prof.max_calls = max_calls;
    g_prof.calls = 0;
    g_prof.active = true;
    return PA_OK;
}

int paged_attn_profile_end(double* partition_ms, double* reduce_ms, int32_t* calls) {
    using namespace pa;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_prof.active) return fail(PA_ERR_ARG, "profile_end without profile_begin");
    double part = 0, red = 0;
    int st = PA_OK;
    for (int c = 0; c < g_prof.calls; ++c) {
        float ms = 0.f;
        if (hipEventSynchronize(g_prof.ev[3 * c + 2]) != hipSuccess) { st = PA_ERR_HIP; break; }
        if (hipEventElapsedTime(&ms, g_prof.ev[3 * c], g_prof.ev[3 * c + 1]) == hipSuccess) part += ms;
        if (g_prof.has_reduce[c] &&
            hipEventElapsedTime(&ms, g_prof.ev[3 * c + 1], g_prof.ev[3 * c + 2]) == hipSuccess)
            red += ms;
    }
    if (partition_ms) *partition_ms = part;
    if (reduce_ms) *reduce_ms = red;
    if (calls) *calls = g_prof.calls;
    for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
    g_prof.ev.clear();
    g_prof.active = false;
    if (st) return fail(st, "profile_end: hipEventSynchronize failed");
    return PA_OK;
}

}  // extern "C"
