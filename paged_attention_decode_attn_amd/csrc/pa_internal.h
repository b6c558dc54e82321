// Internal interface between the host-side validation/planning code
// (pa_host.cpp, plain C++) and the HIP launch code (pa_device.hip).
#pragma once

#include <atomic>
#include <cstdint>

#include "paged_attn.h"
#include "paged_attn_tuning.h"

namespace pa {

// A fully validated call, with every stride converted to the units the
// kernels use.  Element strides unless the name says bytes.
struct Problem {
    int64_t B, Qmax, Hq, Hkv, G, D, NB, W;
    int64_t BS;                                        // tokens per block (a multiple of 16)
    bool fp8;
    float scale;
    int32_t window;                                    // sliding window in tokens, 0 = none
    const float* sinks; int64_t sinks_s;               // fp32 per query head, may be null

    const void* q;  int64_t q_sb, q_st, q_sh;          // bf16 elements
    void* out;      int64_t o_sb, o_st, o_sh;          // bf16 elements
    const void* k;  int64_t k_sblk, k_stok, k_sh;      // bytes
    const void* v;  int64_t v_sblk, v_stok, v_sh;      // bytes
    const float* ks; int64_t ks_sblk, ks_sh;           // fp32 elements (slot stride 1)
    const float* vs; int64_t vs_sblk, vs_sh;
    const int32_t* bt; int64_t bt_sb;                  // int32 elements
    const int32_t* ctx; int64_t ctx_s;
    const int32_t* ql;  int64_t ql_s;                  // ql may be null
};

// A validated cache write (paged_attn_reshape_and_cache).
struct WriteProblem {
    int64_t T, Hkv, D, NB, BS;
    bool fp8;
    const void* k_new; int64_t kn_st, kn_sh;           // bytes
    const void* v_new; int64_t vn_st, vn_sh;           // bytes
    const int32_t* slots; int64_t slot_s;              // int32 elements
    void* kc; int64_t k_sblk, k_stok, k_sh;            // bytes
    void* vc; int64_t v_sblk, v_stok, v_sh;            // bytes
    float* ks; int64_t ks_sblk, ks_sh;                 // fp32 elements (slot stride 1)
    float* vs; int64_t vs_sblk, vs_sh;
};

int validate_write(const pa_tensor* k_new, const pa_tensor* v_new, const pa_tensor* slot_mapping,
                   const pa_tensor* k_cache, const pa_tensor* v_cache, const pa_tensor* k_scale,
                   const pa_tensor* v_scale, WriteProblem* p);

// Host-only validation shared by the check and decode entry points.
int validate(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
             const pa_tensor* block_tables, const pa_tensor* context_lens,
             const pa_tensor* query_lens, float scale, const pa_tensor* k_scale,
             const pa_tensor* v_scale, int32_t sliding_window, const pa_tensor* sinks,
             const pa_tensor* out, Problem* pr);

// The most cache tokens one sequence's rows can read: the table's reach,
// or the window plus the query rows when a window is set.
int64_t max_context_tokens(int64_t block_size, int64_t table_width, int32_t window, int64_t Qmax);

// The split-context plan (see pa_plan in paged_attn.h).
int make_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t Qmax, int64_t max_context,
              bool fp8, int32_t num_cus, pa_plan* plan);

// Cache-write pieces per thread override (paged_attn_tuning.h; 0 = automatic).
extern std::atomic<int32_t> g_write_pieces;

// Records a failure description for paged_attn_last_error() and returns `status`.
int fail(int status, const char* fmt, ...);

// Descriptor checks shared by the entry points' validation.
int64_t elem_bytes(int32_t dtype);
const char* dtype_name(int32_t dtype);
bool aligned(const void* p, uintptr_t a);
// rank in [ndim_lo, ndim_hi], the dtype, non-negative sizes and strides, and
// (need_data) a data pointer when the tensor is not empty
int check_desc(const pa_tensor* t, const char* name, int32_t dtype, int ndim_lo, int ndim_hi, bool need_data);
// inner stride 1, other strides multiples of 16 bytes, base 16-byte aligned
int check_rows16(const pa_tensor* t, const char* name);
// Saturating arithmetic on non-negative sizes: a result past INT64_MAX reads
// as INT64_MAX, so a limit check on it rejects the input.
int64_t sat_mul(int64_t a, int64_t b);
int64_t sat_add(int64_t a, int64_t b);
// The stride of dim i as the kernels use it: 0 for a dim of size 1, whose
// only index is 0 whatever the caller's stride.
int64_t used_stride(const pa_tensor* t, int i);

constexpr int kChunkTokens = 32;            // tokens per chunk: the unit of work splitting
constexpr int kMaxBlockSize = 4096;         // largest tokens-per-block (a multiple of 16)
constexpr int64_t kMaxContext = int64_t(1) << 30;   // tokens a block-table row may reach
constexpr int kDefaultMinShare = 1;         // smallest share of chunks per workgroup
constexpr int kStepsPerWave = 8;            // planner's target chunks per wave
constexpr int kWholeSegmentChunks = 2 * kStepsPerWave;   // longest segment run whole
constexpr int kMaxBatch = 16384;            // per-sequence chunk counts live in LDS
constexpr int64_t kMaxHeads = int64_t(1) << 16;          // kv heads (and query heads per kv head, far fewer)
constexpr int64_t kMaxSize = int64_t(1) << 48;           // any size, and any tensor's extent in bytes
constexpr int64_t kMaxBlocks = (int64_t(1) << 31) - 1;   // int32 block ids
constexpr int kRedThreads = 256;            // merge workgroup size (reduce_kernel)
constexpr int kRedUnroll = 8;               // partial loads in flight per merge lane

}  // namespace pa
