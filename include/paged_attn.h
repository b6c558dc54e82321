/*
 * paged_attn.h -- C ABI of the MI355X (gfx950) paged-KV decode-attention library.
 *
 * The operation: one or a few new query tokens per sequence attend, with
 * softmax attention, over that sequence's tokens in a paged KV cache that a
 * per-sequence block table addresses.  Sources (web pages):
 *   - ATOM model operations guide, "Attention operations" (decode dispatch to
 *     paged-attention kernels; the q_heads / kv_heads ratio and the query
 *     length that bound each kernel's envelope; per-token quantised layers
 *     must not be served by a one-descale kernel) and "KV cache operations"
 *     (bf16 cache writes, fp8 writes with per-token quantisation);
 *   - ATOM configuration guide, "Master configuration (Config)"
 *     (kv_cache_block_size: 16 by default, a multiple of 16; kv_cache_dtype
 *     "bf16" or "fp8") and "Quick reference" (per-layer k/v caches and
 *     their scales);
 *   - ROCm blog "Optimizing ATOM and vLLM-ATOM for High-Interactivity
 *     Inference", "Attention Decode: Split Memory Work to Fill the Device"
 *     (split the KV range so a single query fills the device; per-split
 *     log-sum-exp kept in fp32) and "Host-Overhead Elimination: Keep Decode
 *     Graph-Safe" (caller-provided outputs, no host-device synchronisation).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors are described by pa_tensor: a data pointer, a dtype code, a rank
 * and per-dimension sizes and strides (strides in ELEMENTS, not bytes).  The
 * library never copies a descriptor's memory and keeps no pointer after a
 * call returns; all device tensors stay owned by the caller.  Work is
 * enqueued asynchronously on the given HIP stream (void* so this header is
 * HIP-free; NULL = the default stream): inputs must stay alive and
 * unmodified, and outputs unread, until the stream passes the call.
 *
 * Every entry point returns PA_OK (0) or a negative pa_status.  A negative
 * status from paged_attn_decode means nothing was enqueued, except
 * PA_ERR_HIP, which reports a launch failure.  paged_attn_strerror() maps a
 * status to a fixed string; paged_attn_last_error() returns the calling
 * thread's description of its most recent failure (which argument, which
 * check).
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_BLOCK_SIZE 16      /* default tokens per KV-cache block; a block
                                 holds any multiple of 16 up to 4096 tokens  */
#define PA_MAX_ROWS   64      /* max (q_heads / kv_heads) * query_len       */
#define PA_MAX_ROWS_D256 16   /* prefill at head_dim 256: max q_heads /
                                 kv_heads (decode serves PA_MAX_ROWS)       */

typedef enum pa_dtype {
    PA_DTYPE_BF16        = 1,  /* bfloat16                                  */
    PA_DTYPE_FP8_E4M3FN  = 2,  /* OCP float8 e4m3fn (bias 7, max 448, no inf) */
    PA_DTYPE_FP32        = 3,
    PA_DTYPE_INT32       = 4
} pa_dtype;

typedef enum pa_status {
    PA_OK              = 0,
    PA_ERR_NULL        = -1,  /* a required tensor or data pointer is NULL   */
    PA_ERR_DTYPE       = -2,  /* a tensor has the wrong dtype                */
    PA_ERR_SHAPE       = -3,  /* ranks or sizes disagree between tensors     */
    PA_ERR_UNSUPPORTED = -4,  /* block size not a multiple of 16, head_dim
                                 not 64/128/256,
                                 q_heads % kv_heads != 0, rows > 64, a size
                                 or a tensor's byte extent of 2^48 or more,
                                 more than 65536 kv heads, 2^31 or more
                                 cache blocks, ...                           */
    PA_ERR_LAYOUT      = -5,  /* inner stride != 1, misaligned base/stride   */
    PA_ERR_CAPTURE     = -6,  /* workspace would have to grow while the
                                 stream is being captured into a graph       */
    PA_ERR_HIP         = -7,  /* a HIP runtime call or launch failed         */
    PA_ERR_NOMEM       = -8,  /* workspace allocation failed                 */
    PA_ERR_ARG         = -9   /* any other invalid argument                  */
} pa_status;

typedef struct pa_tensor {
    void*   data;       /* device pointer (host pointer only where stated)   */
    int32_t dtype;      /* pa_dtype                                          */
    int32_t ndim;       /* 1..4                                              */
    int64_t shape[4];
    int64_t stride[4];  /* in elements                                       */
} pa_tensor;

/*
 * paged_attn_decode -- softmax attention of the new query rows over a paged
 * KV cache, written to `out`.
 *
 *   q             bf16 [B, Qmax, Hq, D] (rank 4) or [B, Hq, D] (rank 3,
 *                 Qmax = 1).  Row (b, t) is the t-th new token of sequence
 *                 b (the rectangular speculative-decode layout).
 *   k_cache,      [NB, BS, Hkv, D], both bf16 or both fp8 e4m3fn; the block
 *   v_cache       size BS is a multiple of 16 (16 by default, up to 4096).
 *                 Token j of sequence b is slot j % BS of physical block
 *                 block_tables[b, j / BS].
 *   block_tables  int32 [B, W].  Only the first ceil(context_lens[b] / BS)
 *                 entries of row b are read; the rest may hold anything.
 *                 Entries may repeat within and across rows (shared
 *                 prefix blocks); the cache is only read.
 *   context_lens  int32 [B]: L_b = number of tokens of sequence b in the
 *                 cache, the new query tokens included (their K/V are
 *                 written before this call).
 *   query_lens    int32 [B]: n_b = number of new query rows of sequence b
 *                 (0 <= n_b <= Qmax).  NULL means n_b = Qmax for all b.
 *                 Query row t (t < n_b) is at position L_b - n_b + t and
 *                 attends to keys 0 .. L_b - n_b + t (causal among the new
 *                 tokens).  Rows t >= n_b are neither read nor written.
 *   scale         softmax scale applied to q.k (e.g. 1/sqrt(D)); finite.
 *   k_scale,      fp32, logically [NB, BS, Hkv]: one dequantisation scale
 *   v_scale       per (block, slot, kv head), i.e. per token and head;
 *                 required iff the cache is fp8, else must be NULL.  The
 *                 slot dimension must be contiguous (stride[1] == 1), e.g.
 *                 a [NB, Hkv, BS] tensor viewed as [NB, BS, Hkv].
 *   out           bf16, same shape as q (its own strides); rows t < n_b
 *                 receive the attention output rounded to nearest even.
 *   stream        hipStream_t as void*, NULL = default stream.
 *
 * Query head h reads KV head h / (Hq / Hkv).  D must be 64, 128 or 256,
 * (Hq / Hkv) * Qmax <= 64.  Inner strides of q, out, caches and block_tables
 * must be 1, the other strides of q/out/caches multiples of 16 bytes, data
 * pointers 16-byte aligned; k_scale/v_scale strides of dims 0 and 2
 * multiples of 4 and data 16-byte aligned.
 *
 * Device-side preconditions, not checked (checking would need a
 * host-device synchronisation): n_b <= L_b <= BS * W and
 * 0 <= block_tables[b, i] < NB for i < ceil(L_b / BS).  Violations give
 * unspecified output values but never an out-of-bounds access: the kernels
 * clamp lengths to the tensors' extents and block ids into [0, NB).
 * `out` must not overlap any input.
 *
 * Uses a per-(device, stream) workspace owned by the library for split-
 * context partial results (fp32 partial outputs and log-sum-exp values,
 * and the per-sequence chunk scan the merge kernel reads);
 * it grows on demand with hipMalloc outside stream capture.  Capture a
 * call into a graph only after paged_attn_reserve() or an uncaptured call
 * of the same or larger size on that stream; otherwise PA_ERR_CAPTURE.
 * Growth never frees a buffer that a call used during capture: graphs
 * captured earlier keep replaying into their own buffer, which stays
 * allocated until the process ends (a buffer never used under capture is
 * freed once the stream has passed the calls that used it).  Calls on one
 * stream are ordered; calls on different streams use different
 * workspaces.
 */
int paged_attn_decode(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                      const pa_tensor* block_tables, const pa_tensor* context_lens,
                      const pa_tensor* query_lens, float scale, const pa_tensor* k_scale,
                      const pa_tensor* v_scale, pa_tensor* out, void* stream);

/*
 * paged_attn_decode_noalloc -- paged_attn_decode for callers that cannot
 * allocate device memory (code under HIP graph capture with no workspace
 * reserved beforehand, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, semantics, output and errors as
 * paged_attn_decode (the same kernels run), except for the workspace: the
 * partial results live in a static array of 48 MiB (50331648 bytes) in the
 * library's own device memory, one per device, held until the process ends.
 * A call whose plan needs more (pa_plan.workspace_bytes) returns
 * PA_ERR_UNSUPPORTED before launching anything.  The call allocates
 * nothing: no hipMalloc or hipFree, no library allocation; its first call
 * on a device looks the array's device address up (hipGetSymbolAddress).
 * Every call on one device shares that device's array (nothing in it has
 * to start cleared: each call writes every element it reads), so calls
 * that may overlap on one device (different streams without ordering
 * between them) race and give unspecified output; calls on one stream are
 * ordered and safe.
 */
int paged_attn_decode_noalloc(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                              const pa_tensor* block_tables, const pa_tensor* context_lens,
                              const pa_tensor* query_lens, float scale, const pa_tensor* k_scale,
                              const pa_tensor* v_scale, pa_tensor* out, void* stream);

/*
 * paged_attn_decode_ext -- paged_attn_decode with a sliding window and
 * attention sinks.  Sources: ATOM model operations guide, "Attention
 * operations" (the decode dispatch takes a sliding_window, -1 for none);
 * the ATOM landing page's model table (GPT-OSS: sliding window + attention
 * sinks).  The pages give no formulas; the definitions below are the
 * common ones.  With sliding_window <= 0 and sinks NULL the call is
 * paged_attn_decode.
 *
 *   sliding_window  w > 0: query row t at position p = L_b - n_b + t sees
 *                 only keys max(0, p - w + 1) .. p (its w most recent
 *                 positions).  w <= 0: no window.  Block-table entries
 *                 wholly below the earliest row's window may hold anything
 *                 (e.g. blocks already freed): the kernels clamp them into
 *                 [0, NB) and never use what they address.
 *   sinks         NULL, or fp32 [Hq] (any stride, 4-byte aligned): one
 *                 logit s_h per query head, in the units of scale * q.k,
 *                 added to the softmax normaliser only:
 *                 out = sum_j e^{x_j} v_j / (e^{s_h} + sum_j e^{x_j}).
 *                 -inf turns a head's sink off; +inf and NaN are not
 *                 allowed (not checked: device data).
 *
 * Every other argument, rule and error as for paged_attn_decode.
 */
int paged_attn_decode_ext(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                          const pa_tensor* block_tables, const pa_tensor* context_lens,
                          const pa_tensor* query_lens, float scale, const pa_tensor* k_scale,
                          const pa_tensor* v_scale, int32_t sliding_window, const pa_tensor* sinks,
                          pa_tensor* out, void* stream);

/*
 * paged_attn_check -- the host-side argument validation of
 * paged_attn_decode, without touching the GPU or dereferencing any data
 * pointer.  Same arguments (no stream); returns the status that
 * paged_attn_decode would return for them before launching.
 */
int paged_attn_check(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                     const pa_tensor* block_tables, const pa_tensor* context_lens,
                     const pa_tensor* query_lens, float scale, const pa_tensor* k_scale,
                     const pa_tensor* v_scale, const pa_tensor* out);

/* paged_attn_check_ext -- the same for paged_attn_decode_ext. */
int paged_attn_check_ext(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                         const pa_tensor* block_tables, const pa_tensor* context_lens,
                         const pa_tensor* query_lens, float scale, const pa_tensor* k_scale,
                         const pa_tensor* v_scale, int32_t sliding_window, const pa_tensor* sinks,
                         const pa_tensor* out);

/*
 * paged_attn_prefill -- causal attention of packed prefill chunks over the
 * paged KV cache (prefill and chunked prefill).  Sources: ATOM model
 * operations guide, "Attention operations" (prefill always runs a
 * variable-length flash-attention call; a unified paged prefill kernel is
 * also listed), "Backend abstraction" (block tables and cumulative
 * sequence lengths prepared for every prefill step) and its source-file
 * list (a ragged prefill chunk's tokens placed in their own sequences).
 *
 *   q, out        bf16 [T, Hq, D] (D 64, 128 or 256): the new tokens of
 *                 all sequences packed row after row.
 *   cu_seqlens_q  int32 [B + 1]: sequence b owns rows cu[b] .. cu[b+1]-1
 *                 (n_b = cu[b+1] - cu[b] rows; cu[0] = 0, non-decreasing).
 *                 They are the last n_b of its L_b = context_lens[b] tokens,
 *                 whose K/V are already in the cache (the chunk's own rows
 *                 written before the call; earlier chunks or a cached
 *                 prefix make up the rest).  Row t sits at position
 *                 L_b - n_b + t and attends to keys 0 .. L_b - n_b + t.
 *   max_query_len the largest n_b (a bound is enough; it sizes the grid).
 *   k_cache, v_cache, block_tables, context_lens, scale, k_scale, v_scale:
 *                 as for paged_attn_decode: bf16 caches (scales NULL), or
 *                 e4m3fn caches with fp32 per-(token, kv head) scales
 *                 [NB, BS, Hkv] (slot dimension contiguous, 4-byte aligned).
 *                 With fp8, K enters the scores exactly (its scale multiplies
 *                 the score) and V is scaled and rounded to bf16 once.
 *   stream        hipStream_t as void*, NULL = default stream.
 *
 * Device-side preconditions, not checked: cu non-decreasing with
 * cu[B] <= T, n_b <= L_b <= BS * W, max_query_len >= every n_b, table
 * entries holding keys in [0, NB).  Rows t < n_b of every sequence are
 * written; a row count clamped by these bounds leaves the rest unwritten,
 * and no access leaves the tensors' extents.  No workspace; nothing is
 * allocated.  Layout rules and errors as for paged_attn_decode; (Hq / Hkv)
 * <= 64 (<= 16 for D 256).
 */
int paged_attn_prefill(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                       const pa_tensor* block_tables, const pa_tensor* context_lens,
                       const pa_tensor* cu_seqlens_q, int32_t max_query_len, float scale,
                       const pa_tensor* k_scale, const pa_tensor* v_scale, pa_tensor* out, void* stream);

/* paged_attn_check_prefill -- the host-side validation of paged_attn_prefill. */
int paged_attn_check_prefill(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                             const pa_tensor* block_tables, const pa_tensor* context_lens,
                             const pa_tensor* cu_seqlens_q, int32_t max_query_len, float scale,
                             const pa_tensor* k_scale, const pa_tensor* v_scale, const pa_tensor* out);

/*
 * paged_attn_prefill_ext -- paged_attn_prefill with a sliding window and
 * attention sinks, as paged_attn_decode_ext adds them to the decode call
 * (ATOM model operations guide, "Attention operations": the attention
 * dispatch takes a sliding window; ATOM README model table: GPT-OSS uses
 * a sliding window and attention sinks).
 *
 *   sliding_window  w > 0: the row at position a sees keys max(0, a - w + 1)
 *                   .. a only; w <= 0: no window.  Blocks wholly below every
 *                   row's window may be freed (their table entries are not
 *                   dereferenced past the pool: ids are clamped into it, and
 *                   their keys are never read into a result).
 *   sinks           NULL or fp32 [Hq], any stride: one logit s_h per query
 *                   head, in the units of scale * q.k, added to the softmax
 *                   normaliser only: out = sum e^{x_j} v_j / (e^{s_h} +
 *                   sum e^{x_j}); -inf disables a head's sink.
 *
 * Everything else, and the error behaviour, as paged_attn_prefill, which is
 * this call with sliding_window = 0 and sinks = NULL.
 */
int paged_attn_prefill_ext(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                           const pa_tensor* block_tables, const pa_tensor* context_lens,
                           const pa_tensor* cu_seqlens_q, int32_t max_query_len, float scale,
                           const pa_tensor* k_scale, const pa_tensor* v_scale, int32_t sliding_window,
                           const pa_tensor* sinks, pa_tensor* out, void* stream);

/* paged_attn_check_prefill_ext -- the host-side validation of paged_attn_prefill_ext. */
int paged_attn_check_prefill_ext(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                                 const pa_tensor* block_tables, const pa_tensor* context_lens,
                                 const pa_tensor* cu_seqlens_q, int32_t max_query_len, float scale,
                                 const pa_tensor* k_scale, const pa_tensor* v_scale, int32_t sliding_window,
                                 const pa_tensor* sinks, const pa_tensor* out);

/*
 * paged_attn_reshape_and_cache -- write the new tokens' K and V rows into
 * the paged cache (the step that precedes paged_attn_decode in a decode
 * step).  Sources: ATOM model operations guide, "KV cache operations" (the
 * standard write for a bf16 cache, the fp8 write with per-token
 * quantisation) and its slot-mapping file (which KV slot a token is
 * written to); ROCm blog "Optimizing ATOM and vLLM-ATOM for
 * High-Interactivity Inference", "Attention Input Fusion" (fp8 scales are
 * calculated as K/V are written into the paged cache).
 *
 *   k_new, v_new  bf16 [T, Hkv, D]: the new tokens' rows (D 64, 128 or 256).
 *   slot_mapping  int32 [T]: slot s of token t is position s % BS of block
 *                 s / BS.  Entries < 0 (padding tokens) and >= NB * BS are
 *                 skipped; the others must be distinct (two tokens on one
 *                 slot leave either token's row).
 *   k_cache,      [NB, BS, Hkv, D], both bf16 or both fp8 e4m3fn, BS a
 *   v_cache       multiple of 16 (up to 4096); written at the mapped slots
 *                 only.
 *   k_scale,      fp32, logically [NB, BS, Hkv], slot dimension contiguous;
 *   v_scale       required iff the cache is fp8, else NULL.  For an fp8
 *                 cache every written (token, kv head) row gets
 *                 scale = max_d |x_d| / 448 (1 for an all-zero row) and
 *                 codes e4m3fn(clamp(x_d / scale, -448, 448)), rounded to
 *                 nearest, ties to even; both divisions correctly rounded
 *                 IEEE float32 (subnormal quotients kept).
 *                 A bf16 cache receives the rows bit for bit.
 *   stream        hipStream_t as void*, NULL = default stream.
 *
 * Layout rules as for paged_attn_decode (inner stride 1, other strides of
 * the bf16 and cache tensors multiples of 16 bytes, 16-byte aligned data);
 * scale data 4-byte aligned.  No workspace; nothing is allocated.  Returns
 * PA_OK or a negative pa_status (nothing enqueued except on PA_ERR_HIP).
 */
int paged_attn_reshape_and_cache(const pa_tensor* k_new, const pa_tensor* v_new,
                                 const pa_tensor* slot_mapping, pa_tensor* k_cache,
                                 pa_tensor* v_cache, pa_tensor* k_scale, pa_tensor* v_scale,
                                 void* stream);

/*
 * paged_attn_check_reshape_and_cache -- the host-side argument validation
 * of paged_attn_reshape_and_cache, without touching the GPU or any data.
 */
int paged_attn_check_reshape_and_cache(const pa_tensor* k_new, const pa_tensor* v_new,
                                       const pa_tensor* slot_mapping, const pa_tensor* k_cache,
                                       const pa_tensor* v_cache, const pa_tensor* k_scale,
                                       const pa_tensor* v_scale);

/*
 * Split-context plan: how paged_attn_decode divides the work so that one
 * call fills the GPU whatever the batch and the ragged context lengths.
 * Every (sequence, kv-head group) pair is a segment of ceil(L_b / 32)
 * chunks of 32 tokens (with a sliding window, the chunks from the one that
 * holds the earliest row's first key); the chunks of all segments,
 * sequence-major, are
 * dealt out in equal contiguous shares (to within one chunk) to
 * `workgroups` workgroups of `heads_per_group` kv heads, each served by
 * `row_waves` waves (one; at head_dim 256 one per 16-row tile).  A share may start and end inside a sequence, so each
 * workgroup leaves at most two fp32 partial results (online-softmax state
 * of the segments cut by its share boundaries) per wave and query row; a
 * segment inside one share is written to `out` directly.  The merge kernel
 * combines a row's partials by their log-sum-exp.  Chosen from shapes and
 * the device's compute-unit count only (never from device data): the grid
 * is one workgroup per resident slot, fewer when shares would drop under
 * min_share_chunks chunks even at the longest contexts the table allows;
 * the kernel lowers it further for the actual lengths by the same rule.
 * When every segment is short (at most 2 * 8 chunks: a short table or a
 * sliding window) and there are enough of them to give every compute unit
 * a workgroup, the plan takes whole segments instead: one workgroup per
 * segment, output written directly, no partials and no merge.
 */
typedef struct pa_plan {
    int32_t rows;               /* (Hq / Hkv) * Qmax query rows per kv head */
    int32_t row_tiles;          /* ceil(rows / 16)                         */
    int32_t heads_per_group;    /* kv heads per workgroup                  */
    int32_t min_share_chunks;   /* smallest share, in 32-token chunks      */
    int32_t reduce_rows;        /* merge workgroup: query rows,            */
    int32_t reduce_col4;        /*   float4 columns per row,               */
    int32_t reduce_lanes;       /*   partial lanes per (row, column)       */
    int32_t expected_partials;  /* partials per row for alike lengths      */
    int32_t whole_segments;     /* 1: one workgroup per segment, no merge  */
    int32_t row_waves;          /* waves per kv head: row_tiles at head_dim
                                   256 (a wave holds one 16-row tile), else 1 */
    int64_t workgroups;         /* partition-kernel grid                   */
    int64_t reduce_groups;      /* workgroups of the merge kernel (0: none) */
    int64_t workspace_bytes;    /* fp32 partials + log-sum-exp + chunk scan */
} pa_plan;

/*
 * paged_attn_plan -- the plan for the given sizes on a device with
 * num_cus compute units (host only; no GPU access).  kv_dtype is a
 * pa_dtype of the cache.  max_context is the most cache tokens one
 * sequence's rows can read: block size x table width, or with a sliding
 * window w at most 32 * (ceil((w + query_len - 1) / 32) + 1) of them
 * (1 <= max_context <= 2^30).  Honors the overrides of
 * paged_attn_tuning.h.
 */
int paged_attn_plan(int64_t batch, int64_t q_heads, int64_t kv_heads, int64_t head_dim,
                    int64_t query_len, int64_t max_context, int32_t kv_dtype,
                    int32_t num_cus, pa_plan* plan);

/*
 * paged_attn_reserve -- grow the current device's workspace for `stream`
 * to at least `bytes` (see pa_plan.workspace_bytes) so that later calls of
 * that size can be captured into a HIP graph.  Allocates with hipMalloc;
 * must not be called while `stream` is capturing.
 */
int paged_attn_reserve(int64_t bytes, void* stream);

/*
 * paged_attn_check_metadata -- host-side check of the device-side
 * preconditions on HOST copies of the metadata: 0 <= query_lens[b] <= Qmax,
 * query_lens[b] <= context_lens[b] <= block_size * W, and every table
 * entry that holds a key some row sees (all of the first
 * ceil(L_b / block_size) without a window; with sliding_window > 0 those
 * from the block of the earliest row's first key) in [0, NB).  query_lens
 * may be NULL (all Qmax).  table_row_stride is in elements.  Returns PA_OK
 * or PA_ERR_ARG (with the first offending sequence in
 * paged_attn_last_error()).
 */
int paged_attn_check_metadata(const int32_t* context_lens, const int32_t* query_lens,
                              const int32_t* block_tables, int64_t batch, int64_t table_width,
                              int64_t table_row_stride, int64_t query_len, int64_t num_blocks,
                              int64_t block_size, int32_t sliding_window);

const char* paged_attn_strerror(int status);
const char* paged_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
