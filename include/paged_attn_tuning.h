/*
 * paged_attn_tuning.h -- measurement and tuning hooks of the paged-KV
 * decode-attention library (libpaged_attn.so), for tests and benchmarks
 * only.  They change process-global state that every later decode call
 * reads (the overrides are plain atomics: a call running concurrently with
 * a change sees either value), so a serving process must not call them.
 * The product interface is paged_attn.h; nothing there depends on these.
 */
#ifndef PAGED_ATTN_TUNING_H
#define PAGED_ATTN_TUNING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * paged_attn_set_workgroups -- override the planner's partition-kernel
 * grid for every later call in the process (positive; the min-share rule
 * still lowers it), or 0 for the automatic choice.  A test and tuning
 * hook.
 */
int paged_attn_set_workgroups(int32_t workgroups);

/*
 * paged_attn_set_min_share -- override the smallest share of 32-token
 * chunks per workgroup (positive), or 0 for the default of 1.  A tuning hook.
 */
int paged_attn_set_min_share(int32_t chunks);

/*
 * paged_attn_set_heads_per_group -- override the planner's kv heads per
 * partition workgroup for every later call in the process (1..8; it must
 * divide kv_heads, and be at most 4 when (Hq / Hkv) * Qmax > 16, at most
 * 4 / ceil((Hq / Hkv) * Qmax / 16) at head_dim 256, or the call fails with
 * PA_ERR_ARG), or 0 for the automatic choice.  A tuning hook.
 */
int paged_attn_set_heads_per_group(int32_t heads);

/*
 * paged_attn_set_write_pieces -- override how many 16-byte row pieces each
 * thread of paged_attn_reshape_and_cache moves (1, 2 or 4), or 0 for the
 * automatic choice (1).
 */
int paged_attn_set_write_pieces(int32_t pieces);

/*
 * Kernel timing for measurement: after paged_attn_profile_begin(n), the
 * next n calls of paged_attn_decode or paged_attn_decode_ext (on any
 * stream) record HIP events
 * before and after each kernel they launch, on the call's stream.
 * paged_attn_profile_end() waits for those events and returns the summed
 * durations in milliseconds of the partition kernel and of the merge
 * kernel and the number of calls recorded, then stops recording.
 */
int paged_attn_profile_begin(int32_t max_calls);
int paged_attn_profile_end(double* partition_ms, double* reduce_ms, int32_t* calls);

/*
 * paged_attn_probe_stream_read -- the streaming-read probe the benchmark
 * uses for the achievable HBM read rate: reads `bytes` (a positive multiple
 * of 16; `src` 16-byte aligned device memory) with 16-byte loads, `unroll`
 * (1, 2, 4, 8 or 16) in flight per thread, in `workgroups` workgroups of
 * `threads` threads (a multiple of 64, at most 1024); grid_stride 0: each
 * workgroup streams its own contiguous range, 1: all workgroups sweep the
 * buffer together.  `sink` is 4 bytes of device memory that the probe may
 * write (it does only if the loaded words fold to one fixed constant).
 * Enqueued on `stream`; returns PA_OK or a negative pa_status.
 */
int paged_attn_probe_stream_read(const void* src, int64_t bytes, int32_t workgroups, int32_t threads,
                                 int32_t unroll, int32_t grid_stride, void* sink, void* stream);

/*
 * paged_attn_probe_gather_read -- the gather probe: reads, for each of the
 * n block ids (device int32, clamped into [0, num_blocks)), block_bytes[j]
 * bytes at arrays[j] + id * block_strides[j] for j = 0..3 (block_bytes[j]
 * a multiple of 16, 0 for an unused array; arrays 16-byte aligned device
 * memory of num_blocks blocks each), in `workgroups` workgroups of
 * `threads` threads with `unroll` (4, 8 or 16) 16-byte loads in flight per
 * thread.  With a cache's K and V (and its two scale arrays) and the block
 * ids a decode call reads, it moves the same bytes from the same places.
 * `sink`: 4 bytes of device memory the probe may write.
 */
int paged_attn_probe_gather_read(const void* const* arrays, const int64_t* block_strides,
                                 const int32_t* block_bytes, const int32_t* block_ids, int32_t n,
                                 int32_t num_blocks, int32_t workgroups, int32_t threads, int32_t unroll,
                                 void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_TUNING_H */
