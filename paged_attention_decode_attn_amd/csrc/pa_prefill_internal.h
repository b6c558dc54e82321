// Internal interface between the prefill call's host-side validation
// (pa_prefill_host.cpp, plain C++) and its launch code (pa_prefill.hip).
#pragma once

#include "pa_internal.h"

namespace pa {

// The validated call: byte strides of the tensors, the scale arrays of an
// fp8 cache in floats.
struct PrefillProblem {
    int64_t B, T, Hq, Hkv, G, D, NB, W, BS;
    float scale;
    const void* q;  int64_t q_st, q_sh;                // bytes
    void* out;      int64_t o_st, o_sh;                // bytes
    const void* k;  int64_t k_sblk, k_stok, k_sh;      // bytes
    const void* v;  int64_t v_sblk, v_stok, v_sh;      // bytes
    const int32_t* bt; int64_t bt_sb;                  // int32 elements
    const int32_t* ctx; int64_t ctx_s;
    const int32_t* cu;  int64_t cu_s;
    int32_t window;                                    // sliding window in tokens, 0 = none
    const float* sinks; int64_t sinks_s;               // per query head, may be null
    bool fp8;                                          // e4m3fn cache with per-token scales
    const float* ks; int64_t ks_sblk, ks_sh;           // floats
    const float* vs; int64_t vs_sblk, vs_sh;
};

// Host-side validation of the prefill call (no device access): descriptors,
// shapes, dtypes and layouts; fills *pr when given.
int validate_prefill(const pa_tensor* q, const pa_tensor* kc, const pa_tensor* vc, const pa_tensor* bt,
                     const pa_tensor* ctx, const pa_tensor* cu, int32_t max_query_len, float scale,
                     const pa_tensor* ks, const pa_tensor* vs, int32_t window, const pa_tensor* sinks,
                     const pa_tensor* out, PrefillProblem* pr);

}  // namespace pa
