// Host-side validation of the paged prefill call (plain C++, no device
// access): descriptors, shapes, dtypes and layouts, with the limits the
// kernels' 32-bit offsets and grid set; and the check entry points.
#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "pa_prefill_internal.h"

namespace pa {

int validate_prefill(const pa_tensor* q, const pa_tensor* kc, const pa_tensor* vc, const pa_tensor* bt,
                     const pa_tensor* ctx, const pa_tensor* cu, int32_t max_query_len, float scale,
                     const pa_tensor* ks, const pa_tensor* vs, int32_t window, const pa_tensor* sinks,
                     const pa_tensor* out, PrefillProblem* pr) {
    int st;
    if ((st = check_desc(q, "q", PA_DTYPE_BF16, 3, 3, true))) return st;
    if ((st = check_desc(out, "out", PA_DTYPE_BF16, 3, 3, true))) return st;
    if (!kc) return fail(PA_ERR_NULL, "k_cache: descriptor is NULL");
    if (!vc) return fail(PA_ERR_NULL, "v_cache: descriptor is NULL");
    const int32_t kvt = kc->dtype;
    if (kvt != PA_DTYPE_BF16 && kvt != PA_DTYPE_FP8_E4M3FN)
        return fail(PA_ERR_DTYPE, "k_cache: dtype %s, expected BF16 or FP8_E4M3FN", dtype_name(kvt));
    if ((st = check_desc(kc, "k_cache", kvt, 4, 4, true))) return st;
    if ((st = check_desc(vc, "v_cache", kvt, 4, 4, true))) return st;
    if ((st = check_desc(bt, "block_tables", PA_DTYPE_INT32, 2, 2, true))) return st;
    if ((st = check_desc(ctx, "context_lens", PA_DTYPE_INT32, 1, 1, true))) return st;
    if ((st = check_desc(cu, "cu_seqlens_q", PA_DTYPE_INT32, 1, 1, true))) return st;
    const bool fp8 = kvt == PA_DTYPE_FP8_E4M3FN;
    if (fp8) {
        if (!ks || !vs) return fail(PA_ERR_NULL, "fp8 cache needs k_scale and v_scale");
        if ((st = check_desc(ks, "k_scale", PA_DTYPE_FP32, 3, 3, true))) return st;
        if ((st = check_desc(vs, "v_scale", PA_DTYPE_FP32, 3, 3, true))) return st;
    } else if (ks || vs) {
        return fail(PA_ERR_ARG, "k_scale/v_scale are only accepted with an fp8 cache");
    }
    if (!std::isfinite(scale)) return fail(PA_ERR_ARG, "scale is not finite");
    if (max_query_len < 0) return fail(PA_ERR_ARG, "max_query_len is negative");
    if (sinks && (st = check_desc(sinks, "sinks", PA_DTYPE_FP32, 1, 1, true))) return st;

    const int64_t T = q->shape[0], Hq = q->shape[1], D = q->shape[2];
    for (int i = 0; i < 3; ++i)
        if (out->shape[i] != q->shape[i])
            return fail(PA_ERR_SHAPE, "out: size %lld in dim %d, q has %lld", (long long)out->shape[i], i,
                        (long long)q->shape[i]);
    for (int i = 0; i < 4; ++i)
        if (kc->shape[i] != vc->shape[i])
            return fail(PA_ERR_SHAPE, "v_cache: size %lld in dim %d, k_cache has %lld", (long long)vc->shape[i], i,
                        (long long)kc->shape[i]);
    const int64_t NB = kc->shape[0], BS = kc->shape[1], Hkv = kc->shape[2];
    if (BS < PA_BLOCK_SIZE || BS % PA_BLOCK_SIZE || BS > kMaxBlockSize)
        return fail(PA_ERR_UNSUPPORTED, "k_cache: block size %lld, expected a multiple of 16 up to %d",
                    (long long)BS, kMaxBlockSize);
    if (kc->shape[3] != D)
        return fail(PA_ERR_SHAPE, "k_cache: head_dim %lld, q has %lld", (long long)kc->shape[3], (long long)D);
    if (D != 64 && D != 128 && D != 256)
        return fail(PA_ERR_UNSUPPORTED, "prefill: head_dim %lld, only 64, 128 and 256 are supported", (long long)D);
    if (Hkv < 1) return fail(PA_ERR_SHAPE, "k_cache: no kv heads");
    if (Hkv > kMaxHeads) return fail(PA_ERR_UNSUPPORTED, "k_cache: more than %lld kv heads", (long long)kMaxHeads);
    if (NB > kMaxBlocks) return fail(PA_ERR_UNSUPPORTED, "k_cache: 2^31 blocks or more");
    if (Hq % Hkv != 0 || Hq == 0)
        return fail(PA_ERR_UNSUPPORTED, "q_heads %lld is not a positive multiple of kv_heads %lld",
                    (long long)Hq, (long long)Hkv);
    const int64_t G = Hq / Hkv;
    if (G > PA_MAX_ROWS)
        return fail(PA_ERR_UNSUPPORTED, "prefill: q_heads / kv_heads = %lld exceeds %d", (long long)G, PA_MAX_ROWS);
    if (D == 256 && G > PA_MAX_ROWS_D256)
        return fail(PA_ERR_UNSUPPORTED, "prefill: head_dim 256 takes q_heads / kv_heads up to %d, not %lld",
                    PA_MAX_ROWS_D256, (long long)G);
    const int64_t B = bt->shape[0], W = bt->shape[1];
    if (B >= (int64_t(1) << 31)) return fail(PA_ERR_UNSUPPORTED, "prefill: 2^31 sequences or more");
    if (ctx->shape[0] != B)
        return fail(PA_ERR_SHAPE, "context_lens: %lld entries, block_tables has %lld rows", (long long)ctx->shape[0],
                    (long long)B);
    if (cu->shape[0] != B + 1)
        return fail(PA_ERR_SHAPE, "cu_seqlens_q: %lld entries, expected batch + 1 = %lld", (long long)cu->shape[0],
                    (long long)(B + 1));
    if (T >= (int64_t(1) << 31)) return fail(PA_ERR_UNSUPPORTED, "prefill: too many query rows");
    if (fp8) {
        for (const pa_tensor* s : {ks, vs}) {
            const char* nm = s == ks ? "k_scale" : "v_scale";
            if (s->shape[0] != NB || s->shape[1] != BS || s->shape[2] != Hkv)
                return fail(PA_ERR_SHAPE, "%s: shape must be [num_blocks, block_size, kv_heads]", nm);
            if (s->stride[1] != 1) return fail(PA_ERR_LAYOUT, "%s: the slot dimension must be contiguous", nm);
            if (!aligned(s->data, 4)) return fail(PA_ERR_LAYOUT, "%s: data is not 4-byte aligned", nm);
            if (used_stride(s, 0) * 4 >= (int64_t(1) << 32) || used_stride(s, 2) * 4 >= (int64_t(1) << 32))
                return fail(PA_ERR_LAYOUT, "%s: block or head stride of 4 GiB or more", nm);
        }
    }
    if (sinks) {
        if (sinks->shape[0] != Hq)
            return fail(PA_ERR_SHAPE, "sinks: %lld entries, q has %lld heads", (long long)sinks->shape[0], (long long)Hq);
        if (!aligned(sinks->data, 4)) return fail(PA_ERR_LAYOUT, "sinks: data is not 4-byte aligned");
    }
    if (B > 0 && T > 0) {
        if (W < 1) return fail(PA_ERR_SHAPE, "block_tables: width must be >= 1");
        if (NB < 1) return fail(PA_ERR_SHAPE, "k_cache: the pool has no blocks");
        if (W > kMaxContext / BS) return fail(PA_ERR_UNSUPPORTED, "block_tables: width x block size too large");
    }
    if ((st = check_rows16(q, "q"))) return st;
    if ((st = check_rows16(out, "out"))) return st;
    if ((st = check_rows16(kc, "k_cache"))) return st;
    if ((st = check_rows16(vc, "v_cache"))) return st;
    if (bt->stride[1] != 1 && W > 1) return fail(PA_ERR_LAYOUT, "block_tables: innermost stride must be 1");
    if (!aligned(bt->data, 4) || !aligned(ctx->data, 4) || !aligned(cu->data, 4))
        return fail(PA_ERR_LAYOUT, "int32 metadata must be 4-byte aligned");
    const int64_t eb = fp8 ? 1 : 2;
    for (const pa_tensor* c : {kc, vc}) {
        const int64_t span = sat_add(sat_add(sat_mul(BS - 1, used_stride(c, 1)), sat_mul(Hkv - 1, used_stride(c, 2))), D) * eb;
        if (span >= (int64_t(1) << 31))
            return fail(PA_ERR_LAYOUT, "%s: one block spans more than 2 GiB", c == kc ? "k_cache" : "v_cache");
        if (used_stride(c, 0) * eb >= (int64_t(1) << 32))
            return fail(PA_ERR_LAYOUT, "%s: block stride of 4 GiB or more", c == kc ? "k_cache" : "v_cache");
    }
    if (pr) {
        PrefillProblem& p = *pr;
        p.B = B; p.T = T; p.Hq = Hq; p.Hkv = Hkv; p.G = G; p.D = D; p.NB = NB; p.W = W; p.BS = BS;
        p.scale = scale;
        p.q = q->data; p.q_st = used_stride(q, 0) * 2; p.q_sh = used_stride(q, 1) * 2;
        p.out = out->data; p.o_st = used_stride(out, 0) * 2; p.o_sh = used_stride(out, 1) * 2;
        p.k = kc->data;
        p.k_sblk = used_stride(kc, 0) * eb; p.k_stok = used_stride(kc, 1) * eb; p.k_sh = used_stride(kc, 2) * eb;
        p.v = vc->data;
        p.v_sblk = used_stride(vc, 0) * eb; p.v_stok = used_stride(vc, 1) * eb; p.v_sh = used_stride(vc, 2) * eb;
        p.fp8 = fp8;
        p.ks = fp8 ? static_cast<const float*>(ks->data) : nullptr;
        p.vs = fp8 ? static_cast<const float*>(vs->data) : nullptr;
        p.ks_sblk = fp8 ? used_stride(ks, 0) : 0; p.ks_sh = fp8 ? used_stride(ks, 2) : 0;
        p.vs_sblk = fp8 ? used_stride(vs, 0) : 0; p.vs_sh = fp8 ? used_stride(vs, 2) : 0;
        p.bt = static_cast<const int32_t*>(bt->data); p.bt_sb = used_stride(bt, 0);
        p.ctx = static_cast<const int32_t*>(ctx->data); p.ctx_s = used_stride(ctx, 0);
        p.cu = static_cast<const int32_t*>(cu->data); p.cu_s = used_stride(cu, 0);
        p.window = window > 0 ? window : 0;
        p.sinks = sinks ? static_cast<const float*>(sinks->data) : nullptr;
        p.sinks_s = sinks ? used_stride(sinks, 0) : 0;
    }
    return PA_OK;
}

}  // namespace pa

extern "C" {

int paged_attn_check_prefill(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                             const pa_tensor* block_tables, const pa_tensor* context_lens,
                             const pa_tensor* cu_seqlens_q, int32_t max_query_len, float scale,
                             const pa_tensor* k_scale, const pa_tensor* v_scale, const pa_tensor* out) {
    return pa::validate_prefill(q, k_cache, v_cache, block_tables, context_lens, cu_seqlens_q, max_query_len,
                                scale, k_scale, v_scale, 0, nullptr, out, nullptr);
}

int paged_attn_check_prefill_ext(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                                 const pa_tensor* block_tables, const pa_tensor* context_lens,
                                 const pa_tensor* cu_seqlens_q, int32_t max_query_len, float scale,
                                 const pa_tensor* k_scale, const pa_tensor* v_scale, int32_t sliding_window,
                                 const pa_tensor* sinks, const pa_tensor* out) {
    return pa::validate_prefill(q, k_cache, v_cache, block_tables, context_lens, cu_seqlens_q, max_query_len,
                                scale, k_scale, v_scale, sliding_window, sinks, out, nullptr);
}

}  // extern "C"
