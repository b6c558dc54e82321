// Host-side half of the decode path and shared checks: argument validation, the split-context
// planner, metadata checks and error strings.  Plain C++ with no HIP calls,
// so every function here runs (and is tested) on a machine without a GPU.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "pa_internal.h"

namespace pa {

namespace {
thread_local char g_last_error[512] = "";
std::atomic<int32_t> g_grid_override{0};
std::atomic<int32_t> g_group_override{0};
std::atomic<int32_t> g_share_override{0};

}  // namespace

std::atomic<int32_t> g_write_pieces{0};

int64_t elem_bytes(int32_t dtype) {
    switch (dtype) {
        case PA_DTYPE_BF16: return 2;
        case PA_DTYPE_FP8_E4M3FN: return 1;
        case PA_DTYPE_FP32: return 4;
        case PA_DTYPE_INT32: return 4;
        default: return 0;
    }
}

const char* dtype_name(int32_t dtype) {
    switch (dtype) {
        case PA_DTYPE_BF16: return "BF16";
        case PA_DTYPE_FP8_E4M3FN: return "FP8_E4M3FN";
        case PA_DTYPE_FP32: return "FP32";
        case PA_DTYPE_INT32: return "INT32";
        default: return "unknown";
    }
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t sat_mul(int64_t a, int64_t b) {
    int64_t r;
    return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
}
int64_t sat_add(int64_t a, int64_t b) {
    int64_t r;
    return __builtin_add_overflow(a, b, &r) ? INT64_MAX : r;
}
int64_t used_stride(const pa_tensor* t, int i) { return t->shape[i] > 1 ? t->stride[i] : 0; }

// Rank, dtype, non-negative sizes and strides, sizes and the byte extent
// (the last element's offset plus one) below 2^48, and a data pointer when
// the tensor holds elements.  Every later product of a size or a used
// stride with another bounded size then fits 64 bits.
int check_desc(const pa_tensor* t, const char* name, int32_t dtype, int ndim_lo, int ndim_hi,
               bool need_data) {
    if (!t) return fail(PA_ERR_NULL, "%s: descriptor is NULL", name);
    if (t->ndim < ndim_lo || t->ndim > ndim_hi)
        return fail(PA_ERR_SHAPE, "%s: rank %d, expected %d..%d", name, t->ndim, ndim_lo, ndim_hi);
    if (t->dtype != dtype)
        return fail(PA_ERR_DTYPE, "%s: dtype %s, expected %s", name, dtype_name(t->dtype),
                    dtype_name(dtype));
    bool empty = false;
    int64_t last = 0;                        // element offset of the last element
    for (int i = 0; i < t->ndim; ++i) {
        if (t->shape[i] < 0) return fail(PA_ERR_SHAPE, "%s: negative size in dim %d", name, i);
        if (t->stride[i] < 0) return fail(PA_ERR_LAYOUT, "%s: negative stride in dim %d", name, i);
        if (t->shape[i] >= kMaxSize) return fail(PA_ERR_UNSUPPORTED, "%s: size of dim %d is 2^48 or more", name, i);
        if (t->shape[i] == 0) empty = true;
        else last = sat_add(last, sat_mul(t->shape[i] - 1, used_stride(t, i)));
    }
    if (!empty && sat_mul(sat_add(last, 1), elem_bytes(dtype)) >= kMaxSize)
        return fail(PA_ERR_UNSUPPORTED, "%s: spans 2^48 bytes or more", name);
    if (need_data && !empty && !t->data) return fail(PA_ERR_NULL, "%s: data pointer is NULL", name);
    return PA_OK;
}

// Inner stride 1, other strides multiples of 16 bytes, base 16-byte aligned.
int check_rows16(const pa_tensor* t, const char* name) {
    const int64_t eb = elem_bytes(t->dtype);   // 1, 2 or 4: a divisor of 16
    if (t->stride[t->ndim - 1] != 1 && t->shape[t->ndim - 1] > 1)
        return fail(PA_ERR_LAYOUT, "%s: innermost stride must be 1", name);
    for (int i = 0; i + 1 < t->ndim; ++i)
        if (t->stride[i] % (16 / eb) != 0 && t->shape[i] > 1)
            return fail(PA_ERR_LAYOUT, "%s: stride of dim %d is not a multiple of 16 bytes", name, i);
    if (!aligned(t->data, 16)) return fail(PA_ERR_LAYOUT, "%s: data is not 16-byte aligned", name);
    return PA_OK;
}


int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

int validate(const pa_tensor* q, const pa_tensor* kc, const pa_tensor* vc, const pa_tensor* bt,
             const pa_tensor* ctx, const pa_tensor* ql, float scale, const pa_tensor* ks,
             const pa_tensor* vs, int32_t window, const pa_tensor* sinks, const pa_tensor* out,
             Problem* pr) {
    int st;
    if ((st = check_desc(q, "q", PA_DTYPE_BF16, 3, 4, true))) return st;
    if ((st = check_desc(out, "out", PA_DTYPE_BF16, 3, 4, true))) return st;
    if (!kc) return fail(PA_ERR_NULL, "k_cache: descriptor is NULL");
    if (!vc) return fail(PA_ERR_NULL, "v_cache: descriptor is NULL");
    const int32_t kvt = kc->dtype;
    if (kvt != PA_DTYPE_BF16 && kvt != PA_DTYPE_FP8_E4M3FN)
        return fail(PA_ERR_DTYPE, "k_cache: dtype %s, expected BF16 or FP8_E4M3FN", dtype_name(kvt));
    if ((st = check_desc(kc, "k_cache", kvt, 4, 4, true))) return st;
    if ((st = check_desc(vc, "v_cache", kvt, 4, 4, true))) return st;
    if ((st = check_desc(bt, "block_tables", PA_DTYPE_INT32, 2, 2, true))) return st;
    if ((st = check_desc(ctx, "context_lens", PA_DTYPE_INT32, 1, 1, true))) return st;
    if (ql && (st = check_desc(ql, "query_lens", PA_DTYPE_INT32, 1, 1, true))) return st;
    const bool fp8 = kvt == PA_DTYPE_FP8_E4M3FN;
    if (fp8) {
        if (!ks || !vs) return fail(PA_ERR_NULL, "fp8 cache needs k_scale and v_scale");
        if ((st = check_desc(ks, "k_scale", PA_DTYPE_FP32, 3, 3, true))) return st;
        if ((st = check_desc(vs, "v_scale", PA_DTYPE_FP32, 3, 3, true))) return st;
    } else if (ks || vs) {
        return fail(PA_ERR_ARG, "k_scale/v_scale are only accepted with an fp8 cache");
    }
    if (!std::isfinite(scale)) return fail(PA_ERR_ARG, "scale is not finite");
    if (sinks && (st = check_desc(sinks, "sinks", PA_DTYPE_FP32, 1, 1, true))) return st;

    // ---- sizes
    const bool q3 = q->ndim == 3;
    const int64_t B = q->shape[0];
    const int64_t Qmax = q3 ? 1 : q->shape[1];
    const int64_t Hq = q->shape[q3 ? 1 : 2];
    const int64_t D = q->shape[q3 ? 2 : 3];
    if (out->ndim != q->ndim)
        return fail(PA_ERR_SHAPE, "out: rank %d, q has rank %d", out->ndim, q->ndim);
    for (int i = 0; i < q->ndim; ++i)
        if (out->shape[i] != q->shape[i])
            return fail(PA_ERR_SHAPE, "out: size %lld in dim %d, q has %lld", (long long)out->shape[i],
                        i, (long long)q->shape[i]);
    for (int i = 0; i < 4; ++i)
        if (kc->shape[i] != vc->shape[i])
            return fail(PA_ERR_SHAPE, "v_cache: size %lld in dim %d, k_cache has %lld",
                        (long long)vc->shape[i], i, (long long)kc->shape[i]);
    const int64_t NB = kc->shape[0], BS = kc->shape[1], Hkv = kc->shape[2];
    if (BS < PA_BLOCK_SIZE || BS % PA_BLOCK_SIZE || BS > kMaxBlockSize)
        return fail(PA_ERR_UNSUPPORTED, "k_cache: block size %lld, expected a multiple of 16 up to %d",
                    (long long)BS, kMaxBlockSize);
    if (kc->shape[3] != D)
        return fail(PA_ERR_SHAPE, "k_cache: head_dim %lld, q has %lld", (long long)kc->shape[3], (long long)D);
    if (D != 64 && D != 128 && D != 256)
        return fail(PA_ERR_UNSUPPORTED, "head_dim %lld, only 64, 128 and 256 are supported", (long long)D);
    if (Hkv < 1) return fail(PA_ERR_SHAPE, "k_cache: no kv heads");
    if (Hkv > kMaxHeads) return fail(PA_ERR_UNSUPPORTED, "k_cache: more than %lld kv heads", (long long)kMaxHeads);
    if (NB > kMaxBlocks) return fail(PA_ERR_UNSUPPORTED, "k_cache: 2^31 blocks or more");
    if (Hq % Hkv != 0 || Hq == 0)
        return fail(PA_ERR_UNSUPPORTED, "q_heads %lld is not a positive multiple of kv_heads %lld",
                    (long long)Hq, (long long)Hkv);
    const int64_t G = Hq / Hkv;
    if (Qmax < 1) return fail(PA_ERR_SHAPE, "q: query length must be >= 1");
    if (G > PA_MAX_ROWS || Qmax > PA_MAX_ROWS || G * Qmax > PA_MAX_ROWS)
        return fail(PA_ERR_UNSUPPORTED, "(q_heads / kv_heads) * query_len = %lld exceeds %d",
                    (long long)(G * Qmax), PA_MAX_ROWS);
    if (bt->shape[0] != B)
        return fail(PA_ERR_SHAPE, "block_tables: %lld rows, batch is %lld", (long long)bt->shape[0], (long long)B);
    if (B > kMaxBatch)
        return fail(PA_ERR_UNSUPPORTED, "batch %lld exceeds %d sequences", (long long)B, kMaxBatch);
    const int64_t W = bt->shape[1];
    if (ctx->shape[0] != B)
        return fail(PA_ERR_SHAPE, "context_lens: %lld entries, batch is %lld", (long long)ctx->shape[0], (long long)B);
    if (ql && ql->shape[0] != B)
        return fail(PA_ERR_SHAPE, "query_lens: %lld entries, batch is %lld", (long long)ql->shape[0], (long long)B);
    if (fp8) {
        for (const pa_tensor* s : {ks, vs}) {
            const char* nm = s == ks ? "k_scale" : "v_scale";
            if (s->shape[0] != NB || s->shape[1] != BS || s->shape[2] != Hkv)
                return fail(PA_ERR_SHAPE, "%s: shape must be [num_blocks, block_size, kv_heads]", nm);
            if (s->stride[1] != 1)
                return fail(PA_ERR_LAYOUT, "%s: the slot dimension must be contiguous", nm);
            if (s->stride[0] % 4 || s->stride[2] % 4 || !aligned(s->data, 16))
                return fail(PA_ERR_LAYOUT, "%s: strides of dims 0 and 2 must be multiples of 4 and data 16-byte aligned", nm);
        }
    }
    if (sinks) {
        if (sinks->shape[0] != Hq)
            return fail(PA_ERR_SHAPE, "sinks: %lld entries, q has %lld heads", (long long)sinks->shape[0], (long long)Hq);
        if (!aligned(sinks->data, 4)) return fail(PA_ERR_LAYOUT, "sinks: data is not 4-byte aligned");
    }
    if (B > 0) {
        if (W < 1) return fail(PA_ERR_SHAPE, "block_tables: width must be >= 1");
        if (NB < 1) return fail(PA_ERR_SHAPE, "k_cache: the pool has no blocks");
        if (W > kMaxContext / BS) return fail(PA_ERR_UNSUPPORTED, "block_tables: width x block size too large");
    }

    // ---- layouts
    if ((st = check_rows16(q, "q"))) return st;
    if ((st = check_rows16(out, "out"))) return st;
    if ((st = check_rows16(kc, "k_cache"))) return st;
    if ((st = check_rows16(vc, "v_cache"))) return st;
    if (bt->stride[1] != 1 && W > 1) return fail(PA_ERR_LAYOUT, "block_tables: innermost stride must be 1");
    if (!aligned(bt->data, 4) || !aligned(ctx->data, 4) || (ql && !aligned(ql->data, 4)))
        return fail(PA_ERR_LAYOUT, "int32 metadata must be 4-byte aligned");
    const int64_t eb = fp8 ? 1 : 2;
    // in-block byte offsets of the kernels are 32-bit
    for (const pa_tensor* c : {kc, vc}) {
        const int64_t span = sat_add(sat_add(sat_mul(BS - 1, used_stride(c, 1)), sat_mul(Hkv - 1, used_stride(c, 2))), D) * eb;
        if (span >= (int64_t(1) << 31))
            return fail(PA_ERR_LAYOUT, "%s: one block spans more than 2 GiB", c == kc ? "k_cache" : "v_cache");
        // block strides are 32-bit byte counts in the kernels
        if (used_stride(c, 0) * eb >= (int64_t(1) << 32))
            return fail(PA_ERR_LAYOUT, "%s: block stride of 4 GiB or more", c == kc ? "k_cache" : "v_cache");
    }
    if (fp8)
        for (const pa_tensor* s : {ks, vs})
            if (used_stride(s, 0) * 4 >= (int64_t(1) << 32) || used_stride(s, 2) * 4 >= (int64_t(1) << 31))
                return fail(PA_ERR_LAYOUT, "%s: block stride of 4 GiB or more", s == ks ? "k_scale" : "v_scale");

    if (pr) {
        Problem& p = *pr;
        p.B = B; p.Qmax = Qmax; p.Hq = Hq; p.Hkv = Hkv; p.G = G; p.D = D; p.NB = NB; p.W = W; p.BS = BS;
        p.fp8 = fp8; p.scale = scale;
        p.window = window > 0 ? window : 0;
        p.sinks = sinks ? static_cast<const float*>(sinks->data) : nullptr;
        p.sinks_s = sinks ? used_stride(sinks, 0) : 0;
        p.q = q->data;
        p.q_sb = used_stride(q, 0); p.q_st = q3 ? 0 : used_stride(q, 1); p.q_sh = used_stride(q, q3 ? 1 : 2);
        p.out = out->data;
        p.o_sb = used_stride(out, 0); p.o_st = q3 ? 0 : used_stride(out, 1); p.o_sh = used_stride(out, q3 ? 1 : 2);
        p.k = kc->data;
        p.k_sblk = used_stride(kc, 0) * eb; p.k_stok = used_stride(kc, 1) * eb; p.k_sh = used_stride(kc, 2) * eb;
        p.v = vc->data;
        p.v_sblk = used_stride(vc, 0) * eb; p.v_stok = used_stride(vc, 1) * eb; p.v_sh = used_stride(vc, 2) * eb;
        p.ks = fp8 ? static_cast<const float*>(ks->data) : nullptr;
        p.vs = fp8 ? static_cast<const float*>(vs->data) : nullptr;
        p.ks_sblk = fp8 ? used_stride(ks, 0) : 0; p.ks_sh = fp8 ? used_stride(ks, 2) : 0;
        p.vs_sblk = fp8 ? used_stride(vs, 0) : 0; p.vs_sh = fp8 ? used_stride(vs, 2) : 0;
        p.bt = static_cast<const int32_t*>(bt->data); p.bt_sb = used_stride(bt, 0);
        p.ctx = static_cast<const int32_t*>(ctx->data); p.ctx_s = used_stride(ctx, 0);
        p.ql = ql ? static_cast<const int32_t*>(ql->data) : nullptr; p.ql_s = ql ? used_stride(ql, 0) : 0;
    }
    return PA_OK;
}

int validate_write(const pa_tensor* kn, const pa_tensor* vn, const pa_tensor* sm, const pa_tensor* kc,
                   const pa_tensor* vc, const pa_tensor* ks, const pa_tensor* vs, WriteProblem* pr) {
    int st;
    if ((st = check_desc(kn, "k_new", PA_DTYPE_BF16, 3, 3, true))) return st;
    if ((st = check_desc(vn, "v_new", PA_DTYPE_BF16, 3, 3, true))) return st;
    if ((st = check_desc(sm, "slot_mapping", PA_DTYPE_INT32, 1, 1, true))) return st;
    if (!kc) return fail(PA_ERR_NULL, "k_cache: descriptor is NULL");
    if (!vc) return fail(PA_ERR_NULL, "v_cache: descriptor is NULL");
    const int32_t kvt = kc->dtype;
    if (kvt != PA_DTYPE_BF16 && kvt != PA_DTYPE_FP8_E4M3FN)
        return fail(PA_ERR_DTYPE, "k_cache: dtype %s, expected BF16 or FP8_E4M3FN", dtype_name(kvt));
    if ((st = check_desc(kc, "k_cache", kvt, 4, 4, true))) return st;
    if ((st = check_desc(vc, "v_cache", kvt, 4, 4, true))) return st;
    const bool fp8 = kvt == PA_DTYPE_FP8_E4M3FN;
    if (fp8) {
        if (!ks || !vs) return fail(PA_ERR_NULL, "fp8 cache needs k_scale and v_scale");
        if ((st = check_desc(ks, "k_scale", PA_DTYPE_FP32, 3, 3, true))) return st;
        if ((st = check_desc(vs, "v_scale", PA_DTYPE_FP32, 3, 3, true))) return st;
    } else if (ks || vs) {
        return fail(PA_ERR_ARG, "k_scale/v_scale are only accepted with an fp8 cache");
    }
    const int64_t T = kn->shape[0], Hkv = kn->shape[1], D = kn->shape[2];
    for (int i = 0; i < 3; ++i)
        if (vn->shape[i] != kn->shape[i])
            return fail(PA_ERR_SHAPE, "v_new: size %lld in dim %d, k_new has %lld", (long long)vn->shape[i], i,
                        (long long)kn->shape[i]);
    if (sm->shape[0] != T)
        return fail(PA_ERR_SHAPE, "slot_mapping: %lld entries, %lld new tokens", (long long)sm->shape[0], (long long)T);
    for (int i = 0; i < 4; ++i)
        if (kc->shape[i] != vc->shape[i])
            return fail(PA_ERR_SHAPE, "v_cache: size %lld in dim %d, k_cache has %lld", (long long)vc->shape[i], i,
                        (long long)kc->shape[i]);
    const int64_t NB = kc->shape[0], BS = kc->shape[1];
    if (BS < PA_BLOCK_SIZE || BS % PA_BLOCK_SIZE || BS > kMaxBlockSize)
        return fail(PA_ERR_UNSUPPORTED, "k_cache: block size %lld, expected a multiple of 16 up to %d",
                    (long long)BS, kMaxBlockSize);
    if (kc->shape[2] != Hkv || kc->shape[3] != D)
        return fail(PA_ERR_SHAPE, "k_cache: [%lld, %lld, %lld, %lld], new tokens are [T, %lld, %lld]",
                    (long long)NB, (long long)BS, (long long)kc->shape[2], (long long)kc->shape[3], (long long)Hkv,
                    (long long)D);
    if (D != 64 && D != 128 && D != 256)
        return fail(PA_ERR_UNSUPPORTED, "head_dim %lld, only 64, 128 and 256 are supported", (long long)D);
    if (Hkv < 1) return fail(PA_ERR_SHAPE, "no kv heads");
    if (Hkv > kMaxHeads) return fail(PA_ERR_UNSUPPORTED, "more than %lld kv heads", (long long)kMaxHeads);
    if (NB * BS >= (int64_t(1) << 31))
        return fail(PA_ERR_UNSUPPORTED, "pool of %lld blocks: slots do not fit int32", (long long)NB);
    if (sat_mul(T, Hkv * (D / 8)) >= (int64_t(1) << 40)) return fail(PA_ERR_UNSUPPORTED, "too many new tokens");
    if (fp8) {
        for (const pa_tensor* s : {ks, vs}) {
            const char* nm = s == ks ? "k_scale" : "v_scale";
            if (s->shape[0] != NB || s->shape[1] != BS || s->shape[2] != Hkv)
                return fail(PA_ERR_SHAPE, "%s: shape must be [num_blocks, block_size, kv_heads]", nm);
            if (s->stride[1] != 1) return fail(PA_ERR_LAYOUT, "%s: the slot dimension must be contiguous", nm);
            if (!aligned(s->data, 4)) return fail(PA_ERR_LAYOUT, "%s: data is not 4-byte aligned", nm);
        }
    }
    if ((st = check_rows16(kn, "k_new"))) return st;
    if ((st = check_rows16(vn, "v_new"))) return st;
    if ((st = check_rows16(kc, "k_cache"))) return st;
    if ((st = check_rows16(vc, "v_cache"))) return st;
    if (!aligned(sm->data, 4)) return fail(PA_ERR_LAYOUT, "slot_mapping: data is not 4-byte aligned");
    if (pr) {
        WriteProblem& p = *pr;
        const int64_t eb = fp8 ? 1 : 2;
        p.T = T; p.Hkv = Hkv; p.D = D; p.NB = NB; p.BS = BS; p.fp8 = fp8;
        p.k_new = kn->data; p.kn_st = used_stride(kn, 0) * 2; p.kn_sh = used_stride(kn, 1) * 2;
        p.v_new = vn->data; p.vn_st = used_stride(vn, 0) * 2; p.vn_sh = used_stride(vn, 1) * 2;
        p.slots = static_cast<const int32_t*>(sm->data); p.slot_s = used_stride(sm, 0);
        p.kc = kc->data;
        p.k_sblk = used_stride(kc, 0) * eb; p.k_stok = used_stride(kc, 1) * eb; p.k_sh = used_stride(kc, 2) * eb;
        p.vc = vc->data;
        p.v_sblk = used_stride(vc, 0) * eb; p.v_stok = used_stride(vc, 1) * eb; p.v_sh = used_stride(vc, 2) * eb;
        p.ks = fp8 ? static_cast<float*>(ks->data) : nullptr;
        p.vs = fp8 ? static_cast<float*>(vs->data) : nullptr;
        p.ks_sblk = fp8 ? used_stride(ks, 0) : 0; p.ks_sh = fp8 ? used_stride(ks, 2) : 0;
        p.vs_sblk = fp8 ? used_stride(vs, 0) : 0; p.vs_sh = fp8 ? used_stride(vs, 2) : 0;
    }
    return PA_OK;
}

int64_t max_context_tokens(int64_t block_size, int64_t table_width, int32_t window, int64_t Qmax) {
    const int64_t reach = block_size * table_width;
    if (window <= 0) return reach;
    // rows t < Qmax read keys from L - Qmax - window + 1 to L - 1: at most
    // window + Qmax - 1 tokens, over one more chunk when not aligned
    const int64_t span = int64_t(window) + Qmax - 1;
    return std::min<int64_t>(reach, ((span + kChunkTokens - 1) / kChunkTokens + 1) * kChunkTokens);
}

int make_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t Qmax, int64_t max_context, bool fp8,
              int32_t num_cus, pa_plan* plan) {
    if (!plan) return fail(PA_ERR_NULL, "plan: NULL");
    if (B < 0 || Hkv < 1 || Hq < Hkv || Hq % Hkv || Qmax < 1 || max_context < 1 || max_context > kMaxContext ||
        num_cus < 1 || D < 1)
        return fail(PA_ERR_ARG, "plan: invalid sizes");
    if (B > kMaxBatch || Hkv > kMaxHeads || Hq / Hkv > PA_MAX_ROWS || Qmax > PA_MAX_ROWS ||
        (Hq / Hkv) * Qmax > PA_MAX_ROWS || (D != 64 && D != 128 && D != 256))
        return fail(PA_ERR_UNSUPPORTED, "plan: sizes outside what the kernels serve");
    const int64_t rows = (Hq / Hkv) * Qmax;
    const int64_t row_tiles = (rows + 15) / 16;
    // waves per kv head: a head_dim-256 wave holds one 16-row tile
    const int64_t P = D == 256 ? row_tiles : 1;
    // waves one CU holds for the kernel variant (register budget) and the
    // largest kv-head group (P waves per head) a workgroup may carry
    const bool one_tile = row_tiles == 1 && D <= 128;
    const int64_t cu_waves = one_tile ? (fp8 && D == 64 ? 12 : 8) : 4;
    const int64_t hg_cap = (one_tile ? 8 : 4) / P;
    // waves per CU the plan aims at: what the CU holds, except at head_dim
    // 256, where two waves per CU (more only when one kv head needs more)
    // read faster than four: each wave keeps a 32 KB step in flight, and
    // fewer, longer shares cost less than the extra occupancy (measured:
    // 2 kv heads of 8-32 rows 4-8.5 % faster, 8 kv heads the same)
    const int64_t cu_target = D == 256 ? std::max<int64_t>(2, P) : cu_waves;
    // chunk space: 32-token chunks of every (sequence, head group) segment;
    // only its upper bound is known here (lengths live on the device)
    const int64_t seq_chunks = (max_context + kChunkTokens - 1) / kChunkTokens;
    // Waves: about kStepsPerWave chunks each for the (kv head, chunk) pairs
    // the shapes suggest (the whole table for one sequence, half of it per
    // sequence of a ragged batch), at least a quarter of the CUs, at most
    // what the chip holds.  Each wave has a startup chain (prefix scan,
    // block-table window, first loads) and an epilogue that few steps cannot
    // amortise, while a call that is short overall wants many CUs.
    const int64_t per_seq = B > 1 ? (seq_chunks + 1) / 2 : seq_chunks;
    const int64_t wave_slots = int64_t(num_cus) * cu_waves;
    const int64_t waves = std::max<int64_t>(std::min<int64_t>(B * Hkv * P * per_seq / kStepsPerWave, wave_slots),
                                            std::max<int64_t>(1, num_cus / 4));
    // Heads per workgroup: the largest group that divides kv_heads, fits the
    // CU and still leaves a workgroup for every CU.  The waves of a workgroup
    // read the adjacent head rows of the same tokens (all heads of a token
    // are adjacent in the cache), which the memory system serves faster
    // than the same bytes in per-head pieces.
    const int64_t hg_over = g_group_override.load();
    int64_t HG = 1;
    if (hg_over > 0) {
        HG = hg_over;
    } else {
        for (int64_t h = hg_cap; h >= 1; --h)
            if (Hkv % h == 0 && h * P <= cu_target && waves / (h * P) >= num_cus) { HG = h; break; }
    }
    if (Hkv % HG || HG > hg_cap) return fail(PA_ERR_ARG, "plan: heads per group must divide kv_heads and fit the kernel");
    const int64_t max_chunks = B * (Hkv / HG) * seq_chunks;
    if (max_chunks >= (int64_t(1) << 31)) return fail(PA_ERR_UNSUPPORTED, "batch x context too large for the chunk index");
    // Whole segments: every segment is short and there is one for every CU
    // (the head group chosen so), so splitting would only add partials and
    // a merge.  Overrides of the grid or the share keep the split.
    if (seq_chunks <= kWholeSegmentChunks && g_grid_override.load() <= 0 && g_share_override.load() <= 0) {
        int64_t hg = hg_over > 0 ? HG : 1;
        if (hg_over <= 0)
            for (int64_t h = hg_cap; h >= 1; --h)
                if (Hkv % h == 0 && h * P <= cu_target && B * (Hkv / h) >= num_cus) { hg = h; break; }
        if (B * (Hkv / hg) >= num_cus) {
            plan->rows = int32_t(rows);
            plan->row_tiles = int32_t(row_tiles);
            plan->heads_per_group = int32_t(hg);
            plan->min_share_chunks = int32_t(seq_chunks);
            plan->reduce_rows = plan->reduce_col4 = plan->reduce_lanes = 1;
            plan->expected_partials = 0;
            plan->whole_segments = 1;
            plan->row_waves = int32_t(P);
            plan->workgroups = B * (Hkv / hg);
            plan->reduce_groups = 0;
            plan->workspace_bytes = 0;
            return PA_OK;
        }
    }
    const int64_t share_over = g_share_override.load();
    const int64_t min_share = share_over > 0 ? share_over : kDefaultMinShare;
    const int64_t slots = int64_t(num_cus) * std::max<int64_t>(1, cu_target / (HG * P));
    const int64_t grid_over = g_grid_override.load();
    int64_t n = grid_over > 0 ? grid_over : std::min<int64_t>(std::max<int64_t>(1, waves / (HG * P)), slots);
    n = std::max<int64_t>(1, std::min<int64_t>(n, max_chunks / min_share));
    // Two waves per SIMD whose token-head rows are 256 bytes or more: the
    // same grid with half the heads per workgroup, one wave per SIMD, each
    // wave streaming twice as many chunks.  One wave keeps enough bytes in
    // flight at these row sizes and no longer shares its SIMD's issue and
    // memory arbitration (measured: 131072-token calls 3.8 % faster, with
    // 256-token blocks 10 % faster and no longer placement-sensitive, MTP
    // verify 2 % faster, MHA unchanged; head_dim-64 rows of 64 or 128 bytes
    // lose).
    // (Halving doubles the segments, so the chunk index must still fit.)
    if (hg_over <= 0 && HG % 2 == 0 && n * HG >= 8 * int64_t(num_cus) && D * (fp8 ? 1 : 2) >= 256 &&
        2 * max_chunks < (int64_t(1) << 31))
        HG /= 2;
    // Merge shape.  Expected partials per row: one per workgroup whose share
    // meets the row's segment, about n / (B * groups) + 1 when the lengths are
    // alike (a lopsided batch only takes more rounds of loads), exactly n for
    // a single segment.  PL lanes with 8 loads in flight each cover that in
    // one round; the rest of the 256 threads go to float4 columns (CB, at
    // least 8: 128 contiguous bytes of each partial) and rows of the same
    // segment (RG).
    const int64_t segs = std::max<int64_t>(1, B * (Hkv / HG));
    const int64_t expected = segs == 1 ? n : (n + segs - 1) / segs + 1;
    int64_t PL = 1;
    while (PL * kRedUnroll < expected && PL < 32) PL *= 2;
    const int64_t G = Hq / Hkv;
    const int64_t col4 = D / 4;
    const int64_t CB = std::min<int64_t>(col4, kRedThreads / PL);
    int64_t RG = 1;
    while (RG * 2 * CB * PL <= kRedThreads && G % (RG * 2) == 0) RG *= 2;
    plan->rows = int32_t(rows);
    plan->row_tiles = int32_t(row_tiles);
    plan->heads_per_group = int32_t(HG);
    plan->min_share_chunks = int32_t(min_share);
    plan->reduce_rows = int32_t(RG);
    plan->reduce_col4 = int32_t(CB);
    plan->reduce_lanes = int32_t(PL);
    plan->expected_partials = int32_t(std::min<int64_t>(expected, INT32_MAX));
    plan->whole_segments = 0;
    plan->row_waves = int32_t(P);
    plan->workgroups = n;
    plan->reduce_groups = n > 1 ? B * Qmax * Hkv * (G / RG) * (col4 / CB) : 0;
    plan->workspace_bytes = n > 1 ? 2 * n * HG * rows * (D + 1) * int64_t(sizeof(float)) + B * int64_t(sizeof(int32_t)) : 0;
    if (plan->reduce_groups >= (int64_t(1) << 31)) return fail(PA_ERR_UNSUPPORTED, "grid too large");
    return PA_OK;
}

}  // namespace pa

extern "C" {

int paged_attn_check(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                     const pa_tensor* block_tables, const pa_tensor* context_lens,
                     const pa_tensor* query_lens, float scale, const pa_tensor* k_scale,
                     const pa_tensor* v_scale, const pa_tensor* out) {
    return pa::validate(q, k_cache, v_cache, block_tables, context_lens, query_lens, scale, k_scale,
                        v_scale, 0, nullptr, out, nullptr);
}

int paged_attn_check_ext(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                         const pa_tensor* block_tables, const pa_tensor* context_lens,
                         const pa_tensor* query_lens, float scale, const pa_tensor* k_scale,
                         const pa_tensor* v_scale, int32_t sliding_window, const pa_tensor* sinks,
                         const pa_tensor* out) {
    return pa::validate(q, k_cache, v_cache, block_tables, context_lens, query_lens, scale, k_scale,
                        v_scale, sliding_window, sinks, out, nullptr);
}

int paged_attn_check_reshape_and_cache(const pa_tensor* k_new, const pa_tensor* v_new,
                                       const pa_tensor* slot_mapping, const pa_tensor* k_cache,
                                       const pa_tensor* v_cache, const pa_tensor* k_scale,
                                       const pa_tensor* v_scale) {
    return pa::validate_write(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, nullptr);
}

int paged_attn_plan(int64_t batch, int64_t q_heads, int64_t kv_heads, int64_t head_dim,
                    int64_t query_len, int64_t max_context, int32_t kv_dtype, int32_t num_cus,
                    pa_plan* plan) {
    if (kv_dtype != PA_DTYPE_BF16 && kv_dtype != PA_DTYPE_FP8_E4M3FN)
        return pa::fail(PA_ERR_DTYPE, "plan: kv dtype must be BF16 or FP8_E4M3FN");
    return pa::make_plan(batch, q_heads, kv_heads, head_dim, query_len, max_context,
                         kv_dtype == PA_DTYPE_FP8_E4M3FN, num_cus, plan);
}

int paged_attn_set_workgroups(int32_t workgroups) {
    if (workgroups < 0) return pa::fail(PA_ERR_ARG, "workgroups must be 0 (automatic) or positive");
    pa::g_grid_override.store(workgroups);
    return PA_OK;
}

int paged_attn_set_min_share(int32_t chunks) {
    if (chunks < 0) return pa::fail(PA_ERR_ARG, "min share must be 0 (automatic) or positive");
    pa::g_share_override.store(chunks);
    return PA_OK;
}

int paged_attn_set_write_pieces(int32_t pieces) {
    if (pieces != 0 && pieces != 1 && pieces != 2 && pieces != 4)
        return pa::fail(PA_ERR_ARG, "write pieces per thread must be 0 (automatic), 1, 2 or 4");
    pa::g_write_pieces.store(pieces);
    return PA_OK;
}

int paged_attn_set_heads_per_group(int32_t heads) {
    if (heads < 0 || heads > 8) return pa::fail(PA_ERR_ARG, "heads per group must be 0 (automatic) or 1..8");
    pa::g_group_override.store(heads);
    return PA_OK;
}

int paged_attn_check_metadata(const int32_t* context_lens, const int32_t* query_lens,
                              const int32_t* block_tables, int64_t batch, int64_t table_width,
                              int64_t table_row_stride, int64_t query_len, int64_t num_blocks,
                              int64_t block_size, int32_t sliding_window) {
    if (batch < 0 || table_width < 0 || query_len < 1 || num_blocks < 0 || table_row_stride < table_width ||
        block_size < 1)
        return pa::fail(PA_ERR_ARG, "check_metadata: invalid sizes");
    if (batch > 0 && (!context_lens || !block_tables))
        return pa::fail(PA_ERR_NULL, "check_metadata: NULL metadata");
    for (int64_t b = 0; b < batch; ++b) {
        const int64_t L = context_lens[b];
        const int64_t n = query_lens ? query_lens[b] : query_len;
        if (n < 0 || n > query_len)
            return pa::fail(PA_ERR_ARG, "sequence %lld: query_len %lld outside [0, %lld]", (long long)b,
                            (long long)n, (long long)query_len);
        const int64_t reach = pa::sat_mul(block_size, table_width);
        if (L < n || L > reach)
            return pa::fail(PA_ERR_ARG, "sequence %lld: context_len %lld outside [%lld, %lld]", (long long)b,
                            (long long)L, (long long)n, (long long)reach);
        if (n == 0) continue;
        // the entries the kernels read: blocks holding keys some row sees
        const int64_t lo = sliding_window > 0 ? std::max<int64_t>(0, L - n - sliding_window + 1) : 0;
        const int64_t used = L / block_size + (L % block_size != 0);
        for (int64_t i = lo / block_size; i < used; ++i) {
            const int64_t blk = block_tables[b * table_row_stride + i];
            if (blk < 0 || blk >= num_blocks)
                return pa::fail(PA_ERR_ARG, "sequence %lld: block_tables[%lld] = %lld outside [0, %lld)",
                                (long long)b, (long long)i, (long long)blk, (long long)num_blocks);
        }
    }
    return PA_OK;
}

const char* paged_attn_strerror(int status) {
    switch (status) {
        case PA_OK: return "success";
        case PA_ERR_NULL: return "a required tensor or data pointer is NULL";
        case PA_ERR_DTYPE: return "a tensor has the wrong dtype";
        case PA_ERR_SHAPE: return "tensor ranks or sizes are inconsistent";
        case PA_ERR_UNSUPPORTED: return "unsupported configuration";
        case PA_ERR_LAYOUT: return "unsupported memory layout (strides or alignment)";
        case PA_ERR_CAPTURE: return "workspace must grow while the stream is capturing";
        case PA_ERR_HIP: return "HIP runtime error";
        case PA_ERR_NOMEM: return "out of device memory";
        case PA_ERR_ARG: return "invalid argument";
        default: return "unknown status";
    }
}

const char* paged_attn_last_error(void) { return pa::g_last_error; }

}  // extern "C"
