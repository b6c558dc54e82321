/*
 * A C caller of the library: paged decode attention through the C ABI of
 * paged_attn.h, with device buffers from the HIP runtime API and no other
 * dependency.  Reads one problem from a directory of raw little-endian
 * files, runs paged_attn_decode on the default stream and writes the output
 * beside them.
 *
 *   usage: pa_decode_cli DIR
 *   DIR/meta.txt  "B Qmax Hq Hkv D NB BS W fp8 scale"
 *   DIR/q.bin     bf16 [B, Qmax, Hq, D]        DIR/k_cache.bin, v_cache.bin
 *                                              [NB, BS, Hkv, D] bf16 or e4m3fn
 *   DIR/block_tables.bin int32 [B, W]          DIR/context_lens.bin, query_lens.bin int32 [B]
 *   DIR/k_scale.bin, v_scale.bin   fp32 [NB, Hkv, BS] (fp8 only; passed as the
 *                                  logical [NB, BS, Hkv] with strides (Hkv BS, 1, BS))
 *   -> DIR/out.bin bf16 [B, Qmax, Hq, D]
 *
 * Exit status 0 on success, 50 - status for a library error status (which
 * is negative), 101.. for a local error; the library's last error message
 * goes to stderr.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "paged_attn.h"

static void* read_file(const char* dir, const char* name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    void* buf = malloc(bytes ? bytes : 1);
    size_t got = buf ? fread(buf, 1, bytes, f) : 0;
    fclose(f);
    if (got != bytes) {
        free(buf);
        return NULL;
    }
    return buf;
}

/* device copy of `bytes` host bytes, or (host NULL) an uninitialised buffer */
static void* to_device(const void* host, size_t bytes) {
    void* dev = NULL;
    if (hipMalloc(&dev, bytes ? bytes : 16) != hipSuccess) return NULL;
    if (host && bytes && hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
    return dev;
}

static void describe(pa_tensor* t, void* data, int32_t dtype, int ndim, const int64_t* shape) {
    memset(t, 0, sizeof *t);
    t->data = data;
    t->dtype = dtype;
    t->ndim = ndim;
    int64_t st = 1;
    for (int i = ndim - 1; i >= 0; --i) {
        t->shape[i] = shape[i];
        t->stride[i] = st;
        st *= shape[i];
    }
}

int main(int argc, char** argv) {
    if (argc != 2) {
        fprintf(stderr, "usage: %s DIR\n", argv[0]);
        return 101;
    }
    const char* dir = argv[1];
    long long B, Qmax, Hq, Hkv, D, NB, BS, W;
    int fp8;
    float scale;
    char path[4096];
    snprintf(path, sizeof path, "%s/meta.txt", dir);
    FILE* m = fopen(path, "r");
    if (!m || fscanf(m, "%lld %lld %lld %lld %lld %lld %lld %lld %d %f", &B, &Qmax, &Hq, &Hkv, &D, &NB, &BS, &W,
                     &fp8, &scale) != 10) {
        fprintf(stderr, "cannot read %s\n", path);
        return 102;
    }
    fclose(m);
    const size_t eb = fp8 ? 1 : 2;
    const size_t q_bytes = (size_t)(B * Qmax * Hq * D) * 2;
    const size_t kv_bytes = (size_t)(NB * BS * Hkv * D) * eb;
    const size_t sc_bytes = (size_t)(NB * BS * Hkv) * 4;
    void* h_q = read_file(dir, "q.bin", q_bytes);
    void* h_k = read_file(dir, "k_cache.bin", kv_bytes);
    void* h_v = read_file(dir, "v_cache.bin", kv_bytes);
    void* h_bt = read_file(dir, "block_tables.bin", (size_t)(B * W) * 4);
    void* h_ctx = read_file(dir, "context_lens.bin", (size_t)B * 4);
    void* h_ql = read_file(dir, "query_lens.bin", (size_t)B * 4);
    void* h_ks = fp8 ? read_file(dir, "k_scale.bin", sc_bytes) : NULL;
    void* h_vs = fp8 ? read_file(dir, "v_scale.bin", sc_bytes) : NULL;
    if (!h_q || !h_k || !h_v || !h_bt || !h_ctx || !h_ql || (fp8 && (!h_ks || !h_vs))) {
        fprintf(stderr, "missing or short input file in %s\n", dir);
        return 103;
    }
    void* d_q = to_device(h_q, q_bytes);
    void* d_k = to_device(h_k, kv_bytes);
    void* d_v = to_device(h_v, kv_bytes);
    void* d_bt = to_device(h_bt, (size_t)(B * W) * 4);
    void* d_ctx = to_device(h_ctx, (size_t)B * 4);
    void* d_ql = to_device(h_ql, (size_t)B * 4);
    void* d_ks = fp8 ? to_device(h_ks, sc_bytes) : NULL;
    void* d_vs = fp8 ? to_device(h_vs, sc_bytes) : NULL;
    void* d_out = to_device(NULL, q_bytes);
    if (!d_q || !d_k || !d_v || !d_bt || !d_ctx || !d_ql || !d_out || (fp8 && (!d_ks || !d_vs))) {
        fprintf(stderr, "device allocation or copy failed\n");
        return 104;
    }

    const int64_t s_q[4] = {B, Qmax, Hq, D}, s_kv[4] = {NB, BS, Hkv, D}, s_bt[2] = {B, W}, s_b[1] = {B};
    pa_tensor q, k, v, bt, ctx, ql, out, ks, vs;
    describe(&q, d_q, PA_DTYPE_BF16, 4, s_q);
    describe(&out, d_out, PA_DTYPE_BF16, 4, s_q);
    describe(&k, d_k, fp8 ? PA_DTYPE_FP8_E4M3FN : PA_DTYPE_BF16, 4, s_kv);
    describe(&v, d_v, fp8 ? PA_DTYPE_FP8_E4M3FN : PA_DTYPE_BF16, 4, s_kv);
    describe(&bt, d_bt, PA_DTYPE_INT32, 2, s_bt);
    describe(&ctx, d_ctx, PA_DTYPE_INT32, 1, s_b);
    describe(&ql, d_ql, PA_DTYPE_INT32, 1, s_b);
    /* scales: physical [NB, Hkv, BS], described as the logical [NB, BS, Hkv] */
    const int64_t s_sc[3] = {NB, BS, Hkv};
    describe(&ks, d_ks, PA_DTYPE_FP32, 3, s_sc);
    describe(&vs, d_vs, PA_DTYPE_FP32, 3, s_sc);
    ks.stride[0] = vs.stride[0] = Hkv * BS;
    ks.stride[1] = vs.stride[1] = 1;
    ks.stride[2] = vs.stride[2] = BS;

    int st = paged_attn_decode(&q, &k, &v, &bt, &ctx, &ql, scale, fp8 ? &ks : NULL, fp8 ? &vs : NULL, &out, NULL);
    if (st != PA_OK) {
        fprintf(stderr, "paged_attn_decode: %s: %s\n", paged_attn_strerror(st), paged_attn_last_error());
        return 50 - st;
    }
    if (hipDeviceSynchronize() != hipSuccess) {
        fprintf(stderr, "hipDeviceSynchronize failed\n");
        return 105;
    }
    void* h_out = malloc(q_bytes ? q_bytes : 1);
    if (!h_out || hipMemcpy(h_out, d_out, q_bytes, hipMemcpyDeviceToHost) != hipSuccess) return 106;
    snprintf(path, sizeof path, "%s/out.bin", dir);
    FILE* f = fopen(path, "wb");
    if (!f || fwrite(h_out, 1, q_bytes, f) != q_bytes) return 107;
    fclose(f);
    printf("paged_attn_decode from C: ok, %lld x %lld rows of %lld heads written\n", B, Qmax, Hq);
    return 0;
}
