// Randomised calls of the library's host-only entry points (argument
// validation, planning, metadata checks) for a build with AddressSanitizer
// and UndefinedBehaviorSanitizer: valid descriptors with one to three fields
// replaced by edge values (zero, negative, 2^31, 2^62, INT64 limits,
// misaligned or NULL data).  Every call must return a documented status;
// the sanitizers turn any overflow or stray read into a failure.
// Build: g++ -std=c++17 -fsanitize=address,undefined with pa_host.cpp and
// pa_prefill_host.cpp.  Usage: fuzz_validate ITERATIONS SEED
#include <cinttypes>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <random>
#include <vector>

#include "paged_attn.h"

namespace {

std::mt19937_64 rng;

int64_t pick(std::initializer_list<int64_t> v) { return *(v.begin() + rng() % v.size()); }

int64_t edge() {
    return pick({0, 1, 2, 3, 15, 16, 17, 31, 32, 63, 64, 65, 128, 256, 4096, 4097, 65536, (1LL << 31) - 1,
                 1LL << 31, 1LL << 32, 1LL << 40, 1LL << 62, -1, -16, std::numeric_limits<int64_t>::max(),
                 std::numeric_limits<int64_t>::min()});
}

// a contiguous descriptor of a fake device buffer (never dereferenced)
pa_tensor desc(int32_t dtype, std::vector<int64_t> shape) {
    pa_tensor t;
    std::memset(&t, 0, sizeof t);
    t.data = reinterpret_cast<void*>(uintptr_t(1) << 32);
    t.dtype = dtype;
    t.ndim = int32_t(shape.size());
    int64_t s = 1;
    for (int i = t.ndim - 1; i >= 0; --i) {
        t.shape[i] = shape[i];
        t.stride[i] = s;
        s *= shape[i];
    }
    return t;
}

void mutate(pa_tensor& t) {
    switch (rng() % 6) {
        case 0: t.dtype = int32_t(pick({0, 1, 2, 3, 4, 5, -1})); break;
        case 1: t.ndim = int32_t(pick({-1, 0, 1, 2, 3, 4, 5, 1 << 30})); break;
        case 2: t.shape[rng() % 4] = edge(); break;
        case 3: t.stride[rng() % 4] = edge(); break;
        case 4: t.data = reinterpret_cast<void*>(uintptr_t(pick({0, 1, 8, 4096, 1LL << 47}))); break;
        default: t.shape[rng() % 4] = edge(); t.stride[rng() % 4] = edge(); break;
    }
}

bool documented(int st) { return st <= 0 && st >= PA_ERR_ARG; }

int failures = 0;
long counts[5][10];   // per entry point, per status (0 .. -9)
int current = 0;
void expect(int st, const char* what, long it) {
    if (documented(st)) counts[current][-st]++;
    if (!documented(st)) {
        std::fprintf(stderr, "iteration %ld: %s returned undocumented status %d\n", it, what, st);
        ++failures;
    }
}

void fuzz_decode(long it) {
    const int64_t B = 1 + rng() % 4, Q = 1 + rng() % 3, Hkv = pick({1, 2, 8}), G = pick({1, 2, 4, 8});
    const int64_t D = pick({64, 128, 256}), NB = 1 + rng() % 64, BS = pick({16, 32, 256}), W = 1 + rng() % 8;
    const bool fp8 = rng() % 2;
    const int32_t kv = fp8 ? PA_DTYPE_FP8_E4M3FN : PA_DTYPE_BF16;
    pa_tensor t[10] = {
        desc(PA_DTYPE_BF16, {B, Q, Hkv * G, D}),   // q
        desc(kv, {NB, BS, Hkv, D}),                 // k_cache
        desc(kv, {NB, BS, Hkv, D}),                 // v_cache
        desc(PA_DTYPE_INT32, {B, W}),               // block_tables
        desc(PA_DTYPE_INT32, {B}),                  // context_lens
        desc(PA_DTYPE_INT32, {B}),                  // query_lens
        desc(PA_DTYPE_FP32, {NB, BS, Hkv}),         // k_scale
        desc(PA_DTYPE_FP32, {NB, BS, Hkv}),         // v_scale
        desc(PA_DTYPE_FP32, {Hkv * G}),             // sinks
        desc(PA_DTYPE_BF16, {B, Q, Hkv * G, D}),   // out
    };
    for (int s = 6; s <= 7; ++s) {   // [NB, Hkv, BS] viewed as [NB, BS, Hkv]
        t[s].stride[0] = Hkv * BS;
        t[s].stride[1] = 1;
        t[s].stride[2] = BS;
    }
    float scale = 0.125f;
    int32_t window = int32_t(pick({0, 0, 1, 128, 4096}));
    const int n = int(rng() % 4);
    for (int m = 0; m < n; ++m) {
        const int which = int(rng() % 12);
        if (which < 10) mutate(t[which]);
        else if (which == 10) scale = float(pick({0, -1, 1})) * (rng() % 2 ? INFINITY : 1.f) + (rng() % 3 == 0 ? NAN : 0.f);
        else window = int32_t(pick({-1, 1, 1 << 30, std::numeric_limits<int32_t>::max(), std::numeric_limits<int32_t>::min()}));
    }
    const bool ql = rng() % 4, sinks = rng() % 3 == 0, scales = fp8 ^ (rng() % 8 == 0);
    int st = paged_attn_check_ext(&t[0], &t[1], &t[2], &t[3], &t[4], ql ? &t[5] : nullptr, scale,
                                  scales ? &t[6] : nullptr, scales ? &t[7] : nullptr, window,
                                  sinks ? &t[8] : nullptr, &t[9]);
    expect(st, "paged_attn_check_ext", it);
    // the prefill call's checks on the same cache descriptors: q/out as
    // packed rows [T, Hq, D], cu_seqlens_q int32 [B + 1]
    pa_tensor qp = desc(PA_DTYPE_BF16, {B * Q, Hkv * G, D}), op = qp;
    pa_tensor cu = desc(PA_DTYPE_INT32, {B + 1});
    if (rng() % 2) mutate(rng() % 2 ? qp : op);
    if (rng() % 4 == 0) mutate(cu);
    const int32_t mq = int32_t(rng() % 4 ? Q : pick({-1, 0, std::numeric_limits<int32_t>::max()}));
    st = paged_attn_check_prefill_ext(&qp, &t[1], &t[2], &t[3], &t[4], &cu, mq, scale, scales ? &t[6] : nullptr,
                                      scales ? &t[7] : nullptr, window, sinks ? &t[8] : nullptr, &op);
    current = 4;
    expect(st, "paged_attn_check_prefill_ext", it);
}

void fuzz_write(long it) {
    const int64_t T = rng() % 64, Hkv = pick({1, 2, 8}), D = pick({64, 128, 256}), NB = 1 + rng() % 64;
    const int64_t BS = pick({16, 32, 256});
    const bool fp8 = rng() % 2;
    const int32_t kv = fp8 ? PA_DTYPE_FP8_E4M3FN : PA_DTYPE_BF16;
    pa_tensor t[7] = {
        desc(PA_DTYPE_BF16, {T, Hkv, D}), desc(PA_DTYPE_BF16, {T, Hkv, D}), desc(PA_DTYPE_INT32, {T}),
        desc(kv, {NB, BS, Hkv, D}), desc(kv, {NB, BS, Hkv, D}),
        desc(PA_DTYPE_FP32, {NB, BS, Hkv}), desc(PA_DTYPE_FP32, {NB, BS, Hkv}),
    };
    for (int s = 5; s <= 6; ++s) {
        t[s].stride[0] = Hkv * BS;
        t[s].stride[1] = 1;
        t[s].stride[2] = BS;
    }
    const int n = int(rng() % 4);
    for (int m = 0; m < n; ++m) mutate(t[rng() % 7]);
    const bool scales = fp8 ^ (rng() % 8 == 0);
    expect(paged_attn_check_reshape_and_cache(&t[0], &t[1], &t[2], &t[3], &t[4], scales ? &t[5] : nullptr,
                                              scales ? &t[6] : nullptr),
           "paged_attn_check_reshape_and_cache", it);
}

void fuzz_plan(long it) {
    pa_plan p;
    auto v = [](int64_t ok) { return rng() % 3 ? ok : edge(); };
    const int st = paged_attn_plan(v(1 + rng() % 64), v(pick({8, 32, 64})), v(pick({1, 8})), v(pick({64, 128, 256})),
                                   v(1 + rng() % 4), v(16 * (1 + rng() % 8192)),
                                   int32_t(rng() % 5 ? pick({PA_DTYPE_BF16, PA_DTYPE_FP8_E4M3FN}) : edge()),
                                   int32_t(rng() % 4 ? 256 : edge()), rng() % 50 ? &p : nullptr);
    expect(st, "paged_attn_plan", it);
}

void fuzz_metadata(long it) {
    // host arrays of the declared sizes; extreme values only where the
    // arrays do not depend on them
    const int64_t B = rng() % 5, W = 1 + rng() % 8, stride = W + rng() % 3;
    std::vector<int32_t> ctx(B + 1), ql(B + 1), bt(B * stride + 1);
    for (auto& x : ctx) x = int32_t(rng() % 3 ? rng() % 200 : edge());
    for (auto& x : ql) x = int32_t(rng() % 3 ? rng() % 4 : edge());
    for (auto& x : bt) x = int32_t(rng() % 3 ? rng() % 70 : edge());
    const int64_t bs = rng() % 3 ? pick({1, 16, 32}) : edge();
    const int st = paged_attn_check_metadata(ctx.data(), rng() % 2 ? ql.data() : nullptr, bt.data(), B, W, stride,
                                             rng() % 3 ? 1 + rng() % 4 : edge(), rng() % 3 ? 64 : edge(), bs,
                                             int32_t(rng() % 3 ? 0 : edge()));
    expect(st, "paged_attn_check_metadata", it);
}

}  // namespace

int main(int argc, char** argv) {
    const long iters = argc > 1 ? std::atol(argv[1]) : 100000;
    rng.seed(argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 1);
    long ok = 0;
    for (long it = 0; it < iters; ++it) {
        current = int(it % 4);
        switch (it % 4) {
            case 0: fuzz_decode(it); break;
            case 1: fuzz_write(it); break;
            case 2: fuzz_plan(it); break;
            default: fuzz_metadata(it); break;
        }
        ok++;
    }
    std::printf("%ld calls, %d undocumented statuses\n", ok, failures);
    const char* names[5] = {"check_ext", "check_reshape_and_cache", "plan", "check_metadata", "check_prefill_ext"};
    for (int e = 0; e < 5; ++e) {
        std::printf("%-24s", names[e]);
        for (int k = 0; k < 10; ++k) std::printf(" %7ld", counts[e][k]);
        std::printf("\n");
    }
    return failures ? 1 : 0;
}
