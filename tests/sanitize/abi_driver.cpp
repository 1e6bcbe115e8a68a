// CPU driver for the sanitizer build of libtwq's C ABI layer: calls every entry point
// that twq_api.cpp defines, on buffers allocated at exactly the documented sizes (so
// AddressSanitizer sees any access past them; stub_launch.cpp touches every byte the
// kernels would), over ragged and edge-case shapes, then with invalid arguments that
// must be rejected before any launch. Exit status 0 means every call returned the
// expected status and no sanitizer reported an error.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "twq.h"

namespace {

int g_fail = 0;
std::vector<void *> g_blocks;

void *buf(size_t bytes) {
    void *p = nullptr;
    if (posix_memalign(&p, 16, bytes ? bytes : 16)) std::abort();
    std::memset(p, 0, bytes ? bytes : 16);
    g_blocks.push_back(p);
    return p;
}

void release() {
    for (void *p : g_blocks) std::free(p);
    g_blocks.clear();
}

void expect(int got, int want, const char *what, int64_t b, int64_t m, int64_t n, int64_t r) {
    if (got != want) {
        std::fprintf(stderr, "FAIL %s b=%lld m=%lld n=%lld r=%lld: status %d, expected %d\n", what, (long long)b,
                     (long long)m, (long long)n, (long long)r, got, want);
        ++g_fail;
    }
}

#define CHECK(call, want) expect((call), (want), #call, b, m, n, r)

void valid_calls(int64_t b, int64_t m, int64_t n, int64_t r) {
    const int64_t g = 128, ng = m / g;
    void *x = buf(b * m * 2), *w = buf(n * m * 4), *l1t = buf(r * m * 2), *l2t = buf(n * r * 2);
    void *qx = buf(b * m / 2), *qx8 = buf(b * m), *qw = buf(n * m / 2);
    float *sx = (float *)buf(b * 4), *sxg = (float *)buf(ng * b * 4), *sw = (float *)buf(n * 4);
    float *swg = (float *)buf(ng * n * 4), *t = (float *)buf(b * r * 4);
    void *y = buf(b * n * 2);
    int32_t *acc = (int32_t *)buf(b * n * 4);
    const size_t wq = twq_quantize_act_workspace_bytes(b, m, r);
    void *wsq = buf(wq);

    CHECK(twq_pack_weight((const float *)w, n, m, qw, sw, nullptr), TWQ_OK);
    CHECK(twq_quantize_act(x, b, m, qx, sx, r ? l1t : nullptr, r, r ? t : nullptr, wsq, wq, nullptr), TWQ_OK);
    CHECK(twq_dual_linear(qx, sx, qw, sw, r ? t : nullptr, r ? l2t : nullptr, r, y, b, m, n, nullptr), TWQ_OK);
    CHECK(twq_debug_residual_acc(qx, qw, acc, b, m, n, nullptr), TWQ_OK);
    const size_t wl = twq_linear_workspace_bytes(b, m, n, r);
    void *wsl = buf(wl);
    CHECK(twq_linear(x, qw, sw, r ? l1t : nullptr, r ? l2t : nullptr, r, y, b, m, n, wsl, wl, nullptr), TWQ_OK);
    CHECK(twq_debug_linear_main(x, qw, sw, r ? l1t : nullptr, r ? l2t : nullptr, r, y, b, m, n, wsl, wl, nullptr),
          TWQ_OK);

    // group-wise scales
    CHECK(twq_pack_weight_grouped((const float *)w, n, m, g, qw, swg, nullptr), TWQ_OK);
    CHECK(twq_quantize_act_grouped(x, b, m, g, qx, sxg, r ? l1t : nullptr, r, r ? t : nullptr, wsq, wq, nullptr),
          TWQ_OK);
    CHECK(twq_dual_linear_grouped(qx, sxg, qw, swg, r ? t : nullptr, r ? l2t : nullptr, r, y, b, m, n, g, nullptr),
          TWQ_OK);
    const size_t wg = twq_linear_grouped_workspace_bytes(b, m, n, r, g);
    void *wsg = buf(wg);
    CHECK(twq_linear_grouped(x, qw, swg, r ? l1t : nullptr, r ? l2t : nullptr, r, y, b, m, n, g, wsg, wg, nullptr),
          TWQ_OK);
    CHECK(twq_debug_linear_grouped_main(x, qw, swg, r ? l1t : nullptr, r ? l2t : nullptr, r, y, b, m, n, g, wsg, wg,
                                        nullptr),
          TWQ_OK);

    // W4A8
    CHECK(twq_quantize_act_a8(x, b, m, qx8, sx, r ? l1t : nullptr, r, r ? t : nullptr, wsq, wq, nullptr), TWQ_OK);
    CHECK(twq_dual_linear_a8(qx8, sx, qw, sw, r ? t : nullptr, r ? l2t : nullptr, r, y, b, m, n, nullptr), TWQ_OK);
    CHECK(twq_debug_residual_acc_a8(qx8, qw, acc, b, m, n, nullptr), TWQ_OK);
    const size_t wa = twq_linear_a8_workspace_bytes(b, m, n, r);
    void *wsa = buf(wa);
    CHECK(twq_linear_a8(x, qw, sw, r ? l1t : nullptr, r ? l2t : nullptr, r, y, b, m, n, wsa, wa, nullptr), TWQ_OK);
    CHECK(twq_debug_linear_a8_main(x, qw, sw, r ? l1t : nullptr, r ? l2t : nullptr, r, y, b, m, n, wsa, wa, nullptr),
          TWQ_OK);

    // int4 low-rank branch (ranks a multiple of 32)
    if (r > 0 && r % 32 == 0) {
        void *ql1 = buf(r * m / 2), *ql2 = buf(n * r / 2), *qh = buf(b * r / 2);
        float *sl1 = (float *)buf(r * 4), *sl2 = (float *)buf(r * 4), *c = (float *)buf(r * 4);
        float *sh = (float *)buf(b * 4);
        int32_t *h = (int32_t *)buf(b * r * 4);
        CHECK(twq_pack_lowrank_int4(l1t, l2t, r, m, n, ql1, sl1, ql2, sl2, c, nullptr), TWQ_OK);
        CHECK(twq_quantize_act_lr4(x, b, m, ql1, c, r, qx, sx, qh, sh, nullptr), TWQ_OK);
        CHECK(twq_debug_lr4_h(x, b, m, ql1, c, r, h, qx, sx, qh, sh, nullptr), TWQ_OK);
        CHECK(twq_dual_linear_lr4(qx, sx, qw, sw, qh, sh, ql2, r, y, b, m, n, nullptr), TWQ_OK);
        const size_t w4 = twq_linear_lr4_workspace_bytes(b, m, n, r);
        void *ws4 = buf(w4);
        CHECK(twq_linear_lr4(x, qw, sw, ql1, c, ql2, r, y, b, m, n, ws4, w4, nullptr), TWQ_OK);
        CHECK(twq_debug_linear_lr4_main(x, qw, sw, ql1, c, ql2, r, y, b, m, n, ws4, w4, nullptr), TWQ_OK);
    }
    release();
}

void fold_calls(int64_t m, int64_t n, int64_t r) {
    const int64_t b = 0;
    double *w = (double *)buf(n * m * 8), *u = (double *)buf(m * r * 8), *s = (double *)buf(r * 8);
    double *vt = (double *)buf(r * n * 8), *q = (double *)buf(m * m * 8), *g = (double *)buf(r * r * 8);
    void *l1t = buf(r * m * 2), *l2t = buf(n * r * 2);
    float *wr = (float *)buf(n * m * 4);
    const size_t need = twq_fold_workspace_bytes(m, n, r);
    void *ws = buf(need);
    CHECK(twq_fold_lowrank(w, u, s, vt, q, g, m, n, r, l1t, l2t, wr, ws, need, nullptr), TWQ_OK);
    CHECK(twq_fold_lowrank(w, u, s, vt, nullptr, nullptr, m, n, r, l1t, l2t, wr, ws, need, nullptr), TWQ_OK);
    if (need > 0)
        CHECK(twq_fold_lowrank(w, u, s, vt, q, g, m, n, r, l1t, l2t, wr, ws, need - 1, nullptr), TWQ_ERR_WORKSPACE);
    else
        CHECK(twq_fold_lowrank(w, u, s, vt, q, g, m, n, r, l1t, l2t, wr, nullptr, 0, nullptr), TWQ_OK);
    CHECK(twq_fold_lowrank(w, u, s, vt, q, g, m, n, m + 1, l1t, l2t, wr, ws, need, nullptr), TWQ_ERR_SHAPE);
    if (r > 0) CHECK(twq_fold_lowrank(w, nullptr, s, vt, q, g, m, n, r, l1t, l2t, wr, ws, need, nullptr), TWQ_ERR_NULL);
    release();
}

void invalid_calls() {
    const int64_t b = 16, m = 512, n = 64, r = 32;
    char *p = (char *)buf(1 << 16);
    void *a = p, *mis = p + 8;
    const size_t big = 1 << 16;
    CHECK(twq_quantize_act(a, b, 100, a, (float *)a, a, r, (float *)a, a, big, nullptr), TWQ_ERR_SHAPE);
    CHECK(twq_quantize_act(a, b, m, a, (float *)a, a, 24, (float *)a, a, big, nullptr), TWQ_ERR_SHAPE);
    CHECK(twq_quantize_act(a, -1, m, a, (float *)a, a, r, (float *)a, a, big, nullptr), TWQ_ERR_SHAPE);
    CHECK(twq_quantize_act(nullptr, b, m, a, (float *)a, a, r, (float *)a, a, big, nullptr), TWQ_ERR_NULL);
    CHECK(twq_quantize_act(mis, b, m, a, (float *)a, a, r, (float *)a, a, big, nullptr), TWQ_ERR_ALIGN);
    // 16 tokens, K = 4096: T in 8 K slices, whose partial sums need the workspace
    CHECK(twq_quantize_act(a, b, 4096, a, (float *)a, a, r, (float *)a, nullptr, 0, nullptr), TWQ_ERR_WORKSPACE);
    CHECK(twq_dual_linear(a, (float *)a, a, (float *)a, (float *)a, a, r, a, b, m, 24, nullptr), TWQ_ERR_SHAPE);
    CHECK(twq_dual_linear(a, (float *)a, a, (float *)a, nullptr, a, r, a, b, m, n, nullptr), TWQ_ERR_NULL);
    CHECK(twq_linear(a, a, (float *)a, a, a, r, a, b, m, n, a, 16, nullptr), TWQ_ERR_WORKSPACE);
    CHECK(twq_linear(a, a, (float *)a, a, a, r, mis, b, m, n, a, big, nullptr), TWQ_ERR_ALIGN);
    CHECK(twq_linear_grouped(a, a, (float *)a, a, a, r, a, b, m, n, 64, a, big, nullptr), TWQ_ERR_UNSUPPORTED);
    CHECK(twq_quantize_act_lr4(a, b, m, a, (float *)a, 48, a, (float *)a, a, (float *)a, nullptr), TWQ_ERR_SHAPE);
    CHECK(twq_linear_lr4(a, a, (float *)a, a, (float *)a, a, r, a, b, m, n, a, 16, nullptr), TWQ_ERR_WORKSPACE);
    CHECK(twq_debug_lr4_h(a, b, m, a, (float *)a, r, nullptr, a, (float *)a, a, (float *)a, nullptr), TWQ_ERR_NULL);
    CHECK(twq_pack_weight((float *)a, 24, m, a, (float *)a, nullptr), TWQ_ERR_SHAPE);
    // empty calls launch nothing
    CHECK(twq_linear(nullptr, nullptr, nullptr, nullptr, nullptr, r, nullptr, 0, m, n, nullptr, 0, nullptr), TWQ_OK);
    CHECK(twq_dual_linear_lr4(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, r, nullptr, b, m, 0,
                              nullptr),
          TWQ_OK);
    release();
}

}  // namespace

int main() {
    // (b, m, n, r): one token, ragged tokens and channels, the decode tilings, many tokens
    // with K slices of T, the largest rank, and a long K
    const int64_t shapes[][4] = {{1, 128, 16, 0},     {16, 512, 512, 16},   {17, 384, 80, 64},  {33, 1024, 48, 32},
                                 {64, 4096, 2048, 32}, {65, 256, 32, 32},    {129, 256, 32, 32}, {200, 1152, 208, 64},
                                 {300, 2048, 64, 128}, {3, 16384, 256, 256}, {5, 2048, 1024, 96}, {48, 8192, 128, 128}};
    for (const auto &s : shapes) valid_calls(s[0], s[1], s[2], s[3]);
    for (const auto &f : {std::vector<int64_t>{96, 128, 16}, {512, 384, 32}, {64, 64, 0}, {300, 200, 200}})
        fold_calls(f[0], f[1], f[2]);
    invalid_calls();
    if (g_fail) {
        std::fprintf(stderr, "%d call(s) returned an unexpected status\n", g_fail);
        return 1;
    }
    std::printf("abi_driver: all calls returned the expected status\n");
    return 0;
}
