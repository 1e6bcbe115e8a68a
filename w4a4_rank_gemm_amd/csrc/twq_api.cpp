// twq_api.cpp -- the C ABI of libtwq: argument validation, planning and launches.
// Every check happens before the first HIP call, so a rejected call launches nothing.
#include "twq.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>

#include "twq_kernels.h"

namespace {

thread_local char g_last_error[256] = "";

twq_status hip_fail(hipError_t e, const char *where) {
    std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
    return TWQ_ERR_HIP;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxM = 131072;    // keeps 256 * 49 * m below 2^31 in the int32 accumulator
constexpr int64_t kMaxTokens = int64_t(1) << 24;
constexpr int64_t kMaxN = int64_t(1) << 24;
constexpr int64_t kMaxRank = 256;

bool valid_m(int64_t m) { return m > 0 && m % 128 == 0 && m <= kMaxM; }
bool valid_b(int64_t b) { return b >= 0 && b <= kMaxTokens; }
bool valid_n(int64_t n) { return n >= 0 && n % 16 == 0 && n <= kMaxN; }
bool valid_r(int64_t r) { return r >= 0 && r % 16 == 0 && r <= kMaxRank; }
bool valid_r4(int64_t r) { return r >= 0 && r % 32 == 0 && r <= kMaxRank; }  // int4 low-rank variant

// Workspace of twq_linear: Q_X, s_X, T and the partial sums of T, each 256-byte
// aligned. With few tokens the dual launch adds the partial sums of T itself
// (direct), so T is never written.
struct LinearLayout {
    twq::ActPlan plan;
    bool direct;
    size_t qx, sx, t, partials, total;
};

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// group: 0 (one scale per token) or twq::kGroup (s_X group-major [m / kGroup][b])
// a8: 8-bit activation codes, one byte per element
LinearLayout linear_layout(int64_t b, int64_t m, int64_t n, int64_t r, int group, int a8 = 0) {
    LinearLayout L{};
    L.plan = twq::plan_act(b, m, r);
    L.direct = r > 0 && L.plan.mode == 1 && L.plan.ks > 1 && L.plan.ks <= twq::dual_max_t_slices(b, m, n, (int)r);
    L.qx = 0;
    L.sx = align256((size_t)(a8 ? b * m : b * m / 2));
    L.t = L.sx + align256((size_t)b * 4 * (size_t)(group ? m / group : 1));
    L.partials = L.t + (L.direct ? 0 : align256((size_t)(b * r) * 4));
    L.total = L.partials + align256(L.plan.workspace_bytes);
    return L;
}

bool valid_group(int64_t g) { return g == twq::kGroup; }

// The entry points with and without group-wise scales share these bodies; group is 0
// or twq::kGroup and has been validated.
twq_status quantize_act_impl(const void *x, int64_t b, int64_t m, int group, void *qx, float *sx, const void *l1t,
                             int64_t r, float *t, void *workspace, size_t workspace_bytes, void *stream,
                             const char *name, int a8 = 0) {
    if (!valid_b(b) || !valid_m(m) || !valid_r(r)) return TWQ_ERR_SHAPE;
    if (b == 0) return TWQ_OK;
    if (!x || !qx || !sx) return TWQ_ERR_NULL;
    if (r > 0 && (!l1t || !t)) return TWQ_ERR_NULL;
    if (!aligned16(x) || !aligned16(qx) || !aligned16(sx)) return TWQ_ERR_ALIGN;
    if (r > 0 && (!aligned16(l1t) || !aligned16(t))) return TWQ_ERR_ALIGN;
    const twq::ActPlan plan = twq::plan_act(b, m, r);
    if (r > 0 && plan.workspace_bytes > 0) {
        if (!workspace || workspace_bytes < plan.workspace_bytes) return TWQ_ERR_WORKSPACE;
        if (!aligned16(workspace)) return TWQ_ERR_ALIGN;
    }
    twq::ActArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.b = b;
    a.m = m;
    a.qx = static_cast<uint8_t *>(qx);
    a.sx = sx;
    a.l1t = static_cast<const uint16_t *>(l1t);
    a.r = (int)r;
    a.t = t;
    a.group = group;
    a.a8 = a8;
    if (r > 0 && plan.workspace_bytes > 0) a.partials = static_cast<float *>(workspace);
    const hipError_t e = twq::launch_act(a, plan, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TWQ_OK : hip_fail(e, name);
}

twq_status dual_linear_impl(const void *qx, const float *sx, const void *qw, const float *sw, const float *t,
                            const void *l2t, int64_t r, void *y, int64_t b, int64_t m, int64_t n, int group,
                            void *stream, const char *name, int a8 = 0) {
    if (!valid_b(b) || !valid_m(m) || !valid_n(n) || !valid_r(r)) return TWQ_ERR_SHAPE;
    if (b == 0 || n == 0) return TWQ_OK;
    if (!qx || !sx || !qw || !sw || !y) return TWQ_ERR_NULL;
    if (r > 0 && (!t || !l2t)) return TWQ_ERR_NULL;
    if (!aligned16(qx) || !aligned16(sx) || !aligned16(qw) || !aligned16(sw) || !aligned16(y))
        return TWQ_ERR_ALIGN;
    if (r > 0 && (!aligned16(t) || !aligned16(l2t))) return TWQ_ERR_ALIGN;
    twq::DualArgs a{};
    a.qx = static_cast<const uint8_t *>(qx);
    a.sx = sx;
    a.qw = static_cast<const uint8_t *>(qw);
    a.sw = sw;
    a.t = t;
    a.tpart = t;
    a.tks = 1;
    a.l2t = static_cast<const uint16_t *>(l2t);
    a.r = (int)r;
    a.y = static_cast<uint16_t *>(y);
    a.b = b;
    a.m = m;
    a.n = n;
    a.group = group;
    a.a8 = a8;
    const hipError_t e = twq::launch_dual_linear(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TWQ_OK : hip_fail(e, name);
}

}  // namespace

namespace twq {

int linear_check(const void *x, const void *qw, const float *sw, const void *l1t, const void *l2t, int64_t r,
                 const void *y, int64_t b, int64_t m, int64_t n) {
    if (!valid_b(b) || !valid_m(m) || !valid_n(n) || !valid_r(r)) return TWQ_ERR_SHAPE;
    if (b == 0 || n == 0) return TWQ_OK;
    if (!x || !qw || !sw || !y) return TWQ_ERR_NULL;
    if (r > 0 && (!l1t || !l2t)) return TWQ_ERR_NULL;
    if (!aligned16(x) || !aligned16(qw) || !aligned16(sw) || !aligned16(y)) return TWQ_ERR_ALIGN;
    if (r > 0 && (!aligned16(l1t) || !aligned16(l2t))) return TWQ_ERR_ALIGN;
    return TWQ_OK;
}

size_t linear_workspace(int64_t b, int64_t m, int64_t n, int64_t r, int group, int a8) {
    if (!valid_b(b) || !valid_m(m) || !valid_n(n) || !valid_r(r)) return 0;
    return linear_layout(b, m, n, r, group, a8).total;
}

// main_only: skip the activation launch and run the fused launch alone on the Q_X, s_X
// and T (or T's partial sums) an earlier call of the same shape left in the workspace
// (the measurement export twq_debug_linear_main).
int linear_run(const void *x, const void *qw, const float *sw, const void *l1t, const void *l2t, int64_t r, void *y,
               int64_t b, int64_t m, int64_t n, int group, void *workspace, size_t workspace_bytes, void *stream,
               const char *name, int a8, bool main_only) {
    const int st0 = linear_check(x, qw, sw, l1t, l2t, r, y, b, m, n);
    if (st0 != TWQ_OK || b == 0 || n == 0) return st0;
    const LinearLayout L = linear_layout(b, m, n, r, group, a8);
    if (!workspace || workspace_bytes < L.total) return TWQ_ERR_WORKSPACE;
    if (!aligned16(workspace)) return TWQ_ERR_ALIGN;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    const hipStream_t st = static_cast<hipStream_t>(stream);

    twq::ActArgs act{};
    act.x = static_cast<const uint16_t *>(x);
    act.b = b;
    act.m = m;
    act.qx = ws + L.qx;
    act.sx = reinterpret_cast<float *>(ws + L.sx);
    act.l1t = static_cast<const uint16_t *>(l1t);
    act.r = (int)r;
    act.t = reinterpret_cast<float *>(ws + L.t);
    act.partials = reinterpret_cast<float *>(ws + L.partials);
    act.keep_partials = L.direct;
    act.group = group;
    act.a8 = a8;
    // many-token fused launch with T reduced from slices: T is stored as fp16 (in the fp32
    // T's space), which the launch's epilogue streams through its LDS ring
    int dfn, dfm;
    const bool t16 = r > 0 && L.plan.ks > 1 && !L.direct && !twq::decode_shape(b, m, n, dfn, dfm) && !a8;
    act.t16 = t16 ? reinterpret_cast<uint16_t *>(ws + L.t) : nullptr;
    hipError_t e = main_only ? hipSuccess : twq::launch_act(act, L.plan, st);
    if (e != hipSuccess) return hip_fail(e, name);

    twq::DualArgs a{};
    a.qx = act.qx;
    a.sx = act.sx;
    a.qw = static_cast<const uint8_t *>(qw);
    a.sw = sw;
    a.t = act.t;
    a.tpart = L.direct ? act.partials : act.t;
    a.tks = L.direct ? L.plan.ks : 1;
    a.tstride = L.direct ? (int64_t)L.plan.fm * 16 * r : 0;
    a.l2t = static_cast<const uint16_t *>(l2t);
    a.r = (int)r;
    a.y = static_cast<uint16_t *>(y);
    a.b = b;
    a.m = m;
    a.n = n;
    a.group = group;
    a.a8 = a8;
    a.t16 = act.t16;
    e = twq::launch_dual_linear(a, st);
    return e == hipSuccess ? TWQ_OK : hip_fail(e, name);
}

int hip_error(hipError_t e, const char *where) { return hip_fail(e, where); }

}  // namespace twq

namespace {

twq_status linear_impl(const void *x, const void *qw, const float *sw, const void *l1t, const void *l2t, int64_t r,
                       void *y, int64_t b, int64_t m, int64_t n, int group, void *workspace, size_t workspace_bytes,
                       void *stream, const char *name, int a8 = 0, bool main_only = false) {
    return (twq_status)twq::linear_run(x, qw, sw, l1t, l2t, r, y, b, m, n, group, workspace, workspace_bytes, stream,
                                       name, a8, main_only);
}

}  // namespace

extern "C" {

const char *twq_status_string(int status) {
    switch (status) {
        case TWQ_OK: return "ok";
        case TWQ_ERR_NULL: return "null pointer";
        case TWQ_ERR_SHAPE: return "unsupported shape";
        case TWQ_ERR_ALIGN: return "pointer not 16-byte aligned";
        case TWQ_ERR_UNSUPPORTED: return "unsupported argument combination";
        case TWQ_ERR_HIP: return "HIP runtime error";
        case TWQ_ERR_WORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

const char *twq_last_error_string(void) { return g_last_error; }

const char *twq_last_hip_error(void) { return g_last_error; }

int twq_version(void) { return 100; }

size_t twq_quantize_act_workspace_bytes(int64_t b, int64_t m, int64_t r) {
    if (!valid_b(b) || !valid_m(m) || !valid_r(r)) return 0;
    return twq::plan_act(b, m, r).workspace_bytes;
}

twq_status twq_quantize_act(const void *x, int64_t b, int64_t m, void *qx, float *sx, const void *l1t,
                            int64_t r, float *t, void *workspace, size_t workspace_bytes, void *stream) {
    return quantize_act_impl(x, b, m, 0, qx, sx, l1t, r, t, workspace, workspace_bytes, stream, "twq_quantize_act");
}

twq_status twq_quantize_act_grouped(const void *x, int64_t b, int64_t m, int64_t g, void *qx, float *sx,
                                    const void *l1t, int64_t r, float *t, void *workspace, size_t workspace_bytes,
                                    void *stream) {
    if (!valid_group(g)) return TWQ_ERR_UNSUPPORTED;
    return quantize_act_impl(x, b, m, (int)g, qx, sx, l1t, r, t, workspace, workspace_bytes, stream,
                             "twq_quantize_act_grouped");
}

twq_status twq_pack_weight(const float *w_res, int64_t n, int64_t m, void *qw, float *sw, void *stream) {
    if (!valid_n(n) || !valid_m(m)) return TWQ_ERR_SHAPE;
    if (n == 0) return TWQ_OK;
    if (!w_res || !qw || !sw) return TWQ_ERR_NULL;
    if (!aligned16(w_res) || !aligned16(qw) || !aligned16(sw)) return TWQ_ERR_ALIGN;
    const hipError_t e = twq::launch_pack_weight(w_res, n, m, static_cast<uint8_t *>(qw), sw,
                                                 static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TWQ_OK : hip_fail(e, "twq_pack_weight");
}

twq_status twq_pack_weight_grouped(const float *w_res, int64_t n, int64_t m, int64_t g, void *qw, float *sw,
                                   void *stream) {
    if (!valid_group(g)) return TWQ_ERR_UNSUPPORTED;
    if (!valid_n(n) || !valid_m(m)) return TWQ_ERR_SHAPE;
    if (n == 0) return TWQ_OK;
    if (!w_res || !qw || !sw) return TWQ_ERR_NULL;
    if (!aligned16(w_res) || !aligned16(qw) || !aligned16(sw)) return TWQ_ERR_ALIGN;
    const hipError_t e = twq::launch_pack_weight_grouped(w_res, n, m, static_cast<uint8_t *>(qw), sw,
                                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TWQ_OK : hip_fail(e, "twq_pack_weight_grouped");
}

twq_status twq_dual_linear(const void *qx, const float *sx, const void *qw, const float *sw, const float *t,
                           const void *l2t, int64_t r, void *y, int64_t b, int64_t m, int64_t n, void *stream) {
    return dual_linear_impl(qx, sx, qw, sw, t, l2t, r, y, b, m, n, 0, stream, "twq_dual_linear");
}

twq_status twq_dual_linear_grouped(const void *qx, const float *sx, const void *qw, const float *sw, const float *t,
                                   const void *l2t, int64_t r, void *y, int64_t b, int64_t m, int64_t n, int64_t g,
                                   void *stream) {
    if (!valid_group(g)) return TWQ_ERR_UNSUPPORTED;
    return dual_linear_impl(qx, sx, qw, sw, t, l2t, r, y, b, m, n, (int)g, stream, "twq_dual_linear_grouped");
}

twq_status twq_debug_residual_acc(const void *qx, const void *qw, int32_t *acc, int64_t b, int64_t m, int64_t n,
                                  void *stream) {
    if (!valid_b(b) || !valid_m(m) || !valid_n(n)) return TWQ_ERR_SHAPE;
    if (b == 0 || n == 0) return TWQ_OK;
    if (!qx || !qw || !acc) return TWQ_ERR_NULL;
    if (!aligned16(qx) || !aligned16(qw) || !aligned16(acc)) return TWQ_ERR_ALIGN;
    twq::DualArgs a{};
    a.qx = static_cast<const uint8_t *>(qx);
    a.qw = static_cast<const uint8_t *>(qw);
    a.acc = acc;
    a.tks = 1;
    a.b = b;
    a.m = m;
    a.n = n;
    const hipError_t e = twq::launch_dual_linear(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TWQ_OK : hip_fail(e, "twq_debug_residual_acc");
}

twq_status twq_pack_lowrank_int4(const void *l1t, const void *l2t, int64_t r, int64_t m, int64_t n, void *ql1,
                                 float *sl1, void *ql2, float *sl2, float *c, void *stream) {
    if (!valid_r4(r) || !valid_m(m) || !valid_n(n)) return TWQ_ERR_SHAPE;
    if (r == 0) return TWQ_OK;
    if (!l1t || !l2t || !ql1 || !sl1 || !ql2 || !sl2 || !c) return TWQ_ERR_NULL;
    if (!aligned16(l1t) || !aligned16(l2t) || !aligned16(ql1) || !aligned16(sl1) || !aligned16(ql2) ||
        !aligned16(sl2) || !aligned16(c))
        return TWQ_ERR_ALIGN;
    const hipError_t e = twq::launch_pack_lowrank(static_cast<const uint16_t *>(l1t), static_cast<const uint16_t *>(l2t),
                                                  (int)r, m, n, static_cast<uint8_t *>(ql1), sl1,
                                                  static_cast<uint8_t *>(ql2), sl2, c, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TWQ_OK : hip_fail(e, "twq_pack_lowrank_int4");
}

twq_status twq_dual_linear_lr4(const void *qx, const float *sx, const void *qw, const float *sw, const void *qh,
                               const float *sh, const void *ql2, int64_t r, void *y, int64_t b, int64_t m, int64_t n,
                               void *stream) {
    if (!valid_b(b) || !valid_m(m) || !valid_n(n) || !valid_r4(r)) return TWQ_ERR_SHAPE;
    if (b == 0 || n == 0) return TWQ_OK;
    if (!qx || !sx || !qw || !sw || !y) return TWQ_ERR_NULL;
    if (r > 0 && (!qh || !sh || !ql2)) return TWQ_ERR_NULL;
    if (!aligned16(qx) || !aligned16(sx) || !aligned16(qw) || !aligned16(sw) || !aligned16(y)) return TWQ_ERR_ALIGN;
    if (r > 0 && (!aligned16(qh) || !aligned16(sh) || !aligned16(ql2))) return TWQ_ERR_ALIGN;
    twq::DualArgs a{};
    a.qx = static_cast<const uint8_t *>(qx);
    a.sx = sx;
    a.qw = static_cast<const uint8_t *>(qw);
    a.sw = sw;
    a.r = (int)r;
    a.y = static_cast<uint16_t *>(y);
    a.b = b;
    a.m = m;
    a.n = n;
    a.lr4 = 1;
    a.tks = 1;
    a.qh = static_cast<const uint8_t *>(qh);
    a.sh = sh;
    a.ql2 = static_cast<const uint8_t *>(ql2);
    const hipError_t e = twq::launch_dual_linear(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TWQ_OK : hip_fail(e, "twq_dual_linear_lr4");
}

// ---- int4 low-rank branch: the activation launch with Q_H formed on chip ----

namespace {

struct Lr4Layout {
    size_t qx, sx, qh, sh, total;
};

Lr4Layout lr4_layout(int64_t b, int64_t m, int64_t r) {
    Lr4Layout L{};
    L.qx = 0;
    L.sx = align256((size_t)(b * m / 2));
    L.qh = L.sx + align256((size_t)b * 4);
    L.sh = L.qh + align256((size_t)(b * r / 2));
    L.total = L.sh + align256((size_t)b * 4);
    return L;
}

twq_status quantize_act_lr4_impl(const void *x, int64_t b, int64_t m, const void *ql1, const float *c, int64_t r,
                                 void *qx, float *sx, void *qh, float *sh, int32_t *h, void *stream,
                                 const char *name) {
    if (!valid_b(b) || !valid_m(m) || !valid_r4(r) || r == 0) return TWQ_ERR_SHAPE;
    if (b == 0) return TWQ_OK;
    if (!x || !ql1 || !c || !qx || !sx || !qh || !sh) return TWQ_ERR_NULL;
    if (!aligned16(x) || !aligned16(ql1) || !aligned16(c) || !aligned16(qx) || !aligned16(sx) || !aligned16(qh) ||
        !aligned16(sh) || (h && !aligned16(h)))
        return TWQ_ERR_ALIGN;
    // the per-token quantizer (no first low-rank product: r = 0), then H and Q_H on chip;
    // with few tokens (one a CTA) the requantization kernel quantizes its token itself
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    const bool fused = twq::lowrank_requant_quantizes(b);
    if (!fused) {
        twq::ActArgs a{};
        a.x = static_cast<const uint16_t *>(x);
        a.b = b;
        a.m = m;
        a.qx = static_cast<uint8_t *>(qx);
        a.sx = sx;
        e = twq::launch_act(a, twq::plan_act(b, m, 0), st);
    }
    if (e == hipSuccess)
        e = twq::launch_lowrank_requant(fused ? static_cast<const uint16_t *>(x) : nullptr, static_cast<uint8_t *>(qx), sx,
                                        static_cast<const uint8_t *>(ql1), c, (int)r, static_cast<uint8_t *>(qh), sh, h,
                                        b, m, st);
    return e == hipSuccess ? TWQ_OK : hip_fail(e, name);
}

twq_status linear_lr4_impl(const void *x, const void *qw, const float *sw, const void *ql1, const float *c,
                           const void *ql2, int64_t r, void *y, int64_t b, int64_t m, int64_t n, void *workspace,
                           size_t workspace_bytes, void *stream, const char *name, bool main_only) {
    if (!valid_b(b) || !valid_m(m) || !valid_n(n) || !valid_r4(r) || r == 0) return TWQ_ERR_SHAPE;
    if (b == 0 || n == 0) return TWQ_OK;
    if (!x || !qw || !sw || !ql1 || !c || !ql2 || !y) return TWQ_ERR_NULL;
    if (!aligned16(x) || !aligned16(qw) || !aligned16(sw) || !aligned16(ql1) || !aligned16(c) || !aligned16(ql2) ||
        !aligned16(y))
        return TWQ_ERR_ALIGN;
    const Lr4Layout L = lr4_layout(b, m, r);
    if (!workspace || workspace_bytes < L.total) return TWQ_ERR_WORKSPACE;
    if (!aligned16(workspace)) return TWQ_ERR_ALIGN;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    void *qx = ws + L.qx, *qh = ws + L.qh;
    float *sx = reinterpret_cast<float *>(ws + L.sx), *sh = reinterpret_cast<float *>(ws + L.sh);
    if (!main_only) {
        const twq_status st = quantize_act_lr4_impl(x, b, m, ql1, c, r, qx, sx, qh, sh, nullptr, stream, name);
        if (st != TWQ_OK) return st;
    }
    twq::DualArgs a{};
    a.qx = static_cast<const uint8_t *>(qx);
    a.sx = sx;
    a.qw = static_cast<const uint8_t *>(qw);
    a.sw = sw;
    a.r = (int)r;
    a.y = static_cast<uint16_t *>(y);
    a.b = b;
    a.m = m;
    a.n = n;
    a.lr4 = 1;
    a.tks = 1;
    a.qh = static_cast<const uint8_t *>(qh);
    a.sh = sh;
    a.ql2 = static_cast<const uint8_t *>(ql2);
    const hipError_t e = twq::launch_dual_linear(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TWQ_OK : hip_fail(e, name);
}

}  // namespace

twq_status twq_quantize_act_lr4(const void *x, int64_t b, int64_t m, const void *ql1, const float *c, int64_t r,
                                void *qx, float *sx, void *qh, float *sh, void *stream) {
    return quantize_act_lr4_impl(x, b, m, ql1, c, r, qx, sx, qh, sh, nullptr, stream, "twq_quantize_act_lr4");
}

twq_status twq_debug_lr4_h(const void *x, int64_t b, int64_t m, const void *ql1, const float *c, int64_t r,
                           int32_t *h, void *qx, float *sx, void *qh, float *sh, void *stream) {
    if (!h && valid_b(b) && b > 0) return TWQ_ERR_NULL;
    return quantize_act_lr4_impl(x, b, m, ql1, c, r, qx, sx, qh, sh, h, stream, "twq_debug_lr4_h");
}

size_t twq_linear_lr4_workspace_bytes(int64_t b, int64_t m, int64_t n, int64_t r) {
    if (!valid_b(b) || !valid_m(m) || !valid_n(n) || !valid_r4(r)) return 0;
    return lr4_layout(b, m, r).total;
}

twq_status twq_linear_lr4(const void *x, const void *qw, const float *sw, const void *ql1, const float *c,
                          const void *ql2, int64_t r, void *y, int64_t b, int64_t m, int64_t n, void *workspace,
                          size_t workspace_bytes, void *stream) {
    return linear_lr4_impl(x, qw, sw, ql1, c, ql2, r, y, b, m, n, workspace, workspace_bytes, stream,
                           "twq_linear_lr4", false);
}

twq_status twq_debug_linear_lr4_main(const void *x, const void *qw, const float *sw, const void *ql1, const float *c,
                                     const void *ql2, int64_t r, void *y, int64_t b, int64_t m, int64_t n,
                                     void *workspace, size_t workspace_bytes, void *stream) {
    return linear_lr4_impl(x, qw, sw, ql1, c, ql2, r, y, b, m, n, workspace, workspace_bytes, stream,
                           "twq_debug_linear_lr4_main", true);
}

// ---- offline fold (page 1, section 4.1) ----

size_t twq_fold_workspace_bytes(int64_t m, int64_t n, int64_t r) {
    if (m <= 0 || n <= 0 || r < 0 || r > kMaxRank || r > m || r > n || m > kMaxM || n > kMaxN) return 0;
    return twq::fold_layout(m, n, r).total;
}

twq_status twq_fold_lowrank(const double *w, const double *u, const double *s, const double *vt, const double *q,
                            const double *g, int64_t m, int64_t n, int64_t r, void *l1t, void *l2t, float *w_res,
                            void *workspace, size_t workspace_bytes, void *stream) {
    if (m <= 0 || n <= 0 || r < 0 || r > kMaxRank || r > m || r > n || m > kMaxM || n > kMaxN) return TWQ_ERR_SHAPE;
    if (!w || !w_res) return TWQ_ERR_NULL;
    if (r > 0 && (!u || !s || !vt || !l1t || !l2t)) return TWQ_ERR_NULL;
    if (!aligned16(w) || !aligned16(w_res) || (q && !aligned16(q)) || (g && !aligned16(g))) return TWQ_ERR_ALIGN;
    if (r > 0 && (!aligned16(u) || !aligned16(s) || !aligned16(vt) || !aligned16(l1t) || !aligned16(l2t)))
        return TWQ_ERR_ALIGN;
    const size_t need = twq::fold_layout(m, n, r).total;  // 0 for r == 0
    if (need > 0 && (!workspace || workspace_bytes < need)) return TWQ_ERR_WORKSPACE;
    if (need > 0 && !aligned16(workspace)) return TWQ_ERR_ALIGN;
    twq::FoldArgs a{w, u, s, vt, q, r > 0 ? g : nullptr, m, n, r, l1t, l2t, w_res, workspace};
    const hipError_t e = twq::launch_fold(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TWQ_OK : hip_fail(e, "twq_fold_lowrank");
}

size_t twq_linear_workspace_bytes(int64_t b, int64_t m, int64_t n, int64_t r) {
    if (!valid_b(b) || !valid_m(m) || !valid_n(n) || !valid_r(r)) return 0;
    return linear_layout(b, m, n, r, 0).total;
}

twq_status twq_linear(const void *x, const void *qw, const float *sw, const void *l1t, const void *l2t, int64_t r,
                      void *y, int64_t b, int64_t m, int64_t n, void *workspace, size_t workspace_bytes, void *stream) {
    return linear_impl(x, qw, sw, l1t, l2t, r, y, b, m, n, 0, workspace, workspace_bytes, stream, "twq_linear");
}

twq_status twq_debug_linear_main(const void *x, const void *qw, const float *sw, const void *l1t, const void *l2t,
                                 int64_t r, void *y, int64_t b, int64_t m, int64_t n, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    return linear_impl(x, qw, sw, l1t, l2t, r, y, b, m, n, 0, workspace, workspace_bytes, stream,
                       "twq_debug_linear_main", 0, true);
}

size_t twq_linear_grouped_workspace_bytes(int64_t b, int64_t m, int64_t n, int64_t r, int64_t g) {
    if (!valid_group(g) || !valid_b(b) || !valid_m(m) || !valid_n(n) || !valid_r(r)) return 0;
    return linear_layout(b, m, n, r, (int)g).total;
}

twq_status twq_linear_grouped(const void *x, const void *qw, const float *sw, const void *l1t, const void *l2t,
                              int64_t r, void *y, int64_t b, int64_t m, int64_t n, int64_t g, void *workspace,
                              size_t workspace_bytes, void *stream) {
    if (!valid_group(g)) return TWQ_ERR_UNSUPPORTED;
    return linear_impl(x, qw, sw, l1t, l2t, r, y, b, m, n, (int)g, workspace, workspace_bytes, stream,
                       "twq_linear_grouped");
}

twq_status twq_debug_linear_grouped_main(const void *x, const void *qw, const float *sw, const void *l1t,
                                         const void *l2t, int64_t r, void *y, int64_t b, int64_t m, int64_t n,
                                         int64_t g, void *workspace, size_t workspace_bytes, void *stream) {
    if (!valid_group(g)) return TWQ_ERR_UNSUPPORTED;
    return linear_impl(x, qw, sw, l1t, l2t, r, y, b, m, n, (int)g, workspace, workspace_bytes, stream,
                       "twq_debug_linear_grouped_main", 0, true);
}

twq_status twq_quantize_act_a8(const void *x, int64_t b, int64_t m, void *qx, float *sx, const void *l1t, int64_t r,
                               float *t, void *workspace, size_t workspace_bytes, void *stream) {
    return quantize_act_impl(x, b, m, 0, qx, sx, l1t, r, t, workspace, workspace_bytes, stream, "twq_quantize_act_a8", 1);
}

twq_status twq_dual_linear_a8(const void *qx, const float *sx, const void *qw, const float *sw, const float *t,
                              const void *l2t, int64_t r, void *y, int64_t b, int64_t m, int64_t n, void *stream) {
    return dual_linear_impl(qx, sx, qw, sw, t, l2t, r, y, b, m, n, 0, stream, "twq_dual_linear_a8", 1);
}

size_t twq_linear_a8_workspace_bytes(int64_t b, int64_t m, int64_t n, int64_t r) {
    if (!valid_b(b) || !valid_m(m) || !valid_n(n) || !valid_r(r)) return 0;
    return linear_layout(b, m, n, r, 0, 1).total;
}

twq_status twq_linear_a8(const void *x, const void *qw, const float *sw, const void *l1t, const void *l2t, int64_t r,
                         void *y, int64_t b, int64_t m, int64_t n, void *workspace, size_t workspace_bytes,
                         void *stream) {
    return linear_impl(x, qw, sw, l1t, l2t, r, y, b, m, n, 0, workspace, workspace_bytes, stream, "twq_linear_a8", 1);
}

twq_status twq_debug_linear_a8_main(const void *x, const void *qw, const float *sw, const void *l1t, const void *l2t,
                                    int64_t r, void *y, int64_t b, int64_t m, int64_t n, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    return linear_impl(x, qw, sw, l1t, l2t, r, y, b, m, n, 0, workspace, workspace_bytes, stream,
                       "twq_debug_linear_a8_main", 1, true);
}

twq_status twq_debug_residual_acc_a8(const void *qx, const void *qw, int32_t *acc, int64_t b, int64_t m, int64_t n,
                                     void *stream) {
    if (!valid_b(b) || !valid_m(m) || !valid_n(n)) return TWQ_ERR_SHAPE;
    if (b == 0 || n == 0) return TWQ_OK;
    if (!qx || !qw || !acc) return TWQ_ERR_NULL;
    if (!aligned16(qx) || !aligned16(qw) || !aligned16(acc)) return TWQ_ERR_ALIGN;
    twq::DualArgs a{};
    a.qx = static_cast<const uint8_t *>(qx);
    a.qw = static_cast<const uint8_t *>(qw);
    a.acc = acc;
    a.tks = 1;
    a.b = b;
    a.m = m;
    a.n = n;
    a.a8 = 1;
    const hipError_t e = twq::launch_dual_linear(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TWQ_OK : hip_fail(e, "twq_debug_residual_acc_a8");
}

}  // extern "C"
