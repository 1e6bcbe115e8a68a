// Host stand-ins for libtwq's kernel launchers, for the CPU sanitizer build of the C ABI
// layer (twq_api.cpp) and its planning code (plan.cpp). Each stub reads every byte of
// each input region and writes every byte of each output region that the real kernels
// would touch, sized from the shapes it is given, so an argument, size or workspace
// offset that the ABI layer gets wrong shows as an out-of-bounds access under
// AddressSanitizer. Pointers are host memory here; nothing runs on a GPU.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstring>

#include "twq_kernels.h"

namespace {

volatile uint8_t g_sink;

void touch_read(const void *p, size_t bytes) {
    if (!p || !bytes) return;
    const volatile uint8_t *q = static_cast<const volatile uint8_t *>(p);
    uint8_t acc = 0;
    for (size_t i = 0; i < bytes; i += 61) acc ^= q[i];
    acc ^= q[bytes - 1];
    g_sink = acc;
}

void touch_write(void *p, size_t bytes) {
    if (!p || !bytes) return;
    std::memset(p, 0x5a, bytes);
}

}  // namespace

extern "C" const char *hipGetErrorString(hipError_t) { return "stub"; }

namespace twq {

hipError_t launch_act(const ActArgs &a, const ActPlan &pl, hipStream_t) {
    if (a.b == 0) return hipSuccess;
    const size_t b = (size_t)a.b, m = (size_t)a.m, r = (size_t)a.r;
    // the quantizer's share of the grid: nsl >= 1 CTAs a row (1 with many tokens); 1,
    // 2, 4 or 8 chunks of 8 elements a thread covering the row over 256 threads, or 0
    // for rows past 16384 elements
    if (pl.nsl < 1 || (pl.mode == 0 && pl.nsl != 1)) return hipErrorInvalidValue;
    if (pl.jq != 0 && pl.jq != 1 && pl.jq != 2 && pl.jq != 4 && pl.jq != 8) return hipErrorInvalidValue;
    if (pl.jq ? (size_t)pl.jq * 256 * 8 < m || (pl.jq > 1 && (size_t)pl.jq * 128 * 8 >= m) : m <= 16384)
        return hipErrorInvalidValue;
    touch_read(a.x, b * m * 2);
    touch_write(a.qx, a.a8 ? b * m : b * m / 2);
    touch_write(a.sx, (a.group ? m / a.group : 1) * b * 4);
    if (r == 0) return hipSuccess;
    touch_read(a.l1t, r * m * 2);
    if (pl.ks > 1) {
        const size_t rows_pad = pl.mode == 0 ? (size_t)pl.row_tiles * 128 : (size_t)pl.fm * 16;
        if (pl.workspace_bytes < (size_t)pl.ks * rows_pad * r * 4) return hipErrorInvalidValue;
        touch_write(a.partials, (size_t)pl.ks * rows_pad * r * 4);
        if (a.keep_partials) return hipSuccess;
    }
    if (a.t16)
        touch_write(a.t16, b * r * 2);
    else
        touch_write(a.t, b * r * 4);
    return hipSuccess;
}

hipError_t launch_dual_linear(const DualArgs &a, hipStream_t) {
    if (a.b == 0 || a.n == 0) return hipSuccess;
    const size_t b = (size_t)a.b, m = (size_t)a.m, n = (size_t)a.n, r = (size_t)a.r;
    if (a.tks < 1 || (a.tks > 1 && (a.acc || a.lr4 || a.tks > dual_max_t_slices(a.b, a.m, a.n, a.r))))
        return hipErrorInvalidValue;
    touch_read(a.qx, a.a8 ? b * m : b * m / 2);
    touch_read(a.qw, n * m / 2);
    if (a.acc) {
        touch_write(a.acc, b * n * 4);
        return hipSuccess;
    }
    const size_t groups = a.group ? m / a.group : 1;
    touch_read(a.sx, groups * b * 4);
    touch_read(a.sw, groups * n * 4);
    if (a.lr4) {
        if (r) {
            touch_read(a.qh, b * r / 2);
            touch_read(a.sh, b * 4);
            touch_read(a.ql2, n * r / 2);
        }
    } else if (r) {
        touch_read(a.l2t, n * r * 2);
        if (a.tks > 1) {
            // slice s of T's partial sums starts at s * tstride floats
            if ((size_t)a.tstride < b * r) return hipErrorInvalidValue;
            touch_read(a.tpart, ((size_t)(a.tks - 1) * (size_t)a.tstride + b * r) * 4);
        } else if (a.t16) {
            touch_read(a.t16, b * r * 2);  // T already fp16 (many tokens, T reduced from slices)
        } else {
            touch_read(a.t, b * r * 4);
        }
    }
    touch_write(a.y, b * n * 2);
    return hipSuccess;
}

hipError_t launch_pack_weight(const float *w, int64_t n, int64_t m, uint8_t *qw, float *sw, hipStream_t) {
    touch_read(w, (size_t)n * (size_t)m * 4);
    touch_write(qw, (size_t)n * (size_t)m / 2);
    touch_write(sw, (size_t)n * 4);
    return hipSuccess;
}

hipError_t launch_pack_weight_grouped(const float *w, int64_t n, int64_t m, uint8_t *qw, float *sw, hipStream_t) {
    touch_read(w, (size_t)n * (size_t)m * 4);
    touch_write(qw, (size_t)n * (size_t)m / 2);
    touch_write(sw, (size_t)(m / kGroup) * (size_t)n * 4);
    return hipSuccess;
}

hipError_t launch_pack_lowrank(const uint16_t *l1t, const uint16_t *l2t, int r, int64_t m, int64_t n, uint8_t *ql1,
                               float *sl1, uint8_t *ql2, float *sl2, float *c, hipStream_t) {
    touch_read(l1t, (size_t)r * (size_t)m * 2);
    touch_read(l2t, (size_t)n * (size_t)r * 2);
    touch_write(ql1, (size_t)r * (size_t)m / 2);
    touch_write(ql2, (size_t)n * (size_t)r / 2);
    touch_write(sl1, (size_t)r * 4);
    touch_write(sl2, (size_t)r * 4);
    touch_write(c, (size_t)r * 4);
    return hipSuccess;
}

bool lowrank_requant_quantizes(int64_t b) { return b <= 256; }

hipError_t launch_lowrank_requant(const uint16_t *x, uint8_t *qx, float *sx, const uint8_t *ql1, const float *c, int r,
                                  uint8_t *qh, float *sh, int32_t *h, int64_t b, int64_t m, hipStream_t) {
    if (b == 0) return hipSuccess;
    if (r < 32 || r > 256 || r % 32) return hipErrorInvalidValue;
    if (x && b > 256) return hipErrorInvalidValue;
    if (x) {
        touch_read(x, (size_t)b * (size_t)m * 2);
        touch_write(qx, (size_t)b * (size_t)m / 2);
        touch_write(sx, (size_t)b * 4);
    }
    touch_read(qx, (size_t)b * (size_t)m / 2);
    touch_read(sx, (size_t)b * 4);
    touch_read(ql1, (size_t)r * (size_t)m / 2);
    touch_read(c, (size_t)r * 4);
    touch_write(qh, (size_t)b * (size_t)r / 2);
    touch_write(sh, (size_t)b * 4);
    touch_write(h, h ? (size_t)b * (size_t)r * 4 : 0);
    return hipSuccess;
}

hipError_t launch_fold(const FoldArgs &a, hipStream_t) {
    const size_t m = (size_t)a.m, n = (size_t)a.n, r = (size_t)a.r;
    touch_read(a.w, n * m * 8);
    touch_read(a.q, a.q ? m * m * 8 : 0);
    touch_write(a.workspace, fold_layout(a.m, a.n, a.r).total);
    if (r) {
        touch_read(a.u, m * r * 8);
        touch_read(a.s, r * 8);
        touch_read(a.vt, r * n * 8);
        touch_read(a.g, a.g ? r * r * 8 : 0);
        touch_write(a.l1t, r * m * 2);
        touch_write(a.l2t, n * r * 2);
    }
    touch_write(a.w_res, n * m * 4);
    return hipSuccess;
}

}  // namespace twq
