// plan.cpp -- host-side planning of the launches (no device code): how the activation
// launch splits T = X L1 and the quantizer, and which decode tiling a few-token shape
// takes. Kept apart from the kernels so it builds with any host compiler (the CPU
// sanitizer tests build it with g++ -fsanitize=address,undefined).
#include <stddef.h>
#include <stdint.h>

#include "twq_kernels.h"

namespace twq {

static int64_t pow2_floor(int64_t v) {
    int64_t p = 1;
    while (p * 2 <= v) p *= 2;
    return p;
}

ActPlan plan_act(int64_t b, int64_t m, int64_t r) {
    ActPlan pl{};
    pl.ks = 1;
    pl.nsl = 1;
    if (b == 0) return pl;
    if (b > 128) {
        // many tokens: 128-row tiles x all ranks; K slices (steps of 32, at least 512
        // long, at most 32 of them) until about 256 CTAs
        pl.mode = 0;
        pl.row_tile = 128;
        pl.row_tiles = (int)((b + 127) / 128);
        int64_t ks = 1;
        if (r > 0)
            while ((int64_t)pl.row_tiles * ks < 256 && ks < 32 && m / (ks * 2) >= 512 && m % (ks * 2 * 32) == 0)
                ks *= 2;
        pl.ks = (int)ks;
    } else {
        // few tokens: every token x one 16-rank tile x one K slice per CTA, slices of
        // about 32 KB of X and L1 each (a compute unit streams only tens of GB/s, so
        // the read is spread wide; smaller slices measured slower, their partial sums
        // costing more than they spread); each short token row is quantized by nsl CTAs
        pl.mode = 1;
        pl.fm = (int)((b + 15) / 16);
        pl.row_tile = pl.fm * 16;
        pl.row_tiles = (int)(r / 16);
        const int64_t bytes = m * (16 * pl.fm + 16) * 2;
        int64_t ks = pow2_floor(bytes / 32768 > 0 ? bytes / 32768 : 1);
        const int64_t max_ks = m / 128 < 32 ? m / 128 : 32;  // each wave keeps at least one step
        while (ks > max_ks) ks /= 2;
        pl.ks = r > 0 ? (int)ks : 1;
        int64_t nsl = 1;
        while (b * nsl < 128 && (m / 8) / (nsl * 2) >= 32) nsl *= 2;
        pl.nsl = (int)nsl;
    }
    // a row of m fp16 is m / 8 chunks of 16 bytes over 256 threads
    const int64_t per_thread = (m / 8 + 255) / 256;
    pl.jq = per_thread <= 1 ? 1 : per_thread <= 2 ? 2 : per_thread <= 4 ? 4 : per_thread <= 8 ? 8 : 0;
    if (r > 0 && pl.ks > 1) {
        const int64_t rows_pad = pl.mode == 0 ? (int64_t)pl.row_tiles * 128 : (int64_t)pl.fm * 16;
        pl.workspace_bytes = (size_t)pl.ks * rows_pad * r * sizeof(float);
    }
    return pl;
}

// Decode tiles (FN x FM blocks of 16 channels x 16 tokens per CTA, FM = ceil(b / 16)):
// the widest channel tile that still leaves at least 192 CTAs, at most 2 blocks for 16
// tokens and 4 for 64; for 32 tokens 2 blocks, or 8 where the grid stays that wide and
// K is long enough (m >= 8192) for each of the eight waves of such a CTA to stream at
// least 8 pieces. Wider tiles read Q_X from L2 fewer times; fewer CTAs than that leave
// compute units idle. Measured on MI355X (same-process sweeps of 6 tilings on each of
// 37 few-token shapes, m and n from 4096 to 28672, weights cold): within 6% of the best
// tiling on every shape. false: many tokens, the LDS-ring kernel.
bool decode_shape(int64_t b, int64_t m, int64_t n, int &fn, int &fm) {
    if (b > 64) return false;
    fm = b <= 16 ? 1 : b <= 32 ? 2 : 4;
    if (fm == 2) {
        fn = n / 128 >= 192 && m >= 8192 ? 8 : n / 32 >= 192 ? 2 : 1;
        return true;
    }
    const int cap = fm == 1 ? 2 : 4;
    for (fn = 1; fn < cap && n / (32 * fn) >= 192; fn *= 2) {}
    return true;
}

int dual_max_t_slices(int64_t b, int64_t m, int64_t n, int r) {
    int fn, fm;
    if (r == 0 || !decode_shape(b, m, n, fn, fm) || fn * fm > 4) return 1;  // the epilogue reads T whole
    const int rs = r <= 32 ? 1 : r <= 64 ? 2 : r <= 128 ? 4 : 8;
    return kMaxTSlices / rs;
}

FoldLayout fold_layout(int64_t m, int64_t n, int64_t r) {
    auto al = [](size_t v) { return (v + 255) & ~size_t(255); };
    FoldLayout L{};
    L.ur = 0;
    L.vr = L.ur + al((size_t)(m * r) * 8);
    L.t1 = L.vr + al((size_t)(r * n) * 8);
    L.aug = L.t1 + al((size_t)(m * r) * 8);
    L.ginv = L.aug + al((size_t)(2 * r * r) * 8);
    L.total = L.ginv + al((size_t)(r * r) * 8);
    return L;
}

}  // namespace twq
