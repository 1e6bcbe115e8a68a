// twq_kernels.h -- launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace twq {

// ---- activation quantizer + first low-rank product ------------------------------

// How the activation launch is split. T = X L1 is cut into ks K slices whose partial
// sums (in the workspace) a second kernel adds. Many tokens (mode 0): tiles of 128
// token rows x all ranks staged through an LDS ring, 32 rows per wave. Few tokens
// (mode 1): every token x one 16-rank tile per CTA, the four waves splitting the
// CTA's slice. The quantizer takes nsl CTAs per token row.
struct ActPlan {
    int mode;        // 0 or 1, as above
    int fm;          // mode 1: token tiles of 16
    int row_tile;    // token rows of the partial-sum layout per tile: 128 (mode 0) or 16 fm (mode 1)
    int ks;          // K slices; 1 means T is written directly
    int row_tiles;   // mode 0: ceil(b / 128) row tiles; mode 1: r / 16 rank tiles
    int nsl;         // CTAs per token row for the quantizer
    int jq;          // 16-byte chunks of a row each thread holds: 1, 2, 4 or 8 (m <= 16384), else 0
    size_t workspace_bytes;  // partial sums of T: ks slices of [row_tiles * 128 or 16 fm][r] floats
};

ActPlan plan_act(int64_t b, int64_t m, int64_t r);

struct ActArgs {
    const uint16_t *x;
    int64_t b, m;
    uint8_t *qx;
    float *sx;
    const uint16_t *l1t;
    int r;
    float *t;
    float *partials;  // ks > 1: [ks][rows_pad][r], rows_pad = 128 row_tiles (mode 0) or 16 fm (mode 1)
    int keep_partials;  // ks > 1: leave T as partial sums (the caller's dual launch adds them)
    int group;          // 0: one scale per token row, s_X [b]; kGroup: one scale per kGroup
                        // consecutive elements of a row, s_X group-major [m / kGroup][b]
    int a8;             // 8-bit activations (q_max = 127): qx holds one int8 code per element [b][m]
    uint16_t *t16;      // ks > 1: the reduction writes T here as fp16 [b][r] (rounded to nearest
                        // even, as the fused epilogue rounds T) instead of fp32 T; else NULL
};

// Group size of the group-wise variant: one K stage of every main loop.
constexpr int kGroup = 128;

hipError_t launch_act(const ActArgs &a, const ActPlan &plan, hipStream_t stream);
// ---- weight packer -----------------------------------------------------------------

// Packed Q_W ("panel" layout; n is a multiple of 16, m of 128). Channels 16p..16p+15
// form panel p, stored in panel order; a panel holds its m / 128 pieces (128 codes of
// each of its 16 channels, 64 bytes a channel) one after another, and a piece holds the
// 16 channels' 64-byte segments in channel order. So one 16-channel x 128-code MFMA
// operand is 1 KB of contiguous memory, and a CTA that walks K reads each panel as one
// stream. Byte q of channel j's packed codes (elements 2q and 2q + 1, low nibble first)
// is at qw_offset(j, q, m).
constexpr int kPanelRows = 16, kPieceBytes = 64, kPanelPiece = kPanelRows * kPieceBytes;
__host__ __device__ constexpr int64_t qw_offset(int64_t j, int64_t q, int64_t m) {
    return ((j / kPanelRows) * (m / 128) + q / kPieceBytes) * kPanelPiece + (j % kPanelRows) * kPieceBytes + q % kPieceBytes;
}

hipError_t launch_pack_weight(const float *w, int64_t n, int64_t m, uint8_t *qw, float *sw,
                              hipStream_t stream);
// group-wise: s_W group-major [m / kGroup][n]
hipError_t launch_pack_weight_grouped(const float *w, int64_t n, int64_t m, uint8_t *qw, float *sw,
                                      hipStream_t stream);

// ---- fused dual linear ----------------------------------------------------------------

struct DualArgs {
    const uint8_t *qx;
    const float *sx;
    const uint8_t *qw;
    const float *sw;
    const float *t;    // [b][r]; the decode kernels read T through tpart instead
    const uint16_t *l2t;
    int r;
    const float *tpart;  // T as tks partial sums: T[i][c] = sum_s tpart[s tstride + i r + c] (s in order)
    int tks;
    int64_t tstride;
    uint16_t *y;       // fp16 [b][n]
    int32_t *acc;      // int32 [b][n] instead of y (the exact integer sum)
    int64_t b, m, n;
    int lr4;           // int4 low-rank branch: y += s_H (Q_H Q_L2^T) instead of T L2
    const uint8_t *qh; // [b][r/2] packed Q_H
    const float *sh;   // [b]
    const uint8_t *ql2;// [n][r/2] packed Q_L2
    int group;         // kGroup: group-wise scales, sx [m / kGroup][b] and sw [m / kGroup][n]
    int a8;            // 8-bit activation codes: qx int8 [b][m] (W4A8)
    const uint16_t *t16;  // many-token kernels: T already rounded to fp16 [b][r], or NULL (fp32 t)
};

hipError_t launch_dual_linear(const DualArgs &a, hipStream_t stream);

// Most partial sums of T (K slices x 32-rank steps) one lane of a decode epilogue
// holds; a shape with more slices gets T reduced first.
constexpr int kMaxTSlices = 16;

// Largest number of T partial-sum slices the dual launch for this shape adds itself
// (1: it needs T whole).
int dual_max_t_slices(int64_t b, int64_t m, int64_t n, int r);

// Few-token tiling of the dual launch (plan.cpp): fn x fm blocks of 16 channels x 16
// tokens per CTA; false for many tokens (the LDS-ring kernel).
bool decode_shape(int64_t b, int64_t m, int64_t n, int &fn, int &fm);

// ---- int4 low-rank variant ------------------------------------------------------------

// ---- the one-call layer (twq_api.cpp), shared with the allocation-free entry point ----

// Argument checks of twq_linear other than the workspace (a twq_status value).
int linear_check(const void *x, const void *qw, const float *sw, const void *l1t, const void *l2t, int64_t r,
                 const void *y, int64_t b, int64_t m, int64_t n);
// Workspace bytes of the one-call layer (0 for invalid shapes).
size_t linear_workspace(int64_t b, int64_t m, int64_t n, int64_t r, int group, int a8);
// The body of twq_linear / _grouped / _a8 (a twq_status value); main_only: the fused
// launch alone, on what an earlier call of the same shape left in the workspace.
int linear_run(const void *x, const void *qw, const float *sw, const void *l1t, const void *l2t, int64_t r, void *y,
               int64_t b, int64_t m, int64_t n, int group, void *workspace, size_t workspace_bytes, void *stream,
               const char *name, int a8, bool main_only);
// Records the HIP error text for twq_last_error_string; returns TWQ_ERR_HIP.
int hip_error(hipError_t e, const char *where);

// H = Q_X Q_L1^T and its requantization on chip (lowrank_int4.hip): qx packed [b][m/2],
// sx [b], ql1 in the panel layout (r rows), c [r]; writes qh [b][r/2], sh [b] and, if h
// is not NULL, the exact H [b][r] (int32) as well. x (fp16 [b][m]) not NULL: the kernel
// first writes qx and sx itself from x (only where lowrank_requant_quantizes(b)).
bool lowrank_requant_quantizes(int64_t b);
hipError_t launch_lowrank_requant(const uint16_t *x, uint8_t *qx, float *sx, const uint8_t *ql1, const float *c, int r,
                                  uint8_t *qh, float *sh, int32_t *h, int64_t b, int64_t m, hipStream_t stream);

// ---- offline fold of given transforms into the split (fold.hip) ------------------------

struct FoldArgs {
    const double *w;   // W^T [n][m] (W is the pages' m x n weight)
    const double *u;   // [m][r] left singular vectors of W (top r)
    const double *s;   // [r] singular values
    const double *vt;  // [r][n] right singular vectors, transposed
    const double *q;   // [m][m] orthogonal, or NULL (identity)
    const double *g;   // [r][r] invertible, or NULL (identity)
    int64_t m, n, r;
    void *l1t;         // out fp16 [r][m]: U'^T
    void *l2t;         // out fp16 [n][r]: V'^T
    float *w_res;      // out fp32 [n][m]: R'^T
    void *workspace;   // fold_layout(m, n, r).total bytes
};
struct FoldLayout {
    size_t ur, vr, t1, aug, ginv, total;  // byte offsets of the fp64 scratch arrays
};
FoldLayout fold_layout(int64_t m, int64_t n, int64_t r);  // plan.cpp
hipError_t launch_fold(const FoldArgs &a, hipStream_t stream);

hipError_t launch_pack_lowrank(const uint16_t *l1t, const uint16_t *l2t, int r, int64_t m, int64_t n, uint8_t *ql1,
                               float *sl1, uint8_t *ql2, float *sl2, float *c, hipStream_t stream);

}  // namespace twq
