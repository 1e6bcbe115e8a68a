/*
 * twq.h -- C ABI of libtwq, the fused W4A4 + low-rank linear layer for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer is the dual-component linear of TwinQuant ("TwinQuant: Learnable
 * Subspace Decomposition for 4-Bit LLM Quantization"):
 *
 *     Y = s_X s_W (Q_X Q_W) + (X L1) L2
 *
 * page 1, section 2, eq. (2) (a 4-bit x 4-bit product with its scales) and
 * eq. (3) (a residual R quantized to 4 bits plus a low-rank pair U, V), with the
 * symmetric round-to-nearest quantizer of eq. (1): s = max|v| / q_max, q_max = 7,
 * q = round(v / s). Following page 1, section 4.3, the residual and low-rank
 * partial products never reach global memory: one epilogue merges them and
 * stores fp16 once.
 *
 * Conventions for every entry point:
 *  - Pointers are device pointers owned by the caller; the library never frees
 *    or retains them. Entry points that take a workspace document its size.
 *  - All work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *    null stream). No entry point synchronizes. Results are ready when the stream
 *    reaches them.
 *  - Arguments are validated before any HIP call; a rejected call launches
 *    nothing. Kernel launch failures return TWQ_ERR_HIP, and
 *    twq_last_error_string() gives the HIP text (per calling thread).
 *    Faults inside a kernel surface at the caller's next synchronization.
 *  - Non-finite inputs are not supported (the result is unspecified).
 *  - Every pointer must be 16-byte aligned (TWQ_ERR_ALIGN otherwise).
 *  - Shapes: b (tokens) >= 0, m (input channels) a positive multiple of 128 and
 *    at most 131072, n (output channels) >= 0 and a multiple of 16, rank r = 0
 *    or a multiple of 16 up to 256. b == 0 or n == 0 is a valid empty call that
 *    launches nothing.
 *
 * Data formats:
 *  - X: fp16 [b][m], row-major (one token per row). Y: fp16 [b][n].
 *  - Packed 4-bit codes: two per byte, K-contiguous rows; byte t of a row holds
 *    code 2t in its low nibble and code 2t+1 in its high nibble, each a 4-bit
 *    two's complement value in [-7, 7]. Q_X (and the low-rank codes) are stored
 *    row by row, m/2 bytes a row.
 *  - Q_W is stored in 16-channel panels, n m / 2 bytes in all: channels
 *    16p .. 16p+15 form panel p (panels in channel order); a panel holds its m/128
 *    pieces in K order, and a piece holds bytes 64c .. 64c+63 of each of the 16
 *    channels' rows, in channel order. Byte t of channel j's row is at offset
 *    ((j / 16) (m / 128) + t / 64) 1024 + (j % 16) 64 + t % 64. A 16-channel x
 *    128-code matrix operand is then 1 KB of contiguous memory. twq_pack_weight
 *    writes this layout; every entry point that takes qw reads it.
 *  - Scales are fp32: s_X one per token, s_W one per output channel.
 *  - Quantization reading of eq. (1): s = fl32(max|v| / 7), q = round-half-even
 *    (fl32(v / s)) with correctly rounded binary32 divisions; an all-zero
 *    vector gets s = 0 and codes 0.
 */
#ifndef TWQ_H
#define TWQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TWQ_OK = 0,
    TWQ_ERR_NULL = 1,        /* a required pointer is NULL */
    TWQ_ERR_SHAPE = 2,       /* a size is out of the supported range */
    TWQ_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
    TWQ_ERR_UNSUPPORTED = 4, /* a valid but unsupported combination */
    TWQ_ERR_HIP = 5,         /* the HIP runtime reported an error */
    TWQ_ERR_WORKSPACE = 6    /* the workspace is missing or too small */
} twq_status;

/* Human-readable name of a status code (static storage). */
const char *twq_status_string(int status);

/* Text of the last TWQ_ERR_HIP on the calling thread ("" if none). The two names
 * return the same per-thread string. */
const char *twq_last_error_string(void);
const char *twq_last_hip_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int twq_version(void);

/*
 * Activation quantizer (eq. (1) per token, page 1, section 2), optionally with
 * the first low-rank product T = X L1 (eq. (3)).
 *
 *   x     fp16 [b][m]                  input activations
 *   qx    u8   [b][m/2]   (out)        packed 4-bit codes Q_X
 *   sx    f32  [b]        (out)        per-token scales s_X = max_k |x[i][k]| / 7
 *   l1t   fp16 [r][m]                  L1 transposed (row t = column t of L1); may be
 *                                      NULL only when r == 0
 *   t     f32  [b][r]     (out)        T = X L1 from the fp16 X, fp32 accumulation;
 *                                      may be NULL only when r == 0
 *   workspace, workspace_bytes         device scratch of at least
 *                                      twq_quantize_act_workspace_bytes(b, m, r)
 *                                      bytes for partial sums of T (may be NULL
 *                                      when that is 0, as it is for r == 0). No
 *                                      initial contents are needed. Calls that
 *                                      share a workspace must not overlap in time.
 */
/* (The size covers each of twq_quantize_act, twq_quantize_act_grouped and
 * twq_quantize_act_a8 for the same b, m, r.) */
size_t twq_quantize_act_workspace_bytes(int64_t b, int64_t m, int64_t r);
twq_status twq_quantize_act(const void *x, int64_t b, int64_t m, void *qx, float *sx,
                            const void *l1t, int64_t r, float *t, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * Offline weight packer (eq. (1) per output channel; the residual R of eq. (3)).
 *
 *   w_res f32 [n][m]                   residual weight, one row per output channel
 *                                      (the transpose of the pages' m x n W)
 *   qw    u8  n m / 2     (out)        packed 4-bit codes Q_W, in panels (above)
 *   sw    f32 [n]         (out)        per-channel scales s_W
 */
twq_status twq_pack_weight(const float *w_res, int64_t n, int64_t m, void *qw, float *sw,
                           void *stream);

/*
 * The fused layer (eqs. (2)-(3), single epilogue of page 1, section 4.3):
 *
 *   Y[i][j] = fp16( s_X[i] s_W[j] sum_k Q_X[i][k] Q_W[j][k] + sum_t T[i][t] L2[t][j] )
 *
 * The integer sum is exact (int32 on int8 matrix cores); T is rounded to fp16
 * for the fp16 matrix cores with fp32 accumulation.
 *
 *   qx, sx                              from twq_quantize_act
 *   qw, sw                              from twq_pack_weight
 *   t     f32  [b][r]                  from twq_quantize_act; NULL iff r == 0
 *   l2t   fp16 [n][r]                  L2 transposed (row j = column j of L2); NULL iff r == 0
 *   y     fp16 [b][n]     (out)
 */
twq_status twq_dual_linear(const void *qx, const float *sx, const void *qw, const float *sw,
                           const float *t, const void *l2t, int64_t r, void *y, int64_t b,
                           int64_t m, int64_t n, void *stream);

/*
 * Test export: the same main loop as twq_dual_linear, but the epilogue stores
 * the exact integer accumulator acc[i][j] = sum_k Q_X[i][k] Q_W[j][k] as int32
 * [b][n] instead of Y. Used to check the integer path bit for bit.
 */
twq_status twq_debug_residual_acc(const void *qx, const void *qw, int32_t *acc, int64_t b,
                                  int64_t m, int64_t n, void *stream);

/*
 * The whole layer in one call: the activation quantizer and T = X L1 (as for
 * twq_quantize_act), then the fused layer (as for twq_dual_linear), with Q_X, s_X
 * and T kept in the workspace. TwinQuant page 1, section 4.3 describes the layer as
 * one fused step; here the first low-rank product and the quantizer still run
 * first, but with few tokens T is never reduced to one array: its partial sums
 * over K slices go straight to the epilogue of the main loop, which adds them in
 * slice order (the same order and values twq_quantize_act would give T), saving a
 * launch. Y is bitwise the result of twq_quantize_act + twq_dual_linear.
 *
 *   x     fp16 [b][m];  qw, sw from twq_pack_weight;  l1t, l2t as above (NULL iff r == 0)
 *   y     fp16 [b][n]     (out)
 *   workspace, workspace_bytes         at least twq_linear_workspace_bytes(b, m, n, r)
 *                                      bytes; no initial contents are needed. Calls
 *                                      that share a workspace must not overlap in time.
 */
size_t twq_linear_workspace_bytes(int64_t b, int64_t m, int64_t n, int64_t r);
twq_status twq_linear(const void *x, const void *qw, const float *sw, const void *l1t, const void *l2t,
                      int64_t r, void *y, int64_t b, int64_t m, int64_t n, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * twq_linear for callers that cannot allocate memory: code under HIP graph (stream)
 * capture, serving loops and harnesses that forbid hipMalloc. It computes exactly
 * what twq_linear computes (the same kernels; Y bitwise equal), but takes its scratch
 * memory -- Q_X, s_X and T or T's partial sums between the two launches -- from a
 * device array inside the library instead of a workspace argument, and calls no
 * allocating routine.
 *
 *  - The array holds twq_linear_noalloc_max_bytes() bytes (64 MiB) on each GPU the
 *    library runs this entry point on, from the first call there until the process
 *    ends. A call whose scratch would exceed it (twq_linear_workspace_bytes(b, m, n,
 *    r) > twq_linear_noalloc_max_bytes()) returns TWQ_ERR_WORKSPACE before any HIP
 *    call.
 *  - The array of the calling thread's current device (hipGetDevice) is used; the
 *    stream must belong to that device.
 *  - Every call on one GPU shares that GPU's array, which keeps the last call's
 *    contents; no initial contents are needed. Calls that may overlap in time on one
 *    GPU (other streams, other threads) race on it and must be serialized by the
 *    caller; calls on one stream never overlap.
 *  - The first call on a device looks up the array's device address (not an
 *    allocation); a failure there returns TWQ_ERR_HIP.
 * Other arguments, checks and errors are those of twq_linear.
 */
size_t twq_linear_noalloc_max_bytes(void);
twq_status twq_linear_noalloc(const void *x, const void *qw, const float *sw, const void *l1t,
                              const void *l2t, int64_t r, void *y, int64_t b, int64_t m, int64_t n,
                              void *stream);

/*
 * Measurement export: the second launch of twq_linear alone -- the fused main loop
 * and epilogue, with exactly the kernel, grid and arguments twq_linear uses for this
 * shape -- reading Q_X, s_X and T (or T's partial sums over K slices) from a
 * workspace that a twq_linear call with the same b, m, n and r has filled. Its
 * duration is the duration of that launch inside twq_linear. Arguments, checks and
 * errors are those of twq_linear; x and l1t are validated but not read. On a
 * workspace twq_linear has not filled for this shape, Y is unspecified.
 */
twq_status twq_debug_linear_main(const void *x, const void *qw, const float *sw, const void *l1t,
                                 const void *l2t, int64_t r, void *y, int64_t b, int64_t m, int64_t n,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * ---- group-wise scales (TwinQuant page 1, section 5.1 and page 2, section 5.1:
 * weights and activations quantized group-wise, groups of 128) ----
 *
 * Reading: a group is g consecutive elements along K (the input dimension) of one
 * token row of X or one output channel of W_res; eq. (1) quantizes each group with
 * its own scale, and the integer sum of eq. (2) splits into one sum per group:
 *
 *   Y[i][j] = fp16( sum_G s_X[G][i] s_W[G][j] sum_{k in G} Q_X[i][k] Q_W[j][k]
 *                   + sum_t T[i][t] L2[t][j] )
 *
 * Each group's integer sum is exact (int32); the scaled group sums are added in
 * fp32. The codes use the packed format above. Scales are group-major (one row of
 * the array per group), the layout the main loops read a group's scales of a whole
 * tile in one piece from:
 *   s_X  f32 [m/g][b]    s_X[G][i] of token i, group G (elements G g .. G g + g - 1)
 *   s_W  f32 [m/g][n]    s_W[G][j] of output channel j, group G
 * g must be 128 (TWQ_ERR_UNSUPPORTED otherwise). The other arguments, the
 * workspace rules and the errors are those of the per-token entry points.
 */
twq_status twq_quantize_act_grouped(const void *x, int64_t b, int64_t m, int64_t g, void *qx,
                                    float *sx, const void *l1t, int64_t r, float *t,
                                    void *workspace, size_t workspace_bytes, void *stream);
twq_status twq_pack_weight_grouped(const float *w_res, int64_t n, int64_t m, int64_t g, void *qw,
                                   float *sw, void *stream);
twq_status twq_dual_linear_grouped(const void *qx, const float *sx, const void *qw, const float *sw,
                                   const float *t, const void *l2t, int64_t r, void *y, int64_t b,
                                   int64_t m, int64_t n, int64_t g, void *stream);
size_t twq_linear_grouped_workspace_bytes(int64_t b, int64_t m, int64_t n, int64_t r, int64_t g);
twq_status twq_linear_grouped(const void *x, const void *qw, const float *sw, const void *l1t,
                              const void *l2t, int64_t r, void *y, int64_t b, int64_t m, int64_t n,
                              int64_t g, void *workspace, size_t workspace_bytes, void *stream);
/* Measurement export: the second launch of twq_linear_grouped alone (as twq_debug_linear_main). */
twq_status twq_debug_linear_grouped_main(const void *x, const void *qw, const float *sw, const void *l1t,
                                         const void *l2t, int64_t r, void *y, int64_t b, int64_t m,
                                         int64_t n, int64_t g, void *workspace, size_t workspace_bytes,
                                         void *stream);

/*
 * ---- W4A8 (TwinQuant page 1, section 5.1: WxAy names x-bit weights and y-bit
 * activations; W4A8 results in page 1, section 5.2 and page 2, section A.3) ----
 *
 * The activations are quantized per token by eq. (1) with k = 8 bits, q_max = 127,
 * and stored one int8 code per element, K-contiguous:
 *   qx    i8  [b][m]      codes Q_X in [-127, 127]
 *   sx    f32 [b]         s_X = max_k |x[i][k]| / 127
 * The residual weight is the 4-bit Q_W, s_W of twq_pack_weight. The integer sum is
 * exact (int32; |acc| <= 889 m). Everything else (T, the low-rank branch, the
 * workspace rules, the errors) is as for the 4-bit entry points of the same name.
 */
twq_status twq_quantize_act_a8(const void *x, int64_t b, int64_t m, void *qx, float *sx,
                               const void *l1t, int64_t r, float *t, void *workspace,
                               size_t workspace_bytes, void *stream);
twq_status twq_dual_linear_a8(const void *qx, const float *sx, const void *qw, const float *sw,
                              const float *t, const void *l2t, int64_t r, void *y, int64_t b,
                              int64_t m, int64_t n, void *stream);
size_t twq_linear_a8_workspace_bytes(int64_t b, int64_t m, int64_t n, int64_t r);
twq_status twq_linear_a8(const void *x, const void *qw, const float *sw, const void *l1t,
                         const void *l2t, int64_t r, void *y, int64_t b, int64_t m, int64_t n,
                         void *workspace, size_t workspace_bytes, void *stream);
/* Measurement export: the second launch of twq_linear_a8 alone (as twq_debug_linear_main). */
twq_status twq_debug_linear_a8_main(const void *x, const void *qw, const float *sw, const void *l1t,
                                    const void *l2t, int64_t r, void *y, int64_t b, int64_t m, int64_t n,
                                    void *workspace, size_t workspace_bytes, void *stream);
/* Test export: the W4A8 main loop storing the exact int32 acc[i][j] = sum_k Q_X[i][k] Q_W[j][k]. */
twq_status twq_debug_residual_acc_a8(const void *qx, const void *qw, int32_t *acc, int64_t b,
                                     int64_t m, int64_t n, void *stream);

/*
 * ---- int4 low-rank variant (TwinQuant page 1, section 4.3) ----
 *
 * Both low-rank factors in 4 bits: the first low-rank GEMM gives INT32 H = Q_X Q_L1,
 * which gets a scale s_H from the accumulators and is requantized to packed 4-bit
 * Q_H for the second GEMM; one epilogue merges both branches:
 *
 *   Y[i][j] = fp16( s_X[i] s_W[j] (Q_X Q_W^T)[i][j] + s_H[i] (Q_H Q_L2^T)[i][j] )
 *
 * Readings: L1 (m x r) is quantized with one scale per column t and L2 (r x n) with
 * one per row t (eq. (1) each); s_L2[t] cannot stay inside the integer sum over t,
 * so both factor scales fold into H before requantization: h[i][t] =
 * (s_X[i] H[i][t]) c[t], c[t] = s_L1[t] s_L2[t], binary32 in that order; s_H[i] =
 * max_t |h[i][t]| / 7 (one scale per token), Q_H = round(h / s_H) by eq. (1).
 * Ranks: r = 0 or a multiple of 32 up to 256.
 */

/*
 *   l1t   fp16 [r][m], l2t fp16 [n][r]   as for twq_quantize_act / twq_dual_linear
 *   ql1   u8  r m / 2   (out)            codes of L1 per rank t (row t = column t of L1),
 *                                        in the panel layout of Q_W (r output channels of H)
 *   sl1   f32 [r]       (out)            s_L1[t] = max_k |L1[k][t]| / 7
 *   ql2   u8  [n][r/2]  (out)            codes of L2, K = r contiguous per output channel
 *   sl2   f32 [r]       (out)            s_L2[t] = max_j |L2[t][j]| / 7
 *   c     f32 [r]       (out)            c[t] = s_L1[t] s_L2[t]
 */
twq_status twq_pack_lowrank_int4(const void *l1t, const void *l2t, int64_t r, int64_t m, int64_t n,
                                 void *ql1, float *sl1, void *ql2, float *sl2, float *c, void *stream);

/*
 * The activation side of the int4 low-rank branch: per-token quantization of X (the
 * codes and scales of twq_quantize_act), then H = Q_X Q_L1^T (exact, int32 on int8
 * matrix cores) requantized on chip as described above, by CTAs that each hold every
 * rank of their tokens (TwinQuant page 1, section 4.3: the low-rank intermediate is
 * requantized on the fly and never written to global memory). Only Q_X, s_X, Q_H and
 * s_H are stored. Up to 256 tokens this is one launch (each CTA first quantizes its one
 * token); above, the quantizer is a launch of its own.
 *   x     fp16 [b][m];  ql1, c  from twq_pack_lowrank_int4;  r a multiple of 32, 32..256
 *   qx    u8  [b][m/2]  (out)          packed Q_X
 *   sx    f32 [b]       (out)          s_X per token
 *   qh    u8  [b][r/2]  (out)          packed Q_H (K = r contiguous per token)
 *   sh    f32 [b]       (out)          s_H per token
 */
twq_status twq_quantize_act_lr4(const void *x, int64_t b, int64_t m, const void *ql1, const float *c,
                                int64_t r, void *qx, float *sx, void *qh, float *sh, void *stream);

/*
 * Test export: twq_quantize_act_lr4 (the same kernels, one template argument apart)
 * that also stores the exact integer H [b][r] (int32) it requantizes, so the
 * integer path can be checked bit for bit. The product path never stores H.
 */
twq_status twq_debug_lr4_h(const void *x, int64_t b, int64_t m, const void *ql1, const float *c,
                           int64_t r, int32_t *h, void *qx, float *sx, void *qh, float *sh,
                           void *stream);

/*
 * The fused layer with the int4 low-rank branch (see above); qx, sx, qh, sh from
 * twq_quantize_act_lr4, ql2 from twq_pack_lowrank_int4; qh, sh, ql2 may be NULL when
 * r == 0.
 */
twq_status twq_dual_linear_lr4(const void *qx, const float *sx, const void *qw, const float *sw,
                               const void *qh, const float *sh, const void *ql2, int64_t r,
                               void *y, int64_t b, int64_t m, int64_t n, void *stream);

/*
 * The whole layer with the int4 low-rank branch in one call: twq_quantize_act_lr4 then
 * twq_dual_linear_lr4 (two launches up to 256 tokens, three above), with Q_X, s_X, Q_H and
 * s_H kept in the workspace.
 * Y is bitwise the result of those two calls.
 *   x fp16 [b][m]; qw, sw from twq_pack_weight; ql1, c, ql2 from twq_pack_lowrank_int4;
 *   r a multiple of 32, 32..256; y fp16 [b][n] (out)
 *   workspace, workspace_bytes         at least twq_linear_lr4_workspace_bytes(b, m, n, r)
 *                                      bytes; no initial contents are needed. Calls that
 *                                      share a workspace must not overlap in time.
 */
size_t twq_linear_lr4_workspace_bytes(int64_t b, int64_t m, int64_t n, int64_t r);
twq_status twq_linear_lr4(const void *x, const void *qw, const float *sw, const void *ql1,
                          const float *c, const void *ql2, int64_t r, void *y, int64_t b, int64_t m,
                          int64_t n, void *workspace, size_t workspace_bytes, void *stream);
/* Measurement export: the second launch of twq_linear_lr4 alone (as twq_debug_linear_main). */
twq_status twq_debug_linear_lr4_main(const void *x, const void *qw, const float *sw, const void *ql1,
                                     const float *c, const void *ql2, int64_t r, void *y, int64_t b,
                                     int64_t m, int64_t n, void *workspace, size_t workspace_bytes,
                                     void *stream);

/*
 * ---- offline preparation: folding given transforms into the split (TwinQuant page 1,
 * section 4.1) ----
 *
 * With the weight split W = U V + R (eq. (3)) and given an orthogonal Q (m x m, applied
 * to the activations: the layer is then fed X Q) and an invertible G (r x r, on the rank
 * space), the folded operands are
 *
 *   U' = Q^T U_r G,   V' = G^-1 V_r,   R' = Q^T W - U' V',
 *
 * with U_r = U sqrt(S) and V_r = sqrt(S) V^T from the top-r SVD of W, which the caller
 * computes with any dense linear algebra library. U' and V' are rounded to fp16 (one
 * correctly rounded conversion each); R' is formed in binary64 from those rounded
 * factors, so the split is exact against what the layer is given, and rounded to fp32.
 * All arithmetic (the scalings, the products, G^-1 by Gauss-Jordan elimination with
 * partial pivoting) runs in binary64 on the GPU. A singular G gives non-finite outputs.
 * Runs once per layer, offline.
 *
 *   w     f64 [n][m]   W^T (one row per output channel; W is the pages' m x n weight)
 *   u     f64 [m][r]   the top r left singular vectors of W (columns)
 *   s     f64 [r]      the top r singular values
 *   vt    f64 [r][n]   the top r right singular vectors (rows)
 *   q     f64 [m][m]   orthogonal, or NULL for the identity
 *   g     f64 [r][r]   invertible, or NULL for the identity
 *   l1t   fp16 [r][m]  (out) U'^T, the layer's L1 transposed
 *   l2t   fp16 [n][r]  (out) V'^T, the layer's L2 transposed
 *   w_res f32 [n][m]   (out) R'^T, the residual for twq_pack_weight
 *   workspace          at least twq_fold_workspace_bytes(m, n, r) bytes of scratch
 * Shapes: 0 <= r <= min(m, n, 256); m, n >= 1 (any multiple; the layer's own limits
 * apply when the outputs are packed). u, s, vt, l1t, l2t may be NULL when r == 0.
 */
size_t twq_fold_workspace_bytes(int64_t m, int64_t n, int64_t r);
twq_status twq_fold_lowrank(const double *w, const double *u, const double *s, const double *vt,
                            const double *q, const double *g, int64_t m, int64_t n, int64_t r,
                            void *l1t, void *l2t, float *w_res, void *workspace,
                            size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TWQ_H */
