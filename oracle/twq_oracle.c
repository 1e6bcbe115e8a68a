/*
 * twq_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU definition of the fused W4A4 + low-rank
 * linear layer of TwinQuant ("TwinQuant: Learnable Subspace Decomposition for
 * 4-Bit LLM Quantization"):
 *
 *   Y = s_X s_W (Q_X Q_W) + (X L1) L2
 *
 * It exists to check the HIP library against. Only the test-suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it; the product
 * path never does. It shares no code, header or table with the HIP sources.
 *
 * Every floating-point decision that produces an integer (a scale, a code) is
 * taken in IEEE binary32, because that is the precision the layer itself uses
 * to quantize; everything else (the low-rank product, the merge) is carried in
 * binary64, and the integer GEMM in int64. Build with -O2 -fno-fast-math
 * -ffp-contract=off so every float operation below is one IEEE operation.
 *
 * Readings of the pages taken here (the pages leave these open):
 *  - round() in eq. (1) is round-half-to-even (the IEEE default);
 *  - the code is rint(x / s) with s = amax / 7 computed first, both as correctly
 *    rounded binary32 divisions (eq. (1) writes X / s_X with s_X = max|X| / q_max);
 *  - scales are binary32; an all-zero row has s = 0 and all codes 0;
 *  - codes are clamped to [-7, 7] (q_max = 2^(k-1) - 1 = 7 for k = 4);
 *  - granularity: one scale per token row of X, one per output channel of W_res;
 *  - the fp16 low-rank branch is fed the unquantized fp16 X;
 *  - packed layout: byte t of a row holds code 2t in its low nibble and code
 *    2t+1 in its high nibble, each as 4-bit two's complement.
 *
 * What pins each function (tests marked "not gpu"): hand-worked vectors of
 * eq. (1) with their tie cases, the invariants max|q| = 7, q(-x) = -q(x) and
 * q(2^e x) = q(x), exact-rational nearest-integer bounds, pure-Python brute
 * force of the integer GEMM, the identities r = 0 (plain W4A4, a library int64
 * matmul) and W_res = 0 (pure low-rank, a library fp64 matmul), a hand-worked
 * whole layer, and for the int4 low-rank variant a hand-worked case plus the
 * identity that exactly representable factors reproduce the fp16 branch; for
 * group-wise scales a hand-worked two-group layer, the identities g = m (one
 * group: the per-token layer) and grouped rows = per-row quantization of the
 * rows cut into groups, and brute force with exact rationals; for W4A8 a
 * hand-worked layer with ties at q_max = 127, the rational model at 8 bits, the
 * largest code reached for every fp16 amax, and a library int64 matmul.
 * The pages' own kernel numerics (its s_H granularity in particular) print no
 * example and stay a reading, not a pin.
 */
#include <math.h>
#include <stdio.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define Q_MAX 7 /* 2^(k-1) - 1 for k = 4 bits: TwinQuant page 1, section 2, eq. (1) */

/* Every integer sum of the layer must fit the int32 accumulator of the matrix cores
 * (|acc| < 2^31; with |q| <= 7 and m <= 131072 it is at most 49 m). The sums here are
 * int64, so a violation is detected rather than wrapped: it aborts with a message. */
int64_t orc_require_i32(int64_t v)
{
    if (v >= ((int64_t)1 << 31) || v <= -((int64_t)1 << 31)) {
        fprintf(stderr, "twq_oracle: integer sum %lld outside the int32 accumulator range\n", (long long)v);
        abort();
    }
    return v;
}

/* IEEE 754 binary16 -> binary64, straight from the format's definition:
 * sign 1 bit, exponent 5 bits (bias 15), fraction 10 bits. */
double orc_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24); /* subnormal: f * 2^-10 * 2^-14 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* eq. (1) on one vector held in binary32 with q_max = 2^(k-1) - 1 for k bits:
 * s = max|v| / q_max, q = round(v / s). */
static void quantize_vector_q(const float *v, int64_t len, int q_max, int8_t *q, float *s_out)
{
    float amax = 0.0f;
    for (int64_t k = 0; k < len; k++) {
        float a = fabsf(v[k]);
        if (a > amax)
            amax = a;
    }
    float s = amax / (float)q_max;
    *s_out = s;
    for (int64_t k = 0; k < len; k++) {
        if (amax == 0.0f) {
            q[k] = 0;
            continue;
        }
        float ratio = v[k] / s;      /* one binary32 division */
        float r = rintf(ratio);      /* round half to even */
        if (r > q_max)
            r = (float)q_max;
        if (r < -q_max)
            r = (float)-q_max;
        q[k] = (int8_t)r;
    }
}

/* the 4-bit case of eq. (1) */
static void quantize_vector(const float *v, int64_t len, int8_t *q, float *s_out)
{
    quantize_vector_q(v, len, Q_MAX, q, s_out);
}

/* two codes per byte: element 2t in the low nibble, element 2t+1 in the high nibble */
static void pack_codes(const int8_t *q, int64_t len, uint8_t *packed)
{
    for (int64_t t = 0; t < len / 2; t++) {
        unsigned lo = (unsigned)q[2 * t] & 0xFu;
        unsigned hi = (unsigned)q[2 * t + 1] & 0xFu;
        packed[t] = (uint8_t)(lo | (hi << 4));
    }
}

/* Activation quantizer: X fp16 [b][m] -> codes int8 [b][m], packed u8 [b][m/2], s_X f32 [b].
 * One scale per token (row). packed may be NULL. */
void orc_quantize_act(const uint16_t *x, int64_t b, int64_t m, int8_t *qx, uint8_t *qx_packed,
                      float *sx)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < b; i++) {
        float *row = (float *)malloc(sizeof(float) * (size_t)m);
        for (int64_t k = 0; k < m; k++)
            row[k] = (float)orc_half_to_double(x[i * m + k]); /* exact: fp16 fits binary32 */
        quantize_vector(row, m, qx + i * m, sx + i);
        if (qx_packed)
            pack_codes(qx + i * m, m, qx_packed + i * (m / 2));
        free(row);
    }
}

/* Weight quantizer: W_res f32 [n][m] -> codes int8 [n][m], packed u8 [n][m/2], s_W f32 [n].
 * One scale per output channel (row of this storage). packed may be NULL. */
void orc_quantize_weight(const float *w, int64_t n, int64_t m, int8_t *qw, uint8_t *qw_packed,
                         float *sw)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; j++) {
        quantize_vector(w + j * m, m, qw + j * m, sw + j);
        if (qw_packed)
            pack_codes(qw + j * m, m, qw_packed + j * (m / 2));
    }
}

/* Integer part of eq. (2): acc[i][j] = sum_k Q_X[i][k] * Q_W[j][k], in int64. */
void orc_residual_acc(const int8_t *qx, const int8_t *qw, int64_t b, int64_t m, int64_t n,
                      int64_t *acc)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < b; i++)
        for (int64_t j = 0; j < n; j++) {
            int64_t sum = 0;
            for (int64_t k = 0; k < m; k++)
                sum += (int64_t)qx[i * m + k] * (int64_t)qw[j * m + k];
            acc[i * n + j] = orc_require_i32(sum);
        }
}

/* First low-rank product: T[i][t] = sum_k X[i][k] * L1[k][t], binary64.
 * L1 is given transposed, l1t [r][m]. */
void orc_lowrank_t(const uint16_t *x, const uint16_t *l1t, int64_t b, int64_t m, int64_t r,
                   double *t)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < b; i++)
        for (int64_t u = 0; u < r; u++) {
            double sum = 0.0;
            for (int64_t k = 0; k < m; k++)
                sum += orc_half_to_double(x[i * m + k]) * orc_half_to_double(l1t[u * m + k]);
            t[i * r + u] = sum;
        }
}

/* Second low-rank product: LR[i][j] = sum_t T[i][t] * L2[t][j], binary64.
 * L2 is given transposed, l2t [n][r]. */
void orc_lowrank_out(const double *t, const uint16_t *l2t, int64_t b, int64_t n, int64_t r,
                     double *lr)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < b; i++)
        for (int64_t j = 0; j < n; j++) {
            double sum = 0.0;
            for (int64_t u = 0; u < r; u++)
                sum += t[i * r + u] * orc_half_to_double(l2t[j * r + u]);
            lr[i * n + j] = sum;
        }
}

/* The whole layer (eqs. (2) and (3) of page 1, section 2, with the fp16 low-rank
 * branch): Y[i][j] = s_X[i] s_W[j] acc[i][j] + LR[i][j], binary64.
 * Inputs: x fp16 [b][m], w_res f32 [n][m], l1t fp16 [r][m], l2t fp16 [n][r].
 * Outputs (any may be NULL except y): the codes, packed codes, scales, acc, T, Y. */
int orc_dual_linear(const uint16_t *x, const float *w_res, const uint16_t *l1t,
                    const uint16_t *l2t, int64_t b, int64_t m, int64_t n, int64_t r,
                    uint8_t *qx_packed, float *sx, uint8_t *qw_packed, float *sw,
                    int64_t *acc_out, double *t_out, double *y)
{
    int8_t *qx = (int8_t *)malloc((size_t)(b * m));
    int8_t *qw = (int8_t *)malloc((size_t)(n * m));
    float *sx_l = (float *)malloc(sizeof(float) * (size_t)b);
    float *sw_l = (float *)malloc(sizeof(float) * (size_t)n);
    int64_t *acc = (int64_t *)malloc(sizeof(int64_t) * (size_t)(b * n));
    double *t = (double *)malloc(sizeof(double) * (size_t)(b * (r > 0 ? r : 1)));
    double *lr = (double *)malloc(sizeof(double) * (size_t)(b * n));
    if (!qx || !qw || !sx_l || !sw_l || !acc || !t || !lr)
        return 1;
    orc_quantize_act(x, b, m, qx, qx_packed, sx_l);
    orc_quantize_weight(w_res, n, m, qw, qw_packed, sw_l);
    orc_residual_acc(qx, qw, b, m, n, acc);
    if (r > 0) {
        orc_lowrank_t(x, l1t, b, m, r, t);
        orc_lowrank_out(t, l2t, b, n, r, lr);
    } else {
        memset(lr, 0, sizeof(double) * (size_t)(b * n));
    }
    for (int64_t i = 0; i < b; i++)
        for (int64_t j = 0; j < n; j++)
            y[i * n + j] = (double)sx_l[i] * (double)sw_l[j] * (double)acc[i * n + j] + lr[i * n + j];
    if (sx)
        memcpy(sx, sx_l, sizeof(float) * (size_t)b);
    if (sw)
        memcpy(sw, sw_l, sizeof(float) * (size_t)n);
    if (acc_out)
        memcpy(acc_out, acc, sizeof(int64_t) * (size_t)(b * n));
    if (t_out && r > 0)
        memcpy(t_out, t, sizeof(double) * (size_t)(b * r));
    free(qx); free(qw); free(sx_l); free(sw_l); free(acc); free(t); free(lr);
    return 0;
}

/* Y at sampled positions only, for full-size shapes: Y[rows[p]][cols[p]] for
 * p < count, from the same definition. Only the rows of X and W_res that the
 * samples touch are quantized. Also returns acc at those positions. */
int orc_dual_linear_sampled(const uint16_t *x, const float *w_res, const uint16_t *l1t,
                            const uint16_t *l2t, int64_t b, int64_t m, int64_t n, int64_t r,
                            const int64_t *rows, const int64_t *cols, int64_t count,
                            int64_t *acc_out, double *y_out)
{
    (void)b;
    (void)n;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < count; p++) {
        int64_t i = rows[p], j = cols[p];
        float *xr = (float *)malloc(sizeof(float) * (size_t)m);
        int8_t *qx = (int8_t *)malloc((size_t)m);
        int8_t *qw = (int8_t *)malloc((size_t)m);
        if (!xr || !qx || !qw) {
            fail = 1;
            continue;
        }
        float sxi, swj;
        for (int64_t k = 0; k < m; k++)
            xr[k] = (float)orc_half_to_double(x[i * m + k]);
        quantize_vector(xr, m, qx, &sxi);
        quantize_vector(w_res + j * m, m, qw, &swj);
        int64_t acc = 0;
        for (int64_t k = 0; k < m; k++)
            acc += (int64_t)qx[k] * (int64_t)qw[k];
        double lr = 0.0;
        for (int64_t u = 0; u < r; u++) {
            double tu = 0.0;
            for (int64_t k = 0; k < m; k++)
                tu += orc_half_to_double(x[i * m + k]) * orc_half_to_double(l1t[u * m + k]);
            lr += tu * orc_half_to_double(l2t[j * r + u]);
        }
        acc_out[p] = orc_require_i32(acc);
        y_out[p] = (double)sxi * (double)swj * (double)acc + lr;
        free(xr); free(qx); free(qw);
    }
    return fail;
}

/* ---- int4 low-rank variant (TwinQuant page 1, section 4.3: both low-rank
 * factors in 4 bits, the INT32 intermediate H requantized on the fly) ----
 *
 * Readings: L1 (m x r) is quantized per column (one scale per rank index t),
 * L2 (r x n) per row (again one scale per t). Because s_L2[t] cannot leave an
 * integer sum over t, both factor scales are folded into H before it is
 * requantized: h[i][t] = (s_X[i] * H[i][t]) * c[t], c[t] = s_L1[t] * s_L2[t],
 * all binary32 in that order; s_H is one scale per token over its r values. */

/* l1t fp16 [r][m] (row t = column t of L1), l2t fp16 [n][r] (column t = row t of L2).
 * Outputs: ql1 codes int8 [r][m] (+ packed [r][m/2]), sl1 [r];
 *          ql2 codes int8 [n][r] (+ packed [n][r/2], K = r contiguous), sl2 [r]; c [r]. */
int orc_quantize_lowrank(const uint16_t *l1t, const uint16_t *l2t, int64_t r, int64_t m,
                         int64_t n, int8_t *ql1, uint8_t *ql1_packed, float *sl1, int8_t *ql2,
                         uint8_t *ql2_packed, float *sl2, float *c)
{
    float *row = (float *)malloc(sizeof(float) * (size_t)(m > n ? m : n));
    int8_t *col_q = (int8_t *)malloc((size_t)n);
    if (!row || !col_q)
        return 1;
    for (int64_t t = 0; t < r; t++) {
        for (int64_t k = 0; k < m; k++)
            row[k] = (float)orc_half_to_double(l1t[t * m + k]);
        quantize_vector(row, m, ql1 + t * m, sl1 + t);
        if (ql1_packed)
            pack_codes(ql1 + t * m, m, ql1_packed + t * (m / 2));
        for (int64_t j = 0; j < n; j++)
            row[j] = (float)orc_half_to_double(l2t[j * r + t]);
        quantize_vector(row, n, col_q, sl2 + t);
        for (int64_t j = 0; j < n; j++)
            ql2[j * r + t] = col_q[j];
        c[t] = sl1[t] * sl2[t];
    }
    if (ql2_packed)
        for (int64_t j = 0; j < n; j++)
            pack_codes(ql2 + j * r, r, ql2_packed + j * (r / 2));
    free(row);
    free(col_q);
    return 0;
}

/* Requantized intermediate: H = Q_X Q_L1 (int64), h = (s_X H) c, s_H = max_t|h| / 7,
 * Q_H = round(h / s_H). qx int8 [b][m], ql1 int8 [r][m]. Outputs qh int8 [b][r]
 * (+ packed [b][r/2]), sh [b], and H itself if h_out != NULL. */
void orc_lowrank_requant(const int8_t *qx, const float *sx, const int8_t *ql1, const float *c,
                         int64_t b, int64_t m, int64_t r, int8_t *qh, uint8_t *qh_packed,
                         float *sh, int64_t *h_out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < b; i++) {
        float *h = (float *)malloc(sizeof(float) * (size_t)r);
        for (int64_t t = 0; t < r; t++) {
            int64_t hi = 0;
            for (int64_t k = 0; k < m; k++)
                hi += (int64_t)qx[i * m + k] * (int64_t)ql1[t * m + k];
            orc_require_i32(hi);
            if (h_out)
                h_out[i * r + t] = hi;
            float prod = sx[i] * (float)hi; /* (s_X H) first ... */
            h[t] = prod * c[t];             /* ... then times c_t */
        }
        quantize_vector(h, r, qh + i * r, sh + i);
        if (qh_packed)
            pack_codes(qh + i * r, r, qh_packed + i * (r / 2));
        free(h);
    }
}

/* The whole layer with the int4 low-rank branch:
 * Y[i][j] = s_X[i] s_W[j] acc[i][j] + s_H[i] acc2[i][j], acc2 = Q_H Q_L2 (int64). */
int orc_dual_linear_lr4(const uint16_t *x, const float *w_res, const uint16_t *l1t,
                        const uint16_t *l2t, int64_t b, int64_t m, int64_t n, int64_t r,
                        uint8_t *qh_packed, float *sh_out, int64_t *h_out, int64_t *acc2_out,
                        double *y)
{
    int8_t *qx = (int8_t *)malloc((size_t)(b * m));
    int8_t *qw = (int8_t *)malloc((size_t)(n * m));
    int8_t *ql1 = (int8_t *)malloc((size_t)(r * m));
    int8_t *ql2 = (int8_t *)malloc((size_t)(n * r));
    int8_t *qh = (int8_t *)malloc((size_t)(b * r));
    float *sx = (float *)malloc(sizeof(float) * (size_t)b);
    float *sw = (float *)malloc(sizeof(float) * (size_t)n);
    float *sl1 = (float *)malloc(sizeof(float) * (size_t)r);
    float *sl2 = (float *)malloc(sizeof(float) * (size_t)r);
    float *c = (float *)malloc(sizeof(float) * (size_t)r);
    float *sh = (float *)malloc(sizeof(float) * (size_t)b);
    if (!qx || !qw || !ql1 || !ql2 || !qh || !sx || !sw || !sl1 || !sl2 || !c || !sh)
        return 1;
    orc_quantize_act(x, b, m, qx, NULL, sx);
    orc_quantize_weight(w_res, n, m, qw, NULL, sw);
    if (orc_quantize_lowrank(l1t, l2t, r, m, n, ql1, NULL, sl1, ql2, NULL, sl2, c))
        return 1;
    orc_lowrank_requant(qx, sx, ql1, c, b, m, r, qh, qh_packed, sh, h_out);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < b; i++)
        for (int64_t j = 0; j < n; j++) {
            int64_t acc = 0, acc2 = 0;
            for (int64_t k = 0; k < m; k++)
                acc += (int64_t)qx[i * m + k] * (int64_t)qw[j * m + k];
            for (int64_t t = 0; t < r; t++)
                acc2 += (int64_t)qh[i * r + t] * (int64_t)ql2[j * r + t];
            orc_require_i32(acc);
            if (acc2_out)
                acc2_out[i * n + j] = orc_require_i32(acc2);
            y[i * n + j] = (double)sx[i] * (double)sw[j] * (double)acc + (double)sh[i] * (double)acc2;
        }
    if (sh_out)
        memcpy(sh_out, sh, sizeof(float) * (size_t)b);
    free(qx); free(qw); free(ql1); free(ql2); free(qh);
    free(sx); free(sw); free(sl1); free(sl2); free(c); free(sh);
    return 0;
}

/* The int4 low-rank layer at sampled positions (rows[p], cols[p]) only, from the same
 * definition as orc_dual_linear_lr4: the factors are quantized whole (they are small),
 * H and Q_H are formed for the sampled tokens, acc and acc2 at the sampled outputs. */
int orc_dual_linear_lr4_sampled(const uint16_t *x, const float *w_res, const uint16_t *l1t,
                                const uint16_t *l2t, int64_t b, int64_t m, int64_t n, int64_t r,
                                const int64_t *rows, const int64_t *cols, int64_t count,
                                int64_t *acc_out, int64_t *acc2_out, double *y_out)
{
    (void)b;
    int8_t *ql1 = (int8_t *)malloc((size_t)(r * m));
    int8_t *ql2 = (int8_t *)malloc((size_t)(n * r));
    float *sl1 = (float *)malloc(sizeof(float) * (size_t)r);
    float *sl2 = (float *)malloc(sizeof(float) * (size_t)r);
    float *c = (float *)malloc(sizeof(float) * (size_t)r);
    if (!ql1 || !ql2 || !sl1 || !sl2 || !c)
        return 1;
    if (orc_quantize_lowrank(l1t, l2t, r, m, n, ql1, NULL, sl1, ql2, NULL, sl2, c))
        return 1;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < count; p++) {
        int64_t i = rows[p], j = cols[p];
        float *xr = (float *)malloc(sizeof(float) * (size_t)m);
        int8_t *qx = (int8_t *)malloc((size_t)m);
        int8_t *qw = (int8_t *)malloc((size_t)m);
        int8_t *qh = (int8_t *)malloc((size_t)(r > 0 ? r : 1));
        if (!xr || !qx || !qw || !qh) {
            fail = 1;
            continue;
        }
        float sxi, swj, shi;
        for (int64_t k = 0; k < m; k++)
            xr[k] = (float)orc_half_to_double(x[i * m + k]);
        quantize_vector(xr, m, qx, &sxi);
        quantize_vector(w_res + j * m, m, qw, &swj);
        orc_lowrank_requant(qx, &sxi, ql1, c, 1, m, r, qh, NULL, &shi, NULL);
        int64_t acc = 0, acc2 = 0;
        for (int64_t k = 0; k < m; k++)
            acc += (int64_t)qx[k] * (int64_t)qw[k];
        for (int64_t t = 0; t < r; t++)
            acc2 += (int64_t)qh[t] * (int64_t)ql2[j * r + t];
        acc_out[p] = orc_require_i32(acc);
        acc2_out[p] = orc_require_i32(acc2);
        y_out[p] = (double)sxi * (double)swj * (double)acc + (double)shi * (double)acc2;
        free(xr); free(qx); free(qw); free(qh);
    }
    free(ql1); free(ql2); free(sl1); free(sl2); free(c);
    return fail;
}

/* ---- W4A8 (TwinQuant page 1, section 5.1: WxAy names x-bit weights and y-bit
 * activations; W4A8 results in page 1, section 5.2 and page 2, section A.3) ----
 *
 * The residual weight stays 4-bit (q_max = 7); the activations are quantized per
 * token with eq. (1) at k = 8 bits, q_max = 2^7 - 1 = 127, codes stored one int8 per
 * element. Everything else is the layer above:
 *   Y[i][j] = s_X[i] s_W[j] sum_k Q_X[i][k] Q_W[j][k] + LR[i][j]. */
#define Q_MAX_A8 127

/* X fp16 [b][m] -> codes int8 [b][m], s_X f32 [b] */
void orc_quantize_act_a8(const uint16_t *x, int64_t b, int64_t m, int8_t *qx, float *sx)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < b; i++) {
        float *row = (float *)malloc(sizeof(float) * (size_t)m);
        for (int64_t k = 0; k < m; k++)
            row[k] = (float)orc_half_to_double(x[i * m + k]);
        quantize_vector_q(row, m, Q_MAX_A8, qx + i * m, sx + i);
        free(row);
    }
}

/* The W4A8 layer, binary64. Outputs other than y may be NULL. */
int orc_dual_linear_a8(const uint16_t *x, const float *w_res, const uint16_t *l1t,
                       const uint16_t *l2t, int64_t b, int64_t m, int64_t n, int64_t r,
                       int8_t *qx_out, float *sx, uint8_t *qw_packed, float *sw,
                       int64_t *acc_out, double *y)
{
    int8_t *qx = (int8_t *)malloc((size_t)(b * m));
    int8_t *qw = (int8_t *)malloc((size_t)(n * m));
    float *sx_l = (float *)malloc(sizeof(float) * (size_t)b);
    float *sw_l = (float *)malloc(sizeof(float) * (size_t)n);
    int64_t *acc = (int64_t *)malloc(sizeof(int64_t) * (size_t)(b * n));
    double *t = (double *)malloc(sizeof(double) * (size_t)(b * (r > 0 ? r : 1)));
    double *lr = (double *)malloc(sizeof(double) * (size_t)(b * n));
    if (!qx || !qw || !sx_l || !sw_l || !acc || !t || !lr)
        return 1;
    orc_quantize_act_a8(x, b, m, qx, sx_l);
    orc_quantize_weight(w_res, n, m, qw, qw_packed, sw_l);
    orc_residual_acc(qx, qw, b, m, n, acc);
    if (r > 0) {
        orc_lowrank_t(x, l1t, b, m, r, t);
        orc_lowrank_out(t, l2t, b, n, r, lr);
    } else {
        memset(lr, 0, sizeof(double) * (size_t)(b * n));
    }
    for (int64_t i = 0; i < b; i++)
        for (int64_t j = 0; j < n; j++)
            y[i * n + j] = (double)sx_l[i] * (double)sw_l[j] * (double)acc[i * n + j] + lr[i * n + j];
    if (qx_out)
        memcpy(qx_out, qx, (size_t)(b * m));
    if (sx)
        memcpy(sx, sx_l, sizeof(float) * (size_t)b);
    if (sw)
        memcpy(sw, sw_l, sizeof(float) * (size_t)n);
    if (acc_out)
        memcpy(acc_out, acc, sizeof(int64_t) * (size_t)(b * n));
    free(qx); free(qw); free(sx_l); free(sw_l); free(acc); free(t); free(lr);
    return 0;
}

/* The W4A8 layer at sampled positions: acc and Y at (rows[p], cols[p]). */
int orc_dual_linear_a8_sampled(const uint16_t *x, const float *w_res, const uint16_t *l1t,
                               const uint16_t *l2t, int64_t b, int64_t m, int64_t n, int64_t r,
                               const int64_t *rows, const int64_t *cols, int64_t count,
                               int64_t *acc_out, double *y_out)
{
    (void)b;
    (void)n;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < count; p++) {
        int64_t i = rows[p], j = cols[p];
        float *xr = (float *)malloc(sizeof(float) * (size_t)m);
        int8_t *qx = (int8_t *)malloc((size_t)m);
        int8_t *qw = (int8_t *)malloc((size_t)m);
        if (!xr || !qx || !qw) {
            fail = 1;
            continue;
        }
        float sxi, swj;
        for (int64_t k = 0; k < m; k++)
            xr[k] = (float)orc_half_to_double(x[i * m + k]);
        quantize_vector_q(xr, m, Q_MAX_A8, qx, &sxi);
        quantize_vector(w_res + j * m, m, qw, &swj);
        int64_t acc = 0;
        for (int64_t k = 0; k < m; k++)
            acc += (int64_t)qx[k] * (int64_t)qw[k];
        double lr = 0.0;
        for (int64_t u = 0; u < r; u++) {
            double tu = 0.0;
            for (int64_t k = 0; k < m; k++)
                tu += orc_half_to_double(x[i * m + k]) * orc_half_to_double(l1t[u * m + k]);
            lr += tu * orc_half_to_double(l2t[j * r + u]);
        }
        acc_out[p] = orc_require_i32(acc);
        y_out[p] = (double)sxi * (double)swj * (double)acc + lr;
        free(xr); free(qx); free(qw);
    }
    return fail;
}

#ifdef _OPENMP
#include <omp.h>
#endif
/* threads the parallel loops above will use (1 without OpenMP) */
int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- group-wise scales (TwinQuant page 1, section 5.1, and page 2, section 5.1:
 * weights and activations are quantized group-wise, groups of 128) ----
 *
 * Reading: a group is a run of g consecutive elements along the reduction
 * dimension K of one token row of X or one output channel of W_res; eq. (1)
 * applies to each group on its own, with its own binary32 scale. The integer
 * sum of eq. (2) then splits into one sum per group, each carrying the product
 * of its two group scales:
 *
 *   Y[i][j] = sum_G s_X[i][G] s_W[j][G] acc_G[i][j] + LR[i][j],
 *   acc_G[i][j] = sum_{k in G} Q_X[i][k] Q_W[j][k].
 *
 * Scales are stored row by row: s_X [b][m/g], s_W [n][m/g]. */

/* X fp16 [b][m] -> codes int8 [b][m], packed u8 [b][m/2] (may be NULL), s_X f32 [b][m/g] */
void orc_quantize_act_grouped(const uint16_t *x, int64_t b, int64_t m, int64_t g, int8_t *qx,
                              uint8_t *qx_packed, float *sx)
{
    const int64_t ng = m / g;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < b; i++) {
        float *row = (float *)malloc(sizeof(float) * (size_t)m);
        for (int64_t k = 0; k < m; k++)
            row[k] = (float)orc_half_to_double(x[i * m + k]);
        for (int64_t G = 0; G < ng; G++)
            quantize_vector(row + G * g, g, qx + i * m + G * g, sx + i * ng + G);
        if (qx_packed)
            pack_codes(qx + i * m, m, qx_packed + i * (m / 2));
        free(row);
    }
}

/* W_res f32 [n][m] -> codes int8 [n][m], packed u8 [n][m/2] (may be NULL), s_W f32 [n][m/g] */
void orc_quantize_weight_grouped(const float *w, int64_t n, int64_t m, int64_t g, int8_t *qw,
                                 uint8_t *qw_packed, float *sw)
{
    const int64_t ng = m / g;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; j++) {
        for (int64_t G = 0; G < ng; G++)
            quantize_vector(w + j * m + G * g, g, qw + j * m + G * g, sw + j * ng + G);
        if (qw_packed)
            pack_codes(qw + j * m, m, qw_packed + j * (m / 2));
    }
}

/* acc_G[i][j][G] = sum over k in group G of Q_X[i][k] Q_W[j][k], int64, layout [b][n][m/g] */
void orc_residual_acc_grouped(const int8_t *qx, const int8_t *qw, int64_t b, int64_t m, int64_t n,
                              int64_t g, int64_t *acc)
{
    const int64_t ng = m / g;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < b; i++)
        for (int64_t j = 0; j < n; j++)
            for (int64_t G = 0; G < ng; G++) {
                int64_t sum = 0;
                for (int64_t k = G * g; k < (G + 1) * g; k++)
                    sum += (int64_t)qx[i * m + k] * (int64_t)qw[j * m + k];
                acc[(i * n + j) * ng + G] = orc_require_i32(sum);
            }
}

/* The whole layer with group-wise scales and the fp16 low-rank branch, binary64:
 * Y[i][j] = sum_G s_X[i][G] s_W[j][G] acc_G[i][j] + LR[i][j].
 * Outputs other than y may be NULL. */
int orc_dual_linear_grouped(const uint16_t *x, const float *w_res, const uint16_t *l1t,
                            const uint16_t *l2t, int64_t b, int64_t m, int64_t n, int64_t r,
                            int64_t g, uint8_t *qx_packed, float *sx, uint8_t *qw_packed,
                            float *sw, double *y)
{
    const int64_t ng = m / g;
    int8_t *qx = (int8_t *)malloc((size_t)(b * m));
    int8_t *qw = (int8_t *)malloc((size_t)(n * m));
    float *sx_l = (float *)malloc(sizeof(float) * (size_t)(b * ng));
    float *sw_l = (float *)malloc(sizeof(float) * (size_t)(n * ng));
    int64_t *acc = (int64_t *)malloc(sizeof(int64_t) * (size_t)(b * n * ng));
    double *t = (double *)malloc(sizeof(double) * (size_t)(b * (r > 0 ? r : 1)));
    double *lr = (double *)malloc(sizeof(double) * (size_t)(b * n));
    if (!qx || !qw || !sx_l || !sw_l || !acc || !t || !lr)
        return 1;
    orc_quantize_act_grouped(x, b, m, g, qx, qx_packed, sx_l);
    orc_quantize_weight_grouped(w_res, n, m, g, qw, qw_packed, sw_l);
    orc_residual_acc_grouped(qx, qw, b, m, n, g, acc);
    if (r > 0) {
        orc_lowrank_t(x, l1t, b, m, r, t);
        orc_lowrank_out(t, l2t, b, n, r, lr);
    } else {
        memset(lr, 0, sizeof(double) * (size_t)(b * n));
    }
    for (int64_t i = 0; i < b; i++)
        for (int64_t j = 0; j < n; j++) {
            double sum = 0.0;
            for (int64_t G = 0; G < ng; G++)
                sum += (double)sx_l[i * ng + G] * (double)sw_l[j * ng + G] *
                       (double)acc[(i * n + j) * ng + G];
            y[i * n + j] = sum + lr[i * n + j];
        }
    if (sx)
        memcpy(sx, sx_l, sizeof(float) * (size_t)(b * ng));
    if (sw)
        memcpy(sw, sw_l, sizeof(float) * (size_t)(n * ng));
    free(qx); free(qw); free(sx_l); free(sw_l); free(acc); free(t); free(lr);
    return 0;
}

/* Y of the group-wise layer at sampled positions only: Y[rows[p]][cols[p]]. */
int orc_dual_linear_grouped_sampled(const uint16_t *x, const float *w_res, const uint16_t *l1t,
                                    const uint16_t *l2t, int64_t b, int64_t m, int64_t n,
                                    int64_t r, int64_t g, const int64_t *rows,
                                    const int64_t *cols, int64_t count, double *y_out)
{
    (void)b;
    (void)n;
    const int64_t ng = m / g;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < count; p++) {
        int64_t i = rows[p], j = cols[p];
        float *xr = (float *)malloc(sizeof(float) * (size_t)m);
        int8_t *qx = (int8_t *)malloc((size_t)m);
        int8_t *qw = (int8_t *)malloc((size_t)m);
        float *sxi = (float *)malloc(sizeof(float) * (size_t)ng);
        float *swj = (float *)malloc(sizeof(float) * (size_t)ng);
        if (!xr || !qx || !qw || !sxi || !swj) {
            fail = 1;
            continue;
        }
        for (int64_t k = 0; k < m; k++)
            xr[k] = (float)orc_half_to_double(x[i * m + k]);
        double y = 0.0;
        for (int64_t G = 0; G < ng; G++) {
            quantize_vector(xr + G * g, g, qx + G * g, sxi + G);
            quantize_vector(w_res + j * m + G * g, g, qw + G * g, swj + G);
            int64_t acc = 0;
            for (int64_t k = G * g; k < (G + 1) * g; k++)
                acc += (int64_t)qx[k] * (int64_t)qw[k];
            y += (double)sxi[G] * (double)swj[G] * (double)orc_require_i32(acc);
        }
        double lr = 0.0;
        for (int64_t u = 0; u < r; u++) {
            double tu = 0.0;
            for (int64_t k = 0; k < m; k++)
                tu += orc_half_to_double(x[i * m + k]) * orc_half_to_double(l1t[u * m + k]);
            lr += tu * orc_half_to_double(l2t[j * r + u]);
        }
        y_out[p] = y + lr;
        free(xr); free(qx); free(qw); free(sxi); free(swj);
    }
    return fail;
}
