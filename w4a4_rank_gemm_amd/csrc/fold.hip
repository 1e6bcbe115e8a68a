// fold.hip -- offline preparation of a layer: folding given transforms into its split.
//
// TwinQuant page 1, section 4.1: with the weight split W = U V + R (eq. (3), a rank-r
// pair from the SVD and a residual), an orthogonal Q (m x m) applied to the activations
// and an invertible G (r x r) applied to the rank space are folded into the operands:
//
//   U' = Q^-1 U G,   V' = G^-1 V,   R' = Q^-1 R,   and the layer is fed X Q,
//
// which leaves the real product unchanged, (X Q)(U' V' + R') = X W. Here U = U_r
// sqrt(S_r) and V = sqrt(S_r) V_r^T come from the caller's top-r SVD of W (the platform
// library's), Q^-1 = Q^T, the factors are rounded to fp16 as the layer stores them, and
// R' = Q^T W - U' V' is formed from those rounded factors so the split is exact against
// what the layer is given, then rounded to fp32.
//
// The arithmetic is binary64: one tiled GEMM kernel (64 x 64 output tiles, K in steps of
// 16 through LDS, 4 x 4 outputs a thread, fused multiply-adds) for every product, with
// the transposes expressed as strides and the fp16 / fp32 rounding and the transposed
// stores in its epilogue; G^-1 by Gauss-Jordan elimination with partial pivoting in one
// CTA (r <= 256). This runs once per layer, before serving; it is not on the hot path.
#include <hip/hip_runtime.h>

#include "twq_kernels.h"

namespace twq {

namespace {

constexpr int kFT = 64, kFK = 16, kFThreads = 256;

// Operand element (i, k) of a strided matrix: p[i * si + k * sk] (fp64 or fp16 storage).
template <typename T>
__device__ __forceinline__ double fold_at(const T *p, int64_t i, int64_t k, int64_t si, int64_t sk) {
    return (double)p[i * si + k * sk];
}

enum FoldOut { kOutF64 = 0, kOutF16T = 1, kOutF32T = 2 };

// C (M x N) = [C0 +] A1 B1 [- A2 B2], A1 (M x K1), B1 (K1 x N), A2 (M x K2), B2 (K2 x N),
// each addressed through (row, column) strides. c0: optional M x N fp64 addend with
// strides (c0i, c0j). Output: kOutF64 -> out[i * N + j] fp64; kOutF16T -> out[j * M + i]
// fp16 (round to nearest even); kOutF32T -> out[j * M + i] fp32.
template <typename TA2, int OUT>
__global__ __launch_bounds__(kFThreads) void fold_gemm_kernel(
    const double *a1, int64_t a1i, int64_t a1k, const double *b1, int64_t b1k, int64_t b1j, int64_t k1,
    const TA2 *a2, int64_t a2i, int64_t a2k, const TA2 *b2, int64_t b2k, int64_t b2j, int64_t k2,
    const double *c0, int64_t c0i, int64_t c0j, int64_t M, int64_t N, void *out) {
    __shared__ double as[kFK][kFT + 1];
    __shared__ double bs[kFK][kFT + 1];
    const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
    const int64_t i0 = (int64_t)blockIdx.y * kFT, j0 = (int64_t)blockIdx.x * kFT;
    double acc[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t i = i0 + ty * 4 + u, j = j0 + tx * 4 + v;
            acc[u][v] = (c0 && i < M && j < N) ? c0[i * c0i + j * c0j] : 0.0;
        }
    // two products, the second subtracted: sign s, K extent kk
    for (int pass = 0; pass < 2; ++pass) {
        const int64_t kk = pass == 0 ? k1 : k2;
        if (kk == 0 || (pass == 0 ? a1 == nullptr : a2 == nullptr)) continue;
        const double sgn = pass == 0 ? 1.0 : -1.0;
        for (int64_t k0 = 0; k0 < kk; k0 += kFK) {
            // stage A (kFT rows x kFK) and B (kFK x kFT columns), zero past the edges
            for (int e = tid; e < kFT * kFK; e += kFThreads) {
                const int r_ = e / kFK, c_ = e % kFK;
                const int64_t i = i0 + r_, k = k0 + c_;
                double va = 0.0;
                if (i < M && k < kk)
                    va = pass == 0 ? fold_at(a1, i, k, a1i, a1k) : fold_at(a2, i, k, a2i, a2k);
                as[c_][r_] = va;
                const int rb = e / kFT, cb = e % kFT;
                const int64_t kb = k0 + rb, j = j0 + cb;
                double vb = 0.0;
                if (kb < kk && j < N)
                    vb = pass == 0 ? fold_at(b1, kb, j, b1k, b1j) : fold_at(b2, kb, j, b2k, b2j);
                bs[rb][cb] = vb;
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < kFK; ++k) {
                double av[4], bv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) av[u] = sgn * as[k][ty * 4 + u];
#pragma unroll
                for (int v = 0; v < 4; ++v) bv[v] = bs[k][tx * 4 + v];
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[u][v] = __builtin_fma(av[u], bv[v], acc[u][v]);
            }
            __syncthreads();
        }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t i = i0 + ty * 4 + u, j = j0 + tx * 4 + v;
            if (i >= M || j >= N) continue;
            if constexpr (OUT == kOutF64)
                static_cast<double *>(out)[i * N + j] = acc[u][v];
            else if constexpr (OUT == kOutF16T)  // one correctly rounded f64 -> f16 conversion
                static_cast<_Float16 *>(out)[j * M + i] = (_Float16)acc[u][v];
            else
                static_cast<float *>(out)[j * M + i] = (float)acc[u][v];
        }
}

// U_r[i][t] = u[i][t] sqrt(s[t]) (m x r) and V_r[t][j] = sqrt(s[t]) vt[t][j] (r x n).
__global__ __launch_bounds__(kFThreads) void fold_scale_kernel(const double *u, const double *s, const double *vt,
                                                               int64_t m, int64_t n, int64_t r, double *ur,
                                                               double *vr) {
    const int64_t e = (int64_t)blockIdx.x * kFThreads + threadIdx.x;
    if (e < m * r) ur[e] = u[e] * __builtin_sqrt(s[e % r]);
    if (e < r * n) vr[e] = vt[e] * __builtin_sqrt(s[e / n]);
}

// G^-1 by Gauss-Jordan elimination with partial pivoting on [G | I], r x 2r in global
// memory (the workspace), one CTA. A zero pivot (G singular) leaves non-finite values.
__global__ __launch_bounds__(1024) void fold_inverse_kernel(const double *g, int64_t r, double *aug, double *ginv) {
    __shared__ int piv;
    __shared__ double pval;
    __shared__ double fcol[256];  // column c of every row, read before the rows change
    const int tid = threadIdx.x, nt = blockDim.x;
    const int64_t w2 = 2 * r;
    for (int64_t e = tid; e < r * w2; e += nt) {
        const int64_t i = e / w2, j = e % w2;
        aug[e] = j < r ? g[i * r + j] : (j - r == i ? 1.0 : 0.0);
    }
    __syncthreads();
    for (int64_t c = 0; c < r; ++c) {
        if (tid == 0) {  // the largest |entry| of column c at or below the diagonal
            int64_t best = c;
            double bv = __builtin_fabs(aug[c * w2 + c]);
            for (int64_t i = c + 1; i < r; ++i) {
                const double v = __builtin_fabs(aug[i * w2 + c]);
                if (v > bv) {
                    bv = v;
                    best = i;
                }
            }
            piv = (int)best;
        }
        __syncthreads();
        if (piv != c)
            for (int64_t j = tid; j < w2; j += nt) {
                const double t = aug[c * w2 + j];
                aug[c * w2 + j] = aug[piv * w2 + j];
                aug[piv * w2 + j] = t;
            }
        __syncthreads();
        if (tid == 0) pval = aug[c * w2 + c];
        __syncthreads();
        for (int64_t j = tid; j < w2; j += nt) aug[c * w2 + j] /= pval;
        __syncthreads();
        for (int64_t i = tid; i < r; i += nt) fcol[i] = aug[i * w2 + c];
        __syncthreads();
        // row i -= fcol[i] * row c (the pivot row now has 1 in column c, so column c of
        // every other row becomes exactly 0)
        for (int64_t e = tid; e < r * w2; e += nt) {
            const int64_t i = e / w2, j = e % w2;
            if (i != c) aug[e] = __builtin_fma(-fcol[i], aug[c * w2 + j], aug[e]);
        }
        __syncthreads();
    }
    for (int64_t e = tid; e < r * r; e += nt) ginv[e] = aug[(e / r) * w2 + r + e % r];
}

template <typename TA2, int OUT>
hipError_t gemm(const double *a1, int64_t a1i, int64_t a1k, const double *b1, int64_t b1k, int64_t b1j, int64_t k1,
                const TA2 *a2, int64_t a2i, int64_t a2k, const TA2 *b2, int64_t b2k, int64_t b2j, int64_t k2,
                const double *c0, int64_t c0i, int64_t c0j, int64_t M, int64_t N, void *out, hipStream_t s) {
    const dim3 grid((unsigned)((N + kFT - 1) / kFT), (unsigned)((M + kFT - 1) / kFT));
    hipLaunchKernelGGL((fold_gemm_kernel<TA2, OUT>), grid, dim3(kFThreads), 0, s, a1, a1i, a1k, b1, b1k, b1j, k1,
                       a2, a2i, a2k, b2, b2k, b2j, k2, c0, c0i, c0j, M, N, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fold(const FoldArgs &a, hipStream_t s) {
    const int64_t m = a.m, n = a.n, r = a.r;
    const FoldLayout L = fold_layout(m, n, r);
    uint8_t *ws = static_cast<uint8_t *>(a.workspace);
    double *ur = reinterpret_cast<double *>(ws + L.ur), *vr = reinterpret_cast<double *>(ws + L.vr);
    double *t1 = reinterpret_cast<double *>(ws + L.t1);
    double *aug = reinterpret_cast<double *>(ws + L.aug), *ginv = reinterpret_cast<double *>(ws + L.ginv);
    const _Float16 *l1t = static_cast<const _Float16 *>(a.l1t), *l2t = static_cast<const _Float16 *>(a.l2t);
    hipError_t e = hipSuccess;
    if (r > 0) {
        const int64_t cnt = m * r > r * n ? m * r : r * n;
        hipLaunchKernelGGL(fold_scale_kernel, dim3((unsigned)((cnt + kFThreads - 1) / kFThreads)), dim3(kFThreads), 0, s,
                           a.u, a.s, a.vt, m, n, r, ur, vr);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        // T1 = Q^T U_r (m x r): A1(i, k) = Q[k][i]
        const double *uq = ur;
        if (a.q) {
            e = gemm<double, kOutF64>(a.q, 1, m, ur, r, 1, m, nullptr, 0, 0, nullptr, 0, 0, 0, nullptr, 0, 0, m, r, t1, s);
            if (e != hipSuccess) return e;
            uq = t1;
        }
        // U' = T1 G, stored as fp16 L1^T [r][m]; without G, T1 itself
        if (a.g)
            e = gemm<double, kOutF16T>(uq, r, 1, a.g, r, 1, r, nullptr, 0, 0, nullptr, 0, 0, 0, nullptr, 0, 0, m, r,
                                       a.l1t, s);
        else
            e = gemm<double, kOutF16T>(nullptr, 0, 0, nullptr, 0, 0, 0, nullptr, 0, 0, nullptr, 0, 0, 0, uq, r, 1, m, r,
                                       a.l1t, s);
        if (e != hipSuccess) return e;
        // V' = G^-1 V_r, stored as fp16 L2^T [n][r]; without G, V_r itself
        if (a.g) {
            hipLaunchKernelGGL(fold_inverse_kernel, dim3(1), dim3(1024), 0, s, a.g, r, aug, ginv);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            e = gemm<double, kOutF16T>(ginv, r, 1, vr, n, 1, r, nullptr, 0, 0, nullptr, 0, 0, 0, nullptr, 0, 0, r, n,
                                       a.l2t, s);
        } else {
            e = gemm<double, kOutF16T>(nullptr, 0, 0, nullptr, 0, 0, 0, nullptr, 0, 0, nullptr, 0, 0, 0, vr, n, 1, r, n,
                                       a.l2t, s);
        }
        if (e != hipSuccess) return e;
    }
    // R' = Q^T W - L1 L2 (m x n), from the fp16 factors just stored, as fp32 R'^T [n][m].
    // W(k, j) = w[j][k]; without Q the first term is W itself. L1(i, t) = l1t[t][i],
    // L2(t, j) = l2t[j][t].
    if (a.q)
        return gemm<_Float16, kOutF32T>(a.q, 1, m, a.w, 1, m, m, l1t, 1, m, l2t, 1, r, r, nullptr, 0, 0, m, n,
                                        a.w_res, s);
    return gemm<_Float16, kOutF32T>(nullptr, 0, 0, nullptr, 0, 0, 0, l1t, 1, m, l2t, 1, r, r, a.w, 1, m, m, n, a.w_res,
                                    s);
}

}  // namespace twq
