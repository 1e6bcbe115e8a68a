// lowrank_int4.hip -- the int4 low-rank variant of the fused layer (gfx950).
//
// TwinQuant page 1, section 4.3 quantizes both low-rank factors to 4 bits: the first
// low-rank GEMM gives INT32 H, which gets a scale s_H estimated from the
// accumulators and is requantized to packed 4-bit Q_H for the second GEMM. Here:
//  * pack: L1 (m x r) gets one scale per column t and L2 (r x n) one per row t, by
//    eq. (1) (page 1, section 2); c_t = s_L1[t] s_L2[t] is what the second GEMM
//    cannot carry inside its integer sum over t;
//  * requant: per token, h_t = (s_X H_t) c_t in binary32, s_H = max_t |h_t| / 7,
//    Q_H = round(h / s_H) -- one scale per token over its r values;
//  * the fused kernel's epilogue then adds s_H (Q_H Q_L2) (dual_linear.hip).
// H itself is the residual integer GEMM with Q_L1 in place of Q_W (same kernels).
#include "twq_device.h"
#include "twq_kernels.h"

namespace twq {

constexpr int kLrThreads = 256;

__device__ __forceinline__ float block_max(float v, float *red) {
    v = wave_max_f32(v);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int w = 1; w < kLrThreads / kWave; ++w) m = __builtin_fmaxf(m, red[w]);
    __syncthreads();
    return m;
}

// one CTA per rank t: s_L1[t], the codes of row t of L1^T, s_L2[t] and c[t]
__global__ __launch_bounds__(kLrThreads) void lr_scales_kernel(const uint16_t *l1t, const uint16_t *l2t, int r,
                                                               int64_t m, int64_t n, uint8_t *ql1, float *sl1,
                                                               float *sl2, float *c) {
    __shared__ float red[kLrThreads / kWave];
    const int t = blockIdx.x;
    const uint16_t *row = l1t + (int64_t)t * m;
    float mx = 0.0f;
    for (int64_t k = threadIdx.x; k < m; k += kLrThreads) mx = __builtin_fmaxf(mx, __builtin_fabsf(half_bits_to_float(row[k])));
    const float a1 = block_max(mx, red);
    const float s1 = a1 / kQMax;
    for (int64_t c8 = threadIdx.x; c8 < m / 8; c8 += kLrThreads) {  // Q_L1 is H's weight operand: panel layout
        int q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = a1 == 0.0f ? 0 : quant_code(half_bits_to_float(row[c8 * 8 + e]), s1);
        *reinterpret_cast<uint32_t *>(ql1 + qw_offset(t, 4 * c8, m)) = pack8(q);
    }
    mx = 0.0f;
    for (int64_t j = threadIdx.x; j < n; j += kLrThreads)
        mx = __builtin_fmaxf(mx, __builtin_fabsf(half_bits_to_float(l2t[j * r + t])));
    const float a2 = block_max(mx, red);
    const float s2 = a2 / kQMax;
    if (threadIdx.x == 0) {
        sl1[t] = s1;
        sl2[t] = s2;
        c[t] = s1 * s2;
    }
}

// codes of L2 (column t of L2^T quantized with s_L2[t]), packed K = r contiguous per
// output channel: one thread per byte (ranks 2p and 2p + 1 of channel j)
__global__ __launch_bounds__(kLrThreads) void lr_pack_l2_kernel(const uint16_t *l2t, const float *sl2, int r,
                                                                int64_t n, uint8_t *ql2) {
    const int64_t idx = (int64_t)blockIdx.x * kLrThreads + threadIdx.x;
    if (idx >= n * (r / 2)) return;
    const int64_t j = idx / (r / 2);
    const int p = (int)(idx % (r / 2));
    int q[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const float s = sl2[2 * p + e];
        q[e] = s == 0.0f ? 0 : quant_code(half_bits_to_float(l2t[j * r + 2 * p + e]), s);
    }
    ql2[idx] = (uint8_t)((uint32_t(q[0]) & 0xFu) | ((uint32_t(q[1]) & 0xFu) << 4));
}

// one wave per token row i: h_t = (s_X[i] H[i][t]) c[t], s_H[i] = max_t |h_t| / 7,
// Q_H[i][t] = round(h_t / s_H[i]), packed two per byte
__global__ __launch_bounds__(kLrThreads) void lr_requant_kernel(const int32_t *h, const float *sx, const float *c,
                                                                int r, int64_t b, uint8_t *qh, float *sh) {
#pragma clang fp contract(off)
    const int64_t i = (int64_t)blockIdx.x * (kLrThreads / kWave) + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (i >= b) return;
    // r <= 256: lane holds the pairs p = lane and p = lane + 64
    float hv[2][2];
    float mx = 0.0f;
    const float sxi = sx[i];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int p = lane + 64 * k;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int t = 2 * p + e;
            if (t < r) {
                const float prod = sxi * (float)h[i * r + t];  // exact: |H| <= 49 m < 2^24
                hv[k][e] = prod * c[t];
                mx = __builtin_fmaxf(mx, __builtin_fabsf(hv[k][e]));
            } else {
                hv[k][e] = 0.0f;
            }
        }
    }
    mx = wave_max_f32(mx);
    const float s = mx / kQMax;
    if (lane == 0) sh[i] = s;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int p = lane + 64 * k;
        if (2 * p < r) {
            const int q0 = mx == 0.0f ? 0 : quant_code(hv[k][0], s);
            const int q1 = mx == 0.0f ? 0 : quant_code(hv[k][1], s);
            qh[i * (r / 2) + p] = (uint8_t)((uint32_t(q0) & 0xFu) | ((uint32_t(q1) & 0xFu) << 4));
        }
    }
}

hipError_t launch_pack_lowrank(const uint16_t *l1t, const uint16_t *l2t, int r, int64_t m, int64_t n, uint8_t *ql1,
                               float *sl1, uint8_t *ql2, float *sl2, float *c, hipStream_t stream) {
    if (r == 0) return hipSuccess;
    hipLaunchKernelGGL(lr_scales_kernel, dim3(r), dim3(kLrThreads), 0, stream, l1t, l2t, r, m, n, ql1, sl1, sl2, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n == 0) return e;
    const int64_t bytes = n * (r / 2);
    hipLaunchKernelGGL(lr_pack_l2_kernel, dim3((unsigned)((bytes + kLrThreads - 1) / kLrThreads)), dim3(kLrThreads), 0,
                       stream, l2t, sl2, r, n, ql2);
    return hipGetLastError();
}

hipError_t launch_lowrank_requant(const uint8_t *qx, const float *sx, const uint8_t *ql1, const float *c, int r,
                                  int32_t *h, uint8_t *qh, float *sh, int64_t b, int64_t m, hipStream_t stream) {
    DualArgs a{};
    a.qx = qx;
    a.qw = ql1;  // H = Q_X Q_L1^T: the residual integer GEMM with r output channels
    a.acc = h;
    a.b = b;
    a.m = m;
    a.n = r;
    hipError_t e = launch_dual_linear(a, stream);
    if (e != hipSuccess) return e;
    const int per = kLrThreads / kWave;
    hipLaunchKernelGGL(lr_requant_kernel, dim3((unsigned)((b + per - 1) / per)), dim3(kLrThreads), 0, stream, h, sx, c,
                       r, b, qh, sh);
    return hipGetLastError();
}

}  // namespace twq
