// pack_weight.hip -- offline packing of the residual weight (gfx950).
//
// eq. (1) of TwinQuant (page 1, section 2) applied per output channel to the
// residual R of eq. (3): one CTA per row of W_res (fp32 [n][m]) computes
// s_W = max|w| / 7 and writes the packed 4-bit codes in the library's format.
#include "twq_device.h"
#include "twq_kernels.h"

namespace twq {

constexpr int kPackThreads = 256;
constexpr int kPackMaxJ = 8;  // rows of up to 256 * 8 * 8 = 16384 floats stay in registers

__device__ __forceinline__ float absmax8_f32(const float4 a, const float4 b, float mx) {
    mx = __builtin_fmaxf(mx, __builtin_fabsf(a.x)); mx = __builtin_fmaxf(mx, __builtin_fabsf(a.y));
    mx = __builtin_fmaxf(mx, __builtin_fabsf(a.z)); mx = __builtin_fmaxf(mx, __builtin_fabsf(a.w));
    mx = __builtin_fmaxf(mx, __builtin_fabsf(b.x)); mx = __builtin_fmaxf(mx, __builtin_fabsf(b.y));
    mx = __builtin_fmaxf(mx, __builtin_fabsf(b.z)); mx = __builtin_fmaxf(mx, __builtin_fabsf(b.w));
    return mx;
}

__device__ __forceinline__ uint32_t quant8_f32(const float4 a, const float4 b, float s) {
    int q[8];
    q[0] = quant_code(a.x, s); q[1] = quant_code(a.y, s); q[2] = quant_code(a.z, s); q[3] = quant_code(a.w, s);
    q[4] = quant_code(b.x, s); q[5] = quant_code(b.y, s); q[6] = quant_code(b.z, s); q[7] = quant_code(b.w, s);
    return pack8(q);
}

__global__ __launch_bounds__(kPackThreads) void pack_weight_kernel(const float *w, int64_t m, uint8_t *qw,
                                                                   float *sw) {
    __shared__ float red[kPackThreads / kWave];
    const int64_t j = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t nch = m / 8;
    const float4 *wr = reinterpret_cast<const float4 *>(w + j * m);
    uint32_t *qr = reinterpret_cast<uint32_t *>(qw + j * (m / 2));
    const bool cached = nch <= (int64_t)kPackThreads * kPackMaxJ;
    float4 va[kPackMaxJ], vb[kPackMaxJ];
    float mx = 0.0f;
    if (cached) {
#pragma unroll
        for (int i = 0; i < kPackMaxJ; ++i) {
            const int64_t c = tid + (int64_t)i * kPackThreads;
            va[i] = c < nch ? wr[2 * c] : make_float4(0.f, 0.f, 0.f, 0.f);
            vb[i] = c < nch ? wr[2 * c + 1] : make_float4(0.f, 0.f, 0.f, 0.f);
            mx = absmax8_f32(va[i], vb[i], mx);
        }
    } else {
        for (int64_t c = tid; c < nch; c += kPackThreads) mx = absmax8_f32(wr[2 * c], wr[2 * c + 1], mx);
    }
    mx = wave_max_f32(mx);
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int i = 1; i < kPackThreads / kWave; ++i) mx = __builtin_fmaxf(mx, red[i]);
    const float s = mx / kQMax;
    if (tid == 0) sw[j] = s;
    if (cached) {
#pragma unroll
        for (int i = 0; i < kPackMaxJ; ++i) {
            const int64_t c = tid + (int64_t)i * kPackThreads;
            if (c < nch) qr[c] = mx == 0.0f ? 0u : quant8_f32(va[i], vb[i], s);
        }
    } else {
        for (int64_t c = tid; c < nch; c += kPackThreads)
            qr[c] = mx == 0.0f ? 0u : quant8_f32(wr[2 * c], wr[2 * c + 1], s);
    }
}

hipError_t launch_pack_weight(const float *w, int64_t n, int64_t m, uint8_t *qw, float *sw, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_weight_kernel, dim3((unsigned)n), dim3(kPackThreads), 0, stream, w, m, qw, sw);
    return hipGetLastError();
}

}  // namespace twq
