// pack_weight.hip -- offline packing of the residual weight (gfx950).
//
// eq. (1) of TwinQuant (page 1, section 2) applied per output channel to the
// residual R of eq. (3): one CTA per row of W_res (fp32 [n][m]) computes
// s_W = max|w| / 7 and writes the packed 4-bit codes in the library's panel layout
// (qw_offset): a thread's 8 codes are one aligned dword of one 64-byte segment.
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
    auto qr = [&](int64_t c) -> uint32_t & { return *reinterpret_cast<uint32_t *>(qw + qw_offset(j, 4 * c, m)); };
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
            if (c < nch) qr(c) = mx == 0.0f ? 0u : quant8_f32(va[i], vb[i], s);
        }
    } else {
        for (int64_t c = tid; c < nch; c += kPackThreads)
            qr(c) = mx == 0.0f ? 0u : quant8_f32(wr[2 * c], wr[2 * c + 1], s);
    }
}

// Group-wise packing (groups of kGroup = 128 along K, as in TwinQuant page 1, section
// 5.1): one CTA per row, each thread one 8-element chunk at a time. A group is 16
// chunks held by 16 consecutive lanes, so its amax is a 16-lane reduction and the
// group's scale goes to sw[group][row] (group-major).
__global__ __launch_bounds__(kPackThreads) void pack_weight_grouped_kernel(const float *w, int64_t n, int64_t m,
                                                                           uint8_t *qw, float *sw) {
    static_assert(kGroup == 128, "a group is 16 chunks of 8");
    const int64_t j = blockIdx.x;
    const int64_t nch = m / 8;  // a multiple of 16
    const float4 *wr = reinterpret_cast<const float4 *>(w + j * m);
    for (int64_t c = threadIdx.x; c < nch; c += kPackThreads) {  // whole 16-lane groups enter together
        const float4 va = wr[2 * c], vb = wr[2 * c + 1];
        float mx = absmax8_f32(va, vb, 0.0f);
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, off, kWave));
        const float s = mx / kQMax;
        if ((threadIdx.x & 15) == 0) sw[(c / 16) * n + j] = s;
        *reinterpret_cast<uint32_t *>(qw + qw_offset(j, 4 * c, m)) = mx == 0.0f ? 0u : quant8_f32(va, vb, s);
    }
}

hipError_t launch_pack_weight_grouped(const float *w, int64_t n, int64_t m, uint8_t *qw, float *sw,
                                      hipStream_t stream) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_weight_grouped_kernel, dim3((unsigned)n), dim3(kPackThreads), 0, stream, w, n, m, qw, sw);
    return hipGetLastError();
}

hipError_t launch_pack_weight(const float *w, int64_t n, int64_t m, uint8_t *qw, float *sw, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_weight_kernel, dim3((unsigned)n), dim3(kPackThreads), 0, stream, w, m, qw, sw);
    return hipGetLastError();
}

}  // namespace twq
