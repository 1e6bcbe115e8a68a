// twq_device.h -- device-side building blocks shared by the libtwq kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace twq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kQMax = 7.0f;  // 2^(k-1) - 1 for k = 4 (TwinQuant page 1, section 2, eq. (1))

// One code of eq. (1): q = round-half-even(fl32(v / s)) clamped to [-7, 7].
// The division is the correctly rounded binary32 one (the library is built with
// -fhip-fp32-correctly-rounded-divide-sqrt); no contraction may touch it.
__device__ __forceinline__ int quant_code(float v, float s) {
#pragma clang fp contract(off)
    float ratio = v / s;
    float r = __builtin_rintf(ratio);
    r = __builtin_fminf(__builtin_fmaxf(r, -kQMax), kQMax);
    return (int)r;
}

// Eight codes (elements e0..e7 of a row, in order) into one dword of the packed
// format: element 2t in the low nibble of byte t, element 2t+1 in its high nibble.
__device__ __forceinline__ uint32_t pack8(const int q[8]) {
    uint32_t p = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) p |= (uint32_t(q[e]) & 0xFu) << (4 * e);
    return p;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// max over the 64 lanes of a wave
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, kWave);
        v = v > o ? v : o;
    }
    return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// Packed 4-bit codes -> int8 MFMA operands, scaled by 16.
// A dword of packed codes holds 8 nibbles; masking the high nibbles gives the odd
// elements as int8 values 16*q, and shifting left by 4 first gives the even ones.
// The sign comes for free (a 4-bit two's complement nibble in the top of a byte
// is an int8 multiple of 16), so a product of two such operands is 256 * q_a * q_b
// exactly. The lane-local order of K elements this produces is the same for
// every operand unpacked here, so dot products over K are unaffected.
__device__ __forceinline__ void unpack16(const uint4 raw, v4i &lo, v4i &hi) {
    const uint32_t M = 0xF0F0F0F0u;
    lo[0] = (int)(raw.x & M);
    lo[1] = (int)((raw.x << 4) & M);
    lo[2] = (int)(raw.y & M);
    lo[3] = (int)((raw.y << 4) & M);
    hi[0] = (int)(raw.z & M);
    hi[1] = (int)((raw.z << 4) & M);
    hi[2] = (int)(raw.w & M);
    hi[3] = (int)((raw.w << 4) & M);
}

__device__ __forceinline__ void unpack16(const v4i raw, v4i &lo, v4i &hi) {
    unpack16(make_uint4((uint32_t)raw[0], (uint32_t)raw[1], (uint32_t)raw[2], (uint32_t)raw[3]), lo, hi);
}

__device__ __forceinline__ v4i mfma_i8(const v4i a, const v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_f16(const v8h a, const v8h b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8h load_h8(const uint16_t *p) {
    return *reinterpret_cast<const v8h *>(p);
}

__device__ __forceinline__ v8h f32x8_to_h8(const float4 a, const float4 b) {
    v8h r;
    r[0] = (_Float16)a.x; r[1] = (_Float16)a.y; r[2] = (_Float16)a.z; r[3] = (_Float16)a.w;
    r[4] = (_Float16)b.x; r[5] = (_Float16)b.y; r[6] = (_Float16)b.z; r[7] = (_Float16)b.w;
    return r;
}

}  // namespace twq
