// twq_device.h -- device-side building blocks shared by the libtwq kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <utility>
#include <stdint.h>

namespace twq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

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

// quant_code(v, s) without a division per element, given inv = fl32(1 / s) and
// |v| <= 7 s (every element of the vector s was taken from). t = fl32(v inv) is
// within 9e-7 of v / s (two roundings of relative size 2^-24 on a ratio of at most
// 7.5), and the correctly rounded fl32(v / s) within 4.5e-7, so their nearest
// integers can differ only if a half-integer lies within 1.4e-6 of t. Only then
// (|t - rint(t)| >= 0.5 - 2^-18) is the division done.
__device__ __forceinline__ int quant_code_fast(float v, float s, float inv) {
#pragma clang fp contract(off)
    float t = v * inv;
    float r = __builtin_rintf(t);
    if (__builtin_fabsf(t - r) >= 0.5f - 0x1p-18f) r = __builtin_rintf(v / s);
    r = __builtin_fminf(__builtin_fmaxf(r, -kQMax), kQMax);
    return (int)r;
}

// The 8-bit activation code of eq. (1) (q_max = 127) from inv = fl32(1 / s), exact
// in the same way as quant_code_fast: for |v / s| <= 127, t = fl32(v inv) lies within
// 1.6e-5 of v / s and fl32(v / s) within 7.6e-6, so only a t within 2^-15 of a
// half-integer takes the correctly rounded division.
constexpr float kQMax8 = 127.0f;  // 2^(k-1) - 1 for k = 8
__device__ __forceinline__ int quant_code8_fast(float v, float s, float inv) {
#pragma clang fp contract(off)
    float t = v * inv;
    float r = __builtin_rintf(t);
    if (__builtin_fabsf(t - r) >= 0.5f - 0x1p-15f) r = __builtin_rintf(v / s);
    r = __builtin_fminf(__builtin_fmaxf(r, -kQMax8), kQMax8);
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

// The running maximum mx of |x| over the eight fp16 values of a 16-byte chunk, as bit
// patterns: |x| of an fp16 is its pattern without the sign, and for finite values the
// integer order of these patterns is the order of the magnitudes.
__device__ __forceinline__ uint32_t absmax8_bits(const uint4 c, uint32_t mx) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        uint32_t lo = w[e] & 0x7FFFu, hi = (w[e] >> 16) & 0x7FFFu;
        mx = mx > lo ? mx : lo;
        mx = mx > hi ? mx : hi;
    }
    return mx;
}

// The eight 4-bit codes of eq. (1) of a 16-byte chunk of fp16 (quant_code_fast), packed.
__device__ __forceinline__ uint32_t quant8(const uint4 c, float s, float inv) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    int q[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        q[2 * e] = quant_code_fast(half_bits_to_float(w[e] & 0xFFFFu), s, inv);
        q[2 * e + 1] = quant_code_fast(half_bits_to_float(w[e] >> 16), s, inv);
    }
    return pack8(q);
}

// max over the 64 lanes of a wave (every lane active), returned uniform: butterflies
// within each row of 16 lanes by DPP moves (the two quad permutations, then the
// half-row and the row mirror), then the four row maxima read from lanes 0, 16, 32
// and 48. 0 is the identity of the unsigned max, so lanes a move has no source for
// read it harmlessly. Measured on MI355X: 0.16 us shorter than shuffles through LDS
// on the few-token quantizer.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    uint32_t t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1, 0, 3, 2]
    v = v > t ? v : t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2, 3, 0, 1]
    v = v > t ? v : t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    v = v > t ? v : t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);  // row_mirror
    v = v > t ? v : t;
    uint32_t a0 = __builtin_amdgcn_readlane(v, 0), a1 = __builtin_amdgcn_readlane(v, 16);
    uint32_t a2 = __builtin_amdgcn_readlane(v, 32), a3 = __builtin_amdgcn_readlane(v, 48);
    a0 = a0 > a1 ? a0 : a1;
    a2 = a2 > a3 ? a2 : a3;
    return a0 > a2 ? a0 : a2;
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

// 16 int8 codes (elements 0..15 of a K run, in order) -> one int8 MFMA operand in the
// lane-local K order unpack16 gives the packed 4-bit codes (1, 3, 5, 7, 0, 2, 4, 6,
// 9, ..., 8, ...), so an 8-bit operand pairs element for element with a 4-bit one.
__device__ __forceinline__ v4i perm16(const uint4 raw) {
    v4i r;
    r[0] = (int)__builtin_amdgcn_perm(raw.y, raw.x, 0x07050301u);
    r[1] = (int)__builtin_amdgcn_perm(raw.y, raw.x, 0x06040200u);
    r[2] = (int)__builtin_amdgcn_perm(raw.w, raw.z, 0x07050301u);
    r[3] = (int)__builtin_amdgcn_perm(raw.w, raw.z, 0x06040200u);
    return r;
}

__device__ __forceinline__ v4i perm16(const v4i raw) {
    return perm16(make_uint4((uint32_t)raw[0], (uint32_t)raw[1], (uint32_t)raw[2], (uint32_t)raw[3]));
}

__device__ __forceinline__ v4i mfma_i8(const v4i a, const v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_f16(const v8h a, const v8h b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 32 x 32 blocks: lane l supplies row l % 32 of each operand (16 int8 or 8 fp16 of one
// K run); lane l holds column l % 32 of the result, and its register v the row
// 8 (v / 4) + 4 (l / 32) + v % 4.
__device__ __forceinline__ v16i mfma_i8_32(const v4i a, const v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v16f mfma_f16_32(const v8h a, const v8h b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 16 bytes that one launch reads exactly once (the few-token weight stream): a
// non-temporal load, so the stream does not displace from L2 the lines every CTA
// re-reads (measured on MI355X: decode kernels 2.4-8.5% faster).
__device__ __forceinline__ uint4 load_stream16(const uint8_t *p) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p)));
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

// ---- LDS rings filled by direct-to-LDS loads (the prefill main loop and the
// many-token first low-rank product) ----

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // vmcnt = N, expcnt and lgkmcnt left at their maxima (not waited on)
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// LDS byte offset of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// The eight operand reads of one stage: four consecutive 1 KB blocks from address a
// and four from address b (each plus OFF), completed before returning (the wait is
// part of the same asm statement, so no output register is live while its load is in
// flight). Written as one statement because the compiler cannot tell these reads
// apart from the direct-to-LDS loads still in flight into other ring slots, and would
// otherwise wait for all of those first. The offsets ride in the instructions'
// 16-bit immediate field. The outputs are early-clobber ("=&v"): a read can return
// while later reads of the statement are still to issue, so no output may share a
// register with an address (the compiler otherwise may, where the address dies here).
template <int OFF, int BLK>
__device__ __forceinline__ void lds_read_4x4(uint32_t a, uint32_t b, v4i (&r)[8]) {
    static_assert(OFF >= 0 && OFF + 3 * BLK < 65536, "ds_read immediate offset");
    asm volatile(
        "ds_read_b128 %0, %8 offset:%10\n\t"
        "ds_read_b128 %1, %8 offset:%11\n\t"
        "ds_read_b128 %2, %8 offset:%12\n\t"
        "ds_read_b128 %3, %8 offset:%13\n\t"
        "ds_read_b128 %4, %9 offset:%10\n\t"
        "ds_read_b128 %5, %9 offset:%11\n\t"
        "ds_read_b128 %6, %9 offset:%12\n\t"
        "ds_read_b128 %7, %9 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(a), "v"(b), "n"(OFF), "n"(OFF + BLK), "n"(OFF + 2 * BLK), "n"(OFF + 3 * BLK)
        : "memory");
}

// The eight operand reads of one stage of 32 x 32 blocks: from each of the addresses
// a0, a1 (weight rows, the two halves of the stage) and b0, b1 (token rows), the blocks
// at OFF and OFF + STR, completed before returning, for the same reason and in the same
// way as lds_read_4x4. r = {a0, a0 + STR, a1, a1 + STR, b0, b0 + STR, b1, b1 + STR}.
template <int OFF, int STR>
__device__ __forceinline__ void lds_read_2x4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, v4i (&r)[8]) {
    static_assert(OFF >= 0 && OFF + STR < 65536, "ds_read immediate offset");
    asm volatile(
        "ds_read_b128 %0, %8 offset:%12\n\t"
        "ds_read_b128 %1, %8 offset:%13\n\t"
        "ds_read_b128 %2, %9 offset:%12\n\t"
        "ds_read_b128 %3, %9 offset:%13\n\t"
        "ds_read_b128 %4, %10 offset:%12\n\t"
        "ds_read_b128 %5, %10 offset:%13\n\t"
        "ds_read_b128 %6, %11 offset:%12\n\t"
        "ds_read_b128 %7, %11 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(a0), "v"(a1), "v"(b0), "v"(b1), "n"(OFF), "n"(OFF + STR)
        : "memory");
}

// Four operand reads: the blocks at OFF and OFF + STR from address a and from address b,
// completed before returning, for the same reason and in the same way as lds_read_4x4.
// r = {a, a + STR, b, b + STR}.
template <int OFF, int STR>
__device__ __forceinline__ void lds_read_2x2(uint32_t a, uint32_t b, v4i (&r)[4]) {
    static_assert(OFF >= 0 && OFF + STR < 65536, "ds_read immediate offset");
    asm volatile(
        "ds_read_b128 %0, %4 offset:%6\n\t"
        "ds_read_b128 %1, %4 offset:%7\n\t"
        "ds_read_b128 %2, %5 offset:%6\n\t"
        "ds_read_b128 %3, %5 offset:%7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(a), "v"(b), "n"(OFF), "n"(OFF + STR)
        : "memory");
}

// Twelve operand reads of one stage: four consecutive 1 KB blocks from each of the
// addresses a, b0 and b1 (each plus OFF), completed before returning, for the same
// reason and in the same way as lds_read_4x4.
template <int OFF, int BLK>
__device__ __forceinline__ void lds_read_4x4x4(uint32_t a, uint32_t b0, uint32_t b1, v4i (&r)[12]) {
    static_assert(OFF >= 0 && OFF + 3 * BLK < 65536, "ds_read immediate offset");
    asm volatile(
        "ds_read_b128 %0, %12 offset:%15\n\t"
        "ds_read_b128 %1, %12 offset:%16\n\t"
        "ds_read_b128 %2, %12 offset:%17\n\t"
        "ds_read_b128 %3, %12 offset:%18\n\t"
        "ds_read_b128 %4, %13 offset:%15\n\t"
        "ds_read_b128 %5, %13 offset:%16\n\t"
        "ds_read_b128 %6, %13 offset:%17\n\t"
        "ds_read_b128 %7, %13 offset:%18\n\t"
        "ds_read_b128 %8, %14 offset:%15\n\t"
        "ds_read_b128 %9, %14 offset:%16\n\t"
        "ds_read_b128 %10, %14 offset:%17\n\t"
        "ds_read_b128 %11, %14 offset:%18\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
          "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11])
        : "v"(a), "v"(b0), "v"(b1), "n"(OFF), "n"(OFF + BLK), "n"(OFF + 2 * BLK), "n"(OFF + 3 * BLK)
        : "memory");
}

// Workgroup barrier without the memory fence __syncthreads adds (which waits for every
// outstanding load); callers first wait for their own loads of the stage they need.
__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int... I, class F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, I...>, F &&f) {
    (f(std::integral_constant<int, I>{}), ...);
}

// Two 16-byte LDS reads of consecutive blocks at address a (plus OFF), completed
// before returning, for the same reason and in the same way as lds_read_4x4.
template <int OFF, int BLK>
__device__ __forceinline__ void lds_read_2(uint32_t a, v4i (&r)[2]) {
    static_assert(OFF >= 0 && OFF + BLK < 65536, "ds_read immediate offset");
    asm volatile(
        "ds_read_b128 %0, %2 offset:%3\n\t"
        "ds_read_b128 %1, %2 offset:%4\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1])
        : "v"(a), "n"(OFF), "n"(OFF + BLK)
        : "memory");
}

// Four 16-byte LDS reads of consecutive blocks at address a (plus OFF), completed
// before returning, for the same reason and in the same way as lds_read_4x4.
template <int OFF, int BLK>
__device__ __forceinline__ void lds_read_4(uint32_t a, v4i (&r)[4]) {
    static_assert(OFF >= 0 && OFF + 3 * BLK < 65536, "ds_read immediate offset");
    asm volatile(
        "ds_read_b128 %0, %4 offset:%5\n\t"
        "ds_read_b128 %1, %4 offset:%6\n\t"
        "ds_read_b128 %2, %4 offset:%7\n\t"
        "ds_read_b128 %3, %4 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(a), "n"(OFF), "n"(OFF + BLK), "n"(OFF + 2 * BLK), "n"(OFF + 3 * BLK)
        : "memory");
}

// Group scales of one ring stage for a wave's 4 x 4 tiles of 16 x 16: four 16-byte reads
// from address w (s_W of channels 4g..4g+3 of each of four channel blocks, 64 bytes
// apart) and four 4-byte reads from address x (s_X of token li of each of four token
// blocks, 64 bytes apart), each plus OFF, completed before returning for the same
// reason and in the same way as lds_read_4x4.
template <int OFF>
__device__ __forceinline__ void lds_read_scales(uint32_t w, uint32_t x, v4f (&sw)[4], float (&sx)[4]) {
    static_assert(OFF >= 0 && OFF + 192 < 65536, "ds_read immediate offset");
    asm volatile(
        "ds_read_b128 %0, %8 offset:%10\n\t"
        "ds_read_b128 %1, %8 offset:%11\n\t"
        "ds_read_b128 %2, %8 offset:%12\n\t"
        "ds_read_b128 %3, %8 offset:%13\n\t"
        "ds_read_b32 %4, %9 offset:%10\n\t"
        "ds_read_b32 %5, %9 offset:%11\n\t"
        "ds_read_b32 %6, %9 offset:%12\n\t"
        "ds_read_b32 %7, %9 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(sw[0]), "=&v"(sw[1]), "=&v"(sw[2]), "=&v"(sw[3]), "=&v"(sx[0]), "=&v"(sx[1]), "=&v"(sx[2]), "=&v"(sx[3])
        : "v"(w), "v"(x), "n"(OFF), "n"(OFF + 64), "n"(OFF + 128), "n"(OFF + 192)
        : "memory");
}

// Per-channel and per-token scales of one 32-channel block of a wave's 2 x 2 blocks of
// 32 x 32: four 16-byte reads from address w plus OW (s_W of channels 8q + 4 (l / 32)
// .. + 3, q = 0..3, 32 bytes apart) and two 4-byte reads from address x plus OX (s_X of
// token l % 32 of each 32-token block, 128 bytes apart), completed before returning for
// the same reason and in the same way as lds_read_4x4.
template <int OW, int OX>
__device__ __forceinline__ void lds_read_scales32(uint32_t w, uint32_t x, v4f (&sw)[4], float (&sx)[2]) {
    static_assert(OW >= 0 && OW + 96 < 65536 && OX >= 0 && OX + 128 < 65536, "ds_read immediate offset");
    asm volatile(
        "ds_read_b128 %0, %6 offset:%8\n\t"
        "ds_read_b128 %1, %6 offset:%9\n\t"
        "ds_read_b128 %2, %6 offset:%10\n\t"
        "ds_read_b128 %3, %6 offset:%11\n\t"
        "ds_read_b32 %4, %7 offset:%12\n\t"
        "ds_read_b32 %5, %7 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(sw[0]), "=&v"(sw[1]), "=&v"(sw[2]), "=&v"(sw[3]), "=&v"(sx[0]), "=&v"(sx[1])
        : "v"(w), "v"(x), "n"(OW), "n"(OW + 32), "n"(OW + 64), "n"(OW + 96), "n"(OX), "n"(OX + 128)
        : "memory");
}

}  // namespace twq
