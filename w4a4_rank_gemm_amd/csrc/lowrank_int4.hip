// lowrank_int4.hip -- the int4 low-rank variant of the fused layer (gfx950).
//
// TwinQuant page 1, section 4.3 quantizes both low-rank factors to 4 bits: the first
// low-rank GEMM gives INT32 H, which gets a scale s_H estimated from the
// accumulators and is requantized to packed 4-bit Q_H for the second GEMM. Here:
//  * pack (this file): L1 (m x r) gets one scale per column t and L2 (r x n) one per
//    row t, by eq. (1) (page 1, section 2); c_t = s_L1[t] s_L2[t] is what the second
//    GEMM cannot carry inside its integer sum over t;
//  * H = Q_X Q_L1^T and its requantization, per token h_t = (s_X H_t) c_t in binary32,
//    s_H = max_t |h_t| / 7, Q_H = round(h / s_H), happen on chip in lr4_requant_kernel
//    below, which stores only Q_H and s_H (and, with few tokens, quantizes X first);
//  * the fused kernel's epilogue then adds s_H (Q_H Q_L2) (dual_linear.hip).
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

// ---- H = Q_X Q_L1^T and its requantization, on chip ----------------------------------
//
// One CTA of NW waves owns tpc <= BM = 16 TB tokens and all r ranks, so every token's
// whole row of H is formed inside it and s_H needs nothing from another CTA. With few
// tokens a CTA takes fewer than 16 (rows of the matrix operands past tpc repeat the last
// token and are discarded): each CTA must stream all of Q_L1, and one compute unit
// streams only ~45 GB/s from HBM, so the stream is spread over more units, which then
// find Q_L1 in their L2. The waves split K:
// each streams its range of Q_X rows and Q_L1 panel pieces straight into registers, U
// steps of 128 codes at a time in two batches that take turns (the next batch's loads
// are in flight while the current one is used),
// expands the codes to int8 and accumulates on v_mfma_i32_16x16x64_i8. The waves' exact
// integer sums meet in LDS by integer adds (their order cannot change the result). Then
// per token: h_t = (s_X H_t) c_t in binary32 in that order, s_H = max_t |h_t| / 7 and
// Q_H = round(h / s_H) by eq. (1), the maximum taken across the lanes that hold the
// token's ranks. Only Q_H and s_H are written (and H itself for the test export): H
// never reaches global memory (TwinQuant page 1, section 4.3).
struct RequantArgs {
    uint8_t *qx;         // [b][m / 2] packed (written first by the kernel when x is set)
    float *sx;           // [b] (likewise)
    const uint16_t *x;   // fp16 [b][m], or NULL: one token a CTA quantizes its own row first
    const uint8_t *ql1;  // panel layout, r rows
    const float *c;      // [r]
    int r;
    uint8_t *qh;         // [b][r / 2]
    float *sh;           // [b]
    int32_t *h;          // [b][r] or NULL
    int64_t b, m;
    int tpc;             // tokens per CTA, at most 16 TB (the matrix instruction's other rows repeat the last)
};

constexpr int kReqWaves = 8;

constexpr int req_batch(int nr, int tb) {  // steps per batch: two batches and the sums fit ~170 registers
    return (170 - 4 * nr * tb) / (8 * (nr + tb)) < 1 ? 1 : (170 - 4 * nr * tb) / (8 * (nr + tb)) > 4 ? 4
                                                                : (170 - 4 * nr * tb) / (8 * (nr + tb));
}

// QX (one token a CTA): the CTA first quantizes its token's row by eq. (1) exactly as the
// activation quantizer does (amax over the fp16 bit patterns, s_X = amax / 7 correctly
// rounded, quant_code_fast), writes Q_X and s_X, and meets before the H loop reads them
// back; so the few-token call needs no separate quantizer launch.
template <int TB, int NR, bool STORE_H, bool QX = false>
__global__ __launch_bounds__(kReqWaves * 64) void lr4_requant_kernel(RequantArgs a) {
#pragma clang fp contract(off)
    constexpr int NW = kReqWaves, NT = NW * 64, BM = 16 * TB, U = req_batch(NR, TB);
    static_assert(!QX || TB == 1, "the row quantizer takes one token a CTA");
    constexpr int HP = NR * 16 + 1;        // LDS row pitch of H in words (odd: no bank conflicts)
    constexpr int TPT = NT / BM;           // threads per token in the requantization
    constexpr int RPT = NR * 16 / TPT >= 2 ? NR * 16 / TPT : 2;  // ranks per thread (an even count)
    static_assert(TPT <= kWave && (TPT & (TPT - 1)) == 0, "a token's threads share a wave");
    __shared__ int32_t hs[BM * HP];

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int li = lane & 15, g = lane >> 4;
    const int tpc = a.tpc;
    const int64_t tok0 = (int64_t)blockIdx.x * tpc, b = a.b, m = a.m;
    const int nr = a.r / 16;
    for (int i = tid; i < BM * HP; i += NT) hs[i] = 0;
    if constexpr (QX) {
        // the CTA's one token (tpc = 1, blockIdx.x < b): its row's codes and scale
        __shared__ uint32_t red[NW];
        const uint4 *xr = reinterpret_cast<const uint4 *>(a.x + tok0 * m);
        const int64_t nch = m / 8;
        uint32_t mx = 0;
        for (int64_t c = tid; c < nch; c += NT) mx = absmax8_bits(xr[c], mx);
        mx = wave_max_u32(mx);
        if (lane == 0) red[wave] = mx;
        __syncthreads();
        uint32_t m4 = red[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) m4 = m4 > red[w] ? m4 : red[w];
        const float amax = half_bits_to_float(m4);
        const float s = amax / kQMax;  // correctly rounded binary32 division
        const float inv = 1.0f / s;    // only used when amax > 0
        uint32_t *qrow = reinterpret_cast<uint32_t *>(a.qx + tok0 * (m / 2));
        for (int64_t c = tid; c < nch; c += NT) qrow[c] = amax == 0.0f ? 0u : quant8(xr[c], s, inv);
        if (tid == 0) a.sx[tok0] = s;
        __syncthreads();  // Q_X and s_X of the token written for every thread of the CTA
    }

    // this lane's operand addresses: rank block rb (past the live ones: the last live one,
    // unused) and token block tb (rows past b: the last row, never stored)
    const uint8_t *pa = a.ql1 + li * 64 + g * 16;  // + block offset (uniform) + step offset
    const int64_t rstride = (m / 128) * kPanelPiece;
    const uint8_t *pb[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        const int64_t tok = tok0 + (tb * 16 + li < tpc ? tb * 16 + li : tpc - 1);
        pb[tb] = a.qx + (tok < b ? tok : b - 1) * (m / 2) + g * 16;
    }
    v4i acc[NR][TB];
#pragma unroll
    for (int rb = 0; rb < NR; ++rb)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[rb][tb] = v4i{0, 0, 0, 0};
    const int64_t nst = m / 128, c0 = wave * nst / NW, c1 = (wave + 1) * nst / NW;
    // two batches in turn: the loads of the next batch are issued before the current one
    // is used (steps at or past c1 reload step c1 - 1 and are not used)
    struct Batch {
        uint4 wa[U][NR], xb[U][TB];
    };
    auto load = [&](int64_t c, Batch &bt) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t cu = c + u < c1 ? c + u : c1 - 1;
#pragma unroll
            for (int rb = 0; rb < NR; ++rb)
                bt.wa[u][rb] = *reinterpret_cast<const uint4 *>(pa + (rb < nr ? rb : nr - 1) * rstride + cu * kPanelPiece);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) bt.xb[u][tb] = *reinterpret_cast<const uint4 *>(pb[tb] + cu * 64);
        }
    };
    auto use = [&](int64_t c, const Batch &bt) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (c + u >= c1) break;
            v4i blo[TB], bhi[TB];
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) unpack16(bt.xb[u][tb], blo[tb], bhi[tb]);
#pragma unroll
            for (int rb = 0; rb < NR; ++rb) {
                v4i alo, ahi;
                unpack16(bt.wa[u][rb], alo, ahi);
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    acc[rb][tb] = mfma_i8(alo, blo[tb], acc[rb][tb]);
                    acc[rb][tb] = mfma_i8(ahi, bhi[tb], acc[rb][tb]);
                }
            }
        }
    };
    // two batches when their registers fit beside the sums (up to 128 ranks), else one
    constexpr bool PING = 8 * U * (NR + TB) + 4 * NR * TB <= 170;
    if constexpr (!PING) {
        for (int64_t c = c0; c < c1; c += U) {
            Batch ba;
            load(c, ba);
            __builtin_amdgcn_sched_barrier(0);  // the whole batch in flight before the first use
            use(c, ba);
        }
    } else if (c0 < c1) {
        Batch ba, bb;
        load(c0, ba);
        for (int64_t c = c0;; c += 2 * U) {
            load(c + U, bb);
            __builtin_amdgcn_sched_barrier(0);  // the next batch in flight before this one is used
            use(c, ba);
            if (c + U >= c1) break;
            load(c + 2 * U, ba);
            __builtin_amdgcn_sched_barrier(0);
            use(c + U, bb);
            if (c + 2 * U >= c1) break;
        }
    }
    __syncthreads();  // hs cleared by every thread
    // lane (li, g), register v of tile (rb, tb): 256 H of rank 16 rb + 4 g + v, token 16 tb + li
#pragma unroll
    for (int rb = 0; rb < NR; ++rb)
        if (rb < nr) {
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
                if (tb * 16 + li < tpc) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) atomicAdd(&hs[(tb * 16 + li) * HP + rb * 16 + 4 * g + v], acc[rb][tb][v] >> 8);
                }
        }
    __syncthreads();

    // requantization: token tid / TPT, ranks [RPT sub, RPT sub + RPT) of its r
    const int tl = tid / TPT, sub = tid % TPT;
    const int64_t tok = tok0 + tl;
    const int t0 = sub * RPT;
    const bool live = t0 < a.r;  // r is a multiple of 32, so a live thread's ranks are all < r
    const float sxv = a.sx[tok < b ? tok : b - 1];
    float hv[RPT];
    float mx = 0.0f;
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        const int t = live ? t0 + k : 0;
        const float prod = sxv * (float)hs[tl * HP + t];  // exact: |H| <= 49 m < 2^24
        hv[k] = prod * a.c[t];
        if (live) mx = __builtin_fmaxf(mx, __builtin_fabsf(hv[k]));
    }
#pragma unroll
    for (int off = TPT / 2; off > 0; off >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, off, kWave));
    const float s = mx / kQMax;  // correctly rounded binary32 division
    if (tl >= tpc || tok >= b) return;
    if (sub == 0) a.sh[tok] = s;
    if (!live) return;
    // the thread's RPT codes, two per byte (rank 2p in the low nibble), eight per word
    uint32_t words[(RPT + 7) / 8];
#pragma unroll
    for (int w = 0; w < (RPT + 7) / 8; ++w) words[w] = 0;
#pragma unroll
    for (int k = 0; k < RPT; ++k)
        words[k / 8] |= (uint32_t(mx == 0.0f ? 0 : quant_code(hv[k], s)) & 0xFu) << (4 * (k % 8));
    uint8_t *dst = a.qh + tok * (a.r / 2) + t0 / 2;  // RPT / 2 bytes, aligned to that size
    if constexpr (RPT == 2)
        *dst = (uint8_t)words[0];
    else if constexpr (RPT == 4)
        *reinterpret_cast<uint16_t *>(dst) = (uint16_t)words[0];
    else
#pragma unroll
        for (int w = 0; w < RPT / 8; ++w) reinterpret_cast<uint32_t *>(dst)[w] = words[w];
    if constexpr (STORE_H) {
#pragma unroll
        for (int k = 0; k < RPT; ++k) a.h[tok * a.r + t0 + k] = hs[tl * HP + t0 + k];
    }
}

template <int TB, bool STORE_H, bool QX = false>
static hipError_t launch_requant_tb(const RequantArgs &a, hipStream_t s) {
    const int nr = a.r / 16;  // the kernel's NR bounds the live rank blocks
    const dim3 grid((unsigned)((a.b + a.tpc - 1) / a.tpc)), block(kReqWaves * 64);
    if (nr <= 2)
        hipLaunchKernelGGL((lr4_requant_kernel<TB, 2, STORE_H, QX>), grid, block, 0, s, a);
    else if (nr <= 4)
        hipLaunchKernelGGL((lr4_requant_kernel<TB, 4, STORE_H, QX>), grid, block, 0, s, a);
    else if (nr <= 8)
        hipLaunchKernelGGL((lr4_requant_kernel<TB, 8, STORE_H, QX>), grid, block, 0, s, a);
    else if constexpr (TB == 1)
        hipLaunchKernelGGL((lr4_requant_kernel<1, 16, STORE_H, QX>), grid, block, 0, s, a);
    else
        return hipErrorInvalidValue;  // the launcher takes 16-token tiles above 128 ranks
    return hipGetLastError();
}

bool lowrank_requant_quantizes(int64_t b) { return b <= 256; }

hipError_t launch_lowrank_requant(const uint16_t *x, uint8_t *qx, float *sx, const uint8_t *ql1, const float *c, int r,
                                  uint8_t *qh, float *sh, int32_t *h, int64_t b, int64_t m, hipStream_t stream) {
    if (b == 0) return hipSuccess;
    if (r < 32 || r > 256 || r % 32) return hipErrorInvalidValue;
    // 32-token tiles where that still gives every compute unit a tile (up to 128 ranks;
    // above, the sums of two token blocks would not fit the registers), else up to 16
    // tokens a CTA, as few as gives 256 CTAs (one token a CTA at most 256 tokens, where
    // the CTA also quantizes that token when x is given)
    const bool two = (b + 31) / 32 >= 256 && r <= 128;
    int64_t tpc = two ? 32 : (b + 255) / 256;
    if (tpc > 16 && !two) tpc = 16;
    if (x && tpc != 1) return hipErrorInvalidValue;  // callers quantize first above 256 tokens
    RequantArgs a{qx, sx, x, ql1, c, r, qh, sh, h, b, m, (int)tpc};
    if (x) return h ? launch_requant_tb<1, true, true>(a, stream) : launch_requant_tb<1, false, true>(a, stream);
    if (h) return two ? launch_requant_tb<2, true>(a, stream) : launch_requant_tb<1, true>(a, stream);
    return two ? launch_requant_tb<2, false>(a, stream) : launch_requant_tb<1, false>(a, stream);
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

}  // namespace twq
