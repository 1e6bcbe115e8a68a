// dual_linear.hip -- the fused W4A4 + low-rank linear (gfx950).
//
//   Y[i][j] = fp16( s_X[i] s_W[j] sum_k Q_X[i][k] Q_W[j][k] + sum_t T[i][t] L2[t][j] )
//
// TwinQuant page 1, section 2, eqs. (2)-(3), fused as in page 1, section 4.3:
// the residual partial sums and the low-rank product live only in registers and
// are merged in one epilogue that stores fp16 once.
//
// Main loop: a CTA owns a BN x BM tile of Y^T (BN output channels by BM tokens).
// Per stage it stages 256 packed int4 codes (128 bytes) of each of its weight
// rows and token rows through LDS with coalesced 16-byte loads, double
// buffered, the next stage's global loads in flight while the current one is
// consumed. Each wave reads 16-byte pieces back (XOR-swizzled against bank
// conflicts), expands them to int8 (x16, see unpack16) and issues
// v_mfma_i32_16x16x64_i8 -- gfx950 has no int4 matrix instruction. The
// accumulator holds 256 * acc exactly (|acc| <= 49 m, m <= 131072).
//
// Epilogue: acc is dequantized in place to fp32, then used as the C operand of
// v_mfma_f32_16x16x32_f16 over the rank dimension with A = L2^T rows and
// B = T rows (rounded to fp16), so the two branches merge without a second
// accumulator set. The i32 and f32 16x16 results share one register layout.
#include "twq_device.h"
#include "twq_kernels.h"

namespace twq {

constexpr int kRowBytes = 128;  // packed bytes per row per stage (256 codes)
constexpr int kChunks = kRowBytes / 16;

// 16-byte chunk swizzle of an LDS row; conflict-free for 8 or 16 lanes reading
// the same logical chunk of 16 consecutive rows with 32 or 64 banks
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

template <int BM, int BN, int WM, int WN, bool STORE_ACC>
__global__ __launch_bounds__(256) void dual_linear_tiled(DualArgs a, int tiles_n) {
    constexpr int FM = BM / (16 * WM), FN = BN / (16 * WN);
    static_assert(WM * WN == 4 && FM >= 1 && FN >= 1, "four waves, whole 16x16 tiles");
    constexpr int A_CHUNKS = BN * kChunks, TOTAL = (BN + BM) * kChunks;
    constexpr int PER_THREAD = (TOTAL + 255) / 256;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BN + BM) * kRowBytes];

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int li = lane & 15, g = lane >> 4;
    const int wn = wave % WN, wm = wave / WN;
    const int64_t tile = blockIdx.x;
    const int64_t ch0 = (tile % tiles_n) * BN, tok0 = (tile / tiles_n) * BM;
    const int64_t kb = a.m / 2;  // packed bytes per row
    const int stages = (int)((kb + kRowBytes - 1) / kRowBytes);

    uint4 pre[PER_THREAD];
    auto gload = [&](int s) {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const int q = tid + i * 256;
            const int c = q % kChunks;
            const int64_t kbyte = (int64_t)s * kRowBytes + c * 16;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (q < A_CHUNKS) {
                const int64_t ch = ch0 + q / kChunks;
                if (ch < a.n && kbyte < kb) v = *reinterpret_cast<const uint4 *>(a.qw + ch * kb + kbyte);
            } else if (q < TOTAL) {
                const int64_t tok = tok0 + (q - A_CHUNKS) / kChunks;
                if (tok < a.b && kbyte < kb) v = *reinterpret_cast<const uint4 *>(a.qx + tok * kb + kbyte);
            }
            pre[i] = v;
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const int q = tid + i * 256;
            if (q < TOTAL) {
                const int row = q / kChunks, c = q % kChunks;  // A rows, then B rows
                *reinterpret_cast<uint4 *>(&lds[buf][row * kRowBytes + ((c ^ swz(row)) * 16)]) = pre[i];
            }
        }
    };

    v4i acc[FN][FM];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = v4i{0, 0, 0, 0};

    gload(0);
    sstore(0);
    __syncthreads();
    for (int s = 0; s < stages; ++s) {
        if (s + 1 < stages) gload(s + 1);
        const uint8_t *L = lds[s & 1];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int c = kk * 4 + g;
            v4i alo[FN], ahi[FN], blo[FM], bhi[FM];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int row = wn * (BN / WN) + fn * 16 + li;
                unpack16(*reinterpret_cast<const uint4 *>(L + row * kRowBytes + ((c ^ swz(row)) * 16)), alo[fn],
                         ahi[fn]);
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int row = BN + wm * (BM / WM) + fm * 16 + li;
                unpack16(*reinterpret_cast<const uint4 *>(L + row * kRowBytes + ((c ^ swz(row)) * 16)), blo[fm],
                         bhi[fm]);
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    acc[fn][fm] = mfma_i8(alo[fn], blo[fm], acc[fn][fm]);
                    acc[fn][fm] = mfma_i8(ahi[fn], bhi[fm], acc[fn][fm]);
                }
        }
        if (s + 1 < stages) sstore((s + 1) & 1);
        __syncthreads();
    }

    // lane (li, g), register v of tile (fn, fm) holds channel ch_base + 4g + v, token tok_base + li
    if constexpr (STORE_ACC) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int64_t ch = ch0 + wn * (BN / WN) + fn * 16 + 4 * g;
                const int64_t tok = tok0 + wm * (BM / WM) + fm * 16 + li;
                if (ch < a.n && tok < a.b) {
                    v4i o;
#pragma unroll
                    for (int v = 0; v < 4; ++v) o[v] = acc[fn][fm][v] >> 8;  // exact: a multiple of 256
                    *reinterpret_cast<v4i *>(a.acc + tok * a.n + ch) = o;
                }
            }
        return;
    } else {
        v4f y[FN][FM];
        float sxv[FM];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int64_t tok = tok0 + wm * (BM / WM) + fm * 16 + li;
            sxv[fm] = tok < a.b ? a.sx[tok] : 0.0f;
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int64_t ch = ch0 + wn * (BN / WN) + fn * 16 + 4 * g;
            const float4 sw4 = ch < a.n ? *reinterpret_cast<const float4 *>(a.sw + ch) : make_float4(0.f, 0.f, 0.f, 0.f);
            const float swv[4] = {sw4.x, sw4.y, sw4.z, sw4.w};
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int v = 0; v < 4; ++v) y[fn][fm][v] = (sxv[fm] * swv[v]) * (float)(acc[fn][fm][v] >> 8);
        }
        // low-rank branch: y += L2^T (channels x ranks) . T^T (ranks x tokens)
        for (int k0 = 0; k0 < a.r; k0 += 32) {
            const int rank = k0 + g * 8;  // r is a multiple of 16, so rank < r means rank + 8 <= r
            v8h la[FN], tb[FM];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int64_t ch = ch0 + wn * (BN / WN) + fn * 16 + li;
                la[fn] = (rank < a.r && ch < a.n) ? load_h8(a.l2t + ch * a.r + rank) : v8h{};
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int64_t tok = tok0 + wm * (BM / WM) + fm * 16 + li;
                if (rank < a.r && tok < a.b) {
                    const float4 *tp = reinterpret_cast<const float4 *>(a.t + tok * a.r + rank);
                    tb[fm] = f32x8_to_h8(tp[0], tp[1]);
                } else {
                    tb[fm] = v8h{};
                }
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) y[fn][fm] = mfma_f16(la[fn], tb[fm], y[fn][fm]);
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int64_t ch = ch0 + wn * (BN / WN) + fn * 16 + 4 * g;
                const int64_t tok = tok0 + wm * (BM / WM) + fm * 16 + li;
                if (ch < a.n && tok < a.b) {
                    v4h o;
#pragma unroll
                    for (int v = 0; v < 4; ++v) o[v] = (_Float16)y[fn][fm][v];
                    *reinterpret_cast<v4h *>(a.y + tok * a.n + ch) = o;
                }
            }
    }
}

// ---------------------------------------------------------------------------------
// Few tokens (b <= 64): the layer streams Q_W once from HBM and little else. A CTA
// owns FN*16 output channels and all tokens (FM tiles of 16); its NW waves split
// K and feed the matrix cores straight from global memory, U 16-byte loads per
// operand row issued before any is consumed; the NW partial accumulators are
// added through LDS. Loads are unconditional -- rows past n or b are clamped to a
// valid row and their outputs never stored -- so nothing serialises them, and the
// low-rank operands of the epilogue are loaded first so their latency hides under
// the main loop.
template <int FN, int FM, int U, int RS, bool STORE_ACC, int NW = 4>
__global__ __launch_bounds__(NW * 64) void dual_linear_decode(DualArgs a) {
    __shared__ v4i red[NW][FN * FM][kWave];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int li = lane & 15, g = lane >> 4;
    const int64_t ch0 = (int64_t)blockIdx.x * (FN * 16);
    const int64_t kb = a.m / 2;
    const int64_t nch = a.m / 128;  // 64-byte pieces of a packed row
    const int64_t cb = wave * nch / NW, ce = (wave + 1) * nch / NW;

    const uint8_t *wrow[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int64_t ch = ch0 + fn * 16 + li;
        wrow[fn] = a.qw + (ch < a.n ? ch : a.n - 1) * kb + g * 16;
    }
    const uint8_t *xrow[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int64_t tok = fm * 16 + li;
        xrow[fm] = a.qx + (tok < a.b ? tok : a.b - 1) * kb + g * 16;
    }

    // this wave's epilogue tile and its low-rank operands (rank steps past r are
    // loaded from rank 0 and zeroed where they are used)
    const bool has_tile = wave < FN * FM;
    const int fn_e = has_tile ? wave / FM : 0, fm_e = has_tile ? wave % FM : 0;
    v8h l2f[RS > 0 ? RS : 1];
    float4 tf[RS > 0 ? RS : 1][2];
    if constexpr (!STORE_ACC && RS > 0) {
        const int64_t chr = ch0 + fn_e * 16 + li, tokr = fm_e * 16 + li;
        const uint16_t *l2row = a.l2t + (chr < a.n ? chr : a.n - 1) * a.r;
        const float *trow = a.t + (tokr < a.b ? tokr : a.b - 1) * a.r;
#pragma unroll
        for (int s = 0; s < RS; ++s) {
            const int rank = s * 32 + g * 8;
            const int rk = rank < a.r ? rank : 0;
            l2f[s] = load_h8(l2row + rk);
            tf[s][0] = *reinterpret_cast<const float4 *>(trow + rk);
            tf[s][1] = *reinterpret_cast<const float4 *>(trow + rk + 4);
        }
    }

    v4i acc[FN][FM];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = v4i{0, 0, 0, 0};

    auto mma = [&](const uint4 (&bw)[FN], const uint4 (&bx)[FM]) {
        v4i alo[FN], ahi[FN], blo[FM], bhi[FM];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) unpack16(bw[fn], alo[fn], ahi[fn]);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) unpack16(bx[fm], blo[fm], bhi[fm]);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                acc[fn][fm] = mfma_i8(alo[fn], blo[fm], acc[fn][fm]);
                acc[fn][fm] = mfma_i8(ahi[fn], bhi[fm], acc[fn][fm]);
            }
    };
    int64_t c = cb;
    for (; c + U <= ce; c += U) {
        uint4 bw[U][FN], bx[U][FM];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) bw[u][fn] = *reinterpret_cast<const uint4 *>(wrow[fn] + (c + u) * 64);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) bx[u][fm] = *reinterpret_cast<const uint4 *>(xrow[fm] + (c + u) * 64);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep every load of the batch ahead of its first use
#pragma unroll
        for (int u = 0; u < U; ++u) mma(bw[u], bx[u]);
    }
    for (; c < ce; ++c) {
        uint4 bw[FN], bx[FM];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) bw[fn] = *reinterpret_cast<const uint4 *>(wrow[fn] + c * 64);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) bx[fm] = *reinterpret_cast<const uint4 *>(xrow[fm] + c * 64);
        mma(bw, bx);
    }

#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) red[wave][fn * FM + fm][lane] = acc[fn][fm];
    __syncthreads();
    if (!has_tile) return;
    const int tile = fn_e * FM + fm_e;
    v4i sum = red[0][tile][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) sum += red[w][tile][lane];

    const int64_t ch = ch0 + fn_e * 16 + 4 * g;
    const int64_t tok = fm_e * 16 + li;
    const bool store = ch < a.n && tok < a.b;
    if constexpr (STORE_ACC) {
        if (store) *reinterpret_cast<v4i *>(a.acc + tok * a.n + ch) = sum >> 8;
    } else {
        const float sxv = a.sx[tok < a.b ? tok : a.b - 1];
        const float4 sw4 = *reinterpret_cast<const float4 *>(a.sw + (ch < a.n ? ch : a.n - 4));
        const float swv[4] = {sw4.x, sw4.y, sw4.z, sw4.w};
        v4f y;
#pragma unroll
        for (int v = 0; v < 4; ++v) y[v] = (sxv * swv[v]) * (float)(sum[v] >> 8);
#pragma unroll
        for (int s = 0; s < RS; ++s) {
            const bool live = s * 32 + g * 8 < a.r;
            const v8h tb = live ? f32x8_to_h8(tf[s][0], tf[s][1]) : v8h{};
            y = mfma_f16(l2f[s], tb, y);
        }
        if (store) {
            v4h o;
#pragma unroll
            for (int v = 0; v < 4; ++v) o[v] = (_Float16)y[v];
            *reinterpret_cast<v4h *>(a.y + tok * a.n + ch) = o;
        }
    }
}

template <int FN, int FM, int U, int RS>
static hipError_t launch_decode_rs(const DualArgs &a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.n + FN * 16 - 1) / (FN * 16)));
    if (a.acc)
        hipLaunchKernelGGL((dual_linear_decode<FN, FM, U, 0, true>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((dual_linear_decode<FN, FM, U, RS, false>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int FN, int FM, int U>
static hipError_t launch_decode(const DualArgs &a, hipStream_t stream) {
    // rank steps of 32 the epilogue prefetches
    if (a.r == 0) return launch_decode_rs<FN, FM, U, 0>(a, stream);
    if (a.r <= 32) return launch_decode_rs<FN, FM, U, 1>(a, stream);
    if (a.r <= 64) return launch_decode_rs<FN, FM, U, 2>(a, stream);
    if (a.r <= 128) return launch_decode_rs<FN, FM, U, 4>(a, stream);
    return launch_decode_rs<FN, FM, U, 8>(a, stream);
}

template <int BM, int BN, int WM, int WN>
static hipError_t launch_cfg(const DualArgs &a, hipStream_t stream) {
    const int64_t tiles_n = (a.n + BN - 1) / BN, tiles_m = (a.b + BM - 1) / BM;
    const dim3 grid((unsigned)(tiles_n * tiles_m));
    if (a.acc)
        hipLaunchKernelGGL((dual_linear_tiled<BM, BN, WM, WN, true>), grid, dim3(256), 0, stream, a, (int)tiles_n);
    else
        hipLaunchKernelGGL((dual_linear_tiled<BM, BN, WM, WN, false>), grid, dim3(256), 0, stream, a, (int)tiles_n);
    return hipGetLastError();
}

hipError_t launch_dual_linear(const DualArgs &a, hipStream_t stream) {
    if (a.b == 0 || a.n == 0) return hipSuccess;
    // decode tiles: wider channel tiles read Q_X fewer times, as long as the grid
    // still covers the chip (measured on MI355X with HIP graphs, weights cold)
    if (a.b <= 16) return a.n >= 16384 ? launch_decode<2, 1, 8>(a, stream) : launch_decode<1, 1, 8>(a, stream);
    if (a.b <= 32) return a.n >= 8192 ? launch_decode<4, 2, 2>(a, stream) : launch_decode<1, 2, 4>(a, stream);
    if (a.b <= 64) return a.n >= 8192 ? launch_decode<2, 4, 2>(a, stream) : launch_decode<1, 4, 4>(a, stream);
    return launch_cfg<128, 128, 2, 2>(a, stream);
}

}  // namespace twq
