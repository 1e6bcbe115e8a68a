// dual_linear.hip -- the fused W4A4 + low-rank linear (gfx950).
//
//   Y[i][j] = fp16( s_X[i] s_W[j] sum_k Q_X[i][k] Q_W[j][k] + sum_t T[i][t] L2[t][j] )
//
// TwinQuant page 1, section 2, eqs. (2)-(3), fused as in page 1, section 4.3:
// the residual partial sums and the low-rank product live only in registers and
// are merged in one epilogue that stores fp16 once.
//
// Main loops with the same epilogue arithmetic: dual_linear_decode for few tokens
// (HBM-bound, operands straight from global memory) and, for many tokens
// (matrix-core-bound, operands staged through an LDS ring), dual_linear_pf and its
// 32 x 32-block form dual_linear_pf32, which the per-token 4-bit layer runs. All expand
// packed int4 codes to int8 (x16, see unpack16) and issue v_mfma_i32_16x16x64_i8 (or
// v_mfma_i32_32x32x32_i8) -- gfx950 has no int4 matrix instruction. The accumulator
// holds 256 * acc exactly (|acc| <= 49 m, m <= 131072). The group-wise (GRP), W4A8
// (A8) and int4 low-rank (LR4) variants are described at each kernel.
//
// Epilogue: acc is dequantized in place to fp32, then used as the C operand of
// v_mfma_f32_16x16x32_f16 (v_mfma_f32_32x32x16_f16) over the rank dimension with A = L2^T rows and
// B = T rows (rounded to fp16), so the two branches merge without a second
// accumulator set. The i32 and f32 results of one block shape share one register layout. In
// the int4 low-rank variant the epilogue instead adds s_H (Q_H Q_L2^T), a second
// int8 matrix product over the rank dimension.
#include <utility>

#include "twq_device.h"
#include "twq_kernels.h"

namespace twq {

// int4 low-rank term of one 16 x 16 output tile: 256 x sum_t Q_L2[ch][t] Q_H[tok][t]
// (K = r, r a multiple of 32), for this lane's A row ch_row and B row tok_row; the
// result has the layout of the main accumulator. Rows past n or b are clamped.
__device__ __forceinline__ v4i lr4_tile(const DualArgs &a, int64_t ch_row, int64_t tok_row, int g) {
    const int64_t rb = a.r / 2;
    const uint8_t *arow = a.ql2 + (ch_row < a.n ? ch_row : a.n - 1) * rb;
    const uint8_t *brow = a.qh + (tok_row < a.b ? tok_row : a.b - 1) * rb;
    v4i acc2 = v4i{0, 0, 0, 0};
    for (int64_t k0 = 0; k0 < rb; k0 += 64) {  // 64 bytes = 128 ranks per pair of MFMAs
        const int64_t byte = k0 + g * 16;
        const bool live = byte < rb;           // r % 32 == 0: live means byte + 16 <= r / 2
        const uint4 ra = live ? *reinterpret_cast<const uint4 *>(arow + byte) : make_uint4(0, 0, 0, 0);
        const uint4 rq = live ? *reinterpret_cast<const uint4 *>(brow + byte) : make_uint4(0, 0, 0, 0);
        v4i alo, ahi, blo, bhi;
        unpack16(ra, alo, ahi);
        unpack16(rq, blo, bhi);
        acc2 = mfma_i8(alo, blo, acc2);
        acc2 = mfma_i8(ahi, bhi, acc2);
    }
    return acc2;
}

// Block b runs on XCD b % 8 (the hardware deals CTAs out in turn). Give XCD x the
// contiguous range of q + (x < rem) tiles starting at x q + min(x, rem), q = tiles / 8,
// rem = tiles % 8: a bijection of [0, tiles) for any tile count.
__host__ __device__ __forceinline__ int64_t xcd_order(int64_t bid, int64_t ntiles) {
    const int64_t q = ntiles / 8, rem = ntiles % 8, x = bid % 8, j = bid / 8;
    return x * q + (x < rem ? x : rem) + j;
}

// ---------------------------------------------------------------------------------
// Few tokens (b <= 64): the layer streams Q_W once from HBM and little else. A CTA
// owns FN*16 output channels and all tokens (FM tiles of 16); its NW waves split
// K and feed the matrix cores straight from global memory in batches of U 16-byte
// loads per operand row, every load of a batch issued before any is consumed (a
// weight operand is one contiguous 1 KB piece of a panel, so each wave streams FN
// contiguous runs; some variants also issue the next batch before using the current
// one, see PIPE); the NW partial accumulators are added through LDS. Loads are
// unconditional -- rows past n or b are clamped to a valid row and their outputs never
// stored -- so nothing serialises them, and the low-rank operands of the epilogue are
// loaded first so their latency hides under the main loop.

// Group-wise scales (GRP, groups of kGroup = 128 along K): one 64-byte piece of a
// packed row is one group, so each piece's integer sum is formed from zero and added to
// an fp32 accumulator times s_X[group][token] s_W[group][channel], loaded beside the
// piece; the waves' fp32 partial sums are added through LDS in wave order.
//
// W4A8 (A8): the token rows hold one int8 code per element, so a 64-byte piece of a
// weight row pairs with 128 bytes of each token row; those are permuted into the lane
// order of the expanded weight operand (perm16) and used unscaled, so the accumulator
// holds 16 acc.
template <int FN, int FM, int U, int RS, bool STORE_ACC, int TK = 1, int NW = 4, bool GRP = false, bool A8 = false,
          bool XL = false>
__global__ __launch_bounds__(NW * 64) void dual_linear_decode(DualArgs a) {
    static_assert(!(GRP && STORE_ACC), "group-wise sums are stored dequantized only");
    static_assert(!(GRP && A8), "group-wise scales with 4-bit activations only");
    constexpr int XN = A8 ? 2 : 1;       // 16-byte loads per token row per piece
    constexpr int SH = A8 ? 4 : 8;       // log2 of the operands' combined scale
    // LDS: the cross-wave reduction buffer red[NW][FN*FM][kWave]; with XL it also holds
    // each wave's K slice of Q_X (XSLICE bytes a wave) during the main loop
    constexpr int XSLICE = !XL ? 0 : FN * FM * 1024 > 16384 ? FN * FM * 1024 : 16384;
    constexpr int RED_V4 = NW * FN * FM * kWave;
    constexpr int LDS_V4 = NW * XSLICE / 16 > RED_V4 ? NW * XSLICE / 16 : RED_V4;
    __shared__ v4i red_lds[LDS_V4];
    v4i (*const red)[FN * FM][kWave] = reinterpret_cast<v4i (*)[FN * FM][kWave]>(red_lds);
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int li = lane & 15, g = lane >> 4;
    // GRP: neighbouring channel tiles on one XCD, so the two halves of a 128-byte line of
    // s_W (one group row, FN = 4: 64 bytes a tile) are fetched into the same L2 once
    const int64_t ch0 = (GRP ? xcd_order(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x) * (FN * 16);
    const int64_t kb = a.m / 2;
    const int64_t nch = a.m / 128;  // 64-byte pieces of a packed row
    const int64_t cb = wave * nch / NW, ce = (wave + 1) * nch / NW;

    // this lane's 16 bytes of piece c of channel tile fn: wrow[fn] + c kPanelPiece (a
    // piece of a panel is one contiguous 1 KB operand block)
    const uint8_t *wrow[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int64_t ch = ch0 + fn * 16 + li;
        wrow[fn] = a.qw + qw_offset(ch < a.n ? ch : a.n - 1, (int64_t)g * 16 + cb * kPieceBytes, a.m);
    }
    const uint8_t *xrow[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int64_t tok = fm * 16 + li;
        xrow[fm] = a.qx + (tok < a.b ? tok : a.b - 1) * (A8 ? a.m : kb) + g * 16 * XN;
    }
    // XL (K short enough): each wave copies its K slice of Q_X (its pieces x FM token tiles,
    // 1 KB a block) into its own XSLICE bytes of that LDS by direct-to-LDS loads issued
    // ahead of the weight stream; the main loop then reads X from LDS and only the weights
    // (and group scales) stream from memory. Lane l of the copy of block (piece c, tile fm)
    // fetches bytes 64 c + 16 (l % 4) of token row 16 fm + l / 4, so a block holds 64-byte
    // rows in token order, read back by lane (li, g) at 64 li + 16 g. The launcher picks XL
    // only where a wave's slice fits: ceil(m / 128 / NW) FM KB <= XSLICE. Where XSLICE is
    // the wave's own part of red (16-block tiles of eight waves) the wave overwrites only
    // its own slice when it stores its partial sums; otherwise the CTA meets at a barrier
    // first.
    static_assert(!XL || !A8, "X slices in LDS: 4-bit activations");
    uint8_t *const xls = reinterpret_cast<uint8_t *>(red_lds) + wave * XSLICE;

    // Epilogue tiles are dealt to the waves in turn (tile t to wave t % NW). When a
    // wave owns one tile, its low-rank operands are loaded here, ahead of the main
    // loop (rank steps past r are loaded from rank 0 and zeroed where used). T may come
    // as up to TK partial sums over K slices; they are all loaded here and added in
    // slice order in the epilogue.
    constexpr int TILES = FN * FM;
    constexpr bool PREFETCH = !STORE_ACC && RS > 0 && TILES <= NW;  // fp16 low-rank branch only
    constexpr int TKS = PREFETCH ? TK : 1;
    static_assert(TK == 1 || TK * RS <= kMaxTSlices, "partial sums of T held per lane");
    v8h l2f[PREFETCH ? RS : 1];
    float4 tf[PREFETCH ? RS : 1][TKS][2];
    if (PREFETCH && !a.lr4 && wave < TILES) {
        const int t0 = wave;
        const int64_t chr = ch0 + (t0 / FM) * 16 + li, tokr = (t0 % FM) * 16 + li;
        const uint16_t *l2row = a.l2t + (chr < a.n ? chr : a.n - 1) * a.r;
        const float *trow = a.tpart + (tokr < a.b ? tokr : a.b - 1) * a.r;
#pragma unroll
        for (int s = 0; s < RS; ++s) {
            const int rank = s * 32 + g * 8;
            const int rk = rank < a.r ? rank : 0;
            l2f[s] = load_h8(l2row + rk);
#pragma unroll
            for (int k = 0; k < TKS; ++k) {  // unconditional (slices past tks reload slice 0), so none is sunk to its use
                const int64_t kk = k < a.tks ? k : 0;
                tf[s][k][0] = *reinterpret_cast<const float4 *>(trow + kk * a.tstride + rk);
                tf[s][k][1] = *reinterpret_cast<const float4 *>(trow + kk * a.tstride + rk + 4);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    v4i acc[FN][FM];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = v4i{0, 0, 0, 0};

    // GRP: fp32 sums over groups; this lane's s_W (channels 4g..4g+3 of each channel
    // tile) and s_X (token li of each token tile) columns of the group-major scales
    v4f yg[GRP ? FN : 1][GRP ? FM : 1];
    const float *swp[GRP ? FN : 1];
    const float *sxp[GRP ? FM : 1];
    if constexpr (GRP) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int64_t ch = ch0 + fn * 16 + 4 * g;
            swp[fn] = a.sw + (ch < a.n ? ch : a.n - 4);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) yg[fn][fm] = v4f{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int64_t tok = fm * 16 + li;
            sxp[fm] = a.sx + (tok < a.b ? tok : a.b - 1);
        }
    }

    // one 64-byte piece (128 codes, one group) of every operand row; sw4/sx1: that
    // group's scales (GRP only; s_X pre-multiplied by 2^-8, undoing the x16 x16 of the
    // expanded operands exactly)
    auto mma = [&](const uint4 (&bw)[FN], const uint4 (&bx)[FM][XN], const float4 (&sw4)[GRP ? FN : 1],
                   const float (&sx1)[GRP ? FM : 1]) {
        v4i alo[FN], ahi[FN], blo[FM], bhi[FM];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) unpack16(bw[fn], alo[fn], ahi[fn]);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            if constexpr (A8) {
                blo[fm] = perm16(bx[fm][0]);
                bhi[fm] = perm16(bx[fm][XN - 1]);
            } else {
                unpack16(bx[fm][0], blo[fm], bhi[fm]);
            }
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                if constexpr (GRP) {
                    v4i p = mfma_i8(alo[fn], blo[fm], v4i{0, 0, 0, 0});
                    p = mfma_i8(ahi[fn], bhi[fm], p);
                    const float swv[4] = {sw4[fn].x, sw4[fn].y, sw4[fn].z, sw4[fn].w};
#pragma unroll
                    for (int v = 0; v < 4; ++v) yg[fn][fm][v] += (float)p[v] * (sx1[fm] * swv[v]);
                } else {
                    acc[fn][fm] = mfma_i8(alo[fn], blo[fm], acc[fn][fm]);
                    acc[fn][fm] = mfma_i8(ahi[fn], bhi[fm], acc[fn][fm]);
                }
            }
    };
    auto load_scales = [&](int64_t c, float4 (&sw4)[GRP ? FN : 1], float (&sx1)[GRP ? FM : 1]) {
        if constexpr (GRP) {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) sw4[fn] = *reinterpret_cast<const float4 *>(swp[fn] + c * a.n);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) sx1[fm] = sxp[fm][c * a.b] * 0x1p-8f;
        }
    };
    auto load_x = [&](int64_t c, uint4 (&bx)[FM][XN]) {
        if constexpr (XL) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                bx[fm][0] = *reinterpret_cast<const uint4 *>(xls + ((c - cb) * FM + fm) * 1024 + li * 64 + g * 16);
            return;
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int h = 0; h < XN; ++h) bx[fm][h] = *reinterpret_cast<const uint4 *>(xrow[fm] + c * 64 * XN + 16 * h);
    };
    auto copy_x = [&]() {  // this wave's slice of Q_X into LDS (XL)
        const __amdgpu_buffer_rsrc_t rq =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.qx), 0, 0x7fffffff, 0x00020000);
        for (int64_t c = cb; c < ce; ++c)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int64_t tok = fm * 16 + lane / 4;
                const int64_t off = (tok < a.b ? tok : a.b - 1) * kb + c * 64 + (lane % 4) * 16;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rq, (__attribute__((address_space(3))) void *)(xls + ((c - cb) * FM + fm) * 1024), 16, (int)off, 0, 0, 0);
            }
    };
    // Software-pipelined batches: the loads of batch k + 1 are issued before batch k is
    // used (pieces at or past ce reload piece ce - 1 and are not used). Measured on
    // MI355X: per-token W4A4 CTAs of 16 tiles 3.6-4.7% faster, with fewer tiles the wasted
    // look-ahead of the last batch costs more than the overlap gains; the group-wise
    // variant, whose pieces each carry their scales and an fp32 update, 6-67% faster on
    // every tiling but 2 x 1 blocks (3% slower there); W4A8 2-8% slower.
    constexpr bool PIPE = (!GRP && !A8 && FN * FM >= 16) || (GRP && !(FN == 2 && FM == 1));
    if constexpr (PIPE) {
        struct Batch {
            uint4 bw[U][FN], bx[U][FM][XN];
            float4 sw4[U][GRP ? FN : 1];
            float sx1[U][GRP ? FM : 1];
        };
        auto load_batch = [&](int64_t c0, Batch &bt, bool with_x = true) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t cu = c0 + u < ce ? c0 + u : ce - 1;
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    bt.bw[u][fn] = load_stream16(wrow[fn] + (cu - cb) * kPanelPiece);
                if (with_x) load_x(cu, bt.bx[u]);
                load_scales(cu, bt.sw4[u], bt.sx1[u]);
            }
        };
        auto use_batch = [&](int64_t c0, Batch &bt) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (c0 + u < ce) mma(bt.bw[u], bt.bx[u], bt.sw4[u], bt.sx1[u]);
        };
        if (cb < ce) {
            Batch ba, bb;
            if constexpr (XL) {
                // the copy of X first, then the first batch's weights; once at most those
                // weight loads are outstanding the copy has landed and X is read from LDS
                copy_x();
                asm volatile("" ::: "memory");  // the copy stays ahead of the weight loads
                load_batch(cb, ba, false);
                asm volatile("" ::: "memory");  // every load of the batch issued before the wait
                wait_vmcnt<U * (GRP ? 2 * FN + FM : FN)>();
                asm volatile("" ::: "memory");
#pragma unroll
                for (int u = 0; u < U; ++u) load_x(cb + u < ce ? cb + u : ce - 1, ba.bx[u]);
            } else {
                load_batch(cb, ba);
            }
            for (int64_t c = cb;; c += 2 * U) {
                load_batch(c + U, bb);
                __builtin_amdgcn_sched_barrier(0);  // the next batch in flight before this one is used
                use_batch(c, ba);
                if (c + U >= ce) break;
                load_batch(c + 2 * U, ba);
                __builtin_amdgcn_sched_barrier(0);
                use_batch(c + U, bb);
                if (c + 2 * U >= ce) break;
            }
        }
    } else {
        int64_t c = cb;
        if constexpr (XL) {
            if (cb < ce) copy_x();
            asm volatile("" ::: "memory");  // the copy stays ahead of the weight loads
        }
        for (; c + U <= ce; c += U) {
            uint4 bw[U][FN], bx[U][FM][XN];
            float4 sw4[U][GRP ? FN : 1];
            float sx1[U][GRP ? FM : 1];
            if constexpr (XL) {
                // weights (and scales) of the batch first; at the first batch, once at most
                // those loads are outstanding the copy of X has landed
#pragma unroll
                for (int u = 0; u < U; ++u) {
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) bw[u][fn] = load_stream16(wrow[fn] + (c - cb + u) * kPanelPiece);
                    load_scales(c + u, sw4[u], sx1[u]);
                }
                if (c == cb) {
                    asm volatile("" ::: "memory");  // every load of the batch issued before the wait
                    wait_vmcnt<U * (GRP ? 2 * FN + FM : FN)>();
                    asm volatile("" ::: "memory");
                }
#pragma unroll
                for (int u = 0; u < U; ++u) load_x(c + u, bx[u]);
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) {
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) bw[u][fn] = load_stream16(wrow[fn] + (c - cb + u) * kPanelPiece);
                    load_x(c + u, bx[u]);
                    load_scales(c + u, sw4[u], sx1[u]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);  // keep every load of the batch ahead of its first use
#pragma unroll
            for (int u = 0; u < U; ++u) mma(bw[u], bx[u], sw4[u], sx1[u]);
        }
        for (; c < ce; ++c) {
            uint4 bw[FN], bx[FM][XN];
            float4 sw4[GRP ? FN : 1];
            float sx1[GRP ? FM : 1];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) bw[fn] = load_stream16(wrow[fn] + (c - cb) * kPanelPiece);
            if constexpr (XL) {
                load_scales(c, sw4, sx1);
                if (c == cb) {  // no whole batch before: wait for the copy of X here
                    asm volatile("" ::: "memory");
                    wait_vmcnt<GRP ? 2 * FN + FM : FN>();
                    asm volatile("" ::: "memory");
                }
                load_x(c, bx);
            } else {
                load_x(c, bx);
                load_scales(c, sw4, sx1);
            }
            mma(bw, bx, sw4, sx1);
        }
    }

    // Without the prefetch above (a wave owns several epilogue tiles), the low-rank
    // operands of all of the wave's tiles are loaded here, after the main loop and
    // before the reduction, so they arrive together and under the barrier (tile
    // indices past the last tile reload the last one, unused).
    constexpr int TPW = (TILES + NW - 1) / NW;  // epilogue tiles per wave
    constexpr bool LATE = !STORE_ACC && !PREFETCH && RS > 0 && TPW * RS <= 8;  // else: per tile, below
    v8h lal[LATE ? TPW : 1][LATE ? RS : 1];
    float4 tal[LATE ? TPW : 1][LATE ? RS : 1], tbl[LATE ? TPW : 1][LATE ? RS : 1];
    if constexpr (LATE) {
        if (!a.lr4) {
#pragma unroll
            for (int e = 0; e < TPW; ++e) {
                const int tile = wave + e * NW < TILES ? wave + e * NW : TILES - 1;
                const int64_t chr = ch0 + (tile / FM) * 16 + li, tokr = (tile % FM) * 16 + li;
                const uint16_t *l2row = a.l2t + (chr < a.n ? chr : a.n - 1) * a.r;
                const float *trow = a.t + (tokr < a.b ? tokr : a.b - 1) * a.r;
#pragma unroll
                for (int s = 0; s < RS; ++s) {
                    const int rank = s * 32 + g * 8;
                    const int rk = rank < a.r ? rank : 0;
                    lal[e][s] = load_h8(l2row + rk);
                    tal[e][s] = *reinterpret_cast<const float4 *>(trow + rk);
                    tbl[e][s] = *reinterpret_cast<const float4 *>(trow + rk + 4);
                }
            }
        }
    }

    if constexpr (XL && XSLICE != FN * FM * 1024) __syncthreads();  // every wave done with its slice of X
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            if constexpr (GRP)
                red[wave][fn * FM + fm][lane] = __builtin_bit_cast(v4i, yg[fn][fm]);
            else
                red[wave][fn * FM + fm][lane] = acc[fn][fm];
        }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < TPW; ++e) {
        const int tile = wave + e * NW;
        if (tile >= TILES) break;
        const int fn_e = tile / FM, fm_e = tile % FM;
        v4i sum = red[0][tile][lane];
        v4f ysum = __builtin_bit_cast(v4f, red[0][tile][lane]);
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            if constexpr (GRP)
                ysum += __builtin_bit_cast(v4f, red[w][tile][lane]);
            else
                sum += red[w][tile][lane];
        }
        const int64_t ch = ch0 + fn_e * 16 + 4 * g;
        const int64_t tok = fm_e * 16 + li;
        const bool store = ch < a.n && tok < a.b;
        if constexpr (STORE_ACC) {
            if (store) *reinterpret_cast<v4i *>(a.acc + tok * a.n + ch) = sum >> SH;
        } else {
            v4f y;
            if constexpr (GRP) {
                y = ysum;
            } else {
                const float sxv = a.sx[tok < a.b ? tok : a.b - 1];
                const float4 sw4 = *reinterpret_cast<const float4 *>(a.sw + (ch < a.n ? ch : a.n - 4));
                const float swv[4] = {sw4.x, sw4.y, sw4.z, sw4.w};
#pragma unroll
                for (int v = 0; v < 4; ++v) y[v] = (sxv * swv[v]) * (float)(sum[v] >> SH);
            }
            if (a.lr4) {
                if (a.r > 0) {
                    const v4i acc2 = lr4_tile(a, ch0 + fn_e * 16 + li, fm_e * 16 + li, g);
                    const float shv = a.sh[tok < a.b ? tok : a.b - 1];
#pragma unroll
                    for (int v = 0; v < 4; ++v) y[v] += shv * (float)(acc2[v] >> 8);
                }
            } else if constexpr (PREFETCH) {
#pragma unroll
                for (int s = 0; s < RS; ++s) {
                    const bool live = s * 32 + g * 8 < a.r;
                    float4 t0 = tf[s][0][0], t1 = tf[s][0][1];
#pragma unroll
                    for (int k = 1; k < TKS; ++k)
                        if (k < a.tks) {
                            t0.x += tf[s][k][0].x; t0.y += tf[s][k][0].y; t0.z += tf[s][k][0].z; t0.w += tf[s][k][0].w;
                            t1.x += tf[s][k][1].x; t1.y += tf[s][k][1].y; t1.z += tf[s][k][1].z; t1.w += tf[s][k][1].w;
                        }
                    y = mfma_f16(l2f[s], live ? f32x8_to_h8(t0, t1) : v8h{}, y);
                }
            } else if constexpr (LATE) {
#pragma unroll
                for (int s = 0; s < RS; ++s)
                    y = mfma_f16(lal[e][s], s * 32 + g * 8 < a.r ? f32x8_to_h8(tal[e][s], tbl[e][s]) : v8h{}, y);
            } else if constexpr (RS > 0) {
                // every rank step's L2^T and T pieces are loaded before the first is used
                const int64_t chr = ch0 + fn_e * 16 + li, tokr = fm_e * 16 + li;
                const uint16_t *l2row = a.l2t + (chr < a.n ? chr : a.n - 1) * a.r;
                const float *trow = a.t + (tokr < a.b ? tokr : a.b - 1) * a.r;
                v8h la[RS];
                float4 ta[RS], tb[RS];
#pragma unroll
                for (int s = 0; s < RS; ++s) {
                    const int rank = s * 32 + g * 8;
                    const int rk = rank < a.r ? rank : 0;
                    la[s] = load_h8(l2row + rk);
                    ta[s] = *reinterpret_cast<const float4 *>(trow + rk);
                    tb[s] = *reinterpret_cast<const float4 *>(trow + rk + 4);
                }
#pragma unroll
                for (int s = 0; s < RS; ++s)
                    y = mfma_f16(la[s], s * 32 + g * 8 < a.r ? f32x8_to_h8(ta[s], tb[s]) : v8h{}, y);
            }
            if (store) {
                v4h o;
#pragma unroll
                for (int v = 0; v < 4; ++v) o[v] = (_Float16)y[v];
                *reinterpret_cast<v4h *>(a.y + tok * a.n + ch) = o;
            }
        }
    }
}

// A 512-thread CTA gives a wave at most 256 registers. The variants that hold more --
// T's partial sums prefetched for a CTA of several tiles, the group-wise fp32 sums --
// run four waves instead, each over twice the K range: the first with twice the pieces
// in flight (U4), the group-wise one with its own measured count per tiling (UG); every
// instantiation then fits without spilling. W4A8 token rows take registers too, so
// that variant has half the pieces in flight (halved).
constexpr int halved(int u) { return u > 4 ? u / 2 : u; }

// T as a.tks partial sums: the kernel instantiated for the fewest slices (a power of two,
// at most kMaxTSlices / RS) that hold them. Its epilogue loads every slice it is built
// for before the main loop, so unused slices would cost (measured on the o_proj shape:
// 16 slices for 8 used, +0.9 us).
// xl: read X from LDS (per-token 2 x 2 blocks only: 7-8% faster there with T's slices in
// the epilogue, measured on MI355X; 1 x 2 blocks 3% slower, 1 x 4 and group-wise +2-3%)
template <int FN, int FM, int U, int RS, int NWT, bool GRP, bool A8, int TK = 2>
static void launch_decode_tk(const DualArgs &a, const dim3 grid, hipStream_t stream, bool xl = false) {
    if constexpr (2 * TK * RS <= kMaxTSlices) {
        if (a.tks > TK) return launch_decode_tk<FN, FM, U, RS, NWT, GRP, A8, 2 * TK>(a, grid, stream, xl);
    }
    constexpr bool XLK = !GRP && !A8 && FN == 2 && FM == 2;
    if (XLK && xl)
        hipLaunchKernelGGL((dual_linear_decode<FN, FM, U, RS, false, TK, NWT, GRP, A8, XLK>), grid, dim3(NWT * 64), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((dual_linear_decode<FN, FM, U, RS, false, TK, NWT, GRP, A8>), grid, dim3(NWT * 64), 0, stream,
                           a);
}

template <int FN, int FM, int U, int NW, int RS>
static hipError_t launch_decode_rs(const DualArgs &a, hipStream_t stream) {
    constexpr bool TKS = RS > 0 && FN * FM <= 4;  // the epilogue can add T's partial sums itself
    constexpr int U4 = NW == 8 ? (2 * U < 8 ? 2 * U : 8) : U;
    constexpr bool FIT = FN * FM == 1;  // one tile: its prefetched partial sums fit eight waves
    constexpr int NWT = FIT ? NW : 4, UT = FIT ? U : U4;                      // T as partial sums
    constexpr int NWA = RS >= 8 && FN * FM >= 8 ? 4 : NW, UA = NWA == NW ? U : U4;  // W4A8, T whole
    // group-wise (four waves, pipelined but for 2 x 1 blocks): pieces per batch measured per tiling
    constexpr int UG = FN * FM == 1 || (FN == 2 && FM == 1) ? 4 : FM == 2 && FN <= 2 ? 2 : 1;
    const dim3 grid((unsigned)((a.n + FN * 16 - 1) / (FN * 16)));
    const bool tk = TKS && a.tks > 1;
    if (a.a8) {
        if (a.acc)
            hipLaunchKernelGGL((dual_linear_decode<FN, FM, halved(U), 0, true, 1, NW, false, true>), grid, dim3(NW * 64), 0,
                               stream, a);
        else if (tk) {
            if constexpr (TKS) launch_decode_tk<FN, FM, halved(UT), RS, NWT, false, true>(a, grid, stream);
        } else
            hipLaunchKernelGGL((dual_linear_decode<FN, FM, halved(UA), RS, false, 1, NWA, false, true>), grid,
                               dim3(NWA * 64), 0, stream, a);
        return hipGetLastError();
    }
    // X read from LDS (XL) where it measured faster on MI355X (Y bitwise equal), each wave's
    // K slice of Q_X fitting its XSL bytes: per-token tiles of 16 blocks (4 x 4 at 49-64
    // tokens and m <= 4096 21-25% faster, 8 x 2 at 27-32 tokens and m = 8192 6-9%); per-token
    // tiles of 2 or 4 token blocks at m <= 4096, eight-wave ones (128 KB of LDS, one CTA a
    // compute unit) on at most 256 CTAs (4-8%; larger grids 4-22% slower, as was m = 8192);
    // group-wise tiles at m <= 4096 (4-12%). Per-token tiles of one token block ran 1-5%
    // slower and stay on global loads.
    constexpr bool XLT = FN * FM >= 16 || FM >= 2;
    constexpr int64_t XSL = FN * FM * 1024 > 16384 ? FN * FM * 1024 : 16384;
    const int64_t xpieces = (a.m / 128 + NW - 1) / NW;  // most pieces a wave streams
    const bool xl = XLT && xpieces * FM * 1024 <= XSL &&
                    (FN * FM >= 16 || (a.m <= 4096 && (NW == 4 || (int64_t)grid.x <= 256)));
    const bool xlg = (a.m / 128 + 3) / 4 * FM * 1024 <= XSL && a.m <= 4096;  // group-wise: four waves
    if (a.acc) {
        if (xl)
            hipLaunchKernelGGL((dual_linear_decode<FN, FM, U, 0, true, 1, NW, false, false, XLT>), grid, dim3(NW * 64), 0,
                               stream, a);
        else
            hipLaunchKernelGGL((dual_linear_decode<FN, FM, U, 0, true, 1, NW>), grid, dim3(NW * 64), 0, stream, a);
    } else if (a.group && tk) {
        if constexpr (TKS) launch_decode_tk<FN, FM, UG, RS, 4, true, false>(a, grid, stream);
    } else if (a.group && xlg)
        hipLaunchKernelGGL((dual_linear_decode<FN, FM, UG, RS, false, 1, 4, true, false, true>), grid, dim3(256), 0,
                           stream, a);
    else if (a.group)
        hipLaunchKernelGGL((dual_linear_decode<FN, FM, UG, RS, false, 1, 4, true>), grid, dim3(256), 0, stream, a);
    else if (tk) {
        if constexpr (TKS)
            launch_decode_tk<FN, FM, UT, RS, NWT, false, false>(
                a, grid, stream, (a.m / 128 + NWT - 1) / NWT * FM * 1024 <= 16384 && a.m <= 4096);
    } else if (xl)
        hipLaunchKernelGGL((dual_linear_decode<FN, FM, U, RS, false, 1, NW, false, false, XLT>), grid, dim3(NW * 64), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((dual_linear_decode<FN, FM, U, RS, false, 1, NW>), grid, dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

template <int FN, int FM, int U, int NW>
static hipError_t launch_decode(const DualArgs &a, hipStream_t stream) {
    // rank steps of 32 the epilogue prefetches
    if (a.r == 0) return launch_decode_rs<FN, FM, U, NW, 0>(a, stream);
    if (a.r <= 32) return launch_decode_rs<FN, FM, U, NW, 1>(a, stream);
    if (a.r <= 64) return launch_decode_rs<FN, FM, U, NW, 2>(a, stream);
    if (a.r <= 128) return launch_decode_rs<FN, FM, U, NW, 4>(a, stream);
    return launch_decode_rs<FN, FM, U, NW, 8>(a, stream);
}

// ---------------------------------------------------------------------------------
// Many tokens: the main loop is bound by the int8 matrix cores. A CTA owns a BN x BM
// tile of Y^T (BN output channels by BM tokens) and streams K in stages of 128 codes
// (64 bytes per row) through a ring of S stages in LDS, filled by direct-to-LDS buffer
// loads (no register staging, S - 1 stages in flight).
// A stage holds the 128-code K slice of the tile's BN weight rows and BM token rows
// (64 bytes per row) as 1 KB blocks of 16 rows. Inside a block, rows 2s and 2s + 1
// share the 128-byte line s (s = 0..7): the 16-byte chunk c of row 2s + h has logical
// position 4h + c in the line and is stored at position (4h + c) ^ s. Both sides of the
// stage run at full rate with this layout on gfx950 (measured):
//  - the direct-to-LDS loads write a wave's 64 lanes to 64 consecutive 16-byte slots,
//    and with this layout every 4-lane quad fetches one row's contiguous 64 bytes
//    (only the order inside the quad is permuted), which the memory pipeline coalesces;
//  - an MFMA operand wants row li, chunk g in lane li + 16 g; those reads hit every
//    bank group evenly (plain 64-byte rows, swizzled or not, run at half rate).
// Waves read their operands back, expand them to int8 (unpack16) and issue
// v_mfma_i32_16x16x64_i8. Rows past n or b are clamped to a valid row (their outputs
// are never stored); m is a multiple of 128, so stages never run past a row.
// Block indices are mapped to tiles XCD by XCD (the hardware deals consecutive CTAs
// to the eight XCDs in turn): each XCD walks a contiguous range of tiles ordered in
// groups of GM token tiles, so the CTAs an XCD runs at once share W and Q_X tiles in
// that XCD's L2.

// Y of a wave's FN x FM tiles, stored fp16 (rows past n or b not stored).
template <int BN, int BM, int WN, int WM, int FN, int FM>
__device__ __forceinline__ void pf_store(const DualArgs &a, const v4f (&y)[FN][FM], int64_t ch0, int64_t tok0, int wn,
                                         int wm, int li, int g) {
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

// The fp16 low-rank branch with its operands staged through the CTA's LDS ring (T as
// fp16, a.t16). A step of 32 ranks needs the tile's BN rows of L2^T and BM rows of T,
// 64 bytes each: the shape of one main-loop stage, so it is loaded, laid out and read
// exactly as one (direct-to-LDS loads, no register holds a load in flight), and the steps
// continue the main loop's ring: its last S - 1 steps load low-rank steps 0 .. S - 2 into
// the slots they free, and the epilogue keeps S steps in flight. Measured on MI355X at
// b = m = 8192, n = 28672, r = 128: this branch cost 98 us of the 1306 us kernel with its
// operands loaded into registers step by step (each step a round trip to memory); its
// loads barely overlap the few MFMAs a step takes, so the round trips, not the slots,
// are what to save. The buffers' record counts are the operands' exact sizes, so the half
// step past r (r an odd multiple of 16) of the last row reads zeros; other rows' dead ranks
// are zeroed below, as in the register path. The sums are the register path's, in the same
// order, on the same fp16 values: Y is the same bit for bit.

// Low-rank step e (past the last: the last again) of the tile at (ch0, tok0) into ring slot
// `slot`: the main loop's (row, 16-byte chunk) mapping, rows of L2^T (channel rows, first
// BN) or of T (token rows), clamped into the operand. XS: the stages carry group scales,
// and one more 4-byte load lands in the slot's scale area (never read), so a step issues
// as many loads as a stage. The offsets are formed here from a copy of the thread index the
// compiler cannot see through, so they are not kept live across the main loop.
template <int BN, int BM, int NT, int SLOT, int XS, bool ODD = false>
__device__ __forceinline__ void pf_lr_issue(const DualArgs &a, int64_t ch0, int64_t tok0, uint8_t *ring, int slot, int e,
                                            int tid) {
    constexpr int CPR = 4, DPT = (BN + BM) * CPR / NT;
    static_assert((BN * CPR) % NT == 0 && NT % kWave == 0, "each load group in one operand");
    int t = tid;
    asm volatile("" : "+v"(t));
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
    const int last = (a.r + 31) / 32 - 1;
    const int sc = e < last ? e : last;
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a.l2t), 0,
                                                                        (int)(a.n * a.r * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a.t16), 0,
                                                                        (int)(a.b * a.r * 2), 0x00020000);
    uint8_t *dst = ring + slot * SLOT;
    // lane l of load j: row 16 (4 j + wave) + 2 (l / 8) + c / 4 of the step, 16-byte chunk
    // c % 4, c = (l % 8) ^ (l / 8); indices fit 32 bits (n r and b r do)
    // ODD (the 32 x 32 kernel's layout): odd 1 KB blocks -- each wave fills one -- have
    // bit 0 of the chunk position flipped as well
    const int lane = t % kWave, line = lane / 8, logical = (lane % 8) ^ line ^ (ODD ? (wave & 1) : 0);
    const int lrow = 2 * line + logical / 4, lchunk = (logical % 4) * 16;
    const int nlast = (int)a.n - 1, blast = (int)a.b - 1, r2 = a.r * 2;
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
        const int row = (j * (NT / kWave) + wave) * 16 + lrow;  // j * NT / CPR rows before load j
        const int rr = (j * NT) / CPR < BN ? ((int)ch0 + row < nlast ? (int)ch0 + row : nlast)
                                           : ((int)tok0 + row - BN < blast ? (int)tok0 + row - BN : blast);
        __builtin_amdgcn_raw_ptr_buffer_load_lds((j * NT) / CPR < BN ? rl : rt,
                                                 (__attribute__((address_space(3))) void *)(dst + (j * NT + wave * kWave) * 16),
                                                 16, rr * r2 + lchunk, sc * 64, 0, 0);
    }
    if constexpr (XS > 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (__attribute__((address_space(3))) void *)(dst + XS + wave * kWave * 4), 4,
                                                 0, 0, 0, 0);
}

// The low-rank steps after the main loop. nst: main-loop stages; low-rank step e sits in
// slot (nst + e) % S; steps 0 .. S - 2 were issued by the main loop's last steps (LPT
// loads each, as a stage). Step e: wait until it has landed (the later steps still in
// flight), meet, use it, and, if a step is still to load, meet again (every wave is done
// with the slot) and load step e + S into it. Two barriers a step instead of one, but S
// steps in flight instead of S - 1: the MFMAs between them are few.
template <int BN, int BM, int WN, int WM, int S, int SLOT, int LPT, int XS, int FN, int FM>
__device__ __forceinline__ void pf_lowrank_ring(const DualArgs &a, v4f (&y)[FN][FM], int64_t ch0, int64_t tok0, int wn,
                                                int wm, int li, int g, uint8_t *ring, int tid, int nst) {
    constexpr int NT = WN * WM * 64, BLK = 1024;
    static_assert((BN + BM) * 64 <= SLOT && FN == 4 && FM == 4 && S >= 2 && S <= 3, "one step fits a ring slot");
    const int nlr = (a.r + 31) / 32;
    // operand reads: row li, chunk g of a block, as in the main loop
    const uint32_t lane_off = (li / 2) * 128 + ((4 * (li % 2) + g) ^ (li / 2)) * 16;
    const uint32_t rda = lds_offset(ring) + lane_off + (wn * (BN / WN) / 16) * BLK;
    const uint32_t rdb = lds_offset(ring) + lane_off + ((BN + wm * (BM / WM)) / 16) * BLK;

    int slot = nst % S;  // step 0's
    stage_barrier();     // every wave is done with the main loop's last stage, in slot (nst + S - 1) % S
    if (S - 1 < nlr) pf_lr_issue<BN, BM, NT, SLOT, XS>(a, ch0, tok0, ring, slot == 0 ? S - 1 : slot - 1, S - 1, tid);
    for (int e = 0; e < nlr; ++e) {
        // loads issued after step e's: those of the next steps (if fewer, waiting for more is safe)
        const int ahead = nlr - 1 - e;
        if (S > 2 && ahead >= 2)
            wait_vmcnt<(S > 2 ? 2 : 1) * LPT>();
        else if (ahead >= 1)
            wait_vmcnt<LPT>();
        else
            wait_vmcnt<0>();
        stage_barrier();  // step e landed for every thread
        v4i raw[8];
        lds_read_4x4<0, BLK>(rda + slot * SLOT, rdb + slot * SLOT, raw);
        const bool live = e * 32 + g * 8 < a.r;  // r is a multiple of 16
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                y[fn][fm] = mfma_f16(__builtin_bit_cast(v8h, raw[fn]), live ? __builtin_bit_cast(v8h, raw[4 + fm]) : v8h{},
                                     y[fn][fm]);
        if (e + S < nlr) {
            stage_barrier();  // every wave is done with this slot
            pf_lr_issue<BN, BM, NT, SLOT, XS>(a, ch0, tok0, ring, slot, e + S, tid);
        }
        slot = slot + 1 == S ? 0 : slot + 1;
    }
    wait_vmcnt<0>();  // no load may still be writing this CTA's LDS when it ends
}

// Second half of the many-token epilogue, from the dequantized residual y of a wave's
// FN x FM tiles of 16 x 16 (the wave at (wn, wm) of a BN x BM CTA tile at (ch0, tok0)):
// add the low-rank branch and store fp16 (T as fp32, operands loaded into registers; with
// T as fp16 the kernel takes pf_lowrank_ring instead).
template <int BN, int BM, int WN, int WM, bool LR4, int FN, int FM>
__device__ __forceinline__ void pf_finish(const DualArgs &a, v4f (&y)[FN][FM], int64_t ch0, int64_t tok0, int wn, int wm,
                                          int li, int g) {
    if constexpr (LR4) {
        // int4 low-rank branch: y += s_H (Q_H Q_L2^T)
        if (a.r > 0) {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    const int64_t chr = ch0 + wn * (BN / WN) + fn * 16 + li;
                    const int64_t tokr = tok0 + wm * (BM / WM) + fm * 16 + li;
                    const v4i acc2 = lr4_tile(a, chr, tokr, g);
                    const float shv = a.sh[tokr < a.b ? tokr : a.b - 1];
#pragma unroll
                    for (int v = 0; v < 4; ++v) y[fn][fm][v] += shv * (float)(acc2[v] >> 8);
                }
        }
    }
    // fp16 low-rank branch: y += L2^T (channels x ranks) . T^T (ranks x tokens). Rows are
    // addressed by 32-bit element offsets from the uniform bases (n r and b r stay below
    // 2^32 within the ABI's limits) rather than one 64-bit pointer per row.
    const int64_t chb = ch0 + wn * (BN / WN) + li, tkb = tok0 + wm * (BM / WM) + li;
    for (int k0 = 0; k0 < (LR4 ? 0 : a.r); k0 += 32) {
        const int rank = k0 + g * 8;
        const bool live = rank < a.r;  // r is a multiple of 16: live means rank + 8 <= r
        const uint32_t rk = live ? rank : 0;
        v8h la[FN], tb[FM];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int64_t ch = chb + fn * 16;
            la[fn] = load_h8(a.l2t + ((uint32_t)((ch < a.n ? ch : a.n - 1) * a.r) + rk));
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int64_t tok = tkb + fm * 16;
            const float4 *tp = reinterpret_cast<const float4 *>(a.t + ((uint32_t)((tok < a.b ? tok : a.b - 1) * a.r) + rk));
            tb[fm] = live ? f32x8_to_h8(tp[0], tp[1]) : v8h{};
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) y[fn][fm] = mfma_f16(la[fn], tb[fm], y[fn][fm]);
    }
    pf_store<BN, BM, WN, WM>(a, y, ch0, tok0, wn, wm, li, g);
}

// Epilogue of the many-token kernels: dequantize the integer sums, then pf_finish (or
// store the exact integer sums). SH: log2 of the operands' combined scale in acc (8 for
// 4-bit x 4-bit, 4 for W4A8).
template <int BN, int BM, int WN, int WM, bool STORE_ACC, bool LR4, int SH, int FN, int FM>
__device__ __forceinline__ void pf_epilogue(const DualArgs &a, v4i (&acc)[FN][FM], int64_t ch0, int64_t tok0, int wn, int wm,
                                            int li, int g) {
    // lane (li, g), register v of tile (fn, fm) holds channel ch_base + 4g + v, token tok_base + li
    if constexpr (STORE_ACC) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int64_t ch = ch0 + wn * (BN / WN) + fn * 16 + 4 * g;
                const int64_t tok = tok0 + wm * (BM / WM) + fm * 16 + li;
                if (ch < a.n && tok < a.b) *reinterpret_cast<v4i *>(a.acc + tok * a.n + ch) = acc[fn][fm] >> SH;
            }
    } else {
        float sxv[FM];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int64_t tok = tok0 + wm * (BM / WM) + fm * 16 + li;
            sxv[fm] = a.sx[tok < a.b ? tok : a.b - 1];
        }
        v4f y[FN][FM];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int64_t ch = ch0 + wn * (BN / WN) + fn * 16 + 4 * g;
            const float4 sw4 = *reinterpret_cast<const float4 *>(a.sw + (ch < a.n ? ch : a.n - 4));
            const float swv[4] = {sw4.x, sw4.y, sw4.z, sw4.w};
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int v = 0; v < 4; ++v) y[fn][fm][v] = (sxv[fm] * swv[v]) * (float)(acc[fn][fm][v] >> SH);
        }
        pf_finish<BN, BM, WN, WM, LR4>(a, y, ch0, tok0, wn, wm, li, g);
    }
}

// Three CTAs per compute unit (12 waves) fit the LDS ring; the register budget that
// allows is asked for explicitly (measured 7-12% faster than two CTAs on the prefill
// shapes, the group-wise variant (GRP) included, which keeps a second, fp32 set of
// accumulators). W4A8's stages are 24 KB, so it runs a two-stage ring (one stage in
// flight) to fit three CTAs per unit: 2-10% faster than three stages at two CTAs.
// (The per-token 4-bit layer runs dual_linear_pf32 below, which keeps this kernel's ring
// and tile order on 32 x 32 matrix blocks.)
//
// GRP (groups of kGroup = 128 along K): a stage is one group. Each slot of the ring
// also holds the stage's scales, s_W of the tile's BN channels and s_X of its BM tokens
// (one 4-byte direct-to-LDS load per thread, from the group-major scale arrays), and
// each stage's integer sums are formed from zero and added to the fp32 accumulators
// times s_X s_W.
//
// W4A8 (A8): a token row holds one int8 code per element, 128 bytes per stage, stored as
// two 64-byte rows e = 0, 1 (the first BM rows of the token part and the next BM): row e
// holds bytes 32c + 16e .. 32c + 16e + 15 of the token's slice at chunk position c, so the
// layout, the loads and the lane -> address map of the reads above apply unchanged. Lane
// (li, g) needs codes 32g..32g+31 of its token: chunk g of rows 0 and 1, read exactly
// like the 4-bit token operand (splitting the slice into bytes 0-63 and 64-127 instead
// gave lanes g and g + 2 the same banks: LDS bank conflicts, 2-3.6% slower), permuted
// into the expanded weight operand's lane order (perm16); the accumulator holds 16 acc.
template <int BN, int BM, int WN, int WM, int S, int GM, int RB, bool STORE_ACC, bool LR4 = false, bool GRP = false,
          bool A8 = false, bool T16 = false>
__global__ __launch_bounds__(WN * WM * 64, A8 ? (S > 2 ? 2 : 3) : (S == 2 ? 4 : 3))
void dual_linear_pf(DualArgs a, int tiles_n, int tiles_m) {
    constexpr int NT = WN * WM * 64;
    constexpr int FN = BN / (16 * WN), FM = BM / (16 * WM);
    constexpr int XH = A8 ? 2 : 1;              // LDS rows per token row per stage
    constexpr int ROWS = BN + XH * BM;
    static_assert(!A8 || (RB == 64 && !GRP && !LR4), "W4A8: 64-byte weight rows, per-token scales");
    static_assert(RB == 64 || RB == 128, "bytes per row per stage");
    constexpr int CPR = RB / 16;                // 16-byte chunks per row per stage
    constexpr int BLK = 16 * RB;                // one block of 16 rows
    constexpr int STAGE_BYTES = ROWS * RB;
    constexpr int DPT = ROWS * CPR / NT;        // 16-byte DMA loads per thread per stage
    constexpr int LPT = DPT + (GRP ? 1 : 0);    // all loads per thread per stage
    constexpr int SLOT = STAGE_BYTES + (GRP ? 4 * (BN + BM) : 0);
    static_assert(ROWS * 4 % NT == 0 && FN >= 1 && FM >= 1, "tile shape");
    static_assert((S - 2) * LPT < 64, "outstanding loads fit vmcnt");
    static_assert(!GRP || (RB == 64 && BN == 128 && BM == 128 && NT == 256 && !STORE_ACC && !LR4),
                  "group-wise: one group per stage, one scale load per thread");

    static_assert(!T16 || (GRP && !A8 && !LR4 && !STORE_ACC && RB == 64),
                  "fp16 T through the ring: group-wise, 64-byte stages (per-token: dual_linear_pf32)");
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int li = lane & 15, g = lane >> 4;
    const int wn = wave % WN, wm = wave / WN;

    // block -> tile: contiguous per XCD, grouped GM token tiles at a time. The tile count
    // fits 32 bits (the launch grid does), and the tile indices are uniform: they are
    // computed in 32-bit arithmetic and kept in scalar registers, which leaves the vector
    // registers to the main loop.
    const int ntiles = tiles_n * tiles_m;
    const int o = (int)xcd_order(blockIdx.x, ntiles);
    const int gsz = GM * tiles_n;
    const int grp = o / gsz, within = o % gsz;
    const int gm_here = (tiles_m - grp * GM) < GM ? (tiles_m - grp * GM) : GM;
    const int tm = __builtin_amdgcn_readfirstlane(grp * GM + within % gm_here);
    const int tn = __builtin_amdgcn_readfirstlane(within / gm_here);
    const int64_t ch0 = (int64_t)tn * BN, tok0 = (int64_t)tm * BM;
    const int64_t kb = a.m / 2;
    const int nst = (int)(a.m / (2 * RB));  // m is a multiple of 2 RB

    // this thread's DMA sources: slot q = j * NT + tid of each stage is 16-byte position
    // q % 8 of 128-byte line (q % (16 CPR)) / 8 of block q / (16 CPR). Each j lies wholly
    // in the weight rows or wholly in the token rows, so its address is a uniform tile
    // base plus a 32-bit per-lane offset, advanced per stage by RB bytes in a token row
    // and by 16 RB bytes in the weight panels (a stage is RB / 64 pieces of each panel).
    static_assert(NT % 64 == 0 && (BN * CPR) % NT == 0, "each DMA group in one operand");
    const int64_t xb = A8 ? a.m : kb;           // bytes per token row
    const uint8_t *wbase = a.qw + ch0 * kb, *xbase = a.qx + tok0 * xb;
    uint32_t off[DPT];
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
        const int q = j * NT + tid;
        const int line = (q % (16 * CPR)) / 8, logical = (q % 8) ^ (RB == 64 ? line : (line >> 1) & 7);
        const int row = (q / (16 * CPR)) * 16 + (RB == 64 ? 2 * line + logical / 4 : line);
        const int chunk = RB == 64 ? logical % 4 : logical;
        int64_t rel;  // row offset from the tile's first row, clamped into the operand
        if (row < BN) {
            const int64_t ch = ch0 + row;
            rel = (ch < a.n ? ch : a.n - 1) - ch0;
        } else {
            const int64_t tok = tok0 + (row - BN) % BM;
            rel = (tok < a.b ? tok : a.b - 1) - tok0;
        }
        // A8: chunk c of token row BN + e BM + t holds bytes 32 c + 16 e .. + 15 of token t's slice
        off[j] = (uint32_t)(row < BN ? qw_offset(rel, chunk * 16, a.m)
                                     : rel * xb + (A8 ? chunk * 32 + ((row - BN) / BM) * 16 : chunk * 16));
    }
    __shared__ __attribute__((aligned(16))) uint8_t ring[S * SLOT];
    // GRP: this thread's scale: waves 0-1 load s_W of channel ch0 + tid, waves 2-3 s_X of
    // token tok0 + tid - 128 (rows past n or b clamped), into the slot's scale area
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t soff = 0;
    if constexpr (GRP) {
        const int64_t rel = tid < BN ? (ch0 + tid < a.n ? tid : a.n - 1 - ch0)
                                     : (tok0 + tid - BN < a.b ? tid - BN : a.b - 1 - tok0);
        soff = (uint32_t)(rel * 4);
    }
    // buffer loads straight to LDS: one resource per operand tile (raw, 32-bit element
    // format; every offset stays inside the tile's clamped rows), the per-lane offset
    // in a VGPR that never changes and the stage offset in an SGPR
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(wbase), 0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(xbase), 0, 0x7fffffff, 0x00020000);
    auto issue = [&](int st, auto slot) {
        if constexpr (T16) {
            if (st >= nst) {  // past the last stage: the low-rank steps, into the slots it frees
                pf_lr_issue<BN, BM, NT, SLOT, GRP ? STAGE_BYTES : 0>(a, ch0, tok0, ring, decltype(slot)::value, st - nst, tid);
                return;
            }
        }
        uint8_t *dst = ring + decltype(slot)::value * SLOT;
#pragma unroll
        for (int j = 0; j < DPT; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds((j * NT) / CPR < BN ? rw : rx,
                                                     (__attribute__((address_space(3))) void *)(dst + (j * NT + wave_u * kWave) * 16),
                                                     16, (int)off[j], st * RB * ((j * NT) / CPR < BN ? kPanelRows : XH), 0, 0);
        if constexpr (GRP) {
            // group st's row of the group-major scales, from the tile's first channel or token
            const float *sb = wave_u < BN / kWave ? a.sw + (int64_t)st * a.n + ch0 : a.sx + (int64_t)st * a.b + tok0;
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(sb), 0, 0x7fffffff, 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(dst + STAGE_BYTES + wave_u * kWave * 4),
                                                     4, (int)soff, 0, 0, 0);
        }
    };

    v4i acc[FN][FM];
    v4f yg[GRP ? FN : 1][GRP ? FM : 1];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            acc[fn][fm] = v4i{0, 0, 0, 0};
            if constexpr (GRP) yg[fn][fm] = v4f{0.f, 0.f, 0.f, 0.f};
        }
    // GRP: this lane's scale reads in a slot: s_W of channels wn BN/WN + 16 fn + 4g..+3,
    // s_X of token wm BM/WM + 16 fm + li
    const uint32_t rsw = lds_offset(ring) + STAGE_BYTES + (wn * (BN / WN) + 4 * g) * 4;
    const uint32_t rsx = lds_offset(ring) + STAGE_BYTES + (BN + wm * (BM / WM) + li) * 4;

    // this lane's operand addresses, per MFMA k-step h of a stage: FN weight blocks from
    // rda[h], FM token blocks from rdb[h]. Row li, chunk c of a block: with 64-byte rows,
    // line li / 2 at position (4 (li % 2) + c) ^ (li / 2); with 128-byte rows, line li at
    // position c ^ ((li / 2) % 8).
    static_assert(FN == 4 && FM == 4, "the stage reader loads four weight and four token blocks per wave");
    constexpr int KS = RB / 64;  // MFMA k-steps per stage
    uint32_t rda[KS], rdb[KS];
#pragma unroll
    for (int h = 0; h < KS; ++h) {
        const uint32_t lane_off = RB == 64 ? (li / 2) * 128 + ((4 * (li % 2) + g) ^ (li / 2)) * 16
                                           : li * 128 + ((4 * h + g) ^ ((li / 2) % 8)) * 16;
        rda[h] = lds_offset(ring) + lane_off + (wn * (BN / WN) / 16) * BLK;
        rdb[h] = lds_offset(ring) + lane_off + ((BN + wm * (BM / WM)) / 16) * BLK;
    }
    // A8: this lane's chunk g of token rows e = 0, 1 (as the 4-bit token operand: line
    // li / 2, position (4 (li % 2) + g) ^ (li / 2))
    uint32_t rdx[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        rdx[e] = lds_offset(ring) + (li / 2) * 128 + ((4 * (li % 2) + g) ^ (li / 2)) * 16 +
                 ((BN + e * BM + wm * (BM / WM)) / 16) * BLK;
    }

    // Step st issues stage st into slot st % S and consumes stage st - (S - 1). Every
    // step issues (past the last stage it loads the last stage again, into a slot no
    // later step reads, or with T16 the first low-rank steps), so the count of loads in
    // flight is the same at every wait and the compiler sees no branch around a load.
    // The loop is unrolled by the ring depth, so every slot is a compile-time constant.
    for (int s0 = 0; s0 < nst + S - 1; s0 += S) {
        static_for(std::make_integer_sequence<int, S>{}, [&](auto u) {
            const int st = s0 + u, c = st - (S - 1);
            if (c >= nst) return;
            if (c >= 0) {
                wait_vmcnt<(S - 2) * LPT>();
                stage_barrier();  // stage c landed for every thread; stage c - 1 consumed by every wave
            }
            issue(T16 || st < nst ? st : nst - 1, u);
            if (c < 0) return;
            constexpr int OFF = ((u + 1) % S) * SLOT;  // slot of stage c
            v4f swr[4];
            float sxr[4];
            if constexpr (GRP) lds_read_scales<OFF>(rsw, rsx, swr, sxr);
#pragma unroll
            for (int h = 0; h < KS; ++h) {
                v4i alo[FN], ahi[FN], blo[FM], bhi[FM];
                if constexpr (A8) {
                    v4i raw[12];
                    lds_read_4x4x4<OFF, BLK>(rda[h], rdx[0], rdx[1], raw);
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) unpack16(raw[fn], alo[fn], ahi[fn]);
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm) {
                        blo[fm] = perm16(raw[FN + fm]);
                        bhi[fm] = perm16(raw[FN + FM + fm]);
                    }
                } else {
                    v4i raw[8];
                    lds_read_4x4<OFF, BLK>(rda[h], rdb[h], raw);
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) unpack16(raw[fn], alo[fn], ahi[fn]);
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm) unpack16(raw[FN + fm], blo[fm], bhi[fm]);
                }
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm) {
                        if constexpr (GRP) {
                            // the group's sum from zero, scaled in (2^-8 undoes the x16 x16 of the operands)
                            v4i p = mfma_i8(alo[fn], blo[fm], v4i{0, 0, 0, 0});
                            p = mfma_i8(ahi[fn], bhi[fm], p);
                            const float sxs = sxr[fm] * 0x1p-8f;
#pragma unroll
                            for (int v = 0; v < 4; ++v) yg[fn][fm][v] += (float)p[v] * (sxs * swr[fn][v]);
                        } else {
                            acc[fn][fm] = mfma_i8(alo[fn], blo[fm], acc[fn][fm]);
                            acc[fn][fm] = mfma_i8(ahi[fn], bhi[fm], acc[fn][fm]);
                        }
                    }
            }
        });
    }

    // The epilogue's lane coordinates are recomputed from the thread index (one register
    // across the main loop instead of four; the wave's are uniform): with four CTAs a
    // compute unit, keeping all four live through the loop spilled them.
    int te = tid;
    asm volatile("" : "+v"(te));
    const int li_e = te & 15, g_e = (te >> 4) & 3;
    const int wn_e = wave_u % WN, wm_e = wave_u / WN;
    if constexpr (T16) {  // group-wise (static_assert above)
        pf_lowrank_ring<BN, BM, WN, WM, S, SLOT, LPT, STAGE_BYTES>(a, yg, ch0, tok0, wn_e, wm_e, li_e, g_e, ring, te, nst);
        pf_store<BN, BM, WN, WM>(a, yg, ch0, tok0, wn_e, wm_e, li_e, g_e);
    } else if constexpr (GRP) {
        pf_finish<BN, BM, WN, WM, false>(a, yg, ch0, tok0, wn_e, wm_e, li_e, g_e);
    } else {
        pf_epilogue<BN, BM, WN, WM, STORE_ACC, LR4, A8 ? 4 : 8>(a, acc, ch0, tok0, wn_e, wm_e, li_e, g_e);
    }
}

// ---------------------------------------------------------------------------------
// Many tokens, per-token scales, 4-bit activations (the one-call layer, the split call
// with T in fp32, r = 0, and the exact accumulator export): the ring, stages and tile
// order of dual_linear_pf, with each wave's 64 x 64 tile as 2 x 2 blocks of 32 x 32 on
// v_mfma_i32_32x32x32_i8 instead of 4 x 4 blocks of 16 x 16. The operand bytes, the
// expansion work and the matrix-core time per stage are the same; the matrix
// instructions are half as many, and the issue slots they free go to the expansion
// beside them, which is what bounds the loop.
// Lane l reads row l % 32 of a 32-row block (two 16-row LDS blocks), the 16 bytes of
// chunk 2 h + l / 32 for the stage's halves h = 0, 1, with the same (row, chunk) -> LDS
// address map as dual_linear_pf, so the reads stay free of bank conflicts. Both operands
// take the same chunks and expand them the same way, so their codes pair one for one
// whatever order the instruction sums them in. In the result, lane l holds token l % 32
// of its block and register v channel 8 (v / 4) + 4 (l / 32) + v % 4.
//
// The fp16 low-rank branch runs on v_mfma_f32_32x32x16_f16 with the dequantized sums
// as its C operand: T16, its operands through the ring (as pf_lowrank_ring); else T in
// fp32 and L2^T from memory into registers (as pf_finish). Either way each lane takes
// the 8 ranks of chunk 2 k + l / 32 of a 32-rank step (k = 0, 1) for its row.

// Y of a wave's 2 x 2 blocks of 32 x 32 at (chw, tkw), stored fp16 (rows past n or b
// not stored; n is a multiple of 16, so a live channel quad is whole).
__device__ __forceinline__ void pf32_store(const DualArgs &a, const v16f (&y)[2][2], int64_t chw, int64_t tkw, int r32,
                                           int kh) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t ch = chw + rb * 32 + 8 * q + 4 * kh;
                const int64_t tok = tkw + cb * 32 + r32;
                if (ch < a.n && tok < a.b) {
                    v4h o;
#pragma unroll
                    for (int v = 0; v < 4; ++v) o[v] = (_Float16)y[rb][cb][4 * q + v];
                    *reinterpret_cast<v4h *>(a.y + tok * a.n + ch) = o;
                }
            }
}

// The low-rank steps after the main loop, through the ring (pf_lowrank_ring's schedule:
// steps 0 .. S - 2 were issued by the main loop's last steps into the slots they freed;
// step e sits in slot (nst + e) % S; S steps in flight, two barriers a step).
template <int S, int SLOT, int LPT>
__device__ __forceinline__ void pf32_lowrank_ring(const DualArgs &a, v16f (&y)[2][2], int64_t ch0, int64_t tok0,
                                                  const uint32_t (&rda)[2], const uint32_t (&rdb)[2], int kh,
                                                  uint8_t *ring, int tid, int nst) {
    constexpr int BN = 128, BM = 128, NT = 256, STR = 2048;
    static_assert(S >= 2 && S <= 3, "ring depth");
    const int nlr = (a.r + 31) / 32;
    int slot = nst % S;  // step 0's
    stage_barrier();     // every wave is done with the main loop's last stage
    if (S - 1 < nlr) pf_lr_issue<BN, BM, NT, SLOT, 0, true>(a, ch0, tok0, ring, slot == 0 ? S - 1 : slot - 1, S - 1, tid);
    for (int e = 0; e < nlr; ++e) {
        const int ahead = nlr - 1 - e;
        if (S > 2 && ahead >= 2)
            wait_vmcnt<(S > 2 ? 2 : 1) * LPT>();
        else if (ahead >= 1)
            wait_vmcnt<LPT>();
        else
            wait_vmcnt<0>();
        stage_barrier();  // step e landed for every thread
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            // the step's k-th 16 ranks: L2^T rows of the wave's two channel blocks, T rows
            // of its two token blocks (read half a step at a time: registers are short here)
            v4i raw[4];
            lds_read_2x2<0, STR>(rda[k] + slot * SLOT, rdb[k] + slot * SLOT, raw);
            const bool live = e * 32 + (2 * k + kh) * 8 < a.r;  // r is a multiple of 16
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    y[rb][cb] = mfma_f16_32(__builtin_bit_cast(v8h, raw[rb]), live ? __builtin_bit_cast(v8h, raw[2 + cb]) : v8h{},
                                            y[rb][cb]);
        }
        if (e + S < nlr) {
            stage_barrier();  // every wave is done with this slot
            pf_lr_issue<BN, BM, NT, SLOT, 0, true>(a, ch0, tok0, ring, slot, e + S, tid);
        }
        slot = slot + 1 == S ? 0 : slot + 1;
    }
    wait_vmcnt<0>();  // no load may still be writing this CTA's LDS when it ends
}

// The low-rank branch from memory (T in fp32, rounded to fp16 as it is loaded; L2^T
// rows fp16), as pf_finish does for 16 x 16 blocks.
__device__ __forceinline__ void pf32_lowrank_regs(const DualArgs &a, v16f (&y)[2][2], int64_t chw, int64_t tkw, int r32,
                                                  int kh) {
    for (int k0 = 0; k0 < a.r; k0 += 16) {
        const int rank = k0 + kh * 8;
        const bool live = rank < a.r;  // r is a multiple of 16: live means rank + 8 <= r
        const uint32_t rk = live ? rank : 0;
        v8h la[2], tb[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const int64_t ch = chw + rb * 32 + r32;
            la[rb] = load_h8(a.l2t + ((uint32_t)((ch < a.n ? ch : a.n - 1) * a.r) + rk));
        }
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int64_t tok = tkw + cb * 32 + r32;
            const float4 *tp = reinterpret_cast<const float4 *>(a.t + ((uint32_t)((tok < a.b ? tok : a.b - 1) * a.r) + rk));
            tb[cb] = live ? f32x8_to_h8(tp[0], tp[1]) : v8h{};
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) y[rb][cb] = mfma_f16_32(la[rb], tb[cb], y[rb][cb]);
    }
}

template <int S, int GM, bool STORE_ACC, bool T16>
__global__ __launch_bounds__(256, S == 2 ? 4 : 3) void dual_linear_pf32(DualArgs a, int tiles_n, int tiles_m) {
    constexpr int BN = 128, BM = 128, WN = 2, WM = 2, RB = 64, NT = 256;
    constexpr int CPR = RB / 16, BLK = 16 * RB, ROWS = BN + BM, SLOT = ROWS * RB, DPT = ROWS * CPR / NT;
    static_assert(!(STORE_ACC && T16) && (S - 2) * DPT < 64, "one epilogue; loads in flight fit vmcnt");
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wn = wave % WN, wm = wave / WN;

    // block -> tile, as in dual_linear_pf
    const int ntiles = tiles_n * tiles_m;
    const int o = (int)xcd_order(blockIdx.x, ntiles);
    const int gsz = GM * tiles_n;
    const int grp = o / gsz, within = o % gsz;
    const int gm_here = (tiles_m - grp * GM) < GM ? (tiles_m - grp * GM) : GM;
    const int tm = __builtin_amdgcn_readfirstlane(grp * GM + within % gm_here);
    const int tn = __builtin_amdgcn_readfirstlane(within / gm_here);
    const int64_t ch0 = (int64_t)tn * BN, tok0 = (int64_t)tm * BM;
    const int64_t kb = a.m / 2;
    const int nst = (int)(a.m / (2 * RB));

    // DMA sources, as in dual_linear_pf (64-byte rows, 4-bit token rows)
    const uint8_t *wbase = a.qw + ch0 * kb, *xbase = a.qx + tok0 * kb;
    uint32_t off[DPT];
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
        const int q = j * NT + tid;
        // odd 1 KB blocks (the second 16 rows of each 32-row block) have bit 0 of the
        // chunk position flipped as well (see the reads below)
        const int line = (q % (16 * CPR)) / 8, logical = (q % 8) ^ line ^ ((q / (16 * CPR)) & 1);
        const int row = (q / (16 * CPR)) * 16 + 2 * line + logical / 4;
        const int chunk = logical % 4;
        int64_t rel;
        if (row < BN) {
            const int64_t ch = ch0 + row;
            rel = (ch < a.n ? ch : a.n - 1) - ch0;
        } else {
            const int64_t tok = tok0 + (row - BN);
            rel = (tok < a.b ? tok : a.b - 1) - tok0;
        }
        off[j] = (uint32_t)(row < BN ? qw_offset(rel, chunk * 16, a.m) : rel * kb + chunk * 16);
    }
    constexpr int SCL = STORE_ACC ? 0 : 4 * (BN + BM);
    __shared__ __attribute__((aligned(16))) uint8_t ring[S * SLOT + SCL];
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(wbase), 0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(xbase), 0, 0x7fffffff, 0x00020000);
    auto issue = [&](int st, auto slot) {
        if constexpr (T16) {
            if (st >= nst) {  // past the last stage: the first low-rank steps, into the slots it frees
                pf_lr_issue<BN, BM, NT, SLOT, 0, true>(a, ch0, tok0, ring, decltype(slot)::value, st - nst, tid);
                return;
            }
        }
        uint8_t *dst = ring + decltype(slot)::value * SLOT;
#pragma unroll
        for (int j = 0; j < DPT; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds((j * NT) / CPR < BN ? rw : rx,
                                                     (__attribute__((address_space(3))) void *)(dst + (j * NT + wave_u * kWave) * 16),
                                                     16, (int)off[j], st * RB * ((j * NT) / CPR < BN ? kPanelRows : 1), 0, 0);
    };

    v16i acc[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0;

    // this lane's operand addresses for the stage halves h: row r32 of the wave's first
    // 32-row block of weights (rda) and of tokens (rdb), chunk 2 h + kh; the second block
    // is 2 KB further
    const int r32 = lane & 31, kh = lane >> 5, li = r32 & 15;
    uint32_t rda[2], rdb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t lane_off = (li / 2) * 128 + ((4 * (li % 2) + 2 * h + kh) ^ (li / 2) ^ (r32 / 16)) * 16 + (r32 / 16) * BLK;
        rda[h] = lds_offset(ring) + lane_off + (wn * (BN / WN) / 16) * BLK;
        rdb[h] = lds_offset(ring) + lane_off + ((BN + wm * (BM / WM)) / 16) * BLK;
    }

    if constexpr (SCL > 0) {
        // s_W of the tile's channels and s_X of its tokens past the ring (one 4-byte load a
        // thread; rows past n or b clamped), for the epilogue
        const bool wv = wave_u < BN / kWave;
        const int64_t idx = wv ? (ch0 + tid < a.n ? ch0 + tid : a.n - 1) : (tok0 + tid - BN < a.b ? tok0 + tid - BN : a.b - 1);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(wv ? a.sw : a.sx), 0,
                                                                            (int)((wv ? a.n : a.b) * 4), 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(ring + S * SLOT + wave_u * kWave * 4),
                                                 4, (int)(idx * 4), 0, 0, 0);
    }
    // the main loop of dual_linear_pf: step st issues stage st into slot st % S and
    // consumes stage st - (S - 1); every step issues, so each wait counts the same loads
    for (int s0 = 0; s0 < nst + S - 1; s0 += S) {
        static_for(std::make_integer_sequence<int, S>{}, [&](auto u) {
            const int st = s0 + u, c = st - (S - 1);
            if (c >= nst) return;
            if (c >= 0) {
                wait_vmcnt<(S - 2) * DPT>();
                stage_barrier();  // stage c landed for every thread; stage c - 1 consumed by every wave
            }
            issue(T16 || st < nst ? st : nst - 1, u);
            if (c < 0) return;
            constexpr int OFF = ((u + 1) % S) * SLOT;  // slot of stage c
            v4i raw[8];
            lds_read_2x4<OFF, 2 * BLK>(rda[0], rda[1], rdb[0], rdb[1], raw);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                v4i alo[2], ahi[2], blo[2], bhi[2];
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                    unpack16(raw[2 * h + f], alo[f], ahi[f]);
                    unpack16(raw[4 + 2 * h + f], blo[f], bhi[f]);
                }
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb) {
                        acc[rb][cb] = mfma_i8_32(alo[rb], blo[cb], acc[rb][cb]);
                        acc[rb][cb] = mfma_i8_32(ahi[rb], bhi[cb], acc[rb][cb]);
                    }
            }
        });
    }

    // epilogue: lane coordinates recomputed from the thread index (see dual_linear_pf)
    int te = tid;
    asm volatile("" : "+v"(te));
    const int r32e = te & 31, khe = (te >> 5) & 1;
    const int64_t chw = ch0 + (wave_u % WN) * (BN / WN), tkw = tok0 + (wave_u / WN) * (BM / WM);
    if constexpr (STORE_ACC) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t ch = chw + rb * 32 + 8 * q + 4 * khe;
                    const int64_t tok = tkw + cb * 32 + r32e;
                    if (ch < a.n && tok < a.b)
                        *reinterpret_cast<v4i *>(a.acc + tok * a.n + ch) =
                            v4i{acc[rb][cb][4 * q] >> 8, acc[rb][cb][4 * q + 1] >> 8, acc[rb][cb][4 * q + 2] >> 8,
                                acc[rb][cb][4 * q + 3] >> 8};
                }
    } else {
        // dequantize with the scales from LDS (the first wait of the main loop covered
        // them), one 32-channel block at a time
        const uint32_t sw_at = lds_offset(ring) + (uint32_t)((chw - ch0) + 4 * khe) * 4;
        const uint32_t sx_at = lds_offset(ring) + (uint32_t)(BN + (tkw - tok0) + r32e) * 4;
        v16f y[2][2];
        static_for(std::make_integer_sequence<int, 2>{}, [&](auto rb) {
            v4f swr[4];
            float sxr[2];
            lds_read_scales32<S * SLOT + 128 * decltype(rb)::value, S * SLOT>(sw_at, sx_at, swr, sxr);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    y[rb][cb][v] = sxr[cb] * (swr[v / 4][v % 4] * (float)(acc[rb][cb][v] >> 8));
                // one block at a time: the scheduler would otherwise start every block at
                // once and run out of registers
                __builtin_amdgcn_sched_barrier(0);
            }
        });
        if constexpr (T16) {
            // the ring's read addresses again, from the recomputed lane coordinates
            const int lie = r32e & 15;
            uint32_t ea[2], eb[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t lane_off =
                    (lie / 2) * 128 + ((4 * (lie % 2) + 2 * h + khe) ^ (lie / 2) ^ (r32e / 16)) * 16 + (r32e / 16) * BLK;
                ea[h] = lds_offset(ring) + lane_off + (uint32_t)((chw - ch0) / 16) * BLK;
                eb[h] = lds_offset(ring) + lane_off + (uint32_t)((BN + (tkw - tok0)) / 16) * BLK;
            }
            pf32_lowrank_ring<S, SLOT, DPT>(a, y, ch0, tok0, ea, eb, khe, ring, te, nst);
        } else {
            pf32_lowrank_regs(a, y, chw, tkw, r32e, khe);
        }
        pf32_store(a, y, chw, tkw, r32e, khe);
    }
}

template <int S, int GM, bool STORE_ACC, bool T16>
static hipError_t launch_pf32_kernel(const DualArgs &a, hipStream_t stream) {
    const int64_t tiles_n = (a.n + 127) / 128, tiles_m = (a.b + 127) / 128;
    hipLaunchKernelGGL((dual_linear_pf32<S, GM, STORE_ACC, T16>), dim3((unsigned)(tiles_n * tiles_m)), dim3(256), 0, stream,
                       a, (int)tiles_n, (int)tiles_m);
    return hipGetLastError();
}

template <int BN, int BM, int WN, int WM, int S, int GM, int RB, bool STORE_ACC, bool LR4 = false, bool GRP = false,
          bool A8 = false, bool T16 = false>
static hipError_t launch_pf_kernel(const DualArgs &a, hipStream_t stream) {
    const int64_t tiles_n = (a.n + BN - 1) / BN, tiles_m = (a.b + BM - 1) / BM;
    hipLaunchKernelGGL((dual_linear_pf<BN, BM, WN, WM, S, GM, RB, STORE_ACC, LR4, GRP, A8, T16>), dim3((unsigned)(tiles_n * tiles_m)),
                       dim3(WN * WM * 64), 0, stream, a, (int)tiles_n, (int)tiles_m);
    return hipGetLastError();
}

// Many tokens: 128 x 128 tiles, XCD groups of 8 token tiles (the fastest exact variant
// measured on MI355X for the gate/up and down shapes; 4 and 16 were no faster on the 32 x 32
// kernel). The per-token 4-bit layer runs dual_linear_pf32: a two-stage ring at four CTAs
// per compute unit once the grid has at least 4 x 256 tiles, and a three-stage ring at
// three CTAs below that, where the fourth slots would stay partly empty and the deeper ring
// hides more latency (measured on the 16 x 16 kernel: 3-5% faster above, 1-5% slower below,
// on 13 prefill shapes; three stages measured 2.6%, 5.6% and 5.9% slower on the 70B
// gate/up, down and gate/up shapes with the 32 x 32 kernel). The exact accumulator export
// follows the same rule, so it checks the main loop that the same shape runs for Y.
static hipError_t launch_pf(const DualArgs &a, hipStream_t stream) {
    constexpr int BN = 128, BM = 128, WN = 2, WM = 2, GM = 8, RB = 64;
    const int64_t tiles = ((a.n + BN - 1) / BN) * ((a.b + BM - 1) / BM);
    const bool four = tiles >= 4 * 256;
    if (a.a8)  // W4A8: two stages (see dual_linear_pf)
        return a.acc ? launch_pf_kernel<BN, BM, WN, WM, 2, GM, RB, true, false, false, true>(a, stream)
                     : launch_pf_kernel<BN, BM, WN, WM, 2, GM, RB, false, false, false, true>(a, stream);
    if (a.acc)
        return four ? launch_pf32_kernel<2, GM, true, false>(a, stream) : launch_pf32_kernel<3, GM, true, false>(a, stream);
    if (a.group)
        return a.t16 ? launch_pf_kernel<BN, BM, WN, WM, 3, GM, RB, false, false, true, false, true>(a, stream)
                     : launch_pf_kernel<BN, BM, WN, WM, 3, GM, RB, false, false, true>(a, stream);
    if (a.lr4) return launch_pf_kernel<BN, BM, WN, WM, 3, GM, RB, false, true>(a, stream);
    if (a.t16)  // T as fp16: the low-rank operands go through the ring (pf32_lowrank_ring)
        return four ? launch_pf32_kernel<2, GM, false, true>(a, stream) : launch_pf32_kernel<3, GM, false, true>(a, stream);
    return four ? launch_pf32_kernel<2, GM, false, false>(a, stream) : launch_pf32_kernel<3, GM, false, false>(a, stream);
}

hipError_t launch_dual_linear(const DualArgs &a, hipStream_t stream) {
    if (a.b == 0 || a.n == 0) return hipSuccess;
    if (a.tks > 1 && (a.acc || a.lr4 || a.tks > dual_max_t_slices(a.b, a.m, a.n, a.r))) return hipErrorInvalidValue;
    int fn, fm;
    if (!decode_shape(a.b, a.m, a.n, fn, fm)) return launch_pf(a, stream);
    if (a.group && fn > 4) fn = 4;  // group-wise runs four waves a CTA (above): keep twice the CTAs
    // pieces in flight per operand row (U) and waves per CTA (NW), measured per tile
    if (fm == 1) return fn == 1 ? launch_decode<1, 1, 4, 8>(a, stream) : launch_decode<2, 1, 8, 4>(a, stream);
    if (fm == 2) {
        if (fn == 1) return launch_decode<1, 2, 4, 8>(a, stream);
        if (fn == 2) return launch_decode<2, 2, 4, 4>(a, stream);
        return fn == 4 ? launch_decode<4, 2, 1, 8>(a, stream) : launch_decode<8, 2, 1, 8>(a, stream);
    }
    if (fn == 1) return launch_decode<1, 4, 2, 8>(a, stream);
    return fn == 2 ? launch_decode<2, 4, 2, 8>(a, stream) : launch_decode<4, 4, 1, 8>(a, stream);
}

}  // namespace twq
