// act_quant.hip -- activation side of the fused W4A4 + low-rank linear (gfx950).
//
// One launch does two independent jobs that both only read X:
//  * per-token quantization (TwinQuant page 1, section 2, eq. (1)): a CTA of 256
//    threads computes amax over a token row with a wave reduction, s_X =
//    amax / 7, and the packed 4-bit codes of its slice of the row (few tokens:
//    several CTAs per row); rows up to 16384 elements stay in registers between
//    the two passes, longer rows are re-read from cache;
//  * the first low-rank product T = X L1 of eq. (3) on fp16 matrix cores with
//    fp32 accumulation, cut into K slices so the read of X and L1 is spread over
//    many compute units (one unit streams only tens of GB/s from HBM). A second,
//    elementwise kernel adds the slices' partial sums in slice order. Every sum
//    has a fixed order, so T is bitwise reproducible.
// The T CTAs take the low block indices so the longer jobs start first.
#include "twq_device.h"
#include "twq_kernels.h"

namespace twq {

constexpr int kActThreads = 256;

struct ActDev {
    int mode;        // 0: tiles of 128 token rows x all ranks; 1: all tokens x 16 ranks x a K slice
    int row_tile, ks, row_tiles, n_t_ctas;
    int fm;          // mode 1: token tiles of 16 (b <= 128)
    int nsl;         // CTAs per token row for the quantizer
    int jq;          // chunks of a row per thread (0: rows past 16384 elements)
};

// Eight 8-bit codes (q_max = 127) of one 16-byte chunk of fp16, one byte each in order.
__device__ __forceinline__ uint2 quant8_a8(const uint4 c, float s, float inv) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (uint32_t)quant_code8_fast(half_bits_to_float(w[e] & 0xFFFFu), s, inv) & 0xFFu;
        const uint32_t hi = (uint32_t)quant_code8_fast(half_bits_to_float(w[e] >> 16), s, inv) & 0xFFu;
        out[e / 2] |= (lo | (hi << 8)) << (16 * (e % 2));
    }
    return make_uint2(out[0], out[1]);
}

// The chunks of a row that thread tid holds: 16-byte chunk c = tid + 256 j of the row
// (8 fp16), j < J, zero past the row's nch chunks. J is a compile-time count (a loop
// of guarded loads sized at run time measured 0.6 us slower on a 4096-element row).
template <int J>
__device__ __forceinline__ void load_row(const ActArgs &a, int64_t i, uint4 (&v)[J]) {
    const uint4 *xr = reinterpret_cast<const uint4 *>(a.x + i * a.m);
    const int64_t nch = a.m / 8;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int64_t c = threadIdx.x + (int64_t)j * kActThreads;
        v[j] = c < nch ? xr[c] : make_uint4(0, 0, 0, 0);
    }
}

template <int J>
__device__ __forceinline__ uint32_t row_absmax_bits(const uint4 (&v)[J]) {
    uint32_t mx = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) mx = absmax8_bits(v[j], mx);
    return wave_max_u32(mx);
}

// s_X of eq. (1) from the row's amax: the correctly rounded binary32 division
__device__ __forceinline__ float row_scale(float amax, bool a8) { return amax / (a8 ? kQMax8 : kQMax); }

// Chunk c (held in registers) of row i into its codes
template <bool A8>
__device__ __forceinline__ void put_chunk(const ActArgs &a, int64_t i, int64_t c, const uint4 chunk, float amax,
                                          float s, float inv) {
    if constexpr (A8)
        reinterpret_cast<uint2 *>(a.qx + i * a.m)[c] = amax == 0.0f ? make_uint2(0u, 0u) : quant8_a8(chunk, s, inv);
    else
        reinterpret_cast<uint32_t *>(a.qx + i * (a.m / 2))[c] = amax == 0.0f ? 0u : quant8(chunk, s, inv);
}

// Few tokens: slice sl (of nsl) of token row i, by one CTA of 256 threads. amax is
// taken over the whole row (every slice reads it; only the first reads it from HBM),
// codes are written for the slice's chunks [c_lo, c_hi) only, so the divisions of a
// short row are spread over several compute units. Where the slice is 64 or 128 chunks
// it is staged in LDS (stage: 2 KB) beside the amax reduction, so that all 256 threads
// take 2 or 4 codes each, instead of a quarter or a half of the threads taking 8
// (measured on MI355X: the packing ran 0.5 us on one wave). J: chunks a thread holds,
// J * 256 >= m / 8. A8: 8-bit codes (q_max = 127), one byte each.
template <bool A8, int J>
__device__ void quantize_slice(const ActArgs &a, int64_t i, int sl, int nsl, uint32_t *red, uint4 *stage) {
    const int tid = threadIdx.x;
    const int64_t nch = a.m / 8;
    const int64_t c_lo = nch * sl / nsl, c_hi = nch * (sl + 1) / nsl, nc = c_hi - c_lo;
    uint4 v[J];
    load_row<J>(a, i, v);
    const uint32_t mx = row_absmax_bits<J>(v);
    if (tid % kWave == 0) red[tid / kWave] = mx;
    const bool spread = nc == 64 || nc == 128;
    if (spread) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int64_t c = tid + (int64_t)j * kActThreads;
            if (c >= c_lo && c < c_hi) stage[c - c_lo] = v[j];
        }
    }
    __syncthreads();
    uint32_t m4 = red[0];
#pragma unroll
    for (int w = 1; w < kActThreads / kWave; ++w) m4 = m4 > red[w] ? m4 : red[w];
    const float amax = half_bits_to_float(m4);
    const float s = row_scale(amax, A8);
    const float inv = 1.0f / s;  // only used when amax > 0
    if (tid == 0 && sl == 0) a.sx[i] = s;
    if (spread) {
        // thread tid: elements tid K .. tid K + K - 1 of the slice, K = nc / 32
        const uint16_t *st = reinterpret_cast<const uint16_t *>(stage);
        int q[4] = {0, 0, 0, 0};
        const int K = (int)(nc / 32);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (k < K && amax != 0.0f) {
                const float x = half_bits_to_float(st[tid * K + k]);
                q[k] = A8 ? quant_code8_fast(x, s, inv) : quant_code_fast(x, s, inv);
            }
        if constexpr (A8) {
            uint8_t *dst = a.qx + i * a.m + c_lo * 8 + (int64_t)tid * K;
            const uint32_t b01 = (uint32_t(q[0]) & 0xFFu) | ((uint32_t(q[1]) & 0xFFu) << 8);
            if (K == 2)
                *reinterpret_cast<uint16_t *>(dst) = (uint16_t)b01;
            else
                *reinterpret_cast<uint32_t *>(dst) = b01 | ((uint32_t(q[2]) & 0xFFu) << 16) | ((uint32_t(q[3]) & 0xFFu) << 24);
        } else {
            uint8_t *dst = a.qx + i * (a.m / 2) + c_lo * 4 + (int64_t)tid * (K / 2);
            const uint32_t b0 = (uint32_t(q[0]) & 0xFu) | ((uint32_t(q[1]) & 0xFu) << 4);
            if (K == 2)
                *dst = (uint8_t)b0;
            else
                *reinterpret_cast<uint16_t *>(dst) = (uint16_t)(b0 | (((uint32_t(q[2]) & 0xFu) | ((uint32_t(q[3]) & 0xFu) << 4)) << 8));
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int64_t c = tid + (int64_t)j * kActThreads;
        if (c >= c_lo && c < c_hi) put_chunk<A8>(a, i, c, v[j], amax, s, inv);
    }
}

// Rows longer than 256 * 8 chunks (m > 16384): amax in one pass over the row, the
// codes of slice sl (of nsl) in a second, re-read from cache; rows q0, q0 + nq, ...
// (the launch gives every CTA one row: nq = b).
template <bool A8>
__device__ void quantize_long_rows(const ActArgs &a, int64_t q0, int64_t nq, int sl, int nsl, uint32_t *red) {
    const int tid = threadIdx.x;
    const int64_t nch = a.m / 8;
    const int64_t c_lo = nch * sl / nsl, c_hi = nch * (sl + 1) / nsl;
    for (int64_t i = q0; i < a.b; i += nq) {
        const uint4 *xr = reinterpret_cast<const uint4 *>(a.x + i * a.m);
        uint32_t mx = 0;
        for (int64_t c = tid; c < nch; c += kActThreads) mx = absmax8_bits(xr[c], mx);
        mx = wave_max_u32(mx);
        if (tid % kWave == 0) red[tid / kWave] = mx;
        __syncthreads();
        uint32_t m4 = red[0];
#pragma unroll
        for (int w = 1; w < kActThreads / kWave; ++w) m4 = m4 > red[w] ? m4 : red[w];
        __syncthreads();  // every wave has read red before the next row writes it
        const float amax = half_bits_to_float(m4);
        const float s = row_scale(amax, A8);
        const float inv = 1.0f / s;
        if (tid == 0 && sl == 0) a.sx[i] = s;
        for (int64_t c = c_lo + tid; c < c_hi; c += kActThreads) put_chunk<A8>(a, i, c, xr[c], amax, s, inv);
    }
}

// Group-wise scales (groups of kGroup = 128 along K, TwinQuant page 1, section 5.1):
// slice sl (of nsl) of one token row, in whole groups. Each thread takes one 8-element
// chunk at a time; a group is 16 chunks on 16 consecutive lanes, so its amax is a
// 16-lane reduction, and its scale goes to sx[group][row] (group-major).
__device__ void quantize_row_grouped(const ActArgs &a, int64_t i, int sl, int nsl) {
    static_assert(kGroup == 128, "a group is 16 chunks of 8");
    const int64_t ng = a.m / kGroup;
    const int64_t c_lo = 16 * (ng * sl / nsl), c_hi = 16 * (ng * (sl + 1) / nsl);
    const uint4 *xr = reinterpret_cast<const uint4 *>(a.x + i * a.m);
    uint32_t *qr = reinterpret_cast<uint32_t *>(a.qx + i * (a.m / 2));
    for (int64_t c = c_lo + threadIdx.x; c < c_hi; c += kActThreads) {  // whole 16-lane groups enter together
        const uint4 v = xr[c];
        uint32_t mx = absmax8_bits(v, 0u);
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) {
            const uint32_t o = (uint32_t)__shfl_xor((int)mx, off, kWave);
            mx = mx > o ? mx : o;
        }
        const float amax = half_bits_to_float(mx);
        const float s = amax / kQMax;  // correctly rounded binary32 division
        if ((threadIdx.x & 15) == 0) a.sx[(c / 16) * a.b + i] = s;
        qr[c] = amax == 0.0f ? 0u : quant8(v, s, 1.0f / s);
    }
}

// T tile for many tokens: tokens [128 tm, 128 tm + 128) x all r = 16 NR ranks over K
// slice ks, in steps of 32 (64 bytes of fp16 per row). The step's 128 X rows and its
// L1^T rows (NR blocks of 16, padded to a multiple of four blocks with clamped rows)
// go through an LDS ring filled by direct-to-LDS buffer loads, laid out as the prefill
// main loop's ring: 16-row blocks, rows 2s and 2s + 1 sharing 128-byte line s with the
// 16-byte chunk index XORed by s, which makes the loads coalesce and the operand reads
// conflict-free. X rows are read from HBM once and L1 rows once per CTA. Wave w owns
// tokens [32 w, 32 w + 32) x all ranks: A = L1^T block (16 ranks), B = X block (16
// tokens), so lane (li, g) ends with ranks 4g..4g+3 of token li. The ring has three
// slots up to 64 ranks (37 KB) and two above (32-56 KB instead of 49-74 KB): every
// CTA of the launch holds the ring, the quantizer CTAs included, and the smaller ring
// leaves them more slots a compute unit. Measured on MI355X at b = m = 8192, r = 128:
// the T tiles alone take 52 us instead of 33, but the whole launch 74 instead of 79,
// and the benchmark call 1369-1377 us instead of 1380-1384.
template <int NR>
__device__ void t_tiles(const ActArgs &a, const ActDev &p, int tb, uint8_t *ring) {
    constexpr int BM = 128, NRP = (NR + 3) / 4 * 4, ROWS = BM + 16 * NRP;
    constexpr int S = NR > 4 ? 2 : 3, BLK = 1024, STAGE = ROWS * 64, DPT = ROWS * 4 / kActThreads;
    static_assert(ROWS * 4 % kActThreads == 0 && BM * 4 % kActThreads == 0, "DMA groups");
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int li = lane & 15, g = lane >> 4;
    const int tm = tb / p.ks, ks = tb % p.ks;
    const int64_t kslice = a.m / p.ks, kbeg = ks * kslice;
    const int nst = (int)(kslice / 32);
    const int64_t tok0 = (int64_t)tm * BM;

    // slot q of a stage: position q % 8 of line (q % 64) / 8 of block q / 64
    const uint8_t *xb = reinterpret_cast<const uint8_t *>(a.x + tok0 * a.m + kbeg);
    const uint8_t *lb = reinterpret_cast<const uint8_t *>(a.l1t + kbeg);
    uint32_t off[DPT];
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
        const int q = j * kActThreads + tid;
        const int line = (q % 64) / 8, logical = (q % 8) ^ line;
        const int row = (q / 64) * 16 + 2 * line + logical / 4, chunk = logical % 4;
        int64_t rel;
        if (row < BM) {
            const int64_t tok = tok0 + row;
            rel = (tok < a.b ? tok : a.b - 1) - tok0;
        } else {
            const int rank = row - BM;
            rel = rank < a.r ? rank : a.r - 1;
        }
        off[j] = (uint32_t)(rel * a.m * 2 + chunk * 16);
    }
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(xb), 0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(lb), 0, 0x7fffffff, 0x00020000);
    auto issue = [&](int st, auto slot) {
        uint8_t *dst = ring + decltype(slot)::value * STAGE;
#pragma unroll
        for (int j = 0; j < DPT; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds((j * kActThreads) / 4 < BM ? rx : rl,
                                                     (__attribute__((address_space(3))) void *)(dst + (j * kActThreads + wave * kWave) * 16),
                                                     16, (int)off[j], st * 64, 0, 0);
    };

    v4f acc[NR][2];
#pragma unroll
    for (int tt = 0; tt < NR; ++tt) acc[tt][0] = acc[tt][1] = v4f{0.f, 0.f, 0.f, 0.f};
    // row li, chunk g of a block: line li / 2, logical position 4 (li % 2) + g
    const uint32_t lane_off = lds_offset(ring) + (li / 2) * 128 + ((4 * (li % 2) + g) ^ (li / 2)) * 16;
    const uint32_t rdx = lane_off + 2 * wave * BLK, rdl = lane_off + (BM / 16) * BLK;

    for (int s0 = 0; s0 < nst + S - 1; s0 += S) {
        static_for(std::make_integer_sequence<int, S>{}, [&](auto u) {
            const int st = s0 + u, c = st - (S - 1);
            if (c >= nst) return;
            if (c >= 0) {
                wait_vmcnt<(S - 2) * DPT>();
                stage_barrier();  // stage c landed for every thread; stage c - 1 consumed by every wave
            }
            issue(st < nst ? st : nst - 1, u);
            if (c < 0) return;
            constexpr int OFF = ((u + 1) % S) * STAGE;  // slot of stage c
            v4i xr[2];
            lds_read_2<OFF, BLK>(rdx, xr);
            static_for(std::make_integer_sequence<int, NRP / 4>{}, [&](auto q4) {
                constexpr int t0 = 4 * decltype(q4)::value;
                v4i lr[4];
                lds_read_4<OFF + t0 * BLK, BLK>(rdl, lr);
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (t0 + k < NR) {
#pragma unroll
                        for (int f = 0; f < 2; ++f)
                            acc[t0 + k][f] = mfma_f16(__builtin_bit_cast(v8h, lr[k]), __builtin_bit_cast(v8h, xr[f]), acc[t0 + k][f]);
                    }
            });
        });
    }

#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const int64_t row = tok0 + 32 * wave + 16 * f + li;
        float *dst = p.ks == 1 ? a.t + row * a.r : a.partials + ((int64_t)ks * p.row_tiles * BM + row) * a.r;
        if (p.ks > 1 || row < a.b) {
#pragma unroll
            for (int tt = 0; tt < NR; ++tt) *reinterpret_cast<v4f *>(dst + tt * 16 + 4 * g) = acc[tt][f];
        }
    }
}

// T partial for few tokens: all b tokens (FM tiles of 16) x ranks [16 rt, 16 rt + 16)
// over K slice ks, written to partials[ks]; the four waves split the slice and are
// added through LDS in wave order. A = L1^T rows (16 ranks), B = X rows (16 tokens):
// lane (li, g) ends with ranks 4g..4g+3 of token li of each token tile.
template <int FM>
__device__ void t_slices(const ActArgs &a, const ActDev &p, int tb, float *lds) {
    constexpr int U = FM <= 2 ? 4 : 2;
    const int rt = tb % p.row_tiles, ks = tb / p.row_tiles;  // row_tiles = r / 16 rank tiles
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int li = lane & 15, g = lane >> 4;
    const int64_t nsteps = a.m / 32;
    const int64_t s_lo = nsteps * ks / p.ks, s_hi = nsteps * (ks + 1) / p.ks;
    const int64_t sb = s_lo + (s_hi - s_lo) * wave / 4, se = s_lo + (s_hi - s_lo) * (wave + 1) / 4;
    const uint16_t *lp = a.l1t + ((int64_t)rt * 16 + li) * a.m + g * 8;
    const uint16_t *xp[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int64_t tok = fm * 16 + li;
        xp[fm] = a.x + (tok < a.b ? tok : a.b - 1) * a.m + g * 8;  // rows past b: never stored
    }
    v4f acc[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) acc[fm] = v4f{0.f, 0.f, 0.f, 0.f};
    int64_t st = sb;
    for (; st + U <= se; st += U) {
        v8h la[U], xb[U][FM];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            la[u] = load_h8(lp + (st + u) * 32);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) xb[u][fm] = load_h8(xp[fm] + (st + u) * 32);
        }
        __builtin_amdgcn_sched_barrier(0);  // every load of the batch in flight before the first use
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) acc[fm] = mfma_f16(la[u], xb[u][fm], acc[fm]);
    }
    for (; st < se; ++st) {
        const v8h la = load_h8(lp + st * 32);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) acc[fm] = mfma_f16(la, load_h8(xp[fm] + st * 32), acc[fm]);
    }
    if (wave > 0) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            *reinterpret_cast<v4f *>(lds + (((wave - 1) * FM + fm) * kWave + lane) * 4) = acc[fm];
    }
    __syncthreads();
    if (wave != 0) return;
    for (int w = 1; w < 4; ++w)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) acc[fm] += *reinterpret_cast<const v4f *>(lds + (((w - 1) * FM + fm) * kWave + lane) * 4);
    const int64_t rank = (int64_t)rt * 16 + 4 * g;
    const int64_t tpad = (int64_t)FM * 16;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        float *dst = p.ks == 1 ? a.t + (fm * 16 + li) * (int64_t)a.r + rank
                               : a.partials + (ks * tpad + fm * 16 + li) * a.r + rank;
        if (p.ks > 1 || fm * 16 + li < a.b) *reinterpret_cast<v4f *>(dst) = acc[fm];
    }
}

// Quantizer CTA q: token row q / nsl, slice q % nsl (many tokens: nsl = 1). One CTA
// per row measured faster at prefill than a few CTAs per compute unit looping over
// rows in batches (b = m = 8192: 81 against 100-117 us for the whole launch, with 256
// to 2048 looping CTAs; likewise on the gate/up and down shapes).
template <bool A8>
__device__ void quantize_part(const ActArgs &a, const ActDev &p, int64_t q, uint32_t *red, float *lds) {
    const int64_t i = q / p.nsl;
    const int sl = (int)(q % p.nsl);
    uint4 *stage = reinterpret_cast<uint4 *>(lds);  // the T tiles' buffer: quantizer CTAs compute no T
    switch (p.jq) {
        case 1: quantize_slice<A8, 1>(a, i, sl, p.nsl, red, stage); return;
        case 2: quantize_slice<A8, 2>(a, i, sl, p.nsl, red, stage); return;
        case 4: quantize_slice<A8, 4>(a, i, sl, p.nsl, red, stage); return;
        case 8: quantize_slice<A8, 8>(a, i, sl, p.nsl, red, stage); return;
        default: quantize_long_rows<A8>(a, i, a.b, sl, p.nsl, red); return;
    }
}

// Many tokens (MODE 0): T partials by t_tiles<NT = r / 16>. Few tokens (MODE 1): T
// partials by t_slices<NT = FM>. The remaining CTAs quantize, nsl CTAs per token row.
template <int MODE, int NT>
__global__ __launch_bounds__(kActThreads) void act_kernel(ActArgs a, ActDev p) {
    // MODE 1: T's wave sums, or a quantizer CTA's staged slice (128 chunks)
    __shared__ __attribute__((aligned(16))) float lds[MODE == 1 ? (3 * NT * kWave * 4 > 512 ? 3 * NT * kWave * 4 : 512) : 512];
    // T tiles' ring: slots (3, or 2 above 64 ranks) x (128 token rows + the rank rows) x 64 bytes
    __shared__ __attribute__((aligned(16))) uint8_t ring[MODE == 0 ? (NT > 4 ? 2 : 3) * (128 + 16 * ((NT + 3) / 4 * 4)) * 64 : 16];
    __shared__ uint32_t red[kActThreads / kWave];
    const int64_t bid = blockIdx.x;
    if (bid < p.n_t_ctas) {
        if constexpr (MODE == 0)
            t_tiles<NT>(a, p, (int)bid, ring);
        else
            t_slices<NT>(a, p, (int)bid, lds);
    } else {
        const int64_t q = bid - p.n_t_ctas;
        if (a.group)
            quantize_row_grouped(a, q / p.nsl, (int)(q % p.nsl), p.nsl);
        else if (a.a8)
            quantize_part<true>(a, p, q, red, lds);
        else
            quantize_part<false>(a, p, q, red, lds);
    }
}

// T[row][c] = sum over slices s (in slice order) of partials[s][row][c]. The data is
// small and the kernel latency-bound, so every load of a thread is issued before any
// is added (KS_MAX slices in flight; loads past ks re-read slice 0 and are not added).
// t16: T is stored rounded to fp16 (nearest even, the rounding the fused epilogue
// applies to T) instead of in fp32.
template <int KS_MAX>
__global__ __launch_bounds__(256) void t_reduce_kernel(const float *partials, int64_t b, int64_t rows_pad,
                                                       int r, int ks, float *t, uint16_t *t16) {
    const int64_t i4 = (int64_t)blockIdx.x * 256 + threadIdx.x;  // float4 index into T
    const int64_t n4 = b * r / 4;
    if (i4 >= n4) return;
    const int64_t stride = rows_pad * r;
    const float *src = partials + i4 * 4;
    v4f v[KS_MAX];
#pragma unroll
    for (int u = 0; u < KS_MAX; ++u) v[u] = *reinterpret_cast<const v4f *>(src + (u < ks ? u : 0) * stride);
    v4f sum = v[0];
#pragma unroll
    for (int u = 1; u < KS_MAX; ++u)
        if (u < ks) sum += v[u];
    if (t16) {
        v4h h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = (_Float16)sum[e];
        *reinterpret_cast<v4h *>(t16 + i4 * 4) = h;
    } else {
        *reinterpret_cast<v4f *>(t + i4 * 4) = sum;
    }
}

template <int MODE, int NT>
static void launch_one(const ActArgs &a, const ActDev &p, int64_t grid, hipStream_t stream) {
    hipLaunchKernelGGL((act_kernel<MODE, NT>), dim3((unsigned)grid), dim3(kActThreads), 0, stream, a, p);
}

template <int MODE>
static bool launch_nt(int nt, const ActArgs &a, const ActDev &p, int64_t grid, hipStream_t s) {
    switch (nt) {
        case 0: case 1: launch_one<MODE, 1>(a, p, grid, s); return true;
        case 2: launch_one<MODE, 2>(a, p, grid, s); return true;
        case 3: launch_one<MODE, 3>(a, p, grid, s); return true;
        case 4: launch_one<MODE, 4>(a, p, grid, s); return true;
        case 5: launch_one<MODE, 5>(a, p, grid, s); return true;
        case 6: launch_one<MODE, 6>(a, p, grid, s); return true;
        case 7: launch_one<MODE, 7>(a, p, grid, s); return true;
        case 8: launch_one<MODE, 8>(a, p, grid, s); return true;
        default: break;
    }
    if constexpr (MODE == 0) {
        switch (nt) {
            case 9: launch_one<0, 9>(a, p, grid, s); return true;
            case 10: launch_one<0, 10>(a, p, grid, s); return true;
            case 11: launch_one<0, 11>(a, p, grid, s); return true;
            case 12: launch_one<0, 12>(a, p, grid, s); return true;
            case 13: launch_one<0, 13>(a, p, grid, s); return true;
            case 14: launch_one<0, 14>(a, p, grid, s); return true;
            case 15: launch_one<0, 15>(a, p, grid, s); return true;
            case 16: launch_one<0, 16>(a, p, grid, s); return true;
            default: break;
        }
    }
    return false;
}

hipError_t launch_act(const ActArgs &a, const ActPlan &pl, hipStream_t stream) {
    if (a.b == 0) return hipSuccess;
    ActDev p{};
    p.mode = pl.mode;
    p.fm = pl.fm;
    p.row_tile = pl.row_tile;
    p.ks = pl.ks;
    p.row_tiles = pl.row_tiles;
    p.nsl = pl.nsl;
    p.jq = pl.jq;
    p.n_t_ctas = a.r > 0 ? pl.row_tiles * pl.ks : 0;
    const int64_t grid = p.n_t_ctas + a.b * pl.nsl;
    const bool ok = pl.mode == 0 ? launch_nt<0>(a.r / 16, a, p, grid, stream)
                                 : launch_nt<1>(a.r > 0 ? pl.fm : 1, a, p, grid, stream);
    if (!ok) return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.r == 0 || pl.ks == 1 || a.keep_partials) return e;
    const int64_t n4 = a.b * a.r / 4;
    const int64_t rows_pad = pl.mode == 0 ? (int64_t)pl.row_tiles * 128 : (int64_t)pl.fm * 16;
    const dim3 rgrid((unsigned)((n4 + 255) / 256));
    if (pl.ks <= 8)
        hipLaunchKernelGGL(t_reduce_kernel<8>, rgrid, dim3(256), 0, stream, a.partials, a.b, rows_pad, a.r, pl.ks, a.t, a.t16);
    else if (pl.ks <= 16)
        hipLaunchKernelGGL(t_reduce_kernel<16>, rgrid, dim3(256), 0, stream, a.partials, a.b, rows_pad, a.r, pl.ks, a.t, a.t16);
    else if (pl.ks <= 32)
        hipLaunchKernelGGL(t_reduce_kernel<32>, rgrid, dim3(256), 0, stream, a.partials, a.b, rows_pad, a.r, pl.ks, a.t, a.t16);
    else
        return hipErrorInvalidValue;  // plan_act keeps ks <= 32
    return hipGetLastError();
}

}  // namespace twq
