// Fused int8 pointwise 1x1 -> depthwise kxk: the QuantizedPwDw step of the
// yscv "ONNX CPU Kernels (Conv/MatMul) -- Runtime Map" page (section "Hot
// kernel paths", fused INT8 quant-domain chains).  Two symmetric
// QLinearConvs; the int8 tensor between them (the expansion) lives only in
// LDS.  Every integer sum and every requant is the one the two unfused
// QLinearConvs compute, so the output is bitwise theirs.
//
// Workgroup tile: one image, TH depthwise output rows, CE = 32 expanded
// channels, the full width.  The depthwise needs R = (TH-1)*stride +
// (kh-1)*dilation + 1 expanded rows (its halo rows are recomputed by the
// neighbouring tiles rather than exchanged).
//   1. Pointwise on the i8 matrix cores (v_mfma_i32_16x16x64_i8).  The input
//      rows, 64 channels at a time, are staged in LDS pixel-major (a thread
//      loads 4 channels x 4 pixels with 4-byte loads and transposes the block
//      with byte permutes), so a 16-pixel fragment of 64 channels is one
//      16-byte read per lane.  Pixels are the first operand, so a lane's
//      result is 4 consecutive pixels of one expanded channel.  The weights
//      (k-contiguous) come straight from global memory.
//   2. + pointwise bias, requant with the pointwise composite (zero point 0,
//      the pointwise descriptor's rounding and ReLU) into an int8 tile of the
//      expansion, [CE][R][EW] bytes; rows outside the image and the halo
//      columns hold 0, the intermediate's zero point: the depthwise padding
//      applies to the pointwise output.
//   3. Depthwise on the VALU: VO outputs per thread from a register window
//      of the tile's bytes, + depthwise bias, requant with the depthwise
//      composite, y_zp, rounding and ReLU, one packed 4-byte store where the
//      row allows it.
#include "device_common.h"

#include <type_traits>

namespace conv2d {

namespace {

constexpr int kT = 256;          // threads (4 waves)
constexpr int CE = 32;           // expanded channels per workgroup
constexpr int KC = 64;           // input channels per MFMA step
constexpr int XROW = KC + 16;    // LDS bytes per staged pixel (16 pad bytes spread the banks)
constexpr int NFMAX = 12;        // 16-pixel fragments per wave
constexpr int VO = 4;            // depthwise outputs per thread
constexpr int UMAX = 4;          // staged 4x4 blocks per thread and pass

struct QPDArgs {
    ConvArgs pw, dw;
    float comp_pw, comp_dw;
    int32_t y_zp;
    int32_t tile_h, tiles_h, ce_tiles;
    int32_t rows;        // expanded rows per tile
    int32_t off;         // LDS column of image column 0 in the expansion tile (>= dw pad_left, multiple of 4)
    int32_t ew;          // LDS row length of the expansion tile (multiple of 4)
    int32_t vec;         // input rows move as 4-byte words
    int32_t dwf_off;     // LDS byte offset of the depthwise filter words and biases
    uint32_t num_blocks;
    DivU32 dv_ce_tiles, dv_tiles_h;
    FastDiv div_w;       // pixel -> row
    DivU32 dv_uw;        // depthwise unit -> (channel, row) index: by the VO-column groups per row
    DivU32 dv_th, dv_th_last;   // (channel, row) index -> channel: by tile_h, by the last tile's rows
    DivU32 dv_pq;        // unit / 4 -> channel quad group (by the 4-pixel groups of the tile)
};

// Transpose a 4x4 byte block: in[c] holds pixels 0..3 of channel c; out[p]
// holds channels 0..3 of pixel p.
__device__ __forceinline__ void tr4x4(const uint32_t in[4], uint32_t out[4]) {
    const uint32_t t0 = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);
    const uint32_t t1 = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);
    const uint32_t t2 = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);
    const uint32_t t3 = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);
    out[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
    out[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
    out[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
    out[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// Requant of one sum with the rounding mode chosen at run time without a
// branch: rintf rounds ties to even and agrees with rounding half away from
// zero everywhere but at ties, which are the products whose fraction is
// exactly 1/2 (the difference to the truncated value is exact in f32).  The
// saturation (and ReLU) is the clamp of the rounded value to [lo, hi], the
// int8 range shifted by the zero point, as in requant().
__device__ __forceinline__ int rq_sel(int32_t acc, float comp, bool away, float lo, float hi, int zp) {
    float yf = __fmul_rn((float)acc, comp);
    asm volatile("" : "+v"(yf));   // the rounded f32 product decides ties (no fma into the rounding)
    const float t = truncf(yf);
    const float r = (away && fabsf(yf - t) == 0.5f) ? t + copysignf(1.0f, yf) : rintf(yf);
    return (int)__builtin_amdgcn_fmed3f(r, lo, hi) + zp;
}

// The same requant for ties to even: rint.
__device__ __forceinline__ int rq_even(int32_t acc, float comp, float lo, float hi, int zp) {
    float yf = __fmul_rn((float)acc, comp);
    asm volatile("" : "+v"(yf));
    return (int)__builtin_amdgcn_fmed3f(rintf(yf), lo, hi) + zp;
}

// KH/KW/SS: a fixed depthwise window (dilation 1, stride SS) the compiler
// unrolls, or 0 for a runtime window, stride and dilation.
// RNE: both stages round ties to even (the default), so the requant is one
// rint; otherwise each stage's mode is chosen at run time (rq_sel).
template <int NF, int KH, int KW, int SS, bool RNE>
__global__ __launch_bounds__(kT) void qfused_pw_dw_kernel(QPDArgs f) {
    extern __shared__ __align__(16) uint8_t lds[];
    const ConvArgs& P = f.pw;
    const ConvArgs& D = f.dw;
    constexpr bool FIXED = KH > 0;
    const int kh = FIXED ? KH : D.k_h, kw = FIXED ? KW : D.k_w;
    const int sh = FIXED ? SS : D.stride_h, sw = FIXED ? SS : D.stride_w;
    const int dh = FIXED ? 1 : D.dilation_h, dwl = FIXED ? 1 : D.dilation_w;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    uint32_t L = xcd_remap(blockIdx.x, f.num_blocks);
    uint32_t Q = divu(L, f.dv_ce_tiles);
    const int cet = L - Q * f.ce_tiles;
    L = Q; Q = divu(L, f.dv_tiles_h);
    const int tht = L - Q * f.tiles_h;
    const int n = Q;
    const int ce0 = cet * CE;
    const int ce_valid = min(CE, P.c_out - ce0);
    const int ho0 = tht * f.tile_h;
    const int ih_lo = ho0 * sh - D.pad_top;      // image row of expanded row 0
    const int W = P.w, H = P.h, K = P.c_in;
    const int R = f.rows;
    const int npix = R * W;
    const int nfrag = (npix + 15) / 16;
    const int64_t HW = (int64_t)H * W;
    const int8_t* __restrict__ xg = (const int8_t*)P.xptr + ((int64_t)n * P.in_total + P.in_off) * HW;
    const int8_t* __restrict__ wpw = (const int8_t*)P.wptr;

    // Pixel p of the staged rows lives at slot (p % 4) * ceil(npix / 4) + p / 4:
    // a thread's four pixels land in four quarters, and the words of
    // consecutive threads 80 bytes apart.
    uint8_t* xs = lds;   // [4 * ceil(npix / 4)][XROW]

    i32x4 acc[NF][2];
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[j][0] = acc[j][1] = i32x4{0, 0, 0, 0};

    // ---- 1. pointwise, 64 input channels per step ----
    // A step stages the channel quads that hold data (LDS bytes of channels
    // past K keep whatever they held: their weights are zero, so they add
    // exactly 0 to the integer sums).  Every thread requests all of its
    // loads, and the weight fragments, before it writes anything to LDS, so
    // one memory latency covers the whole step.
    const int pq_n = (npix + 3) >> 2;            // 4-pixel groups of the tile
    for (int c0 = 0; c0 < K; c0 += KC) {
        const int kq_n = min(KC, K - c0 + 3) >> 2;
        // Unit u: channel quad 4 * (u / (4 * pq_n)) + u % 4 of the 4-pixel
        // group (u / 4) % pq_n; four consecutive lanes take four channel
        // quads of one group, so a wave's LDS stores cover every bank.
        const int units = ((kq_n + 3) & ~3) * pq_n;
        // B fragments: channel ce0 + 16*cb + lane%16, k = c0 + 16*(lane/16) .. +15.
        i32x4 bw[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int ce = ce0 + 16 * cb + (lane & 15);
            const int k = c0 + 16 * (lane >> 4);
            uint32_t w4[4] = {0, 0, 0, 0};
            if (ce < P.c_out && k < K) {
                const int8_t* src = wpw + (int64_t)ce * K + k;
                if ((K & 15) == 0 && (((uintptr_t)wpw) & 15) == 0) {
                    const uint4 v = *(const uint4*)src;
                    w4[0] = v.x; w4[1] = v.y; w4[2] = v.z; w4[3] = v.w;
                } else {
                    for (int b = 0; b < 16; ++b)
                        if (k + b < K) w4[b >> 2] |= (uint32_t)(uint8_t)src[b] << (8 * (b & 3));
                }
            }
            bw[cb] = i32x4{(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]};
        }
        for (int u0 = 0; u0 < units; u0 += UMAX * kT) {
            uint32_t in[UMAX][4];
#pragma unroll
            for (int i = 0; i < UMAX; ++i) {
                const int u = u0 + tid + i * kT;
                const int hi = (int)divu((uint32_t)(u >> 2), f.dv_pq);
                const int cq = 4 * hi + (u & 3);
                const int p = 4 * ((u >> 2) - hi * pq_n);
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    const int ch = c0 + 4 * cq + cc;
                    uint32_t v = 0;
                    if (u < units && cq < kq_n && ch < K) {
                        const int8_t* src = xg + (int64_t)ch * HW;
                        if (f.vec) {
                            // W % 4 == 0: the 4 pixels share a row.
                            const int r = (int)fdiv((uint32_t)p, f.div_w);
                            const int ih = ih_lo + r;
                            if ((unsigned)ih < (unsigned)H) v = *(const uint32_t*)(src + (int64_t)ih * W + (p - r * W));
                        } else {
#pragma unroll
                            for (int b = 0; b < 4; ++b) {
                                const int pp = p + b;
                                const int r = (int)fdiv((uint32_t)pp, f.div_w);
                                const int ih = ih_lo + r;
                                if (pp < npix && (unsigned)ih < (unsigned)H)
                                    v |= (uint32_t)(uint8_t)src[(int64_t)ih * W + (pp - r * W)] << (8 * b);
                            }
                        }
                    }
                    in[i][cc] = v;
                }
            }
#pragma unroll
            for (int i = 0; i < UMAX; ++i) {
                const int u = u0 + tid + i * kT;
                const int hi = (int)divu((uint32_t)(u >> 2), f.dv_pq);
                const int cq = 4 * hi + (u & 3);
                if (u >= units || cq >= kq_n) continue;
                const int g4 = (u >> 2) - hi * pq_n;
                uint32_t outw[4];
                tr4x4(in[i], outw);
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    if (4 * g4 + b < npix) *(uint32_t*)&xs[(b * pq_n + g4) * XROW + 4 * cq] = outw[b];
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NF; ++j) {
            const int fj = wave + 4 * j;
            if (fj < nfrag) {
                int p = 16 * fj + (lane & 15);
                p = p < npix ? p : 0;   // pixels past the tile read pixel 0 (their results are never stored)
                const i32x4 a = *(const i32x4*)&xs[((p & 3) * pq_n + (p >> 2)) * XROW + 16 * (lane >> 4)];
                acc[j][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bw[0], acc[j][0], 0, 0, 0);
                acc[j][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bw[1], acc[j][1], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // ---- 2. pointwise bias + requant into the expansion tile (aliases xs) ----
    uint8_t* es = lds;   // [CE][R][EW]
    const int EW = f.ew, OFF = f.off;
    const int plane = R * EW;
    {
        const bool away_p = P.rounding == CONV_ROUND_HALF_AWAY;
        const float lo_p = P.act == CONV_ACT_RELU ? 0.0f : -128.0f;
        auto rq_p = [&](int32_t v) __attribute__((always_inline)) {
            return RNE ? rq_even(v, f.comp_pw, lo_p, 127.0f, 0) : rq_sel(v, f.comp_pw, away_p, lo_p, 127.0f, 0);
        };
        // Lane's results: pixels 16*fj + 4*(lane/16) + v (v = 0..3), channel 16*cb + lane%16.
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int ce = 16 * cb + (lane & 15);
            const bool cv = ce < ce_valid;
            const int32_t bb = (P.qbias && cv) ? P.qbias[ce0 + ce] : 0;
            uint8_t* ech = es + ce * plane;
#pragma unroll
            for (int j = 0; j < NF; ++j) {
                const int fj = wave + 4 * j;
                if (fj >= nfrag || !cv) continue;
                const int p0 = 16 * fj + 4 * (lane >> 4);
                if (f.vec && p0 < npix) {
                    // W % 4 == 0: the four pixels share a row; one aligned word.
                    const int r = (int)fdiv((uint32_t)p0, f.div_w);
                    uint32_t word = 0;
                    if ((unsigned)(ih_lo + r) < (unsigned)H) {
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            word |= (uint32_t)(uint8_t)rq_p(acc[j][cb][v] + bb)
                                    << (8 * v);
                    }
                    *(uint32_t*)&ech[r * EW + OFF + (p0 - r * W)] = word;
                } else {
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int p = p0 + v;
                        if (p >= npix) continue;
                        const int r = (int)fdiv((uint32_t)p, f.div_w);
                        const int8_t q = (unsigned)(ih_lo + r) < (unsigned)H
                                             ? (int8_t)rq_p(acc[j][cb][v] + bb)
                                             : (int8_t)0;
                        ech[r * EW + OFF + (p - r * W)] = (uint8_t)q;
                    }
                }
            }
        }
        // Halo columns of every row (one row per thread): the zero point.
        for (int rr = tid; rr < CE * R; rr += kT) {
            uint8_t* row = es + rr * EW;     // rows of all channels are consecutive: plane = R * EW
            for (int c = 0; c < OFF; c += 4) *(uint32_t*)(row + c) = 0u;
            for (int c = OFF + W; c < EW; ++c) row[c] = 0;
        }
    }
    // The depthwise filter rows (3x3: one packed word each) and biases of the
    // tile's channels, once per workgroup, behind the tile.
    uint32_t* dwf = (uint32_t*)(lds + f.dwf_off);      // [CE][3]
    int32_t* dwb = (int32_t*)(dwf + 3 * CE);           // [CE]
    if constexpr (FIXED && KH == 3 && KW == 3) {
        const int8_t* __restrict__ wd = (const int8_t*)D.wptr;
        for (int i = tid; i < CE * 3; i += kT) {
            const int ce = i / 3, r = i - 3 * (i / 3);
            uint32_t v = 0;
            if (ce < ce_valid) {
                const int8_t* w3 = wd + (int64_t)(ce0 + ce) * 9 + 3 * r;
                v = (uint32_t)(uint8_t)w3[0] | (uint32_t)(uint8_t)w3[1] << 8 | (uint32_t)(uint8_t)w3[2] << 16;
            }
            dwf[i] = v;
        }
    }
    for (int i = tid; i < CE; i += kT) dwb[i] = (D.qbias && i < ce_valid) ? D.qbias[ce0 + i] : 0;
    __syncthreads();

    // ---- 3. depthwise, VO outputs per thread ----
    const int th_n = min(f.tile_h, D.ho - ho0);
    const int uw = (D.wo + VO - 1) / VO;
    const int64_t oplane = (int64_t)D.ho * D.wo;
    int8_t* __restrict__ yg = (int8_t*)D.yptr;
    const bool away_d = D.rounding == CONV_ROUND_HALF_AWAY;
    const float lo_d = D.act == CONV_ACT_RELU ? 0.0f : (float)(-128 - f.y_zp), hi_d = (float)(127 - f.y_zp);
    const bool vec_y = (D.wo % 4) == 0 && (((uintptr_t)D.yptr) % 4) == 0;
    const int c_shift = OFF - D.pad_left;   // LDS column of tap 0 of output column 0
    auto rq_d = [&](int32_t v) __attribute__((always_inline)) {
        return RNE ? rq_even(v, f.comp_dw, lo_d, hi_d, f.y_zp) : rq_sel(v, f.comp_dw, away_d, lo_d, hi_d, f.y_zp);
    };
    auto store4 = [&](int8_t* dst, const int32_t (&accd)[VO], int q0) __attribute__((always_inline)) {
        uint32_t word = 0;
#pragma unroll
        for (int q = 0; q < VO; ++q) word |= (uint32_t)(uint8_t)rq_d(accd[q]) << (8 * q);
        if (vec_y && q0 + VO <= D.wo) {
            *(uint32_t*)dst = word;
        } else {
#pragma unroll
            for (int q = 0; q < VO; ++q)
                if (q0 + q < D.wo) dst[q] = (int8_t)(word >> (8 * q));
        }
    };
    if constexpr (FIXED && KH == 3 && KW == 3) {
        // A thread owns one channel and one group of VO output columns and
        // walks down the tile's output rows.  A filter row is one word (w0,
        // w1, w2, 0); the three taps of output q are the bytes from c_shift +
        // (q0+q)*SS on, cut out of two dwords with v_alignbyte (the fourth
        // byte meets the zero weight), and one v_dot4 adds the row's three
        // products.  Each expanded row's dwords are read once: they stay in
        // registers for the next output row that needs them.  SHc is the byte
        // offset of output q0's first tap inside its dword (the same for every
        // column group, as q0 * stride is a multiple of 4), fixed at compile
        // time so that the window dwords stay in registers.
        constexpr int ND = SS == 1 ? 3 : 4;
        auto walk = [&](auto SHc) __attribute__((always_inline)) {
            constexpr int SH = decltype(SHc)::value;
            auto dotrow = [&](const uint32_t (&d)[ND], uint32_t wrow, int32_t (&accd)[VO])
                __attribute__((always_inline)) {
#pragma unroll
                for (int q = 0; q < VO; ++q) {
                    const int idx = SH + SS * q;
                    const uint32_t lo = d[idx >> 2];
                    const uint32_t hi = d[(idx >> 2) + 1 < ND ? (idx >> 2) + 1 : ND - 1];
                    const uint32_t win = (idx & 3) ? __builtin_amdgcn_alignbyte(hi, lo, idx & 3) : lo;
                    accd[q] = __builtin_amdgcn_sdot4((int)win, (int)wrow, accd[q], false);
                }
            };
            const int pairs = ce_valid * uw;
            for (int pr = tid; pr < pairs; pr += kT) {
                const int ce = (int)divu((uint32_t)pr, f.dv_uw);
                const int q0 = (pr - ce * uw) * VO;
                const int cg = ce0 + ce;
                const uint32_t w0 = dwf[3 * ce], w1 = dwf[3 * ce + 1], w2 = dwf[3 * ce + 2];
                const int32_t db = dwb[ce];
                const uint32_t* col = (const uint32_t*)(es + ce * plane) + ((c_shift + q0 * SS) >> 2);
                const int EWD = EW >> 2;
                int8_t* dst = yg + ((int64_t)n * D.out_total + D.out_off + cg) * oplane + (int64_t)ho0 * D.wo + q0;
                auto load = [&](uint32_t (&d)[ND], int row) __attribute__((always_inline)) {
#pragma unroll
                    for (int t = 0; t < ND; ++t) d[t] = col[row * EWD + t];
                };
                uint32_t ra[ND], rb[ND];
                load(ra, 0);
                if constexpr (SS == 1) load(rb, 1);
                for (int o = 0; o < th_n; ++o) {
                    int32_t accd[VO];
#pragma unroll
                    for (int q = 0; q < VO; ++q) accd[q] = db;
                    uint32_t rc[ND];
                    if constexpr (SS == 1) {
                        load(rc, o + 2);
                        dotrow(ra, w0, accd);
                        dotrow(rb, w1, accd);
                        dotrow(rc, w2, accd);
#pragma unroll
                        for (int t = 0; t < ND; ++t) { ra[t] = rb[t]; rb[t] = rc[t]; }
                    } else {
                        load(rb, SS * o + 1);
                        load(rc, SS * o + 2);
                        dotrow(ra, w0, accd);
                        dotrow(rb, w1, accd);
                        dotrow(rc, w2, accd);
#pragma unroll
                        for (int t = 0; t < ND; ++t) ra[t] = rc[t];
                    }
                    store4(dst + (int64_t)o * D.wo, accd, q0);
                }
            }
        };
        switch (c_shift & 3) {
        case 0: walk(std::integral_constant<int, 0>{}); break;
        case 1: walk(std::integral_constant<int, 1>{}); break;
        case 2: walk(std::integral_constant<int, 2>{}); break;
        default: walk(std::integral_constant<int, 3>{}); break;
        }
    } else {
        // Any window, stride and dilation: VO outputs of one row per unit.
        const int units = ce_valid * th_n * uw;
        const DivU32 dvt = th_n == f.tile_h ? f.dv_th : f.dv_th_last;
        const int8_t* __restrict__ wdw = (const int8_t*)D.wptr;
        for (int u = tid; u < units; u += kT) {
            const int ridx = (int)divu((uint32_t)u, f.dv_uw);
            const int q0 = (u - ridx * uw) * VO;
            const int ce = (int)divu((uint32_t)ridx, dvt);
            const int orow = ridx - ce * th_n;
            const int cg = ce0 + ce;
            const uint8_t* ech = es + ce * plane;
            const int8_t* wch = wdw + (int64_t)cg * kh * kw;
            int32_t accd[VO];
#pragma unroll
            for (int q = 0; q < VO; ++q) accd[q] = dwb[ce];
            for (int r = 0; r < kh; ++r) {
                const uint8_t* row = ech + (orow * sh + r * dh) * EW;
                for (int s2 = 0; s2 < kw; ++s2) {
                    const int32_t wv = wch[r * kw + s2];
#pragma unroll
                    for (int q = 0; q < VO; ++q) {
                        // Outputs past the row end are not stored; clamp their reads.
                        const int col = c_shift + min(q0 + q, D.wo - 1) * sw + s2 * dwl;
                        accd[q] += (int32_t)(int8_t)row[col] * wv;
                    }
                }
            }
            store4(yg + ((int64_t)n * D.out_total + D.out_off + cg) * oplane + (int64_t)(ho0 + orow) * D.wo + q0,
                   accd, q0);
        }
    }
}

struct QPDPlan {
    int tile_h, rows, off, ew, lds, nf, dwf_off;
};

// Output rows per tile: the fewest rounds of resident workgroups times
// expanded rows per workgroup (the halo recompute included).
bool qpd_plan(const Desc& pw, const Desc& dw, QPDPlan* out) {
    const conv2d_params_t& d = dw.p;
    const int W = pw.p.w;
    const int off = (d.pad_left + 3) / 4 * 4;
    const int ew = (off + W + d.pad_right + 3) / 4 * 4;
    const long ce_tiles = (pw.p.c_out + CE - 1) / CE;
    bool ok = false;
    long best = 0;
    for (int th = 1; th <= dw.ho; ++th) {
        const int rows = (th - 1) * d.stride_h + (d.k_h - 1) * d.dilation_h + 1;
        const int npix = rows * W;
        const int nf = ((npix + 15) / 16 + 3) / 4;
        if (nf > NFMAX || npix >= 65536) break;
        // 16 bytes past the expansion tile: a unit's window dwords may run
        // past the last row (those bytes meet zero weights or feed outputs
        // that are not stored).
        const int etile = (CE * rows * ew + 16 + 15) / 16 * 16;
        const int dwf_off = max((npix + 3) / 4 * 4 * XROW, etile);
        const int lds = dwf_off + CE * 16;            // 3 filter words and a bias per channel
        if (lds > 64 * 1024) break;
        // The kernel is bound by VALU issue: its time follows the expanded
        // rows the busiest compute unit processes (workgroups per CU, rounded
        // up, times rows per workgroup); ties go to more workgroups.
        const long blocks = ce_tiles * pw.p.n * ((dw.ho + th - 1) / th);
        const long cost = (blocks + device_cu_count() - 1) / device_cu_count() * rows;
        if (!ok || cost < best) {
            *out = QPDPlan{th, rows, off, ew, lds, nf, dwf_off};
            best = cost;
            ok = true;
        }
    }
    return ok;
}

template <int NF, bool RNE>
const void* pick_fn(const conv2d_params_t& d) {
    const bool d1 = d.dilation_h == 1 && d.dilation_w == 1;
    if (d1 && d.k_h == 3 && d.k_w == 3 && d.stride_h == 1 && d.stride_w == 1)
        return (const void*)qfused_pw_dw_kernel<NF, 3, 3, 1, RNE>;
    if (d1 && d.k_h == 3 && d.k_w == 3 && d.stride_h == 2 && d.stride_w == 2)
        return (const void*)qfused_pw_dw_kernel<NF, 3, 3, 2, RNE>;
    return (const void*)qfused_pw_dw_kernel<NF, 0, 0, 0, RNE>;
}

template <int NF>
const void* pick_rne(const conv2d_params_t& d, bool rne) {
    return rne ? pick_fn<NF, true>(d) : pick_fn<NF, false>(d);
}

}  // namespace

bool plan_qfused_pw_dw(const Desc& pw, const Desc& dw) {
    QPDPlan qp{};
    return qpd_plan(pw, dw, &qp);
}

hipError_t launch_qfused_pw_dw(const Desc& pw, const Desc& dw, ConvArgs apw, ConvArgs adw, float comp_pw,
                               float comp_dw, int y_zp, hipStream_t s) {
    QPDPlan qp{};
    if (!qpd_plan(pw, dw, &qp)) return hipErrorInvalidConfiguration;
    QPDArgs f;
    f.pw = apw;
    f.dw = adw;
    f.pw.rounding = pw.p.int8_rounding;
    f.dw.rounding = dw.p.int8_rounding;
    f.comp_pw = comp_pw;
    f.comp_dw = comp_dw;
    f.y_zp = y_zp;
    f.tile_h = qp.tile_h;
    f.tiles_h = (dw.ho + qp.tile_h - 1) / qp.tile_h;
    f.ce_tiles = (pw.p.c_out + CE - 1) / CE;
    f.rows = qp.rows;
    f.off = qp.off;
    f.ew = qp.ew;
    f.dwf_off = qp.dwf_off;
    f.vec = pw.p.w % 4 == 0 && ((uintptr_t)apw.xptr % 4) == 0;
    f.div_w = make_fastdiv((uint32_t)pw.p.w);
    f.dv_pq = make_divu32((uint32_t)((qp.rows * pw.p.w + 3) / 4));
    f.dv_uw = make_divu32((uint32_t)((dw.wo + VO - 1) / VO));
    f.dv_th = make_divu32((uint32_t)qp.tile_h);
    f.dv_th_last = make_divu32((uint32_t)(dw.ho - (f.tiles_h - 1) * qp.tile_h));
    f.dv_ce_tiles = make_divu32((uint32_t)f.ce_tiles);
    f.dv_tiles_h = make_divu32((uint32_t)f.tiles_h);
    const uint64_t blocks = (uint64_t)f.ce_tiles * f.tiles_h * apw.n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0xFFFFFFFFull) return hipErrorInvalidConfiguration;
    f.num_blocks = (uint32_t)blocks;
    const void* fn;
    const bool rne = pw.p.int8_rounding == CONV_ROUND_HALF_EVEN && dw.p.int8_rounding == CONV_ROUND_HALF_EVEN;
    switch (qp.nf) {
    case 1: case 2: fn = pick_rne<2>(dw.p, rne); break;
    case 3: case 4: fn = pick_rne<4>(dw.p, rne); break;
    case 5: case 6: fn = pick_rne<6>(dw.p, rne); break;
    case 7: case 8: fn = pick_rne<8>(dw.p, rne); break;
    default: fn = pick_rne<NFMAX>(dw.p, rne); break;
    }
    void* args[] = {&f};
    return hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(kT), args, qp.lds, s);
}

}  // namespace conv2d
