// int8 fused depthwise kxk -> pointwise 1x1 (the QuantizedDwPw step of the
// yscv "ONNX CPU Kernels" page, section "Hot kernel paths": the depthwise
// int32 sums are requantised to int8 in on-chip memory and feed the int8
// pointwise GEMM; the intermediate tensor never reaches main memory).
//
// The intermediate is exactly the int8 tensor the unfused depthwise would
// store (same integer sums, same requant), so the result is bitwise that of
// the two QLinearConvs run one after the other.
//
// Workgroup tile: one image, TH output rows of full width (TH * Wo <= 256
// pixels), MI x 16 pointwise output channels.  Depthwise channels (= the
// pointwise K) are walked in chunks of KC = 64, one MFMA K step:
//   1. the chunk's input rows go to LDS as bytes (pad rows and columns hold
//      the zero point, 0, written once); its depthwise weights and biases too;
//   2. a thread owns 4 consecutive channels of the chunk and walks the tile's
//      pixels 16 apart: int32 sums of the window, + bias, requant to int8, the
//      4 channel bytes of a pixel written as one word of the pixel-major
//      operand tile [pixel][k] (16 consecutive k per MFMA lane);
//   3. v_mfma_i32_16x16x64_i8: A = pointwise weights (k-contiguous OIHW rows,
//      16 bytes per lane straight from memory), B = that tile.
// The epilogue adds the pointwise bias and requantises (ties to even or away,
// y_zp, optional ReLU) into channel out_off + co of the output buffer.
#include "device_common.h"

namespace conv2d {

namespace {

constexpr int kT = 256;
constexpr int kWaves = kT / 64;
constexpr int KC = 64;          // depthwise channels per chunk = one MFMA K step
constexpr int XROW = KC + 16;   // LDS bytes per pixel of the operand tile
constexpr int KHW_MAX = 25;

struct QFArgs {
    ConvArgs dw, pw;
    float comp_dw, comp_pw;
    int32_t rnd_dw, rnd_pw, relu_dw, relu_pw, y_zp;
    int32_t th, tiles_h, co_tiles;
    int32_t ir;        // input rows per tile
    int32_t xw;        // LDS bytes per input row (pad_left + w + pad_right, rounded to 4)
    int32_t xplane;    // LDS bytes per channel of the input tile (= 4 mod 64... see plan)
    int32_t npx, nf;   // tile pixels, 16-pixel fragments
    int32_t vec;       // input rows move as 4-byte words
    uint32_t num_blocks;
};

template <int MI, int NJ>
__global__ __launch_bounds__(kT) void qfused_dw_pw_kernel(QFArgs f) {
    extern __shared__ __align__(16) uint8_t lds8[];
    const ConvArgs& D = f.dw;
    const ConvArgs& P = f.pw;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    uint32_t L = blockIdx.x;
    const int cot = L % f.co_tiles;  L /= f.co_tiles;
    const int tht = L % f.tiles_h;   L /= f.tiles_h;
    const int n = L;
    const int co0 = cot * MI * 16;
    const int ho0 = tht * f.th;
    const int th_n = min(f.th, D.ho - ho0);
    const int npx_n = th_n * D.wo;
    const int kh = D.k_h, kw = D.k_w, khw = kh * kw;
    const int sh = D.stride_h, sw = D.stride_w, dh = D.dilation_h, dwl = D.dilation_w;
    const int ih0 = ho0 * sh - D.pad_top;
    const int C = D.c_out, H = D.h, W = D.w, WO = D.wo;
    const int64_t HW = (int64_t)H * W;

    uint8_t* xs = lds8;                                        // [KC][ir][xw]
    uint8_t* es = xs + KC * f.xplane;                          // [nf*16][XROW]
    int8_t* wd = (int8_t*)(es + f.nf * 16 * XROW);             // [KC][khw]
    int32_t* bd = (int32_t*)(wd + (KC * KHW_MAX + 3) / 4 * 4); // [KC]

    const int8_t* __restrict__ xg = (const int8_t*)D.xptr + ((int64_t)n * D.in_total + D.in_off) * HW;
    const int8_t* __restrict__ wdg = (const int8_t*)D.wptr;
    const int8_t* __restrict__ wpg = (const int8_t*)P.wptr;
    const bool vec_w = (C % 16) == 0 && ((uintptr_t)P.wptr % 16) == 0;

    // Pad rows and columns of the input tile hold the zero point (0): written
    // once, the chunk copies below only write in-image bytes.
    for (int e = tid; e < KC * f.xplane / 4; e += kT) ((uint32_t*)xs)[e] = 0u;
    __syncthreads();

    i32x4 acc[MI][NJ];
#pragma unroll
    for (int m = 0; m < MI; ++m)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[m][j] = i32x4{0, 0, 0, 0};

    const int cq = tid & 15;          // channels 4*cq .. 4*cq+3 of the chunk
    const int pg = tid >> 4;          // pixels pg, pg+16, ...
    const int xoff = D.pad_left;      // LDS column of image column 0

    for (int c0 = 0; c0 < C; c0 += KC) {
        // ---- 1. chunk -> LDS: input rows, depthwise weights and biases ----
        if (f.vec) {
            const int w4 = W >> 2;
            const int units = KC * f.ir * w4;
            for (int u = tid; u < units; u += kT) {
                const int ch = u / (f.ir * w4), rem = u - ch * (f.ir * w4);
                const int row = rem / w4, c4 = rem - row * w4;
                const int ih = ih0 + row;
                if (c0 + ch < C && (unsigned)ih < (unsigned)H) {
                    const uint32_t v = *(const uint32_t*)(xg + (int64_t)(c0 + ch) * HW + (int64_t)ih * W + 4 * c4);
                    uint8_t* dst = xs + ch * f.xplane + row * f.xw + xoff + 4 * c4;
#pragma unroll
                    for (int b = 0; b < 4; ++b) dst[b] = (uint8_t)(v >> (8 * b));
                }
            }
        } else {
            const int units = KC * f.ir * W;
            for (int u = tid; u < units; u += kT) {
                const int ch = u / (f.ir * W), rem = u - ch * (f.ir * W);
                const int row = rem / W, col = rem - row * W;
                const int ih = ih0 + row;
                if (c0 + ch < C && (unsigned)ih < (unsigned)H)
                    xs[ch * f.xplane + row * f.xw + xoff + col] = (uint8_t)xg[(int64_t)(c0 + ch) * HW + (int64_t)ih * W + col];
            }
        }
        for (int e = tid; e < KC * khw; e += kT) wd[e] = c0 * khw + e < C * khw ? wdg[(int64_t)c0 * khw + e] : (int8_t)0;
        if (tid < KC) bd[tid] = (D.qbias && c0 + tid < C) ? D.qbias[c0 + tid] : 0;
        __syncthreads();

        // ---- 2. depthwise, requant, pixel-major int8 operand tile ----
        for (int p = pg; p < f.nf * 16; p += kT / 16) {
            uint32_t word = 0;
            if (p < npx_n) {
                const int r = p / WO, c = p - r * WO;
                const uint8_t* base = xs + r * sh * f.xw + xoff - D.pad_left + c * sw;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int ch = 4 * cq + k;
                    if (c0 + ch >= C) continue;              // byte stays 0 (zero weights in the GEMM too)
                    const uint8_t* src = base + ch * f.xplane;
                    const int8_t* wch = wd + ch * khw;
                    int32_t s = bd[ch];
                    for (int i = 0; i < kh; ++i)
                        for (int j = 0; j < kw; ++j)
                            s += (int32_t)(int8_t)src[i * dh * f.xw + j * dwl] * (int32_t)wch[i * kw + j];
                    const uint32_t q = (uint32_t)(uint8_t)requant(s, f.comp_dw, f.rnd_dw, 0, f.relu_dw != 0);
                    word |= q << (8 * k);
                }
            }
            *(uint32_t*)(es + p * XROW + 4 * cq) = word;
        }
        __syncthreads();

        // ---- 3. pointwise on the i8 matrix cores ----
        // B: pixel fj*16 + lane%16, k = 16*(lane/16) .. +15 of the chunk;
        // A: output channel co0 + m*16 + lane%16, the same k.
        const int kk = c0 + 16 * (lane >> 4);
        i32x4 afrag[MI];
#pragma unroll
        for (int m = 0; m < MI; ++m) {
            const int co = co0 + m * 16 + (lane & 15);
            afrag[m] = i32x4{0, 0, 0, 0};
            if (co < P.c_out) {
                const int8_t* src = wpg + (int64_t)co * C + kk;
                if (vec_w && kk + 16 <= C) {
                    afrag[m] = *(const i32x4*)src;
                } else {
                    uint32_t w4[4] = {0, 0, 0, 0};
                    for (int b = 0; b < 16; ++b)
                        if (kk + b < C) w4[b >> 2] |= (uint32_t)(uint8_t)src[b] << (8 * (b & 3));
                    afrag[m] = i32x4{(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]};
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int fj = wave + kWaves * j;
            if (fj < f.nf) {
                const i32x4 bfrag = *(const i32x4*)(es + (fj * 16 + (lane & 15)) * XROW + 16 * (lane >> 4));
#pragma unroll
                for (int m = 0; m < MI; ++m)
                    acc[m][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(afrag[m], bfrag, acc[m][j], 0, 0, 0);
            }
        }
        __syncthreads();   // the next chunk rewrites the input tile and the operand tile
    }

    // ---- epilogue: lane holds output channels 4*(lane/16)+v of pixel lane%16 ----
    int8_t* __restrict__ yg = (int8_t*)P.yptr;
    const int64_t oplane = (int64_t)P.ho * P.wo;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int fj = wave + kWaves * j;
        const int p = fj * 16 + (lane & 15);
        if (fj >= f.nf || p >= npx_n) continue;
#pragma unroll
        for (int m = 0; m < MI; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int co = co0 + m * 16 + (lane >> 4) * 4 + v;
                if (co >= P.c_out) continue;
                const int32_t val = acc[m][j][v] + (P.qbias ? P.qbias[co] : 0);
                yg[((int64_t)n * P.out_total + P.out_off + co) * oplane + (int64_t)ho0 * WO + p] =
                    requant(val, f.comp_pw, f.rnd_pw, f.y_zp, f.relu_pw != 0);
            }
    }
}

struct QPlan {
    int th, ir, xw, xplane, npx, nf, nj, lds;
};

// ---------------------------------------------------------------------------
// Fast path: 3x3 or 5x5 window, stride 1 or 2, dilation 1, input rows a
// multiple of 16 bytes, 16-byte aligned input and pointwise weights.
//
//   * A chunk's input rows are copied as 16-byte vectors into LDS rows whose
//     image column 0 sits FM bytes in (the margins, the right pad and the rows
//     outside the image hold the zero point 0, written once).  Each thread's
//     copy slots (global and LDS offsets) are fixed for the whole kernel; the
//     loads run two chunks ahead in registers, issued unconditionally (a slot
//     outside the tile reads the image's first bytes and is dropped at the LDS
//     write), so the compiler's waits leave the later chunk in flight.
//   * Depthwise: a unit is 4 channels x 4 consecutive output columns of one
//     row.  Per filter row it reads the covering LDS dwords once, shifts them
//     by the pad's byte offset (v_alignbyte), and each output takes its window
//     with v_dot4_i32_i8 against the packed filter row (w0, w1, w2, 0), plus a
//     second dot4 for the fifth tap of a 5x5 window: exact int32 sums.  After
//     the requant the 4 x 4 bytes are transposed in registers into 4 words,
//     one per pixel holding its 4 channels, the layout the i8 MFMA operand
//     wants (16 consecutive k per lane).
//   * Pointwise: v_mfma_i32_16x16x64_i8 with the depthwise tile as the first
//     operand (pixels) and the chunk's pointwise weights, staged in LDS and
//     double-buffered, as the second; a lane ends up holding 4 consecutive
//     pixels of one output channel and stores them as one packed word.
constexpr int FM = 16;      // LDS bytes left of image column 0
constexpr int FROW = 80;    // LDS bytes per row of an MFMA operand tile (64 k; rows 20 dwords apart)
constexpr int FNF = 4;      // MFMA fragments per wave

struct QFastArgs {
    ConvArgs dw, pw;
    float comp_dw, comp_pw;
    int32_t rnd_dw, rnd_pw, relu_dw, relu_pw, y_zp;
    int32_t th, tiles_h, co_tiles, cot, mt;   // output rows per tile, row tiles, channel tiles, channels and fragments per tile
    int32_t ir, rb, pb;     // input rows per tile, LDS bytes per input row and per channel plane
    int32_t q0, off;        // dword and byte of column group 0's first tap in an LDS row
    int32_t nf, wq;         // 16-pixel fragments per tile, 4-column groups per output row
    int32_t out_vec;        // outputs stored as packed 4-byte words
    uint32_t num_blocks;
    DivU32 dv_co_tiles, dv_tiles_h;
    FastDiv div_wq, div_per_ch, div_w16, div_mt;   // numerators below 2^16
};

// The depthwise requant with the rounding fixed at compile time; lo is the
// lower clamp (-128, or the zero point 0 under ReLU).  The clamp runs on the
// rounded float (an integer value, so it equals clamping the int); the int8
// result is the low byte of the returned int.
template <int RND>
__device__ __forceinline__ int rq_dw(int32_t acc, float comp, float lo) {
    float yf = __fmul_rn((float)acc, comp);
    asm volatile("" : "+v"(yf));   // the rounded f32 product decides ties (no fma into roundf)
    const float r = RND == CONV_ROUND_HALF_AWAY ? roundf(yf) : rintf(yf);
    return (int)__builtin_amdgcn_fmed3f(r, lo, 127.0f);
}

template <int SS, int KK, int NQ, int RND>
__global__ __launch_bounds__(kT) void qfused_fast_kernel(QFastArgs f) {
    extern __shared__ __align__(16) uint8_t lds8[];
    const ConvArgs& D = f.dw;
    const ConvArgs& P = f.pw;
    constexpr int NWIN = (KK + 3) / 4;                       // dot4 windows per filter row
    constexpr int NE = (SS * 3 + 4 * (NWIN - 1)) / 4 + 2;    // shifted dwords under 4 outputs' windows
    constexpr int NWS = (KC * KK + kT - 1) / kT;             // filter rows per thread and chunk
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    uint32_t L = xcd_remap(blockIdx.x, f.num_blocks);
    uint32_t Q = divu(L, f.dv_co_tiles);
    const int cot = L - Q * f.co_tiles;
    L = Q;
    Q = divu(L, f.dv_tiles_h);
    const int tht = L - Q * f.tiles_h;
    const int n = Q;
    const int co0 = cot * f.cot;
    const int ho0 = tht * f.th;
    const int th_n = min(f.th, D.ho - ho0);
    const int ih0 = ho0 * SS - D.pad_top;
    const int C = D.c_out, H = D.h, W = D.w, WO = D.wo;
    const int HW = H * W;                                    // C * H * W < 2^31 (planner)
    const int nch = (C + KC - 1) / KC;
    const int w16 = W >> 4;

    uint8_t* xs = lds8;                                      // [KC][pb]
    uint8_t* at = xs + KC * f.pb;                            // [nf * 16][FROW] depthwise result
    uint8_t* wt0 = at + f.nf * 16 * FROW;                    // [64][FROW] x 2 pointwise weights
    int32_t* wpk = (int32_t*)(wt0 + 2 * 64 * FROW);          // [KC][KK][NWIN] packed filter rows
    int32_t* bd = wpk + KC * KK * NWIN;                      // [KC] depthwise bias

    const int8_t* __restrict__ xg = (const int8_t*)D.xptr + ((int64_t)n * D.in_total + D.in_off) * HW;
    const int8_t* __restrict__ wdg = (const int8_t*)D.wptr;
    const int8_t* __restrict__ wpg = (const int8_t*)P.wptr;
    const int32_t* __restrict__ bsrc = D.qbias ? D.qbias : (const int32_t*)xg;

    // Copy slots: u = tid + i*kT -> (channel, tile row, 16-byte column).
    const int per_ch = f.ir * w16;
    const int units_x = KC * per_ch;
    int goff[NQ], loff[NQ], chs[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const int u = tid + i * kT;
        const int ch = (int)fdiv((uint32_t)u, f.div_per_ch), rem = u - ch * per_ch;
        const int row = (int)fdiv((uint32_t)rem, f.div_w16), j = rem - row * w16;
        const int ih = ih0 + row;
        const bool ok = u < units_x && (unsigned)ih < (unsigned)H;
        goff[i] = ch * HW + ih * W + 16 * j;
        loff[i] = ok ? ch * f.pb + row * f.rb + FM + 16 * j : -1;
        chs[i] = ch;
    }

    struct Regs {
        i32x4 x[NQ];
        i32x4 pw;
        uint32_t wb[NWS][2];   // the two aligned dwords under a filter row
        int32_t bias;
    };
    auto load_chunk = [&](int c, Regs& R) __attribute__((always_inline)) {
        const int c0 = c * KC;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const bool ok = loff[i] >= 0 && c0 + chs[i] < C;
            R.x[i] = *(const i32x4*)(xg + (ok ? (int64_t)c0 * HW + goff[i] : 0));
        }
        {
            const int co = tid >> 2, kq = tid & 3;
            const bool ok = co < f.cot && co0 + co < P.c_out && c0 + 16 * kq < C;
            R.pw = *(const i32x4*)(wpg + (ok ? (int64_t)(co0 + co) * C + c0 + 16 * kq : 0));
        }
        // A filter row (KK bytes at any byte offset) lies within the two
        // aligned dwords from its offset rounded down; the weight tensor's
        // size is a multiple of 4 (C % 16 == 0), so the second dword is in
        // bounds whenever the row needs it and is clamped otherwise.
#pragma unroll
        for (int s = 0; s < NWS; ++s) {
            const int e = tid + s * kT;                      // channel * KK + filter row
            const int ch = e / KK;
            const bool ok = e < KC * KK && c0 + ch < C;
            const int64_t b = ok ? (int64_t)(c0 + ch) * KK * KK + (e - ch * KK) * KK : 0;
            const int64_t a0 = b & ~(int64_t)3;
            const int64_t a1 = a0 + 4 < (int64_t)C * KK * KK ? a0 + 4 : a0;
            R.wb[s][0] = *(const uint32_t*)(wdg + a0);
            R.wb[s][1] = *(const uint32_t*)(wdg + a1);
        }
        R.bias = bsrc[D.qbias && tid < KC && c0 + tid < C ? c0 + tid : 0];
    };
    // The empty asm statements pin each prefetched register to this point:
    // no operation on it (a byte shift, a select) can be scheduled earlier,
    // where its wait would also cover the loads of the chunk behind it.
    auto store_chunk = [&](int c, Regs& R, uint8_t* wt) __attribute__((always_inline)) {
        const int c0 = c * KC;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            asm volatile("" : "+v"(R.x[i]));
            if (loff[i] >= 0 && c0 + chs[i] < C) *(i32x4*)(xs + loff[i]) = R.x[i];
        }
        asm volatile("" : "+v"(R.pw));
        *(i32x4*)(wt + (tid >> 2) * FROW + 16 * (tid & 3)) = R.pw;
#pragma unroll
        for (int s = 0; s < NWS; ++s) {
            asm volatile("" : "+v"(R.wb[s][0]));
            asm volatile("" : "+v"(R.wb[s][1]));
        }
        asm volatile("" : "+v"(R.bias));
#pragma unroll
        for (int s = 0; s < NWS; ++s) {
            const int e = tid + s * kT;
            if (e < KC * KK) {
                // Channels past the last one get zero weights (and a zero bias
                // below): their sums are 0 and requantise to 0.
                const bool live = c0 + e / KK < C;
                const uint32_t sh = (uint32_t)((c0 * KK * KK + e * KK) & 3);   // the row's byte in dword 0
                const uint32_t w4 = __builtin_amdgcn_alignbyte(R.wb[s][1], R.wb[s][0], sh);
                wpk[e * NWIN] = live ? (int32_t)(KK == 3 ? (w4 & 0x00FFFFFFu) : w4) : 0;
                if (NWIN > 1) wpk[e * NWIN + 1] = live ? (int32_t)((R.wb[s][1] >> (8 * sh)) & 0xFFu) : 0;
            }
        }
        if (tid < KC) bd[tid] = D.qbias && c0 + tid < C ? R.bias : 0;
    };

    // Depthwise of chunk c into the pixel-major operand tile.  Unit u: channel
    // quad u % 16 (the 16 lanes of a quarter-wave hold the chunk's 64
    // channels, so their operand writes fill one 64-byte pixel row), then
    // column group and output row.
    const int du = 16 * th_n * f.wq;
    const float lo_dw = f.relu_dw ? 0.0f : -128.0f;
    // The chunk's input tile and filter rows are the ones in LDS (a single
    // buffer, rewritten each chunk), so the depthwise needs no chunk index.
    auto depthwise = [&]() __attribute__((always_inline)) {
        for (int u = tid; u < du; u += kT) {
            const int cq = u & 15;
            const int pu = u >> 4;
            const int r = (int)fdiv((uint32_t)pu, f.div_wq);
            const int k = pu - r * f.wq;
            // Two channels per pass; their bytes of pixel j are packed with one
            // v_perm, the two passes' halves with one shift-or.
            uint32_t outw[4] = {0u, 0u, 0u, 0u};
#pragma unroll 1
            for (int pr = 0; pr < 2; ++pr) {
                int q[2][4];
#pragma unroll
                for (int ii = 0; ii < 2; ++ii) {
                    const int ch = 4 * cq + 2 * pr + ii;
                    int32_t acc[4];
                    const int32_t b = bd[ch];
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[j] = b;
                    const uint8_t* prow = xs + ch * f.pb + r * SS * f.rb + 4 * (SS * k + f.q0);
#pragma unroll
                    for (int rr = 0; rr < KK; ++rr) {
                        const uint32_t* src = (const uint32_t*)(prow + rr * f.rb);
                        uint32_t d[NE + 1], e[NE];
#pragma unroll
                        for (int t = 0; t <= NE; ++t) d[t] = src[t];
#pragma unroll
                        for (int t = 0; t < NE; ++t) e[t] = __builtin_amdgcn_alignbyte(d[t + 1], d[t], (uint32_t)f.off);
                        const int32_t* wr = wpk + (ch * KK + rr) * NWIN;
#pragma unroll
                        for (int w = 0; w < NWIN; ++w) {
                            const int32_t wv = wr[w];
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const int idx = SS * j + 4 * w;    // byte of output j's window in e[]
                                const uint32_t lo = e[idx >> 2];
                                const uint32_t win = (idx & 3) ? __builtin_amdgcn_alignbyte(e[(idx >> 2) + 1], lo, idx & 3) : lo;
                                acc[j] = __builtin_amdgcn_sdot4((int)win, wv, acc[j], false);
                            }
                        }
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) q[ii][j] = rq_dw<RND>(acc[j], f.comp_dw, lo_dw);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    outw[j] |= __builtin_amdgcn_perm((uint32_t)q[1][j], (uint32_t)q[0][j], 0x0c0c0400u) << (16 * pr);
            }
            const int p = r * WO + 4 * k;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (4 * k + j < WO) *(uint32_t*)(at + (p + j) * FROW + 4 * cq) = outw[j];
        }
    };

    // Fragments of this wave: fi = wave + kWaves * s -> (pixel fragment, channel fragment).
    const int nfr = f.nf * f.mt;
    int pfo[FNF], cfo[FNF];
#pragma unroll
    for (int s = 0; s < FNF; ++s) {
        const int fi = wave + kWaves * s;
        const int pf = (int)fdiv((uint32_t)fi, f.div_mt);
        pfo[s] = (pf * 16 + (lane & 15)) * FROW + 16 * (lane >> 4);
        cfo[s] = ((fi - pf * f.mt) * 16 + (lane & 15)) * FROW + 16 * (lane >> 4);
    }
    i32x4 acc[FNF];
#pragma unroll
    for (int s = 0; s < FNF; ++s) acc[s] = i32x4{0, 0, 0, 0};
    auto pointwise = [&](const uint8_t* wt) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < FNF; ++s) {
            if (wave + kWaves * s < nfr) {
                const i32x4 a = *(const i32x4*)(at + pfo[s]);
                const i32x4 b = *(const i32x4*)(wt + cfo[s]);
                acc[s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[s], 0, 0, 0);
            }
        }
    };

    // Chunk c: registers -> LDS (the input tile and the filter rows were last
    // read by chunk c-1's depthwise, before the barrier that preceded its
    // MFMAs; weight buffer c%2 by chunk c-2's MFMAs), barrier, loads of chunk
    // cn (two ahead) into the same registers, depthwise, barrier, MFMAs.
    auto compute = [&](int c, const uint8_t* wt) __attribute__((always_inline)) {
        if (c < nch) {
            depthwise();
            __syncthreads();
            pointwise(wt);
        }
    };
    auto step = [&](int c, Regs& R, int cn) __attribute__((always_inline)) {
        uint8_t* wt = wt0 + (c & 1) * 64 * FROW;
        store_chunk(c, R, wt);
        __syncthreads();
        load_chunk(cn, R);
        compute(c, wt);
    };
    // An odd number of steps S >= nch: step 0 is peeled, the rest go in pairs
    // with fixed register sets, and every step issues loads (the last ones
    // reload chunk S-1), so no load sits behind a condition.  Step 0 stores
    // chunk 0 before chunk 1's loads are issued: with every workgroup's
    // first loads in flight at once, a wave would otherwise stall issuing
    // chunk 1 until most of chunk 0 had arrived anyway, and start later.
    const int S = nch | 1;
    Regs R0, R1;
    load_chunk(0, R0);
    for (int e = tid; e < KC * f.pb / 16; e += kT) ((i32x4*)xs)[e] = i32x4{0, 0, 0, 0};
    __syncthreads();
    store_chunk(0, R0, wt0);
    load_chunk(min(1, S - 1), R1);
    __syncthreads();
    load_chunk(min(2, S - 1), R0);
    compute(0, wt0);
    for (int c = 1; c < S; c += 2) {
        step(c, R1, min(c + 2, S - 1));
        step(c + 1, R0, min(c + 3, S - 1));
    }

    // ---- epilogue: fragment s of this wave, lane holds pixels p0 .. p0+3 of
    // output channel co; + bias, requant, one packed word per lane ----
    int8_t* __restrict__ yg = (int8_t*)P.yptr;
    const int64_t oplane = (int64_t)P.ho * P.wo;
    const int npx_n = th_n * WO;
    const bool relu_pw = f.relu_pw != 0;
#pragma unroll
    for (int s = 0; s < FNF; ++s) {
        const int fi = wave + kWaves * s;
        if (fi >= nfr) continue;
        const int pf = (int)fdiv((uint32_t)fi, f.div_mt);
        const int col = (fi - pf * f.mt) * 16 + (lane & 15);
        const int co = co0 + col;
        const int p0 = pf * 16 + 4 * (lane >> 4);
        if (col >= f.cot || co >= P.c_out || p0 >= npx_n) continue;
        const int32_t bias = P.qbias ? P.qbias[co] : 0;
        int8_t* dst = yg + ((int64_t)n * P.out_total + P.out_off + co) * oplane + (int64_t)ho0 * WO + p0;
        int8_t q[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) q[v] = requant(acc[s][v] + bias, f.comp_pw, f.rnd_pw, f.y_zp, relu_pw);
        if (f.out_vec) {
            *(uint32_t*)dst = (uint32_t)(uint8_t)q[0] | ((uint32_t)(uint8_t)q[1] << 8) |
                              ((uint32_t)(uint8_t)q[2] << 16) | ((uint32_t)(uint8_t)q[3] << 24);
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (p0 + v < npx_n) dst[v] = q[v];
        }
    }
}

struct QFastPlan {
    int th, cot, mt, nf, ir, rb, pb, q0, off, wq, nq, lds;
};

// Fast-path plan, or false when the layer or its tensors do not fit it.
bool qfast_plan(const Desc& dw, const Desc& pw, const void* x, const void* w_dw, const void* w_pw, QFastPlan* out) {
    const conv2d_params_t& d = dw.p;
    const int kk = d.k_h, ss = d.stride_h;
    if (d.k_w != kk || (kk != 3 && kk != 5) || d.stride_w != ss || (ss != 1 && ss != 2)) return false;
    if (d.dilation_h != 1 || d.dilation_w != 1 || d.w % 16 != 0 || d.pad_left > FM) return false;
    if (d.c_out % 16 != 0 || (int64_t)d.c_out * d.h * d.w >= INT32_MAX) return false;
    if (x == nullptr || w_pw == nullptr || (uintptr_t)x % 16 != 0 || (uintptr_t)w_pw % 16 != 0) return false;
    if (w_dw == nullptr || (uintptr_t)w_dw % 4 != 0) return false;
    const int nwin = (kk + 3) / 4;
    const int ne = (ss * 3 + 4 * (nwin - 1)) / 4 + 2;
    const int wq = (dw.wo + 3) / 4;
    const int q0 = (FM - d.pad_left) >> 2;
    int rb = FM + d.w;
    const int last = 4 * (ss * (wq - 1) + q0 + ne + 1);
    if (last > rb) rb = last;
    rb = (rb + 15) / 16 * 16;
    const int co = pw.p.c_out;
    const int cot = co <= 64 ? (co + 15) / 16 * 16 : 64;
    const int mt = cot / 16;
    const int co_tiles = (co + cot - 1) / cot;
    bool ok = false;
    long best = 0;
    for (int th = 1; th <= dw.ho; ++th) {
        const int nf = (th * dw.wo + 15) / 16;
        if (nf * mt > FNF * kWaves) break;
        const int ir = (th - 1) * ss + kk;
        const int units = KC * ir * (d.w / 16);
        if (units > 8 * kT) break;
        const int pb = ir * rb + 4;                         // an odd number of dwords
        const int lds = KC * pb + nf * 16 * FROW + 2 * 64 * FROW + 4 * KC * kk * nwin + 4 * KC;
        if (lds > 80 * 1024) break;
        const long blocks = (long)d.n * ((dw.ho + th - 1) / th) * co_tiles;
        const long cost = (blocks + device_cu_count() - 1) / device_cu_count() * (ir + th);
        if (!ok || cost < best) {
            *out = QFastPlan{th, cot, mt, nf, ir, rb, pb, q0, (FM - d.pad_left) & 3, wq, units <= 4 * kT ? 4 : 8, lds};
            best = cost;
            ok = true;
        }
    }
    return ok;
}

template <int SS, int KK, int RND>
const void* pick_fast_nq(int nq) {
    return nq == 4 ? (const void*)qfused_fast_kernel<SS, KK, 4, RND> : (const void*)qfused_fast_kernel<SS, KK, 8, RND>;
}

template <int RND>
const void* pick_fast(int ss, int kk, int nq) {
    return ss == 1 ? (kk == 3 ? pick_fast_nq<1, 3, RND>(nq) : pick_fast_nq<1, 5, RND>(nq))
                   : (kk == 3 ? pick_fast_nq<2, 3, RND>(nq) : pick_fast_nq<2, 5, RND>(nq));
}

hipError_t launch_qfast(const Desc& dw, const Desc& pw, const QFastPlan& pl, ConvArgs adw, ConvArgs apw, float comp_dw,
                        float comp_pw, int y_zp, hipStream_t s) {
    QFastArgs f;
    f.dw = adw;
    f.pw = apw;
    f.comp_dw = comp_dw;
    f.comp_pw = comp_pw;
    f.rnd_dw = dw.p.int8_rounding;
    f.rnd_pw = pw.p.int8_rounding;
    f.relu_dw = dw.p.act_type == CONV_ACT_RELU;
    f.relu_pw = pw.p.act_type == CONV_ACT_RELU;
    f.y_zp = y_zp;
    f.th = pl.th;
    f.tiles_h = (dw.ho + pl.th - 1) / pl.th;
    f.cot = pl.cot;
    f.mt = pl.mt;
    f.co_tiles = (pw.p.c_out + pl.cot - 1) / pl.cot;
    f.ir = pl.ir;
    f.rb = pl.rb;
    f.pb = pl.pb;
    f.q0 = pl.q0;
    f.off = pl.off;
    f.nf = pl.nf;
    f.wq = pl.wq;
    const int64_t ohw = (int64_t)pw.ho * pw.wo;
    f.out_vec = pw.wo % 4 == 0 && ((uintptr_t)apw.yptr % 4) == 0 && ((int64_t)apw.out_off * ohw) % 4 == 0 &&
                ((int64_t)apw.out_total * ohw) % 4 == 0;
    const uint64_t blocks = (uint64_t)f.co_tiles * f.tiles_h * adw.n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0xFFFFFFFFull) return hipErrorInvalidConfiguration;
    f.num_blocks = (uint32_t)blocks;
    f.dv_co_tiles = make_divu32((uint32_t)f.co_tiles);
    f.dv_tiles_h = make_divu32((uint32_t)f.tiles_h);
    f.div_wq = make_fastdiv((uint32_t)pl.wq);
    f.div_per_ch = make_fastdiv((uint32_t)(pl.ir * (dw.p.w / 16)));
    f.div_w16 = make_fastdiv((uint32_t)(dw.p.w / 16));
    f.div_mt = make_fastdiv((uint32_t)pl.mt);
    const int ss = dw.p.stride_h, kk = dw.p.k_h;
    const void* fn = dw.p.int8_rounding == CONV_ROUND_HALF_AWAY ? pick_fast<CONV_ROUND_HALF_AWAY>(ss, kk, pl.nq)
                                                                : pick_fast<CONV_ROUND_HALF_EVEN>(ss, kk, pl.nq);
    if (pl.lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, pl.lds);
        if (e != hipSuccess) return e;
    }
    void* args[] = {&f};
    return hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(kT), args, pl.lds, s);
}

bool qplan(const Desc& dw, const Desc& pw, QPlan* out) {
    const conv2d_params_t& d = dw.p;
    const int mi = pw.p.c_out <= 16 ? 1 : pw.p.c_out <= 32 ? 2 : pw.p.c_out <= 48 ? 3 : 4;
    const int co_tiles = (pw.p.c_out + 16 * mi - 1) / (16 * mi);
    const int xw = (d.pad_left + d.w + d.pad_right + 3) / 4 * 4;
    bool ok = false;
    long best = 0;
    for (int th = 1; th <= dw.ho; ++th) {
        const int npx = th * dw.wo;
        const int nf = (npx + 15) / 16;
        const int nj = (nf + kWaves - 1) / kWaves;
        if (nj > 4) break;
        const int ir = (th - 1) * d.stride_h + (d.k_h - 1) * d.dilation_h + 1;
        // Channel planes 4 (mod 64) bytes apart spread a thread group's reads over the banks.
        const int xplane = (ir * xw + 59) / 64 * 64 + 4;
        const int lds = KC * xplane + nf * 16 * XROW + (KC * KHW_MAX + 3) / 4 * 4 + 4 * KC;
        if (lds > 64 * 1024) break;
        const long blocks = (long)d.n * ((dw.ho + th - 1) / th) * co_tiles;
        long per_cu = (160 * 1024) / lds;
        if (per_cu > 4) per_cu = 4;
        const long rounds = (blocks + per_cu * device_cu_count() - 1) / (per_cu * device_cu_count());
        const long cost = rounds * ir;
        if (!ok || cost < best) {
            *out = QPlan{th, ir, xw, xplane, npx, nf, nj <= 1 ? 1 : (nj <= 2 ? 2 : 4), lds};
            best = cost;
            ok = true;
        }
    }
    return ok;
}

template <int MI>
const void* pick_nj(int nj) {
    if (nj == 1) return (const void*)qfused_dw_pw_kernel<MI, 1>;
    if (nj == 2) return (const void*)qfused_dw_pw_kernel<MI, 2>;
    return (const void*)qfused_dw_pw_kernel<MI, 4>;
}

}  // namespace

bool plan_qfused_dw_pw(const Desc& dw, const Desc& pw) {
    if (dw.p.k_h * dw.p.k_w > KHW_MAX) return false;
    if ((int64_t)dw.p.h * dw.p.w >= INT32_MAX / 2 || (int64_t)dw.ho * dw.wo >= INT32_MAX / 2) return false;
    QPlan pl{};
    return qplan(dw, pw, &pl);
}

hipError_t launch_qfused_dw_pw(const Desc& dw, const Desc& pw, ConvArgs adw, ConvArgs apw, float comp_dw,
                               float comp_pw, int y_zp, hipStream_t s) {
    QFastPlan fp{};
    if (qfast_plan(dw, pw, adw.xptr, adw.wptr, apw.wptr, &fp)) return launch_qfast(dw, pw, fp, adw, apw, comp_dw, comp_pw, y_zp, s);
    QPlan pl{};
    if (!qplan(dw, pw, &pl)) return hipErrorInvalidConfiguration;
    QFArgs f;
    f.dw = adw;
    f.pw = apw;
    f.comp_dw = comp_dw;
    f.comp_pw = comp_pw;
    f.rnd_dw = dw.p.int8_rounding;
    f.rnd_pw = pw.p.int8_rounding;
    f.relu_dw = dw.p.act_type == CONV_ACT_RELU;
    f.relu_pw = pw.p.act_type == CONV_ACT_RELU;
    f.y_zp = y_zp;
    const int mi = pw.p.c_out <= 16 ? 1 : pw.p.c_out <= 32 ? 2 : pw.p.c_out <= 48 ? 3 : 4;
    f.th = pl.th;
    f.tiles_h = (dw.ho + pl.th - 1) / pl.th;
    f.co_tiles = (pw.p.c_out + 16 * mi - 1) / (16 * mi);
    f.ir = pl.ir;
    f.xw = pl.xw;
    f.xplane = pl.xplane;
    f.npx = pl.npx;
    f.nf = pl.nf;
    const int64_t hw = (int64_t)dw.p.h * dw.p.w;
    f.vec = dw.p.w % 4 == 0 && ((uintptr_t)adw.xptr % 4) == 0 && ((int64_t)adw.in_off * hw) % 4 == 0 &&
            ((int64_t)adw.in_total * hw) % 4 == 0;
    const uint64_t blocks = (uint64_t)f.co_tiles * f.tiles_h * adw.n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0xFFFFFFFFull) return hipErrorInvalidConfiguration;
    f.num_blocks = (uint32_t)blocks;
    const void* fn = mi == 1 ? pick_nj<1>(pl.nj) : mi == 2 ? pick_nj<2>(pl.nj) : mi == 3 ? pick_nj<3>(pl.nj) : pick_nj<4>(pl.nj);
    void* args[] = {&f};
    return hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(kT), args, pl.lds, s);
}

}  // namespace conv2d
