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

int cu_count_q() {
    static int cached = 0;
    if (cached == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            cached = v;
        else
            cached = 256;
    }
    return cached;
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
        const long rounds = (blocks + per_cu * cu_count_q() - 1) / (per_cu * cu_count_q());
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
