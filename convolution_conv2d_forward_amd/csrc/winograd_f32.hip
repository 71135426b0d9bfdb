// Winograd F(2x2, 3x3) convolution, fp32: 3x3 windows, stride 1, dilation 1,
// one group.  The Go package doc "ops" (section WorkerPool) names "Winograd
// cells" among its conv fan-out sites without describing them; the transforms
// here are the minimal-filtering algorithm F(2x2, 3x3) of Lavin and Gray,
// "Fast Algorithms for Convolutional Neural Networks" (CVPR 2016):
//   U = G g G^T     G   = [1 0 0; 1/2 1/2 1/2; 1/2 -1/2 1/2; 0 0 1]
//   V = B^T d B     B^T = [1 0 -1 0; 0 1 1 0; 0 -1 1 0; 0 1 0 -1]
//   M = sum over input channels of U (.) V   (16 independent GEMMs)
//   Y = A^T M A     A^T = [1 1 1 0; 0 1 -1 -1]
// for every 4x4 input tile d (tiles 2 apart) and its 2x2 output tile Y.
// In exact arithmetic Y is the 3x3 correlation; in fp32 it differs from it by
// rounding only (9 multiplies per output become 4 per tile and channel).
//
// Workgroup: 512 threads (8 waves), TR x TC = 2 x 8 output tiles (4 x 16
// pixels) of one image, COT = 32 output channels.  Input channels are walked
// in chunks of KC = 16:
//   1. the chunk's 6 x 18 input patch (pads hold pad_value) and its 3x3
//      filters are loaded into registers two chunks ahead; the patch goes to
//      LDS;
//   2. threads 0..255 transform one (channel, tile) patch each into V, all
//      512 threads one (output channel, input channel) filter each into U,
//      both written to LDS as [position][k][column];
//   3. wave w multiplies positions 2w and 2w+1 on the fp32 matrix cores
//      (v_mfma_f32_16x16x4f32, U as the first operand: a lane ends up
//      holding output channels 4*(lane/16)+v of tile lane%16).
// At the end the 16 positions of every (channel, tile) are gathered through
// LDS, and one thread per (channel, tile) applies A^T M A, the bias and the
// activation and stores its 2x2 pixels (ConcatFusedTail offsets included).
#include "device_common.h"

namespace conv2d {

namespace {

constexpr int kT = 512;
constexpr int TR = 2, TC = 8;              // output tiles per workgroup (rows, columns)
constexpr int NT = TR * TC;                // 16: one MFMA column fragment
constexpr int PH = 2 * TR + 2;             // input patch rows
constexpr int PW = 2 * TC + 2;             // input patch columns
constexpr int PPL = PH * PW;               // patch floats per channel
constexpr int KC = 16;                     // input channels per chunk
constexpr int COT = 32;                    // output channels per workgroup
constexpr int NX = (KC * PPL + kT - 1) / kT;   // patch loads per thread and chunk
constexpr int VS = NT;                     // V row stride: 16 floats (4 k-rows hit 64 banks)
constexpr int US = 48;                     // U row stride: 32 channels padded to 48 (= 16 mod 32)
constexpr int MS = 20;                     // gathered M row stride
constexpr int LDS_PATCH = KC * PPL;                    // floats
constexpr int LDS_V = 16 * KC * VS;
constexpr int LDS_U = 16 * KC * US;
constexpr int LDS_M = 16 * COT * MS;
constexpr int LDS_FLOATS = LDS_PATCH + (LDS_V + LDS_U > LDS_M ? LDS_V + LDS_U : LDS_M);

struct WinoArgs {
    ConvArgs a;
    int32_t tiles_h, tiles_w;        // output tiles per image (rows, columns)
    int32_t bh, bw, co_tiles;        // workgroup tiles per image (rows, columns), channel tiles
    uint32_t num_blocks;
    DivU32 dv_co_tiles, dv_bw, dv_bh;
};

template <int N>
struct WRegs {
    float x[N];
    float g[9];
};

__global__ __launch_bounds__(kT) void winograd_f32_kernel(WinoArgs f) {
    extern __shared__ __align__(16) float lds[];
    const ConvArgs& a = f.a;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    uint32_t L = xcd_remap(blockIdx.x, f.num_blocks);
    uint32_t Q = divu(L, f.dv_co_tiles);
    const int cot = L - Q * f.co_tiles;
    L = Q;
    Q = divu(L, f.dv_bw);
    const int bx = L - Q * f.bw;
    L = Q;
    Q = divu(L, f.dv_bh);
    const int by = L - Q * f.bh;
    const int n = Q;
    const int co0 = cot * COT;
    const int ty0 = by * TR, tx0 = bx * TC;            // first output tile
    const int ih0 = 2 * ty0 - a.pad_top, iw0 = 2 * tx0 - a.pad_left;
    const int C = a.c_in, H = a.h, W = a.w;
    const int64_t HW = (int64_t)H * W;
    const int nch = (C + KC - 1) / KC;

    float* patch = lds;                                // [KC][PH][PW]
    float* vs = lds + LDS_PATCH;                       // [16][KC][VS]
    float* us = vs + LDS_V;                            // [16][KC][US]
    float* ms = lds + LDS_PATCH;                       // [16][COT][MS] (after the last chunk)

    const float* __restrict__ xg = (const float*)a.xptr + ((int64_t)n * a.in_total + a.in_off) * HW;
    const float* __restrict__ wg = (const float*)a.wptr;
    const float pv = a.pad_value;

    // ---- chunk loads: issued unconditionally (slots outside the patch or the
    // channels read the image's first element and are replaced when stored),
    // each register pinned to its use so no wait covers the next chunk ----
    using Regs = WRegs<NX>;
    const int fco = tid & 31, fci = tid >> 5;          // this thread's filter: (output, input) channel
    auto load_chunk = [&](int c, Regs& R) __attribute__((always_inline)) {
        const int c0 = c * KC;
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int u = tid + i * kT;
            const int ch = u / PPL, rem = u - ch * PPL;
            const int r = rem / PW, col = rem - r * PW;
            const int ih = ih0 + r, iw = iw0 + col;
            const bool ok = u < KC * PPL && c0 + ch < C && (unsigned)ih < (unsigned)H && (unsigned)iw < (unsigned)W;
            R.x[i] = xg[ok ? (int64_t)(c0 + ch) * HW + (int64_t)ih * W + iw : 0];
        }
        const bool okw = co0 + fco < a.c_out && c0 + fci < C;
        const float* src = wg + (okw ? ((int64_t)(co0 + fco) * C + c0 + fci) * 9 : 0);
#pragma unroll
        for (int t = 0; t < 9; ++t) R.g[t] = src[t];
    };
    auto store_patch = [&](int c, Regs& R) __attribute__((always_inline)) {
        const int c0 = c * KC;
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            asm volatile("" : "+v"(R.x[i]));
            const int u = tid + i * kT;
            if (u < KC * PPL) {
                const int ch = u / PPL, rem = u - ch * PPL;
                const int r = rem / PW, col = rem - r * PW;
                const int ih = ih0 + r, iw = iw0 + col;
                float v = R.x[i];
                if (c0 + ch >= C) v = 0.0f;                                   // past the channels: no term
                else if ((unsigned)ih >= (unsigned)H || (unsigned)iw >= (unsigned)W) v = pv;   // padded tap
                patch[u] = v;
            }
        }
    };
    // U = G g G^T of this thread's filter (zero past the channels).
    auto filter_transform = [&](int c, Regs& R) __attribute__((always_inline)) {
        const int c0 = c * KC;
        const bool okw = co0 + fco < a.c_out && c0 + fci < C;
        float g[9];
#pragma unroll
        for (int t = 0; t < 9; ++t) {
            asm volatile("" : "+v"(R.g[t]));
            g[t] = okw ? R.g[t] : 0.0f;
        }
        float t4[4][3];                                // G g: rows of the 4x3 product
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const float g0 = g[j], g1 = g[3 + j], g2 = g[6 + j];
            t4[0][j] = g0;
            t4[1][j] = 0.5f * (g0 + g1 + g2);
            t4[2][j] = 0.5f * (g0 - g1 + g2);
            t4[3][j] = g2;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float r0 = t4[i][0], r1 = t4[i][1], r2 = t4[i][2];
            float* dst = us + (4 * i) * KC * US + fci * US + fco;
            dst[0 * KC * US] = r0;
            dst[1 * KC * US] = 0.5f * (r0 + r1 + r2);
            dst[2 * KC * US] = 0.5f * (r0 - r1 + r2);
            dst[3 * KC * US] = r2;
        }
    };
    // V = B^T d B of one (channel, tile) patch.
    auto input_transform = [&]() __attribute__((always_inline)) {
        if (tid < KC * NT) {
            const int ci = tid >> 4, t = tid & 15;
            const int tr = t / TC, tc = t - tr * TC;
            const float* p = patch + ci * PPL + (2 * tr) * PW + 2 * tc;
            float d[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) d[i][j] = p[i * PW + j];
            float b[4][4];                             // B^T d
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                b[0][j] = d[0][j] - d[2][j];
                b[1][j] = d[1][j] + d[2][j];
                b[2][j] = d[2][j] - d[1][j];
                b[3][j] = d[1][j] - d[3][j];
            }
            float* dst = vs + ci * VS + t;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dst[(4 * i + 0) * KC * VS] = b[i][0] - b[i][2];
                dst[(4 * i + 1) * KC * VS] = b[i][1] + b[i][2];
                dst[(4 * i + 2) * KC * VS] = b[i][2] - b[i][1];
                dst[(4 * i + 3) * KC * VS] = b[i][1] - b[i][3];
            }
        }
    };

    // ---- the 16 GEMMs: wave w owns positions 2w, 2w+1 ----
    f32x4 acc[2][2];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int m = 0; m < 2; ++m) acc[e][m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int kq = lane >> 4, l16 = lane & 15;
    auto gemm = [&]() __attribute__((always_inline)) {
        float av[2][KC / 4][2], bv[2][KC / 4];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int pos = 2 * wave + e;
#pragma unroll
            for (int ks = 0; ks < KC / 4; ++ks) {
                const int k = 4 * ks + kq;
                bv[e][ks] = vs[(pos * KC + k) * VS + l16];
#pragma unroll
                for (int m = 0; m < 2; ++m) av[e][ks][m] = us[(pos * KC + k) * US + 16 * m + l16];
            }
        }
#pragma unroll
        for (int ks = 0; ks < KC / 4; ++ks)
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    acc[e][m] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e][ks][m], bv[e][ks], acc[e][m], 0, 0, 0);
    };

    // Chunk c: patch registers -> LDS, barrier (the previous chunk's MFMAs have
    // read U and V), loads of chunk cn into the same registers, transforms,
    // barrier, MFMAs.  An even number of steps with fixed register sets, loads
    // in every step (the last ones reload the last chunk): no load sits behind
    // a condition.
    auto step = [&](int c, Regs& R, int cn) __attribute__((always_inline)) {
        store_patch(c, R);
        __syncthreads();
        filter_transform(c, R);
        load_chunk(cn, R);
        if (c < nch) {
            input_transform();
            __syncthreads();
            gemm();
        }
    };
    const int nch2 = (nch + 1) & ~1;
    Regs R0, R1;
    load_chunk(0, R0);
    load_chunk(1, R1);
    for (int c = 0; c < nch2; c += 2) {
        step(c, R0, min(c + 2, nch2 - 1));
        step(c + 1, R1, min(c + 3, nch2 - 1));
    }

    // ---- gather M[position][channel][tile] through LDS ----
    __syncthreads();                                   // every wave is done with U and V
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int pos = 2 * wave + e;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v) ms[(pos * COT + 16 * m + 4 * kq + v) * MS + l16] = acc[e][m][v];
    }
    __syncthreads();

    // ---- Y = A^T M A, bias, activation, store: thread = (channel, tile) ----
    const int oc = tid >> 4, t = tid & 15;
    const int co = co0 + oc;
    const int tr = t / TC, tc = t - tr * TC;
    const int oy = 2 * (ty0 + tr), ox = 2 * (tx0 + tc);
    if (co < a.c_out && oy < a.ho && ox < a.wo) {
        float m4[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) m4[i][j] = ms[((4 * i + j) * COT + oc) * MS + t];
        float r[2][4];                                 // A^T M
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            r[0][j] = m4[0][j] + m4[1][j] + m4[2][j];
            r[1][j] = m4[1][j] - m4[2][j] - m4[3][j];
        }
        float y[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            y[i][0] = bias_act(a, r[i][0] + r[i][1] + r[i][2], co);
            y[i][1] = bias_act(a, r[i][1] - r[i][2] - r[i][3], co);
        }
        float* yc = (float*)a.yptr + ((int64_t)n * a.out_total + a.out_off + co) * ((int64_t)a.ho * a.wo);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (oy + i >= a.ho) continue;
            float* row = yc + (int64_t)(oy + i) * a.wo + ox;
            if (ox + 1 < a.wo && (((uintptr_t)row) & 7) == 0) {
                *(float2*)row = make_float2(y[i][0], y[i][1]);
            } else {
                row[0] = y[i][0];
                if (ox + 1 < a.wo) row[1] = y[i][1];
            }
        }
    }
}

}  // namespace

bool plan_winograd_f32(const Desc& d) {
    const conv2d_params_t& p = d.p;
    if (p.dtype != CONV_DTYPE_F32 || p.k_h != 3 || p.k_w != 3 || p.stride_h != 1 || p.stride_w != 1) return false;
    if (p.dilation_h != 1 || p.dilation_w != 1 || p.groups != 1) return false;
    if ((int64_t)p.c_out * p.c_in * 9 >= INT32_MAX) return false;
    const int64_t tiles_h = (d.ho + 1) / 2, tiles_w = (d.wo + 1) / 2;
    const int64_t blocks = (int64_t)p.n * ((tiles_h + TR - 1) / TR) * ((tiles_w + TC - 1) / TC) *
                           ((p.c_out + COT - 1) / COT);
    return blocks > 0 && blocks <= 0x7FFFFFFF;
}

hipError_t launch_winograd_f32(const Desc& d, ConvArgs a, hipStream_t s) {
    WinoArgs f;
    f.a = a;
    f.tiles_h = (d.ho + 1) / 2;
    f.tiles_w = (d.wo + 1) / 2;
    f.bh = (f.tiles_h + TR - 1) / TR;
    f.bw = (f.tiles_w + TC - 1) / TC;
    f.co_tiles = (d.p.c_out + COT - 1) / COT;
    const uint64_t blocks = (uint64_t)a.n * f.bh * f.bw * f.co_tiles;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
    f.num_blocks = (uint32_t)blocks;
    f.dv_co_tiles = make_divu32((uint32_t)f.co_tiles);
    f.dv_bw = make_divu32((uint32_t)f.bw);
    f.dv_bh = make_divu32((uint32_t)f.bh);
    const int lds = LDS_FLOATS * 4;
    const void* fn = (const void*)winograd_f32_kernel;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
    }
    void* args[] = {&f};
    return hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(kT), args, lds, s);
}

}  // namespace conv2d
