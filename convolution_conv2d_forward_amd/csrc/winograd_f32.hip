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

// U = G g G^T of one 3x3 filter g (row-major): u[4*i + j], i, j = 0..3.  The
// forward kernel (weights given at each call) and the bound-weight pack use
// this one function, so both paths multiply the same U.
__device__ __forceinline__ void filter_u(const float (&g)[9], float (&u)[16]) {
    float t4[4][3];                                    // G g: rows of the 4x3 product
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
        u[4 * i + 0] = r0;
        u[4 * i + 1] = 0.5f * (r0 + r1 + r2);
        u[4 * i + 2] = 0.5f * (r0 - r1 + r2);
        u[4 * i + 3] = r2;
    }
}

// Packed U (bound weights): for each output-channel tile, chunk, wave and
// lane, the 16 values the lane's MFMAs take, in the order (e, ks, m):
// position 2*wave + e, input channel chunk*KC + 4*ks + lane/16, output
// channel tile*COT + 16*m + lane%16; zero past the channels.  One wave's
// chunk is 4 KB, read as four coalesced 16-byte loads per lane.
// MB blocks of 16 output channels per workgroup tile (2 or 4): 8 * MB floats
// per lane and chunk, in the order (e, ks, m).
template <int MB>
__global__ __launch_bounds__(256) void pack_winograd_u(const float* __restrict__ w, float* __restrict__ out,
                                                       int cin, int cout, int nch, int co_tiles) {
    constexpr int NPU = 8 * MB;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)co_tiles * nch * 8 * 64;
    if (idx >= total) return;
    const int lane = (int)(idx & 63);
    const int wave = (int)((idx >> 6) & 7);
    const int64_t rest = idx >> 9;
    const int c = (int)(rest % nch);
    const int ct = (int)(rest / nch);
    const int kq = lane >> 4, l16 = lane & 15;
    float v[NPU];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int ks = 0; ks < KC / 4; ++ks) {
            const int co = ct * 16 * MB + 16 * m + l16, ci = c * KC + 4 * ks + kq;
            float g[9], u[16];
            const bool ok = co < cout && ci < cin;
#pragma unroll
            for (int t = 0; t < 9; ++t) g[t] = ok ? w[((int64_t)co * cin + ci) * 9 + t] : 0.0f;
            filter_u(g, u);
#pragma unroll
            for (int e = 0; e < 2; ++e) v[(e * (KC / 4) + ks) * MB + m] = u[2 * wave + e];
        }
    float4* dst = (float4*)(out + idx * NPU);
#pragma unroll
    for (int q = 0; q < NPU / 4; ++q) dst[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
}

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
        float g[9], u[16];
#pragma unroll
        for (int t = 0; t < 9; ++t) {
            asm volatile("" : "+v"(R.g[t]));
            g[t] = okw ? R.g[t] : 0.0f;
        }
        filter_u(g, u);
        float* dst = us + fci * US + fco;
#pragma unroll
        for (int pos = 0; pos < 16; ++pos) dst[pos * KC * US] = u[pos];
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

// Bound weights (U packed by pack_winograd_u<MB>), pipelined: one barrier
// per input-channel chunk.  Iteration c multiplies chunk c (V from one LDS
// buffer, U from registers) while every thread transforms half of one
// (channel, tile) patch of chunk c+1 into the other V buffer and stores the
// patch of chunk c+2 (loaded one iteration earlier) into the free patch
// buffer; the loads of chunk c+3 and the U of chunk c+1 are in flight over
// the same iteration.  MFMAs and transforms share the waves, so the matrix
// core works while the VALU and LDS transform the next chunk.  The
// transforms, the 16 channel sums and the output transform are those of
// winograd_f32_kernel (same U, same V, same order of accumulation), so the
// results are bitwise equal for the same descriptor.  CO = 16*MB output
// channels per workgroup.
template <int MB>
__global__ __launch_bounds__(kT) void winograd_pu_kernel(WinoArgs f) {
    constexpr int CO = 16 * MB;
    constexpr int NPU = 8 * MB;
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
    const int co0 = cot * CO;
    const int ty0 = by * TR, tx0 = bx * TC;
    const int ih0 = 2 * ty0 - a.pad_top, iw0 = 2 * tx0 - a.pad_left;
    const int C = a.c_in, H = a.h, W = a.w;
    const int64_t HW = (int64_t)H * W;
    const int nch = (C + KC - 1) / KC;

    float* patch = lds;                                // [2][KC][PH][PW]
    float* vs = lds + 2 * LDS_PATCH;                   // [2][16][KC][VS]
    float* ms = lds;                                   // [16][CO][MS] (after the last chunk)

    const float* __restrict__ xg = (const float*)a.xptr + ((int64_t)n * a.in_total + a.in_off) * HW;
    const float* __restrict__ wu = (const float*)a.wptr;
    const float pv = a.pad_value;

    // Patch of chunk c -> registers: unconditional loads (slots outside the
    // patch or the channels read the image's first element, replaced on store).
    float px[NX];
    auto load_patch = [&](int c) __attribute__((always_inline)) {
        const int c0 = c * KC;
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int u = tid + i * kT;
            const int ch = u / PPL, rem = u - ch * PPL;
            const int r = rem / PW, col = rem - r * PW;
            const int ih = ih0 + r, iw = iw0 + col;
            const bool ok = u < KC * PPL && c0 + ch < C && (unsigned)ih < (unsigned)H && (unsigned)iw < (unsigned)W;
            px[i] = xg[ok ? (int64_t)(c0 + ch) * HW + (int64_t)ih * W + iw : 0];
        }
    };
    auto store_patch = [&](int c, float* dst) __attribute__((always_inline)) {
        const int c0 = c * KC;
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int u = tid + i * kT;
            if (u < KC * PPL) {
                const int ch = u / PPL, rem = u - ch * PPL;
                const int r = rem / PW, col = rem - r * PW;
                const int ih = ih0 + r, iw = iw0 + col;
                float v = px[i];
                if (c0 + ch >= C) v = 0.0f;                                   // past the channels: no term
                else if ((unsigned)ih >= (unsigned)H || (unsigned)iw >= (unsigned)W) v = pv;   // padded tap
                dst[u] = v;
            }
        }
    };
    // U of chunk c for this wave's lane (NPU floats, order (e, ks, m)).
    auto load_u = [&](int c, float (&u)[NPU]) __attribute__((always_inline)) {
        const float4* src = (const float4*)(wu + ((((int64_t)cot * nch + c) * 8 + wave) * 64 + lane) * NPU);
#pragma unroll
        for (int q = 0; q < NPU / 4; ++q) {
            const float4 v = src[q];
            u[4 * q] = v.x; u[4 * q + 1] = v.y; u[4 * q + 2] = v.z; u[4 * q + 3] = v.w;
        }
    };
    // V = B^T d B, half of one (channel, tile) patch per thread: rows 2h and
    // 2h+1 of B^T d (B^T rows 0, 1 use patch rows 0..2; rows 2, 3 use 1..3).
    auto transform = [&](const float* pin, float* vout) __attribute__((always_inline)) {
        const int ti = tid >> 1, h = tid & 1;
        const int ci = ti >> 4, t = ti & 15;
        const int tr = t / TC, tc = t - tr * TC;
        const float* p = pin + ci * PPL + (2 * tr + h) * PW + 2 * tc;
        float d[3][4];
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) d[i][j] = p[i * PW + j];
        float b[2][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // h = 0: d rows 0,1,2 -> b0 = d0 - d2, b1 = d1 + d2;  h = 1: d rows 1,2,3 -> b2 = d2 - d1, b3 = d1 - d3
            b[0][j] = h ? d[1][j] - d[0][j] : d[0][j] - d[2][j];
            b[1][j] = h ? d[0][j] - d[2][j] : d[1][j] + d[2][j];
        }
        float* dst = vout + ci * VS + t;
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const int i = 2 * h + ii;
            dst[(4 * i + 0) * KC * VS] = b[ii][0] - b[ii][2];
            dst[(4 * i + 1) * KC * VS] = b[ii][1] + b[ii][2];
            dst[(4 * i + 2) * KC * VS] = b[ii][2] - b[ii][1];
            dst[(4 * i + 3) * KC * VS] = b[ii][1] - b[ii][3];
        }
    };

    f32x4 acc[2][MB];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[e][m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int kq = lane >> 4, l16 = lane & 15;
    auto gemm = [&](const float* vin, const float (&u)[NPU]) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < KC / 4; ++ks)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float bv = vin[((2 * wave + e) * KC + 4 * ks + kq) * VS + l16];
#pragma unroll
                for (int m = 0; m < MB; ++m)
                    acc[e][m] = __builtin_amdgcn_mfma_f32_16x16x4f32(u[(e * (KC / 4) + ks) * MB + m], bv, acc[e][m],
                                                                     0, 0, 0);
            }
    };

    // ---- prologue: patches of chunks 0 and 1 in LDS, V of chunk 0, patch of
    // chunk 2 in registers, U of chunk 0 ----
    float ucur[NPU], unext[NPU];
    load_patch(0);
    store_patch(0, patch);
    if (nch > 1) {
        load_patch(1);
        store_patch(1, patch + LDS_PATCH);
    }
    load_u(0, ucur);
    if (nch > 2) load_patch(2);
    __syncthreads();
    transform(patch, vs);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const int b = c & 1;
        if (c + 1 < nch) load_u(c + 1, unext);
        gemm(vs + b * LDS_V, ucur);
        if (c + 1 < nch) transform(patch + (b ^ 1) * LDS_PATCH, vs + (b ^ 1) * LDS_V);
        if (c + 2 < nch) store_patch(c + 2, patch + b * LDS_PATCH);   // chunk c's patch was transformed last iteration
        if (c + 3 < nch) load_patch(c + 3);
        __syncthreads();
        if (c + 1 < nch) {
#pragma unroll
            for (int q = 0; q < NPU; ++q) ucur[q] = unext[q];
        }
    }

    // ---- gather M[position][channel][tile] through LDS ----
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int pos = 2 * wave + e;
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v) ms[(pos * CO + 16 * m + 4 * kq + v) * MS + l16] = acc[e][m][v];
    }
    __syncthreads();

    // ---- Y = A^T M A, bias, activation, store: one (channel, tile) per pass ----
    for (int pr = tid; pr < CO * NT; pr += kT) {
        const int oc = pr >> 4, t = pr & 15;
        const int co = co0 + oc;
        const int tr = t / TC, tc = t - tr * TC;
        const int oy = 2 * (ty0 + tr), ox = 2 * (tx0 + tc);
        if (co >= a.c_out || oy >= a.ho || ox >= a.wo) continue;
        float m4[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) m4[i][j] = ms[((4 * i + j) * CO + oc) * MS + t];
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

// Output channels per workgroup of the bound-weight kernel: 64 when the
// layer has more than 32 and the 32-channel grid would hold at least eight
// workgroups per CU of the 256 (the input transform is then shared by twice
// the output channels without leaving CUs idle), else 32.
int pu_mb(const Desc& d) {
    if (d.p.c_out <= 32) return 2;
    const int64_t tiles = (int64_t)((d.ho + 1) / 2 + TR - 1) / TR * (((d.wo + 1) / 2 + TC - 1) / TC);
    return (int64_t)d.p.n * tiles * ((d.p.c_out + 31) / 32) >= 8 * 256 ? 4 : 2;
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

int64_t winograd_u_bytes(const Desc& d) {
    const int mb = pu_mb(d);
    const int64_t co_tiles = (d.p.c_out + 16 * mb - 1) / (16 * mb), nch = (d.p.c_in + KC - 1) / KC;
    return co_tiles * nch * 8 * 64 * (8 * mb) * 4;
}

hipError_t pack_winograd_f32_weights(const Desc& d, const void* w, void* dst, hipStream_t s) {
    const int mb = pu_mb(d);
    const int co_tiles = (d.p.c_out + 16 * mb - 1) / (16 * mb), nch = (d.p.c_in + KC - 1) / KC;
    const int64_t total = (int64_t)co_tiles * nch * 8 * 64;
    if (total == 0) return hipSuccess;
    const float* wp = (const float*)w;
    float* op = (float*)dst;
    int cin = d.p.c_in, cout = d.p.c_out, nc = nch, ct = co_tiles;
    void* args[] = {(void*)&wp, &op, &cin, &cout, &nc, &ct};
    const void* fn = mb == 4 ? (const void*)pack_winograd_u<4> : (const void*)pack_winograd_u<2>;
    return hipLaunchKernel(fn, dim3((uint32_t)((total + 255) / 256)), dim3(256), args, 0, s);
}

hipError_t launch_winograd_f32(const Desc& d, ConvArgs a, hipStream_t s, const void* upacked) {
    WinoArgs f;
    f.a = a;
    f.tiles_h = (d.ho + 1) / 2;
    f.tiles_w = (d.wo + 1) / 2;
    f.bh = (f.tiles_h + TR - 1) / TR;
    f.bw = (f.tiles_w + TC - 1) / TC;
    const int mb = pu_mb(d);
    const bool pu = upacked && (uintptr_t)upacked % 16 == 0;
    f.co_tiles = pu ? (d.p.c_out + 16 * mb - 1) / (16 * mb) : (d.p.c_out + COT - 1) / COT;
    const uint64_t blocks = (uint64_t)a.n * f.bh * f.bw * f.co_tiles;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
    f.num_blocks = (uint32_t)blocks;
    f.dv_co_tiles = make_divu32((uint32_t)f.co_tiles);
    f.dv_bw = make_divu32((uint32_t)f.bw);
    f.dv_bh = make_divu32((uint32_t)f.bh);
    int lds = LDS_FLOATS * 4;
    const void* fn = (const void*)winograd_f32_kernel;
    if (pu) {
        f.a.wptr = upacked;
        fn = mb == 4 ? (const void*)winograd_pu_kernel<4> : (const void*)winograd_pu_kernel<2>;
        const int pipe = 2 * LDS_PATCH + 2 * LDS_V, gather = 16 * 16 * mb * MS;
        lds = 4 * (pipe > gather ? pipe : gather);
    }
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
    }
    void* args[] = {&f};
    return hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(kT), args, lds, s);
}

}  // namespace conv2d
