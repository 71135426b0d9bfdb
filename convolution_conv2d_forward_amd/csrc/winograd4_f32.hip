// Winograd F(4x4, 3x3) convolution, fp32, weights bound to the descriptor:
// 3x3 windows, stride 1, dilation 1, one group.  The Go package doc "ops"
// (section WorkerPool) names "Winograd cells" among its conv fan-out sites;
// this is the larger minimal-filtering tile of Lavin and Gray, "Fast
// Algorithms for Convolutional Neural Networks" (CVPR 2016), whose transform
// matrices for F(4x4, 3x3) are
//   G   = [1/4 0 0; -1/6 -1/6 -1/6; -1/6 1/6 -1/6; 1/24 1/12 1/6;
//          1/24 -1/12 1/6; 0 0 1]                                (6 x 3)
//   B^T = [4 0 -5 0 1 0; 0 -4 -4 1 1 0; 0 4 -4 -1 1 0;
//          0 -2 -1 2 1 0; 0 2 -1 -2 1 0; 0 4 0 -5 0 1]           (6 x 6)
//   A^T = [1 1 1 1 1 0; 0 1 -1 2 -2 0; 0 1 1 4 4 0; 0 1 -1 8 -8 1] (4 x 6)
// U = G g G^T per filter (once, when the weights are bound), V = B^T d B per
// 6x6 input tile d (tiles 4 apart), M = the sum over input channels of
// U (.) V at each of the 36 positions, Y = A^T M A: a 4x4 output tile for
// 36 multiplies per input channel instead of 144.  In exact arithmetic Y is
// the 3x3 correlation; in fp32 it differs by rounding, more than F(2x2)
// since the transforms carry larger constants (the parity tests bound it by
// 1e-4 * (1 + |y|)).
//
// Workgroup: 512 threads (8 waves), 2 x 8 output tiles (8 x 32 pixels) of
// one image and 32 output channels; input channels in chunks of 16.  As in
// the F(2x2) kernel the waves are specialized, one of each kind per SIMD:
//   matrix waves 0-3: wave mw owns positions 9*mw .. 9*mw+8; per chunk it
//     multiplies U (registers, each position reloaded for the next chunk
//     right after its MFMAs) by V (LDS) on the fp32 matrix cores,
//     v_mfma_f32_16x16x4f32 with U as the first operand (a lane ends up
//     holding output channels 4*(lane/16)+v of tile lane%16);
//   transform waves 4-7: load the 10 x 34 input patches three chunks ahead,
//     store them to LDS two chunks ahead and turn the next chunk's patch
//     into V, one (input channel, tile) per thread.
// Patch and V are double-buffered; one barrier per chunk.  At the end the
// 36 positions of every (channel, tile) are gathered through LDS and one
// thread per (channel, tile) applies A^T M A, the bias and the activation
// and stores its 4 x 4 pixels (ConcatFusedTail offsets included).
#include "device_common.h"

namespace conv2d {

namespace {

constexpr int kT = 512;
constexpr int TR = 2, TC = 8;              // output tiles per workgroup (rows, columns)
constexpr int PH = 4 * TR + 2;             // input patch rows
constexpr int PW = 4 * TC + 2;             // input patch columns
constexpr int PPL = PH * PW;               // patch floats per channel
constexpr int KC = 16;                     // input channels per chunk
constexpr int COT = 32;                    // output channels per workgroup
constexpr int NP = 36;                     // Winograd positions
constexpr int PPW = NP / 4;                // positions per matrix wave
constexpr int NX = (KC * PPL + 255) / 256; // patch values per transform thread and chunk
constexpr int MS = 20;                     // gathered M row stride
constexpr int LDS_PATCH = KC * PPL;
constexpr int LDS_V = NP * KC * 16;
constexpr int LDS_M = NP * COT * MS;
constexpr int LDS_FLOATS = 2 * LDS_PATCH + 2 * LDS_V > LDS_M ? 2 * LDS_PATCH + 2 * LDS_V : LDS_M;
constexpr int UCHUNK = 4 * PPW * 64 * 8;   // packed U floats per (channel tile, chunk)

struct Wino4Args {
    ConvArgs a;
    int32_t tiles_h, tiles_w;        // output tiles per image (rows, columns)
    int32_t bh, bw, co_tiles;        // workgroup tiles per image (rows, columns), channel tiles
    int32_t nch;                     // input-channel chunks
    uint32_t num_blocks;
    DivU32 dv_co_tiles, dv_bw, dv_bh;
};

// V is stored [position][channel][tile ^ ((channel >> 1) & 7)]: a transform
// wave's stores (16 channels x 4 tiles) and a matrix wave's operand reads (4
// channels x 16 tiles) both fall on 64 distinct banks.
__device__ __forceinline__ int vswz(int ci) { return (ci >> 1) & 7; }

__global__ __launch_bounds__(kT) void winograd4_kernel(Wino4Args f) {
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
    const int ty0 = by * TR, tx0 = bx * TC;
    const int C = a.c_in;
    const int64_t HW = (int64_t)a.h * a.w;
    const int nch = f.nch;

    float* patch = lds;                                // [2][KC][PH][PW]
    float* vs = lds + 2 * LDS_PATCH;                   // [2][36][KC][16], tile column swizzled
    float* ms = lds;                                   // [36][COT][MS] (after the last chunk)

    if (wave >= 4) {
        // ---------------- transform waves ----------------
        const int tt = tid - 256;
        const float* __restrict__ xg = (const float*)a.xptr + ((int64_t)n * a.in_total + a.in_off) * HW;
        const float pv = a.pad_value;
        const int ih0 = 4 * ty0 - a.pad_top, iw0 = 4 * tx0 - a.pad_left;
        // Patch slot u = tt + 256*i (its LDS offset within a buffer): channel
        // chn[i] of the chunk, image offset goff[i] when inside the image.
        uint32_t goff[NX];
        int chn[NX];
        uint32_t inimg = 0;
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int u = tt + 256 * i;
            const int ch = u / PPL, rem = u - ch * PPL;
            const int r = rem / PW, col = rem - r * PW;
            const int ih = ih0 + r, iw = iw0 + col;
            const bool in = u < KC * PPL && (unsigned)ih < (unsigned)a.h && (unsigned)iw < (unsigned)a.w;
            chn[i] = u < KC * PPL ? ch : KC;           // slots past the patch: never loaded or stored
            goff[i] = in ? (uint32_t)(ch * HW + (int64_t)ih * a.w + iw) : 0u;
            inimg |= (in ? 1u : 0u) << i;
        }
        float px[NX];
        auto load = [&](int c) __attribute__((always_inline)) {
            const float* __restrict__ xc = xg + (int64_t)c * KC * HW;
            const int lim = min(C - c * KC, KC);
#pragma unroll
            for (int i = 0; i < NX; ++i)
                if (chn[i] < lim && ((inimg >> i) & 1u)) px[i] = xc[goff[i]];
        };
        auto store = [&](int c, float* dst) __attribute__((always_inline)) {
            const int lim = C - c * KC;
#pragma unroll
            for (int i = 0; i < NX; ++i)
                if (chn[i] < KC) dst[tt + 256 * i] = chn[i] < lim ? (((inimg >> i) & 1u) ? px[i] : pv) : 0.0f;
        };
        // V = B^T d B of one (channel, tile): lanes 16 channels x 4 tiles.
        const int ci = tt & 15, t = tt >> 4;
        const int tr = t / TC, tc = t - tr * TC;
        const int rbase = ci * PPL + 4 * tr * PW + 4 * tc;
        const int wbase = ci * 16 + (t ^ vswz(ci));
        // One row (or column) of B^T applied to six values.
        auto bt = [](const float (&x)[6], float (&y)[6]) __attribute__((always_inline)) {
            y[0] = 4.0f * x[0] - 5.0f * x[2] + x[4];
            y[1] = -4.0f * (x[1] + x[2]) + x[3] + x[4];
            y[2] = 4.0f * (x[1] - x[2]) - x[3] + x[4];
            y[3] = 2.0f * (x[3] - x[1]) - x[2] + x[4];
            y[4] = 2.0f * (x[1] - x[3]) - x[2] + x[4];
            y[5] = 4.0f * x[1] - 5.0f * x[3] + x[5];
        };
        auto transform = [&](const float* pin, float* vout) __attribute__((always_inline)) {
            const float* p = pin + rbase;
            float b[6][6];                             // B^T d, column by column
#pragma unroll
            for (int j = 0; j < 6; ++j) {
                float col[6], o[6];
#pragma unroll
                for (int i = 0; i < 6; ++i) col[i] = p[i * PW + j];
                bt(col, o);
#pragma unroll
                for (int i = 0; i < 6; ++i) b[i][j] = o[i];
            }
            float* dst = vout + wbase;
#pragma unroll
            for (int i = 0; i < 6; ++i) {             // (B^T d) B, row by row
                float o[6];
                bt(b[i], o);
#pragma unroll
                for (int j = 0; j < 6; ++j) dst[(6 * i + j) * KC * 16] = o[j];
            }
        };
        load(0);
        store(0, patch);
        if (nch > 1) {
            load(1);
            store(1, patch + LDS_PATCH);
        }
        if (nch > 2) load(2);
        __syncthreads();
        transform(patch, vs);
        __syncthreads();
        for (int c = 0; c < nch; ++c) {
            const int b = c & 1;
            if (c + 1 < nch) transform(patch + (b ^ 1) * LDS_PATCH, vs + (b ^ 1) * LDS_V);
            if (c + 2 < nch) store(c + 2, patch + b * LDS_PATCH);   // chunk c's patch was transformed last iteration
            if (c + 3 < nch) load(c + 3);
            __syncthreads();
        }
        __syncthreads();                               // the matrix waves have gathered M
    } else {
        // ---------------- matrix waves ----------------
        const int mw = wave, kq = lane >> 4, l16 = lane & 15;
        const float4* __restrict__ ub =
            (const float4*)((const float*)a.wptr + (int64_t)cot * nch * UCHUNK + mw * PPW * 64 * 8 + lane * 8);
        int roff[KC / 4];                              // V operand of step ks: row 4*ks + kq, swizzled column
#pragma unroll
        for (int ks = 0; ks < KC / 4; ++ks) roff[ks] = (4 * ks + kq) * 16 + (l16 ^ vswz(4 * ks + kq));
        f32x4 acc[PPW][2];
#pragma unroll
        for (int p = 0; p < PPW; ++p)
#pragma unroll
            for (int m = 0; m < 2; ++m) acc[p][m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        // U of this wave's positions: 8 floats per lane and position, (output
        // channel half m, k step ks) at 4*m + ks.  One register set: as soon
        // as position p of chunk c has been multiplied, its registers are
        // reloaded with position p of chunk c+1, which lands while the rest
        // of the chunk runs.  Past the last chunk the loads repeat it, so
        // every chunk issues the same loads and the waits stay exact.
        float4 u[2 * PPW];
        auto load_pos = [&](int c, int p) __attribute__((always_inline)) {
            const float4* src = ub + (int64_t)c * (UCHUNK / 4) + p * 128;
            u[2 * p] = src[0];
            u[2 * p + 1] = src[1];
        };
#pragma unroll
        for (int p = 0; p < PPW; ++p) load_pos(0, p);
        __syncthreads();
        __syncthreads();
        for (int c = 0; c < nch; ++c) {
            const float* vin = vs + (c & 1) * LDS_V;
            const int cn = min(c + 1, nch - 1);
#pragma unroll
            for (int p = 0; p < PPW; ++p) {
                float bv[KC / 4];
#pragma unroll
                for (int ks = 0; ks < KC / 4; ++ks) bv[ks] = vin[(PPW * mw + p) * KC * 16 + roff[ks]];
                const float ua[8] = {u[2 * p].x, u[2 * p].y, u[2 * p].z, u[2 * p].w,
                                     u[2 * p + 1].x, u[2 * p + 1].y, u[2 * p + 1].z, u[2 * p + 1].w};
#pragma unroll
                for (int ks = 0; ks < KC / 4; ++ks)
#pragma unroll
                    for (int m = 0; m < 2; ++m)
                        acc[p][m] = __builtin_amdgcn_mfma_f32_16x16x4f32(ua[4 * m + ks], bv[ks], acc[p][m], 0, 0, 0);
                load_pos(cn, p);
            }
            __syncthreads();
        }
        // ---- gather M[position][channel][tile] through LDS ----
#pragma unroll
        for (int p = 0; p < PPW; ++p) {
            const int pos = PPW * mw + p;
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int v = 0; v < 4; ++v) ms[(pos * COT + 16 * m + 4 * kq + v) * MS + l16] = acc[p][m][v];
        }
        __syncthreads();
    }

    // ---- Y = A^T M A, bias, activation, store: thread = (channel, tile) ----
    const int oc = tid >> 4, t = tid & 15;
    const int co = co0 + oc;
    const int tr = t / TC, tc = t - tr * TC;
    const int oy = 4 * (ty0 + tr), ox = 4 * (tx0 + tc);
    if (co < a.c_out && oy < a.ho && ox < a.wo) {
        float r[4][6];                                 // A^T M, column by column
#pragma unroll
        for (int j = 0; j < 6; ++j) {
            float m6[6];
#pragma unroll
            for (int i = 0; i < 6; ++i) m6[i] = ms[((6 * i + j) * COT + oc) * MS + t];
            r[0][j] = m6[0] + m6[1] + m6[2] + m6[3] + m6[4];
            r[1][j] = m6[1] - m6[2] + 2.0f * (m6[3] - m6[4]);
            r[2][j] = m6[1] + m6[2] + 4.0f * (m6[3] + m6[4]);
            r[3][j] = m6[1] - m6[2] + 8.0f * (m6[3] - m6[4]) + m6[5];
        }
        float* yc = (float*)a.yptr + ((int64_t)n * a.out_total + a.out_off + co) * ((int64_t)a.ho * a.wo);
        const ChanEpi ce = chan_epi(a, co);   // before the first row's store
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (oy + i >= a.ho) continue;
            const float* q = r[i];
            float y[4];
            y[0] = bias_act_pre(a, q[0] + q[1] + q[2] + q[3] + q[4], ce);
            y[1] = bias_act_pre(a, q[1] - q[2] + 2.0f * (q[3] - q[4]), ce);
            y[2] = bias_act_pre(a, q[1] + q[2] + 4.0f * (q[3] + q[4]), ce);
            y[3] = bias_act_pre(a, q[1] - q[2] + 8.0f * (q[3] - q[4]) + q[5], ce);
            float* row = yc + (int64_t)(oy + i) * a.wo + ox;
            if (ox + 3 < a.wo && (((uintptr_t)row) & 15) == 0) {
                *(float4*)row = make_float4(y[0], y[1], y[2], y[3]);
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (ox + v < a.wo) row[v] = y[v];
            }
        }
    }
}

// U = G g G^T of every (output channel, input channel) filter, scattered to
// the matrix waves' operand order: for (channel tile, chunk, wave mw,
// position p of the wave, lane (kq, l16)) the 8 floats of (half m, step ks)
// at 4*m + ks, lane (kq, l16) holding output channel 16*m + l16 and input
// channel 4*ks + kq of the tile and chunk.  Channels past the layer's get 0.
__global__ __launch_bounds__(256) void pack_winograd4_u(const float* __restrict__ w, float* __restrict__ u, int c_out,
                                                        int c_in, int co_tiles, int nch) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t cis = (int64_t)nch * KC;
    if (idx >= (int64_t)co_tiles * COT * cis) return;
    const int co = (int)(idx / cis), ci = (int)(idx - (int64_t)co * cis);
    float g[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) g[k] = (co < c_out && ci < c_in) ? w[((int64_t)co * c_in + ci) * 9 + k] : 0.0f;
    float t[6][3];                                     // G g
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const float g0 = g[j], g1 = g[3 + j], g2 = g[6 + j];
        t[0][j] = 0.25f * g0;
        t[1][j] = -(g0 + g1 + g2) / 6.0f;
        t[2][j] = -(g0 - g1 + g2) / 6.0f;
        t[3][j] = g0 / 24.0f + g1 / 12.0f + g2 / 6.0f;
        t[4][j] = g0 / 24.0f - g1 / 12.0f + g2 / 6.0f;
        t[5][j] = g2;
    }
    const int cot = co / COT, m = (co % COT) / 16, l16 = co % 16;
    const int c = ci / KC, ks = (ci % KC) / 4, kq = ci % 4;
    const int ln = kq * 16 + l16;
    float* base = u + ((int64_t)cot * nch + c) * UCHUNK + ln * 8 + 4 * m + ks;
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        const float r0 = t[i][0], r1 = t[i][1], r2 = t[i][2];
        const float v[6] = {0.25f * r0, -(r0 + r1 + r2) / 6.0f, -(r0 - r1 + r2) / 6.0f,
                            r0 / 24.0f + r1 / 12.0f + r2 / 6.0f, r0 / 24.0f - r1 / 12.0f + r2 / 6.0f, r2};
#pragma unroll
        for (int j = 0; j < 6; ++j) {
            const int p = 6 * i + j;
            const int mw = p / PPW, pp = p - mw * PPW;
            base[(int64_t)(mw * PPW + pp) * 64 * 8] = v[j];
        }
    }
}

}  // namespace

bool plan_winograd4_f32(const Desc& d) {
    const conv2d_params_t& p = d.p;
    if (p.dtype != CONV_DTYPE_F32 || p.k_h != 3 || p.k_w != 3 || p.stride_h != 1 || p.stride_w != 1) return false;
    if (p.dilation_h != 1 || p.dilation_w != 1 || p.groups != 1) return false;
    if ((int64_t)p.c_out * p.c_in * 9 >= INT32_MAX) return false;
    if ((int64_t)KC * p.h * p.w > (int64_t)UINT32_MAX) return false;   // 32-bit patch offsets within a chunk
    const int64_t tiles_h = (d.ho + 3) / 4, tiles_w = (d.wo + 3) / 4;
    const int64_t blocks = (int64_t)p.n * ((tiles_h + TR - 1) / TR) * ((tiles_w + TC - 1) / TC) *
                           ((p.c_out + COT - 1) / COT);
    return blocks > 0 && blocks <= 0x7FFFFFFF;
}

// AUTO with bound weights: measured faster than F(2x2) and the implicit GEMM
// with packed weights once the grid fills the GPU (batch 4-32 layers of
// 64-256 channels on 56x56 to 128x128 images: 0.82-0.91 of F(2x2)'s time);
// with fewer workgroups than CUs (the single-image dense-block layers, 64 or
// 128 of them) it is up to 2x slower, and F(2x2) keeps those.
bool winograd4_bound_preferred(const Desc& d) {
    if (!plan_winograd4_f32(d) || d.p.c_in < 32) return false;
    const int64_t blocks = (int64_t)d.p.n * (((d.ho + 3) / 4 + TR - 1) / TR) * (((d.wo + 3) / 4 + TC - 1) / TC) *
                           ((d.p.c_out + COT - 1) / COT);
    return blocks >= device_cu_count();
}

int64_t winograd4_u_bytes(const Desc& d) {
    const int64_t co_tiles = (d.p.c_out + COT - 1) / COT, nch = (d.p.c_in + KC - 1) / KC;
    return 4 * co_tiles * nch * UCHUNK;
}

hipError_t pack_winograd4_f32_weights(const Desc& d, const void* w, void* dst, hipStream_t s) {
    const int co_tiles = (d.p.c_out + COT - 1) / COT, nch = (d.p.c_in + KC - 1) / KC;
    const int64_t total = (int64_t)co_tiles * COT * nch * KC;
    if (total == 0) return hipSuccess;
    const float* wp = (const float*)w;
    float* up = (float*)dst;
    int c_out = d.p.c_out, c_in = d.p.c_in, ct = co_tiles, nc = nch;
    void* args[] = {&wp, &up, &c_out, &c_in, &ct, &nc};
    return hipLaunchKernel((const void*)pack_winograd4_u, dim3((uint32_t)((total + 255) / 256)), dim3(256), args, 0,
                           s);
}

hipError_t launch_winograd4_f32(const Desc& d, ConvArgs a, hipStream_t s, const void* upacked) {
    if (!upacked) return hipErrorInvalidValue;
    Wino4Args f;
    f.a = a;
    f.a.wptr = upacked;
    f.tiles_h = (d.ho + 3) / 4;
    f.tiles_w = (d.wo + 3) / 4;
    f.bh = (f.tiles_h + TR - 1) / TR;
    f.bw = (f.tiles_w + TC - 1) / TC;
    f.co_tiles = (d.p.c_out + COT - 1) / COT;
    f.nch = (d.p.c_in + KC - 1) / KC;
    f.dv_co_tiles = make_divu32((uint32_t)f.co_tiles);
    f.dv_bw = make_divu32((uint32_t)f.bw);
    f.dv_bh = make_divu32((uint32_t)f.bh);
    const uint64_t blocks = (uint64_t)a.n * f.bh * f.bw * f.co_tiles;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
    f.num_blocks = (uint32_t)blocks;
    const void* fn = (const void*)winograd4_kernel;
    const int lds = 4 * LDS_FLOATS;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
    }
    void* args[] = {&f};
    return hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(kT), args, lds, s);
}

}  // namespace conv2d
