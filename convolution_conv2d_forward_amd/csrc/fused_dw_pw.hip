// Fused depthwise kxk -> pointwise 1x1 (the FusedDwPw step of the yscv
// "ONNX CPU Kernels" page, section "Hot kernel paths": the depthwise rows
// feed the pointwise GEMM from on-chip memory, so the depthwise output is
// never written to main memory).
//
// Workgroup tile: one image, TH output rows of full width, COT (32 or 64)
// pointwise output channels.  The depthwise channels (= the pointwise K) are
// walked in chunks of KC = 32:
//   1. the chunk's input rows (TH rows of output need IR input rows, halo
//      included) are loaded into registers one chunk ahead and written to an
//      LDS tile whose pad rows and columns hold the depthwise pad_value
//      (written once: they are the same for every chunk); the chunk's
//      pointwise weights go to LDS as [k][co] at the same time;
//   2. the depthwise conv reads VO outputs of one row per thread unit out of
//      that tile (register window), adds its bias, applies its activation and
//      writes the result to LDS as the GEMM's B operand, [k][pixel];
//   3. Y[co, pixel] += W_pw[co, k] * D[k, pixel] runs on the fp32 matrix
//      cores (v_mfma_f32_16x16x4f32, the pixel fragment as first operand so a
//      lane ends up holding 4 consecutive pixels of one output channel).
// The depthwise result and the pointwise weights are double-buffered, so a
// chunk costs two workgroup barriers.  The epilogue adds the pointwise bias,
// applies its activation and stores 16-byte vectors into channel
// out_off + co of a buffer with out_total channels (ConcatFusedTail).
// With more output channels than one tile holds, each channel tile redoes the
// depthwise conv of its pixels (the planner counts that).
#include "device_common.h"

namespace conv2d {

namespace {

constexpr int kT = 512;
constexpr int kWaves = kT / 64;
constexpr int KC = 32;        // depthwise channels per chunk
constexpr int VO = 4;         // depthwise outputs per thread unit (one row)
constexpr int NXV = 8;        // 16-byte input loads per thread and chunk (upper bound)
constexpr int NSC = 8;        // scalar-path input elements per thread and chunk, in units of kT

struct DwPwArgs {
    ConvArgs dw, pw;
    int32_t th, tiles_h, co_tiles, cot;
    int32_t ir;            // input rows per tile
    int32_t xoff;          // LDS column of image column 0 (a multiple of 4, >= pad_left)
    int32_t xw;            // LDS row stride of the input tile
    int32_t xs_plane;      // LDS floats per channel of the input tile
    int32_t npx, nf;       // pixels of a tile (th * wo) and 16-pixel fragments
    int32_t es_stride;     // LDS floats per channel of the depthwise result (= 16 mod 64)
    int32_t cop;           // LDS row stride of the pointwise weight chunk (= 16 mod 64)
    int32_t vec;           // input rows move as 16-byte vectors
    uint32_t num_blocks;
    DivU32 dv_co_tiles, dv_tiles_h;
};

__host__ __device__ inline int stride16(int n) {   // smallest s >= n with s % 64 == 16
    int s = (n + 47) / 64 * 64 + 16;
    return s < n ? s + 64 : s;
}

// KH/KW/SS > 0: fixed 3x3 window with stride SS and dilation 1 (the reads are
// constant offsets); 0: any window up to 5x5 with the descriptor's stride and
// dilation.  MI: 16-channel output fragments (COT / 16).  NJ: pixel fragments
// per wave.
template <int KH, int KW, int SS, int MI, int NJ>
__global__ __launch_bounds__(kT) void fused_dw_pw_kernel(DwPwArgs f) {
    extern __shared__ __align__(16) float lds[];
    const ConvArgs& D = f.dw;
    const ConvArgs& P = f.pw;
    constexpr bool FIXED = KH > 0;
    const int kh = FIXED ? KH : D.k_h, kw = FIXED ? KW : D.k_w;
    const int sh = FIXED ? SS : D.stride_h, sw = FIXED ? SS : D.stride_w;
    const int dh = FIXED ? 1 : D.dilation_h, dwl = FIXED ? 1 : D.dilation_w;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, l16 = lane & 15;

    uint32_t L = xcd_remap(blockIdx.x, f.num_blocks);
    uint32_t Q = divu(L, f.dv_co_tiles);
    const int cot = L - Q * f.co_tiles;
    L = Q; Q = divu(L, f.dv_tiles_h);
    const int tht = L - Q * f.tiles_h;
    const int n = Q;
    const int co0 = cot * f.cot;
    const int ho0 = tht * f.th;
    const int th_n = min(f.th, D.ho - ho0);                 // output rows of this tile
    const int ih0 = ho0 * sh - D.pad_top;                   // image row of tile input row 0
    const int C = D.c_out, W = D.w, H = D.h, WO = D.wo;
    const int64_t HW = (int64_t)H * W;
    const int nch = (C + KC - 1) / KC;

    float* xs = lds;                                        // [KC][ir][xw]
    float* es0 = xs + KC * f.xs_plane;                      // [KC][es_stride] x 2
    float* ws0 = es0 + 2 * KC * f.es_stride;                // [KC][cop] x 2
    const float* __restrict__ xg = (const float*)D.xptr + ((int64_t)n * D.in_total + D.in_off) * HW;
    const float* __restrict__ wdw = (const float*)D.wptr;
    const float* __restrict__ wpw = (const float*)P.wptr;
    const float pv = D.pad_value;

    // Pad rows (outside the image) and pad columns of the input tile: the
    // same for every chunk, written once.
    for (int e = tid; e < KC * f.ir * f.xw; e += kT) {
        const int row = (e / f.xw) % f.ir, col = e % f.xw;
        const int ih = ih0 + row, iw = col - f.xoff;
        if ((unsigned)ih >= (unsigned)H || (unsigned)iw >= (unsigned)W) xs[(e / (f.ir * f.xw)) * f.xs_plane + row * f.xw + col] = pv;
    }

    // ---- chunk loads: input rows and pointwise weights into registers ----
    const int w4 = W >> 2;
    const int vunits = KC * f.ir * w4;                      // 4-pixel units of a chunk (vector path)
    float4 xr[NXV];
    float sr[NSC];
    float wr[KC * 64 / kT];                                 // pointwise weights: KC x COT (<= 64) / kT per thread
    auto load_chunk = [&](int c) __attribute__((always_inline)) {
        const int c0 = c * KC;
        if (f.vec) {
#pragma unroll
            for (int i = 0; i < NXV; ++i) {
                const int u = tid + i * kT;
                const int ch = u / (f.ir * w4), rem = u - ch * (f.ir * w4);
                const int row = rem / w4, c4 = rem - row * w4;
                const int ih = ih0 + row;
                xr[i] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (u < vunits && c0 + ch < C && (unsigned)ih < (unsigned)H)
                    xr[i] = *(const float4*)(xg + (int64_t)(c0 + ch) * HW + (int64_t)ih * W + 4 * c4);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NSC; ++i) {
                const int e = tid + i * kT;
                const int ch = e / (f.ir * W), rem = e - ch * (f.ir * W);
                const int row = rem / W, col = rem - row * W;
                const int ih = ih0 + row;
                sr[i] = 0.0f;
                if (e < KC * f.ir * W && c0 + ch < C && (unsigned)ih < (unsigned)H)
                    sr[i] = xg[(int64_t)(c0 + ch) * HW + (int64_t)ih * W + col];
            }
        }
#pragma unroll
        for (int i = 0; i < KC * 64 / kT; ++i) {
            const int e = tid + i * kT;                     // k-major: e = k * 64 + co
            const int k = e >> 6, co = e & 63;
            wr[i] = (co < f.cot && co0 + co < P.c_out && c0 + k < C) ? wpw[(int64_t)(co0 + co) * C + c0 + k] : 0.0f;
        }
    };
    auto store_chunk = [&](float* ws) __attribute__((always_inline)) {
        if (f.vec) {
#pragma unroll
            for (int i = 0; i < NXV; ++i) {
                const int u = tid + i * kT;
                const int ch = u / (f.ir * w4), rem = u - ch * (f.ir * w4);
                const int row = rem / w4, c4 = rem - row * w4;
                if (u < vunits && (unsigned)(ih0 + row) < (unsigned)H)
                    *(float4*)(xs + ch * f.xs_plane + row * f.xw + f.xoff + 4 * c4) = xr[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < NSC; ++i) {
                const int e = tid + i * kT;
                const int ch = e / (f.ir * W), rem = e - ch * (f.ir * W);
                const int row = rem / W, col = rem - row * W;
                if (e < KC * f.ir * W && (unsigned)(ih0 + row) < (unsigned)H)
                    xs[ch * f.xs_plane + row * f.xw + f.xoff + col] = sr[i];
            }
        }
#pragma unroll
        for (int i = 0; i < KC * 64 / kT; ++i) {
            const int e = tid + i * kT;
            const int k = e >> 6, co = e & 63;
            if (co < f.cot) ws[k * f.cop + co] = wr[i];
        }
    };

    f32x4 acc[MI][NJ];
#pragma unroll
    for (int m = 0; m < MI; ++m)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[m][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int uw = (WO + VO - 1) / VO;
    const int units = KC * th_n * uw;
    load_chunk(0);
    for (int c = 0; c < nch; ++c) {
        float* es = es0 + (c & 1) * KC * f.es_stride;
        float* ws = ws0 + (c & 1) * KC * f.cop;
        store_chunk(ws);
        __syncthreads();                                    // input tile and weights of chunk c are in LDS
        if (c + 1 < nch) load_chunk(c + 1);

        // ---- 2. depthwise into the GEMM operand ----
        const int c0 = c * KC;
        for (int u = tid; u < units; u += kT) {
            const int ch = u / (th_n * uw), rem = u - ch * (th_n * uw);
            const int r = rem / uw, q0 = (rem - r * uw) * VO;
            const int cg = c0 + ch;
            float outv[VO];
            if (cg < C) {
                float a[VO];
#pragma unroll
                for (int v = 0; v < VO; ++v) a[v] = 0.0f;
                const float* src = xs + ch * f.xs_plane + r * sh * f.xw + f.xoff - D.pad_left + q0 * sw;
                const float* wch = wdw + (int64_t)cg * kh * kw;
                if constexpr (FIXED) {
                    constexpr int CIN = (VO - 1) * SS + KW;
#pragma unroll
                    for (int i = 0; i < KH; ++i) {
                        float win[CIN];
#pragma unroll
                        for (int jj = 0; jj < CIN; ++jj) win[jj] = src[i * f.xw + jj];
#pragma unroll
                        for (int s2 = 0; s2 < KW; ++s2) {
                            const float wv = wch[i * KW + s2];
#pragma unroll
                            for (int v = 0; v < VO; ++v) a[v] = fmaf(win[v * SS + s2], wv, a[v]);
                        }
                    }
                } else {
                    for (int i = 0; i < kh; ++i)
                        for (int s2 = 0; s2 < kw; ++s2) {
                            const float wv = wch[i * kw + s2];
                            const float* rp = src + i * dh * f.xw + s2 * dwl;
#pragma unroll
                            for (int v = 0; v < VO; ++v) a[v] = fmaf(rp[v * sw], wv, a[v]);
                        }
                }
#pragma unroll
                for (int v = 0; v < VO; ++v) outv[v] = bias_act(D, a[v], cg);
            } else {
#pragma unroll
                for (int v = 0; v < VO; ++v) outv[v] = 0.0f;   // past the last channel: zero weights too
            }
            float* dst = es + ch * f.es_stride + r * WO + q0;
#pragma unroll
            for (int v = 0; v < VO; ++v)
                if (q0 + v < WO) dst[v] = outv[v];
        }
        __syncthreads();                                    // the depthwise rows of chunk c are in LDS

        // ---- 3. pointwise on the matrix cores ----
#pragma unroll
        for (int kq = 0; kq < KC; kq += 4) {
            const int kr = kq + q;
            float bv[MI];
#pragma unroll
            for (int m = 0; m < MI; ++m) bv[m] = ws[kr * f.cop + m * 16 + l16];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int fj = wave + kWaves * j;
                if (fj < f.nf) {
                    const float av = es[kr * f.es_stride + fj * 16 + l16];
#pragma unroll
                    for (int m = 0; m < MI; ++m)
                        acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv[m], acc[m][j], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue: lane (q, l16) of fragment (m, j) holds output channel
    // co0 + m*16 + l16 at the 4 pixels j*16 + 4q .. +3 of the tile ----
    const int64_t oplane = (int64_t)P.ho * P.wo;
    float* __restrict__ yg = (float*)P.yptr;
    const bool vec_out = WO % 4 == 0 && ((uintptr_t)P.yptr % 16) == 0;
    const int npx_n = th_n * WO;
#pragma unroll
    for (int m = 0; m < MI; ++m) {
        const int co = co0 + m * 16 + l16;
        if (m * 16 + l16 >= f.cot || co >= P.c_out) continue;
        float* yc = yg + ((int64_t)n * P.out_total + P.out_off + co) * oplane + (int64_t)ho0 * WO;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int fj = wave + kWaves * j;
            const int px = fj * 16 + 4 * q;
            if (fj >= f.nf || px >= npx_n) continue;
            float v4[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) v4[v] = bias_act(P, acc[m][j][v], co);
            if (vec_out) {
                *(float4*)(yc + px) = make_float4(v4[0], v4[1], v4[2], v4[3]);
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (px + v < npx_n) yc[px + v] = v4[v];
            }
        }
    }
}

struct Plan {
    int th, ir, xoff, xw, xs_plane, npx, nf, nj, es_stride, cot, cop, lds_floats, vec;
};

int cu_count_dwpw() {
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

bool plan(const Desc& dw, const Desc& pw, Plan* out) {
    const conv2d_params_t& d = dw.p;
    const int W = d.w, WO = dw.wo;
    const bool vec = W % 4 == 0;
    const int cot = pw.p.c_out <= 32 ? 32 : 64;
    const int co_tiles = (pw.p.c_out + cot - 1) / cot;
    const int xoff = (d.pad_left + 3) / 4 * 4;
    // Columns a tile reads: up to xoff - pad_left + (wo_padded-1)*sw + (kw-1)*dw + 1.
    const int wo_pad = (WO + VO - 1) / VO * VO;
    const int need = xoff - d.pad_left + (wo_pad - 1) * d.stride_w + (d.k_w - 1) * d.dilation_w + 1;
    int xw = xoff + W + d.pad_right;
    if (xw < need) xw = need;
    xw = (xw + 3) / 4 * 4;
    bool ok = false;
    long best = 0;
    for (int th = 1; th <= dw.ho; ++th) {
        const int ir = (th - 1) * d.stride_h + (d.k_h - 1) * d.dilation_h + 1;
        const int npx = th * WO;
        const int nf = (npx + 15) / 16;
        const int nj = (nf + kWaves - 1) / kWaves;
        if (nj > 4) break;
        if (vec ? KC * ir * (W / 4) > NXV * kT : KC * ir * W > NSC * kT) break;
        const int xs_plane = ir * xw;
        const int es_stride = stride16(nf * 16);
        const int cop = stride16(cot);
        const int lds = KC * xs_plane + 2 * KC * es_stride + 2 * KC * cop;
        if (lds * 4 > 160 * 1024) break;
        // One workgroup per compute unit: 8 waves of up to 256 registers.
        const long blocks = (long)d.n * ((dw.ho + th - 1) / th) * co_tiles;
        const long rounds = (blocks + cu_count_dwpw() - 1) / cu_count_dwpw();
        // Time ~ rounds x input rows a workgroup stages (halo included).
        const long cost = rounds * ir;
        if (!ok || cost < best) {
            *out = Plan{th, ir, xoff, xw, xs_plane, npx, nf, nj <= 2 ? 2 : 4, es_stride, cot, cop, lds, vec ? 1 : 0};
            best = cost;
            ok = true;
        }
    }
    return ok;
}

template <int KH, int KW, int SS>
const void* pick_mn(int mi, int nj) {
    if (mi == 2) return nj == 2 ? (const void*)fused_dw_pw_kernel<KH, KW, SS, 2, 2> : (const void*)fused_dw_pw_kernel<KH, KW, SS, 2, 4>;
    return nj == 2 ? (const void*)fused_dw_pw_kernel<KH, KW, SS, 4, 2> : (const void*)fused_dw_pw_kernel<KH, KW, SS, 4, 4>;
}

}  // namespace

bool plan_fused_dw_pw(const Desc& dw, const Desc& pw) {
    if (dw.p.k_h > 5 || dw.p.k_w > 5) return false;
    if ((int64_t)dw.p.h * dw.p.w >= INT32_MAX / 2 || (int64_t)dw.ho * dw.wo >= INT32_MAX / 2) return false;
    Plan pl{};
    return plan(dw, pw, &pl);
}

hipError_t launch_fused_dw_pw(const Desc& dw, const Desc& pw, ConvArgs adw, ConvArgs apw, hipStream_t s) {
    Plan pl{};
    if (!plan(dw, pw, &pl)) return hipErrorInvalidConfiguration;
    DwPwArgs f;
    f.dw = adw;
    f.pw = apw;
    f.th = pl.th;
    f.tiles_h = (dw.ho + pl.th - 1) / pl.th;
    f.cot = pl.cot;
    f.co_tiles = (pw.p.c_out + pl.cot - 1) / pl.cot;
    f.ir = pl.ir;
    f.xoff = pl.xoff;
    f.xw = pl.xw;
    f.xs_plane = pl.xs_plane;
    f.npx = pl.npx;
    f.nf = pl.nf;
    f.es_stride = pl.es_stride;
    f.cop = pl.cop;
    f.vec = pl.vec && ((uintptr_t)adw.xptr % 16) == 0 &&
            ((int64_t)adw.in_off * dw.p.h * dw.p.w) % 4 == 0 && ((int64_t)adw.in_total * dw.p.h * dw.p.w) % 4 == 0;
    f.dv_co_tiles = make_divu32((uint32_t)f.co_tiles);
    f.dv_tiles_h = make_divu32((uint32_t)f.tiles_h);
    const uint64_t blocks = (uint64_t)f.co_tiles * f.tiles_h * adw.n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0xFFFFFFFFull) return hipErrorInvalidConfiguration;
    f.num_blocks = (uint32_t)blocks;
    const conv2d_params_t& d = dw.p;
    const bool k3 = d.k_h == 3 && d.k_w == 3 && d.dilation_h == 1 && d.dilation_w == 1 && d.stride_h == d.stride_w &&
                    (d.stride_h == 1 || d.stride_h == 2);
    const int mi = pl.cot / 16;
    const void* fn = !k3 ? pick_mn<0, 0, 0>(mi, pl.nj)
                         : (d.stride_h == 1 ? pick_mn<3, 3, 1>(mi, pl.nj) : pick_mn<3, 3, 2>(mi, pl.nj));
    const int lds = pl.lds_floats * 4;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
    }
    void* args[] = {&f};
    return hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(kT), args, lds, s);
}

}  // namespace conv2d
