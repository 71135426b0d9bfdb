// Fused pointwise 1x1 -> depthwise kxk (the FusedPwDw step of the yscv
// "ONNX CPU Kernels" page, section "Hot kernel paths": an inverted-bottleneck
// expansion followed by its depthwise conv, with the expanded tensor never
// written to main memory).
//
// Workgroup tile: one image, TH output rows, CE expanded channels.
//   1. For each chunk of KC input channels, stage the input rows the tile
//      needs (TH + (kh-1)*dh rows, full width) and the CE x KC pointwise
//      weights in LDS, and accumulate E = W_pw * X on the fp32 matrix cores
//      (v_mfma_f32_16x16x4f32; M = CE channels, N = flattened row pixels).
//   2. Bias + activation of the pointwise conv; the result goes to LDS as
//      rows of W + pad_left + pad_right floats.  Rows and columns outside the
//      image hold the depthwise pad_value: the depthwise padding applies to
//      the pointwise output, not to pw(pad).
//   3. Depthwise taps from LDS, bias + activation, 16-byte stores of VO
//      consecutive outputs.
// The halo rows are recomputed by the tiles above and below
// ((TH + kh - 1) / TH pointwise work) instead of being exchanged.
#include "device_common.h"

namespace conv2d {

namespace {

constexpr int kThreads = 256;
constexpr int CE = 32;      // expanded channels per workgroup
constexpr int KC = 32;      // input channels per pointwise chunk
constexpr int CEP = CE + 16;
constexpr int NFW = 14;     // max 16x16 pointwise fragments per wave
constexpr int VO = 4;

struct FusedArgs {
    ConvArgs pw, dw;
    int32_t tile_h, tiles_h, ce_tiles;
    int32_t rows;          // pointwise rows per tile: TH + (kh-1)*dh
    int32_t xs_stride;     // LDS floats per input-channel plane (rows * w, padded)
    int32_t ew;            // LDS row length of the expanded tile
    int32_t es_stride;     // LDS floats per expanded channel
    uint32_t num_blocks;
    FastDiv div_w, div_units_row;
};

__device__ __forceinline__ float act_f(int act, float v, float a0, float a1, float slope) {
    switch (act) {
    case CONV_ACT_RELU: return v > 0.0f ? v : 0.0f;
    case CONV_ACT_LEAKY_RELU: return v >= 0.0f ? v : a0 * v;
    case CONV_ACT_PRELU: return v >= 0.0f ? v : slope * v;
    case CONV_ACT_CLIP: return fminf(fmaxf(v, a0), a1);
    default: return v;
    }
}

template <int KH, int KW>
__global__ __launch_bounds__(kThreads) void fused_pw_dw_kernel(FusedArgs f) {
    extern __shared__ float lds[];
    const ConvArgs& P = f.pw;
    const ConvArgs& D = f.dw;
    const int kh = KH ? KH : D.k_h, kw = KW ? KW : D.k_w;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    uint32_t L = xcd_remap(blockIdx.x, f.num_blocks);
    const int cet = L % f.ce_tiles;  L /= f.ce_tiles;
    const int tht = L % f.tiles_h;   L /= f.tiles_h;
    const int n = L;
    const int ce0 = cet * CE;
    const int ho0 = tht * f.tile_h;
    const int ih_lo = ho0 - D.pad_top;          // input row of pointwise row 0
    const int W = P.w, H = P.h;
    const int npix = f.rows * W;                 // pointwise pixels of the tile
    const int nfrag_n = (npix + 15) / 16;
    const int nfrag = (CE / 16) * nfrag_n;
    const int ce_valid = min(CE, P.c_out - ce0);
    const int64_t HW = (int64_t)H * W;

    const float* __restrict__ xg = (const float*)P.xptr + ((int64_t)n * P.in_total + P.in_off) * HW;
    const float* __restrict__ wpw = (const float*)P.wptr;

    float* xs = lds;                       // [KC][xs_stride]
    float* ws = lds + KC * f.xs_stride;    // [KC][CEP]

    f32x4 acc[NFW];
#pragma unroll
    for (int i = 0; i < NFW; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // ---- 1. pointwise on the matrix cores ----
    for (int k0 = 0; k0 < P.c_in; k0 += KC) {
        // input rows (zeros for rows outside the image: replaced in step 2)
        for (int e = tid; e < KC * npix; e += kThreads) {
            const int kc = e / npix;
            const int p = e - kc * npix;
            const int r = (int)fdiv(p, f.div_w);
            const int c = p - r * W;
            const int ih = ih_lo + r;
            float v = 0.0f;
            if (k0 + kc < P.c_in && (unsigned)ih < (unsigned)H) v = xg[(int64_t)(k0 + kc) * HW + (int64_t)ih * W + c];
            xs[kc * f.xs_stride + p] = v;
        }
        for (int e = tid; e < KC * CE; e += kThreads) {
            const int ce = e % CE;
            const int kc = e / CE;
            float v = 0.0f;
            if (ce < ce_valid && k0 + kc < P.c_in) v = wpw[(int64_t)(ce0 + ce) * P.c_in + k0 + kc];
            ws[kc * CEP + ce] = v;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NFW; ++i) {
            const int fi = wave + 4 * i;
            if (fi < nfrag) {
                const int mf = fi % (CE / 16);
                const int nf = fi / (CE / 16);
                f32x4 a = acc[i];
#pragma unroll 8
                for (int kq = 0; kq < KC; kq += 4) {
                    const float av = ws[(kq + (lane >> 4)) * CEP + mf * 16 + (lane & 15)];
                    const float bv = xs[(kq + (lane >> 4)) * f.xs_stride + nf * 16 + (lane & 15)];
                    a = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, a, 0, 0, 0);
                }
                acc[i] = a;
            }
        }
        __syncthreads();
    }

    // ---- 2. pointwise epilogue into the expanded tile (aliases xs/ws) ----
    float* es = lds;   // [CE][es_stride], row r at r*ew, image column c at c + pad_left
    const float dpad = D.pad_value;
#pragma unroll
    for (int i = 0; i < NFW; ++i) {
        const int fi = wave + 4 * i;
        if (fi < nfrag) {
            const int mf = fi % (CE / 16);
            const int nf = fi / (CE / 16);
            const int p = nf * 16 + (lane & 15);
            if (p < npix) {
                const int r = (int)fdiv(p, f.div_w);
                const int c = p - r * W;
                const bool inside = (unsigned)(ih_lo + r) < (unsigned)H;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int ce = mf * 16 + (lane >> 4) * 4 + v;
                    float val = dpad;
                    if (inside && ce < ce_valid) {
                        const int cg = ce0 + ce;
                        float t = acc[i][v] + (P.bias ? P.bias[cg] : 0.0f);
                        const float sl = P.act == CONV_ACT_PRELU ? P.slope[P.slope_count == 1 ? 0 : cg] : 0.0f;
                        val = act_f(P.act, t, P.act_a, P.act_b, sl);
                    }
                    es[ce * f.es_stride + r * f.ew + c + D.pad_left] = val;
                }
            }
        }
    }
    // pad columns of every row
    const int padc = f.ew - W;
    for (int e = tid; e < CE * f.rows * padc; e += kThreads) {
        const int ce = e / (f.rows * padc);
        const int rem = e - ce * f.rows * padc;
        const int r = rem / padc;
        const int j = rem - r * padc;
        const int col = j < D.pad_left ? j : W + j;
        es[ce * f.es_stride + r * f.ew + col] = dpad;
    }
    __syncthreads();

    // ---- 3. depthwise from LDS ----
    const int th_n = min(f.tile_h, D.ho - ho0);
    const int uw = (D.wo + VO - 1) / VO;
    const int units = ce_valid * th_n * uw;
    const int64_t oplane = (int64_t)D.ho * D.wo;
    float* __restrict__ yg = (float*)D.yptr;
    const float* __restrict__ wdw = (const float*)D.wptr;
    const bool vec_ok = (D.wo % VO) == 0 && (((uintptr_t)D.yptr) % 16) == 0;
    for (int u = tid; u < units; u += kThreads) {
        const int ce = u / (th_n * uw);
        const int rem = u - ce * th_n * uw;
        const int th = rem / uw;
        const int q0 = (rem - th * uw) * VO;
        const int cg = ce0 + ce;
        float accd[VO];
#pragma unroll
        for (int q = 0; q < VO; ++q) accd[q] = 0.0f;
        const float* ech = es + ce * f.es_stride;
        const float* wch = wdw + (int64_t)cg * kh * kw;
#pragma unroll
        for (int r = 0; r < kh; ++r) {
            const float* row = ech + (th + r * D.dilation_h) * f.ew;
#pragma unroll
            for (int s2 = 0; s2 < kw; ++s2) {
                const float wv = wch[r * kw + s2];
#pragma unroll
                for (int q = 0; q < VO; ++q) {
                    // Columns past the row end belong to masked outputs; clamp the read.
                    const int col = min(q0 + q, D.wo - 1) + s2 * D.dilation_w;
                    accd[q] = fmaf(row[col], wv, accd[q]);
                }
            }
        }
        float outv[VO];
#pragma unroll
        for (int q = 0; q < VO; ++q) outv[q] = bias_act(D, accd[q], cg);
        float* dst = yg + ((int64_t)n * D.out_total + D.out_off + cg) * oplane + (int64_t)(ho0 + th) * D.wo + q0;
        if (vec_ok && q0 + VO <= D.wo) {
            *(float4*)dst = make_float4(outv[0], outv[1], outv[2], outv[3]);
        } else {
#pragma unroll
            for (int q = 0; q < VO; ++q)
                if (q0 + q < D.wo) dst[q] = outv[q];
        }
    }
}

int xs_stride_for(int npix) {
    int s = ((npix + 63 - 16) / 64) * 64 + 16;
    if (s < npix) s += 64;
    return s;
}

struct FusedPlan {
    int tile_h, rows, xs_stride, ew, es_stride, lds_floats;
};

bool plan(const Desc& pw, const Desc& dw, FusedPlan* out) {
    const conv2d_params_t& d = dw.p;
    const int W = pw.p.w;
    const int ew = W + d.pad_left + d.pad_right;
    bool ok = false;
    long best_cost = 0;
    for (int th = 1; th <= dw.ho; ++th) {
        const int rows = th + (d.k_h - 1) * d.dilation_h;
        const int npix = rows * W;
        if ((CE / 16) * ((npix + 15) / 16) > 4 * NFW) break;
        if (npix >= 65536) break;
        const int xs = xs_stride_for(npix);
        const int es = rows * ew;
        const int fl1 = KC * xs + KC * CEP;
        const int fl2 = CE * es;
        const int lds = fl1 > fl2 ? fl1 : fl2;
        if (lds * 4 > 64 * 1024) break;
        // Pointwise rows computed over the whole image (halo recompute and
        // the ragged last tile included): the smaller the better.
        const long cost = (long)((dw.ho + th - 1) / th) * rows;
        if (!ok || cost <= best_cost) {
            *out = FusedPlan{th, rows, xs, ew, es, lds};
            best_cost = cost;
            ok = true;
        }
    }
    return ok;
}

}  // namespace

bool plan_fused_pw_dw(const Desc& pw, const Desc& dw, int32_t* tile_h, int32_t* lds_bytes) {
    if (dw.p.k_h > 5 || dw.p.k_w > 5) return false;
    FusedPlan fp{};
    if (!plan(pw, dw, &fp)) return false;
    *tile_h = fp.tile_h;
    *lds_bytes = fp.lds_floats * 4;
    return true;
}

hipError_t launch_fused_pw_dw(const Desc& pw, const Desc& dw, ConvArgs apw, ConvArgs adw, hipStream_t s) {
    FusedPlan fp{};
    if (!plan(pw, dw, &fp)) return hipErrorInvalidConfiguration;
    FusedArgs f;
    f.pw = apw;
    f.dw = adw;
    f.tile_h = fp.tile_h;
    f.tiles_h = (dw.ho + fp.tile_h - 1) / fp.tile_h;
    f.ce_tiles = (pw.p.c_out + CE - 1) / CE;
    f.rows = fp.rows;
    f.xs_stride = fp.xs_stride;
    f.ew = fp.ew;
    f.es_stride = fp.es_stride;
    f.div_w = make_fastdiv((uint32_t)pw.p.w);
    f.div_units_row = make_fastdiv(1);
    const uint64_t blocks = (uint64_t)f.ce_tiles * f.tiles_h * apw.n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0xFFFFFFFFull) return hipErrorInvalidConfiguration;
    f.num_blocks = (uint32_t)blocks;
    const void* fn = (dw.p.k_h == 3 && dw.p.k_w == 3) ? (const void*)fused_pw_dw_kernel<3, 3>
                                                     : (const void*)fused_pw_dw_kernel<0, 0>;
    void* args[] = {&f};
    return hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(kThreads), args, fp.lds_floats * 4, s);
}

}  // namespace conv2d
