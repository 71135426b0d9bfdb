// int8 dense and grouped convolution (symmetric QLinearConv: int32
// accumulation, + int32 bias, requant) as an implicit GEMM on the gfx950 i8
// matrix cores (v_mfma_i32_16x16x64_i8), for the windows the depthwise and
// pointwise kernels do not take.  The requant follows the yscv "ONNX CPU
// Kernels (Conv/MatMul) -- Runtime Map" page (section "Hot kernel paths",
// fused INT8 chains); the convolution is ncnn's "convolution" definition
// with the zero point as the pad.
//
// GEMM per group: Y[co, p] = sum_k W[co, k] X^[k, p], with K ordered
// tap-major: k = tap * 64 + c within a chunk of 64 input channels.  An MFMA
// step is one tap of one chunk, so a lane's 16 consecutive k are 16
// consecutive channels at one tap:
//   - the input patch of the tile is staged in LDS pixel-major, [pixel][64
//     channels] (4 channels x 4 pixels per thread: four 4-byte loads,
//     transposed with v_perm), so the pixel operand is one 16-byte LDS read
//     at the tap's patch pixel;
//   - the weights are re-laid per chunk into [tap][co][64 channels] (a thread
//     reads one output channel's 4 input channels x all taps, contiguous in
//     OIHW, and writes one word per tap).
// Workgroup tile: BM = 16*MB output channels of one group x (4*NFW) output
// rows x 16 output columns; wave w owns output rows w, w+4, ...  Pixels are
// the first MFMA operand, so a lane's result is 4 consecutive output columns
// of one channel: + bias, requant, one packed 4-byte store where the row
// allows it.
#include "device_common.h"

namespace conv2d {

namespace {

constexpr int kT = 256;
constexpr int CK = 64;          // input channels per chunk (the MFMA's K)
constexpr int XR = CK + 16;     // LDS bytes per staged pixel / weight row (16 pad bytes spread the banks)
constexpr int TW = 16;          // output columns per tile (one MFMA fragment)
constexpr int QV = 4;           // staged 4x4 blocks per thread and pass

struct I8Args {
    ConvArgs a;
    int32_t khw;            // taps
    int32_t th;             // output rows per tile (4 * NFW)
    int32_t ph, pw;         // patch rows, patch columns (a multiple of 4)
    int32_t pw4;            // pw / 4
    int32_t co_tiles, tiles_h, tiles_w, chunks;
    int32_t xs_bytes;       // LDS bytes of the patch
    int32_t vec_x;          // patch rows move as 4-byte words
    int32_t vec_w;          // filter blocks move as 4-byte words
    int32_t away;           // requant ties away from zero
    uint32_t num_blocks;
    DivU32 dv_co_tiles, dv_groups, dv_tiles_w, dv_tiles_h;
    DivU32 dv_pw4;          // staging unit -> (quad, patch row)
    DivU32 dv_ppix;         // staging unit / 4 -> channel quad group (patch words per quad)
    DivU32 dv_kw;           // tap -> (r, s)
};

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

// Requant, ties to even or (away) away from zero, branch-free; the clamp to
// [lo, hi] (the int8 range shifted by the zero point, raised to 0 under
// ReLU) runs on the rounded value.
__device__ __forceinline__ int rq8(int32_t acc, float comp, bool away, float lo, float hi, int zp) {
    float yf = __fmul_rn((float)acc, comp);
    asm volatile("" : "+v"(yf));   // the rounded f32 product decides ties (no fma into the rounding)
    const float t = truncf(yf);
    const float r = (away && fabsf(yf - t) == 0.5f) ? t + copysignf(1.0f, yf) : rintf(yf);
    return (int)__builtin_amdgcn_fmed3f(r, lo, hi) + zp;
}

template <int NFW, int MB>
__global__ __launch_bounds__(kT) void igemm_i8_kernel(I8Args f) {
    extern __shared__ __align__(16) uint8_t lds[];
    const ConvArgs& a = f.a;
    constexpr int BM = 16 * MB;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    uint32_t L = xcd_remap(blockIdx.x, f.num_blocks);
    uint32_t Q = divu(L, f.dv_co_tiles);
    const int cot = L - Q * f.co_tiles;
    L = Q; Q = divu(L, f.dv_groups);
    const int g = L - Q * a.groups;
    L = Q; Q = divu(L, f.dv_tiles_w);
    const int twi = L - Q * f.tiles_w;
    L = Q; Q = divu(L, f.dv_tiles_h);
    const int thi = L - Q * f.tiles_h;
    const int n = Q;

    const int co0 = cot * BM;
    const int ho0 = thi * f.th, wo0 = twi * TW;
    const int ih0 = ho0 * a.stride_h - a.pad_top;
    const int iw_lo = wo0 * a.stride_w - a.pad_left;
    const int iw_a = iw_lo >= 0 ? iw_lo & ~3 : -((-iw_lo + 3) & ~3);   // patch column 0, a multiple of 4
    const int shift = iw_lo - iw_a;
    const int H = a.h, W = a.w;
    const int64_t HW = (int64_t)H * W;
    const int cin_g = a.cin_g;
    const int khw = f.khw;
    const int PH = f.ph, PW = f.pw;

    const int8_t* __restrict__ xg = (const int8_t*)a.xptr + ((int64_t)n * a.in_total + a.in_off + (int64_t)g * cin_g) * HW;
    const int8_t* __restrict__ wg = (const int8_t*)a.wptr + (int64_t)(g * a.cout_g + co0) * cin_g * khw;

    // Patch pixel p (row-major, PW a multiple of 4) lives at slot
    // (p % 4) * (PH * PW / 4) + p / 4: a thread's four pixels land in four
    // quarters, and the words of consecutive threads 80 bytes apart.
    uint8_t* xs = lds;                    // [PH * PW][XR]
    uint8_t* ws = lds + f.xs_bytes;       // [khw][BM][XR]

    // This lane's pixel in each of its fragments: patch pixel of tap (0, 0).
    int pbase[NFW];
#pragma unroll
    for (int j = 0; j < NFW; ++j) {
        const int oh = wave + 4 * j, ow = lane & 15;
        pbase[j] = oh * a.stride_h * PW + ow * a.stride_w + shift;
    }

    i32x4 acc[NFW][MB];
#pragma unroll
    for (int j = 0; j < NFW; ++j)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[j][m] = i32x4{0, 0, 0, 0};

    const int pq_n = PH * f.pw4;          // 4-pixel words of the patch per channel quad
    for (int kc = 0; kc < f.chunks; ++kc) {
        const int c0 = kc * CK;
        const int kq_n = min(CK, cin_g - c0 + 3) >> 2;   // channel quads holding data
        // ---- patch -> LDS (pixel-major); quads past cin_g are left as they
        // are: their weights are staged as zero ----
        // Unit u: channel quad 4 * (u / (4 * pq_n)) + u % 4 and word rem =
        // (u / 4) % pq_n of the patch (patch row pr, columns 4 * (rem % pw4)
        // ..+3).  Four consecutive lanes take four channel quads of one word,
        // so a wave's LDS stores cover every bank (see slot below).
        const int kq4 = (kq_n + 3) & ~3;
        const int units = kq4 * pq_n;
        for (int u0 = 0; u0 < units; u0 += QV * kT) {
            uint32_t in[QV][4];
#pragma unroll
            for (int i = 0; i < QV; ++i) {
                const int u = u0 + tid + i * kT;
                const int hi = (int)divu((uint32_t)(u >> 2), f.dv_ppix);
                const int cq = 4 * hi + (u & 3);
                const int rem = (u >> 2) - hi * pq_n;
                const int pr = (int)divu((uint32_t)rem, f.dv_pw4);
                const int pc = 4 * (rem - pr * f.pw4);
                const int ih = ih0 + pr, iw = iw_a + pc;
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    const int ch = c0 + 4 * cq + cc;
                    uint32_t v = 0;
                    if (u < units && cq < kq_n && ch < cin_g && (unsigned)ih < (unsigned)H) {
                        const int8_t* src = xg + (int64_t)ch * HW + (int64_t)ih * W;
                        if (f.vec_x) {
                            // W % 4 == 0 and iw % 4 == 0: the word is inside the row or outside it.
                            if (iw >= 0 && iw < W) v = *(const uint32_t*)(src + iw);
                        } else {
#pragma unroll
                            for (int b = 0; b < 4; ++b)
                                if ((unsigned)(iw + b) < (unsigned)W) v |= (uint32_t)(uint8_t)src[iw + b] << (8 * b);
                        }
                    }
                    in[i][cc] = v;
                }
            }
#pragma unroll
            for (int i = 0; i < QV; ++i) {
                const int u = u0 + tid + i * kT;
                const int hi = (int)divu((uint32_t)(u >> 2), f.dv_ppix);
                const int cq = 4 * hi + (u & 3);
                if (u >= units || cq >= kq_n) continue;
                const int rem = (u >> 2) - hi * pq_n;
                uint32_t outw[4];
                tr4x4(in[i], outw);
                // rem = pr * pw4 + pc / 4, so byte b is patch pixel 4 * rem + b,
                // kept at slot b * pq_n + rem.
#pragma unroll
                for (int b = 0; b < 4; ++b) *(uint32_t*)&xs[(b * pq_n + rem) * XR + 4 * cq] = outw[b];
            }
        }
        // ---- weights -> LDS [tap][co][64 channels]; zero past the filter ----
        for (int u = tid; u < BM * (CK / 4); u += kT) {
            const int co = u >> 4, cq = u & 15;
            const int ci = c0 + 4 * cq;
            const bool live = co0 + co < a.cout_g && ci < cin_g;
            const int8_t* src = wg + ((int64_t)co * cin_g + ci) * khw;
            if (live && f.vec_w && ci + 4 <= cin_g) {
                // cin_g % 4 == 0 and an aligned base: the 4 channels x khw taps
                // are 4 * khw contiguous bytes starting on a word.
                const uint32_t* src32 = (const uint32_t*)src;   // the block's khw words
                for (int t0 = 0; t0 < khw; t0 += 4) {
                    // Taps t0 .. t0+3 of channels ci .. ci+3 sit at bytes c * khw + t.
                    // Bytes past the block (taps past the window of the
                    // last channel) are never written below; they read as 0.
                    uint32_t wv[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int b0 = c * khw + t0;
                        const int wi = b0 >> 2;
                        const uint32_t lo = wi < khw ? src32[wi] : 0u;
                        const uint32_t hi = ((b0 & 3) && wi + 1 < khw) ? src32[wi + 1] : 0u;
                        wv[c] = __builtin_amdgcn_alignbyte(hi, lo, b0 & 3);
                    }
                    uint32_t outw[4];
                    tr4x4(wv, outw);      // outw[t] = channels 0..3 at tap t0 + t
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (t0 + t < khw) *(uint32_t*)&ws[((t0 + t) * BM + co) * XR + 4 * cq] = outw[t];
                }
            } else {
                for (int t = 0; t < khw; ++t) {
                    uint32_t v = 0;
                    if (live) {
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            if (ci + c < cin_g) v |= (uint32_t)(uint8_t)src[c * khw + t] << (8 * c);
                    }
                    *(uint32_t*)&ws[(t * BM + co) * XR + 4 * cq] = v;
                }
            }
        }
        __syncthreads();
        // ---- MFMAs: one K step per tap ----
        for (int t = 0; t < khw; ++t) {
            const int r = (int)divu((uint32_t)t, f.dv_kw);
            const int s = t - r * a.k_w;
            const int toff = r * a.dilation_h * PW + s * a.dilation_w;
            i32x4 bw[MB];
#pragma unroll
            for (int m = 0; m < MB; ++m)
                bw[m] = *(const i32x4*)&ws[((t * BM) + 16 * m + (lane & 15)) * XR + 16 * (lane >> 4)];
#pragma unroll
            for (int j = 0; j < NFW; ++j) {
                const int pp = pbase[j] + toff;
                const i32x4 av = *(const i32x4*)&xs[((pp & 3) * pq_n + (pp >> 2)) * XR + 16 * (lane >> 4)];
#pragma unroll
                for (int m = 0; m < MB; ++m)
                    acc[j][m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bw[m], acc[j][m], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // ---- epilogue: + bias, requant, 4 consecutive columns per lane ----
    const bool relu = a.act == CONV_ACT_RELU;
    const float lo = relu ? 0.0f : (float)(-128 - a.y_zp), hi = (float)(127 - a.y_zp);
    const bool away = f.away != 0;
    int8_t* __restrict__ yg = (int8_t*)a.yptr;
    const int64_t oplane = (int64_t)a.ho * a.wo;
    const bool vec_y = (a.wo % 4) == 0 && ((uintptr_t)a.yptr % 4) == 0;
    const int wo = wo0 + 4 * (lane >> 4);
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        const int co = co0 + 16 * m + (lane & 15);
        if (co >= a.cout_g) continue;
        const int cg = g * a.cout_g + co;
        const int32_t bb = a.qbias ? a.qbias[cg] : 0;
        int8_t* yc = yg + ((int64_t)n * a.out_total + a.out_off + cg) * oplane;
#pragma unroll
        for (int j = 0; j < NFW; ++j) {
            const int ho = ho0 + wave + 4 * j;
            if (ho >= a.ho || wo >= a.wo) continue;
            uint32_t word = 0;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                word |= (uint32_t)(uint8_t)rq8(acc[j][m][v] + bb, a.composite, away, lo, hi, a.y_zp) << (8 * v);
            int8_t* dst = yc + (int64_t)ho * a.wo + wo;
            if (vec_y && wo + 4 <= a.wo) {
                *(uint32_t*)dst = word;
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (wo + v < a.wo) dst[v] = (int8_t)(word >> (8 * v));
            }
        }
    }
}

struct I8Plan {
    int nfw, mb, th, ph, pw, xs_bytes, lds;
};

constexpr int kLdsMax = 160 * 1024;

// The largest tile that fits: 8 output rows (two fragments per wave) when
// the patch and the weights fit in LDS, else 4; 64 output channels per
// workgroup for windows of up to 9 taps, 32 for larger ones.
bool i8_plan(const Desc& d, I8Plan* out) {
    const conv2d_params_t& p = d.p;
    const int khw = p.k_h * p.k_w;
    const int mb = khw <= 9 ? 4 : 2;
    for (int nfw = 2; nfw >= 1; --nfw) {
        const int th = 4 * nfw;
        const int ph = (th - 1) * p.stride_h + (p.k_h - 1) * p.dilation_h + 1;
        const int pw = ((3 + (TW - 1) * p.stride_w + (p.k_w - 1) * p.dilation_w + 1) + 3) / 4 * 4;
        const int xs = ph * pw * XR;
        const int lds = xs + khw * 16 * mb * XR;
        if (lds <= 64 * 1024 || (nfw == 1 && lds <= kLdsMax)) {
            *out = I8Plan{nfw, mb, th, ph, pw, xs, lds};
            return true;
        }
    }
    return false;
}

}  // namespace

bool plan_igemm_i8(const Desc& d) {
    const conv2d_params_t& p = d.p;
    if (p.dtype != CONV_DTYPE_I8) return false;
    if ((int64_t)d.cin_g * p.k_h * p.k_w > (1 << 24)) return false;
    I8Plan ip{};
    return i8_plan(d, &ip);
}

hipError_t launch_igemm_i8(const Desc& d, ConvArgs a, hipStream_t s) {
    I8Plan ip{};
    if (!i8_plan(d, &ip)) return hipErrorInvalidConfiguration;
    const conv2d_params_t& p = d.p;
    I8Args f;
    f.a = a;
    f.khw = p.k_h * p.k_w;
    f.th = ip.th;
    f.ph = ip.ph;
    f.pw = ip.pw;
    f.pw4 = ip.pw / 4;
    f.co_tiles = (d.cout_g + 16 * ip.mb - 1) / (16 * ip.mb);
    f.tiles_h = (d.ho + ip.th - 1) / ip.th;
    f.tiles_w = (d.wo + TW - 1) / TW;
    f.chunks = (d.cin_g + CK - 1) / CK;
    f.xs_bytes = ip.xs_bytes;
    f.vec_x = p.w % 4 == 0 && ((uintptr_t)a.xptr % 4) == 0;
    f.vec_w = d.cin_g % 4 == 0 && ((uintptr_t)a.wptr % 4) == 0;
    f.away = p.int8_rounding == CONV_ROUND_HALF_AWAY;
    f.dv_co_tiles = make_divu32((uint32_t)f.co_tiles);
    f.dv_groups = make_divu32((uint32_t)p.groups);
    f.dv_tiles_w = make_divu32((uint32_t)f.tiles_w);
    f.dv_tiles_h = make_divu32((uint32_t)f.tiles_h);
    f.dv_pw4 = make_divu32((uint32_t)f.pw4);
    f.dv_ppix = make_divu32((uint32_t)(ip.ph * f.pw4));
    f.dv_kw = make_divu32((uint32_t)p.k_w);
    const uint64_t blocks = (uint64_t)f.co_tiles * p.groups * f.tiles_w * f.tiles_h * p.n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0xFFFFFFFFull) return hipErrorInvalidConfiguration;
    f.num_blocks = (uint32_t)blocks;
    const void* fn = ip.nfw == 2 ? (ip.mb == 4 ? (const void*)igemm_i8_kernel<2, 4> : (const void*)igemm_i8_kernel<2, 2>)
                                 : (ip.mb == 4 ? (const void*)igemm_i8_kernel<1, 4> : (const void*)igemm_i8_kernel<1, 2>);
    if (ip.lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, ip.lds);
        if (e != hipSuccess) return e;
    }
    void* args[] = {&f};
    return hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(kT), args, ip.lds, s);
}

}  // namespace conv2d
