// Grouped convolution with few channels per group (cin_g == cout_g == 4 or
// 8, 3x3): ncnn "convolution" with group > 1 as a direct VALU kernel.  With
// so few channels per group an implicit GEMM would run mostly empty matrix
// tiles, so the layer is bound by HBM traffic and fp32 FMA issue instead:
//   * a workgroup owns one (image, group) and a TH x 32 output tile; it
//     stages the group's input window (all CIG channels, pad_value outside
//     the image) in LDS as fp32 with coalesced row loads, every load of a
//     thread issued before the first LDS write (the whole grid runs in one
//     round, so a chain of dependent loads per thread would set its time);
//   * the group's weights are staged in LDS as fp32 in [ci][r][co][s] order
//     and read as broadcast 16-byte loads (the same address in every lane);
//   * each thread computes 2 horizontally adjacent output pixels for every
//     output channel of the group (2 * COG accumulators), reading each input
//     channel's window from LDS once for all of them; stride and dilation are
//     template parameters, so the window reads are fixed offsets.
// Bias, activation and the bf16 rounding happen once per output.
#include "device_common.h"

namespace conv2d {

namespace {

constexpr int kTW = 32;   // output columns per tile (16 threads x 2 pixels)
constexpr int kPX = 2;

template <typename T>
__device__ __forceinline__ float ld(const T* p);
template <>
__device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld<__hip_bfloat16>(const __hip_bfloat16* p) { return bf16_to_f32(*p); }

template <typename T, int CG, int SS, int DL, int TH>
__global__ __launch_bounds__(TH * 16) void grouped_kernel(ConvArgs a, float pad_v) {
    constexpr int KH = 3, KW = 3, NT = TH * 16;
    constexpr int PH = (TH - 1) * SS + (KH - 1) * DL + 1;            // patch rows
    constexpr int PW0 = (kTW - 1) * SS + (KW - 1) * DL + 1;          // patch columns
    constexpr int PW = (PW0 + 1) & ~1;                               // even row stride
    __shared__ float xs[CG * PH * PW];
    __shared__ __align__(16) float ws[CG * KH * CG * KW];   // [ci][r][co][s], fp32

    const int ng = blockIdx.y;               // n * groups + g
    const int g = ng % a.groups, n = ng / a.groups;
    const int tiles_w = (a.wo + kTW - 1) / kTW;
    const int ho0 = (blockIdx.x / tiles_w) * TH, wo0 = (blockIdx.x % tiles_w) * kTW;
    const int ih0 = ho0 * SS - a.pad_top, iw0 = wo0 * SS - a.pad_left;
    const int64_t HW = (int64_t)a.h * a.w;
    const T* __restrict__ xg = (const T*)a.xptr + ((int64_t)n * a.in_total + a.in_off + (int64_t)g * CG) * HW;

    // Stage the window: CG planes x PH rows x PW0 columns (pad outside), in
    // batches of up to 24 elements per thread: a batch's loads first
    // (unconditional: a slot outside the image reads the plane's first
    // element), then its LDS writes, where the pad is put in.  The weights'
    // loads go out with the first batch.
    constexpr int NX = (CG * PH * PW0 + NT - 1) / NT;
    constexpr int NB = (NX + 23) / 24;
    constexpr int BX = (NX + NB - 1) / NB;
    constexpr int NWT = (CG * CG * KH * KW + NT - 1) / NT;
    const T* __restrict__ wg = (const T*)a.wptr + (int64_t)g * CG * CG * KH * KW;
    float wv0[NWT];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        float xv0[BX];
#pragma unroll
        for (int i = 0; i < BX; ++i) {
            const int e = threadIdx.x + (b * BX + i) * NT;
            const int ci = e / (PH * PW0);
            const int rem = e - ci * (PH * PW0);
            const int r = rem / PW0, c = rem - r * PW0;
            const int ih = ih0 + r, iw = iw0 + c;
            const bool in = e < CG * PH * PW0 && (unsigned)ih < (unsigned)a.h && (unsigned)iw < (unsigned)a.w;
            xv0[i] = ld<T>(xg + (in ? ci * HW + ih * a.w + iw : 0));
        }
        if (b == 0) {
#pragma unroll
            for (int i = 0; i < NWT; ++i) {
                const int e = threadIdx.x + i * NT;
                wv0[i] = ld<T>(wg + (e < CG * CG * KH * KW ? e : 0));
            }
        }
#pragma unroll
        for (int i = 0; i < BX; ++i) {
            const int e = threadIdx.x + (b * BX + i) * NT;
            if (e < CG * PH * PW0) {
                const int ci = e / (PH * PW0);
                const int rem = e - ci * (PH * PW0);
                const int r = rem / PW0, c = rem - r * PW0;
                const int ih = ih0 + r, iw = iw0 + c;
                const bool in = (unsigned)ih < (unsigned)a.h && (unsigned)iw < (unsigned)a.w;
                xs[(ci * PH + r) * PW + c] = in ? xv0[i] : pad_v;
            }
        }
    }
    // The group's weights, OIHW -> [ci][r][co][s] in fp32: the 3*CG weights
    // one (ci, r) step needs are contiguous, read as broadcast 16-byte LDS
    // loads (every lane of a wave reads the same address).
#pragma unroll
    for (int i = 0; i < NWT; ++i) {
        const int e = threadIdx.x + i * NT;
        if (e < CG * CG * KH * KW) {
            const int s = e % KW, r = (e / KW) % KH, ci = (e / (KW * KH)) % CG, co = e / (KW * KH * CG);
            ws[((ci * KH + r) * CG + co) * KW + s] = wv0[i];
        }
    }
    __syncthreads();

    const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
    const int ho = ho0 + ty, wo = wo0 + kPX * tx;

    float acc[CG][kPX];
#pragma unroll
    for (int co = 0; co < CG; ++co)
#pragma unroll
        for (int p = 0; p < kPX; ++p) acc[co][p] = 0.0f;

    // The channel loop stays rolled: unrolled, the compiler hoists every
    // weight read of the group into registers.
#pragma unroll 1
    for (int ci = 0; ci < CG; ++ci)
#pragma unroll
        for (int r = 0; r < KH; ++r) {
            const float* row = xs + (ci * PH + ty * SS + r * DL) * PW + kPX * tx * SS;
            float xv[kPX][KW];
#pragma unroll
            for (int p = 0; p < kPX; ++p)
#pragma unroll
                for (int s = 0; s < KW; ++s) xv[p][s] = row[p * SS + s * DL];
#pragma unroll
            for (int co = 0; co < CG; ++co)
#pragma unroll
                for (int s = 0; s < KW; ++s) {
                    const float wv = ws[((ci * KH + r) * CG + co) * KW + s];
#pragma unroll
                    for (int p = 0; p < kPX; ++p) acc[co][p] = fmaf(xv[p][s], wv, acc[co][p]);
                }
        }

    if (ho >= a.ho || wo >= a.wo) return;
    const int64_t out_plane = (int64_t)a.ho * a.wo;
    const bool vec = a.wo % 2 == 0 && ((uintptr_t)a.yptr % (2 * sizeof(T))) == 0;
#pragma unroll
    for (int co = 0; co < CG; ++co) {
        const int cg = g * CG + co;
        const float b = a.bias ? a.bias[cg] : 0.0f;
        const float sl = a.act == CONV_ACT_PRELU ? a.slope[a.slope_count == 1 ? 0 : cg] : 0.0f;
        T* y = (T*)a.yptr + ((int64_t)n * a.out_total + a.out_off + cg) * out_plane + (int64_t)ho * a.wo + wo;
        const float v0 = apply_act(a, acc[co][0] + b, sl), v1 = apply_act(a, acc[co][1] + b, sl);
        if constexpr (sizeof(T) == 4) {
            if (vec) {
                *(float2*)y = make_float2(v0, v1);
            } else {
                y[0] = v0;
                if (wo + 1 < a.wo) y[1] = v1;
            }
        } else {
            const uint32_t lo = __bfloat16_as_ushort(f32_to_bf16(v0));
            const uint32_t hi = __bfloat16_as_ushort(f32_to_bf16(v1));
            if (vec) {
                *(uint32_t*)y = lo | (hi << 16);
            } else {
                ((uint16_t*)y)[0] = (uint16_t)lo;
                if (wo + 1 < a.wo) ((uint16_t*)y)[1] = (uint16_t)hi;
            }
        }
    }
}

template <typename T, int CG, int SS, int DL>
hipError_t launch_t(ConvArgs a, hipStream_t s, float pad_v) {
    constexpr int TH = SS == 1 ? 16 : 8;
    const int64_t bx = (int64_t)((a.ho + TH - 1) / TH) * ((a.wo + kTW - 1) / kTW);
    const int64_t by = (int64_t)a.n * a.groups;
    if (bx == 0 || by == 0) return hipSuccess;
    if (bx > 0x7FFFFFFF || by > 65535) return hipErrorInvalidConfiguration;
    void* args[] = {&a, &pad_v};
    return hipLaunchKernel((const void*)grouped_kernel<T, CG, SS, DL, TH>, dim3((uint32_t)bx, (uint32_t)by),
                           dim3(TH * 16), args, 0, s);
}

template <typename T, int CG>
hipError_t launch_cg(const Desc& d, ConvArgs a, hipStream_t s, float pad_v) {
    const int st = d.p.stride_h, dl = d.p.dilation_h;
    if (st == 1 && dl == 1) return launch_t<T, CG, 1, 1>(a, s, pad_v);
    if (st == 1 && dl == 2) return launch_t<T, CG, 1, 2>(a, s, pad_v);
    return launch_t<T, CG, 2, 1>(a, s, pad_v);
}

}  // namespace

bool plan_grouped(const Desc& d) {
    const conv2d_params_t& p = d.p;
    if (p.dtype != CONV_DTYPE_F32 && p.dtype != CONV_DTYPE_BF16) return false;
    if (p.groups < 2 || p.k_h != 3 || p.k_w != 3) return false;
    if (d.cin_g != d.cout_g || (d.cin_g != 4 && d.cin_g != 8)) return false;
    if (p.stride_h != p.stride_w || p.dilation_h != p.dilation_w) return false;
    const bool ok = (p.stride_h == 1 && (p.dilation_h == 1 || p.dilation_h == 2)) ||
                    (p.stride_h == 2 && p.dilation_h == 1);
    if (!ok) return false;
    if ((int64_t)p.n * p.groups > 65535) return false;
    if ((int64_t)d.cin_g * p.h * p.w >= INT32_MAX / 2 || (int64_t)d.ho * d.wo >= INT32_MAX / 2) return false;
    return true;
}

hipError_t launch_grouped(const Desc& d, ConvArgs a, hipStream_t s) {
    if (d.p.dtype == CONV_DTYPE_F32)
        return d.cin_g == 8 ? launch_cg<float, 8>(d, a, s, a.pad_value) : launch_cg<float, 4>(d, a, s, a.pad_value);
    // The pad enters the same storage type as the input (bf16).
    const float pv = bf16_to_f32(f32_to_bf16(a.pad_value));
    return d.cin_g == 8 ? launch_cg<__hip_bfloat16, 8>(d, a, s, pv) : launch_cg<__hip_bfloat16, 4>(d, a, s, pv);
}

}  // namespace conv2d
