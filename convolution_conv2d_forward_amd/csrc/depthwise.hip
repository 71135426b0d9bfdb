// Depthwise convolution (groups == c_in == c_out): ncnn
// "convolutiondepthwise" with one filter per channel, and the yscv int8
// depthwise QLinearConv (3x3 s1 / s2, int32 accumulate, requant).
//
// There is one multiply-add per input byte or so: the kernel is bound by HBM,
// so the design is about moving bytes once, in wide coalesced transactions.
// A workgroup owns a tile of one (n, c) plane: it copies the input window
// (halo included) into LDS with 16-byte loads (pad_value, or zero for int8,
// outside the image), then each thread produces VO consecutive outputs of a
// row from LDS and writes them with one vector store.  No MFMA: there is no
// reduction dimension to feed it.
#include "device_common.h"

namespace conv2d {

namespace {

constexpr int kThreads = 256;
constexpr int VO = 4;   // consecutive outputs per thread

template <typename T> struct Elem;
template <> struct Elem<float> { using lds_t = float; static constexpr int VL = 4; };
template <> struct Elem<__hip_bfloat16> { using lds_t = float; static constexpr int VL = 8; };
template <> struct Elem<int8_t> { using lds_t = int8_t; static constexpr int VL = 16; };

struct DwGeom {
    int rows, cols;      // LDS window
    int col_shift;       // iw_lo - iw_a
};

// VEC: true when rows can be moved as 16-byte vectors (w % VL == 0 and x
// 16-byte aligned); KH/KW/SH/SW: compile-time kernel and stride (0 = runtime).
template <typename T, bool VEC, int KH, int KW, int SH, int SW>
__global__ __launch_bounds__(kThreads) void dw_kernel(ConvArgs a) {
    using LT = typename Elem<T>::lds_t;
    constexpr int VL = VEC ? Elem<T>::VL : 1;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    LT* tile = (LT*)lds_raw;

    const int kh = KH ? KH : a.k_h, kw = KW ? KW : a.k_w;
    const int sh = SH ? SH : a.stride_h, sw = SW ? SW : a.stride_w;
    const int dh = a.dilation_h, dwl = a.dilation_w;

    // block -> (tile col, tile row, channel, image)
    uint32_t L = blockIdx.x;
    const int twi = L % a.tiles_w;  L /= a.tiles_w;
    const int thi = L % a.tiles_h;  L /= a.tiles_h;
    const int c = L % a.c_out;      L /= a.c_out;
    const int n = L;

    const int ho0 = thi * a.tile_h, wo0 = twi * a.tile_w;
    const int th_n = min(a.tile_h, a.ho - ho0);
    const int tw_n = min(a.tile_w, a.wo - wo0);
    const int ih_lo = ho0 * sh - a.pad_top;
    const int iw_lo = wo0 * sw - a.pad_left;
    const int iw_a = VL > 1 ? (iw_lo >= 0 ? iw_lo / VL * VL : -((-iw_lo + VL - 1) / VL) * VL) : iw_lo;
    const int rows = (th_n - 1) * sh + (kh - 1) * dh + 1;
    const int iw_hi = (wo0 + tw_n - 1) * sw - a.pad_left + (kw - 1) * dwl;
    const int lw = (iw_hi + 1 - iw_a + VL - 1) / VL * VL;   // LDS row length (elements)
    const int lwv = lw / VL;
    const int shift = iw_lo - iw_a;

    const int64_t HW = (int64_t)a.h * a.w;
    const T* __restrict__ xp = (const T*)a.xptr + ((int64_t)n * a.in_total + a.in_off + c) * HW;

    LT padv;
    if constexpr (sizeof(T) == 1) padv = 0;          // symmetric int8: the pad is the zero point
    else padv = (LT)a.pad_value;

    // Input window -> LDS.
    const int nvec = rows * lwv;
    for (int v = threadIdx.x; v < nvec; v += kThreads) {
        const int r = v / lwv;
        const int cv = v - r * lwv;
        const int ih = ih_lo + r;
        const int iw = iw_a + cv * VL;
        LT* dst = tile + r * lw + cv * VL;
        const bool row_in = (unsigned)ih < (unsigned)a.h;
        if constexpr (VL > 1) {
            // Vectors never straddle the image edge: w % VL == 0 and iw % VL == 0.
            if (row_in && iw >= 0 && iw < a.w) {
                const T* src = xp + (int64_t)ih * a.w + iw;
                if constexpr (sizeof(T) == 4) {
                    *(float4*)dst = *(const float4*)src;
                } else if constexpr (sizeof(T) == 1) {
                    *(int4*)dst = *(const int4*)src;
                } else {
                    const uint4 raw = *(const uint4*)src;
                    const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        dst[2 * q] = __uint_as_float(wv[q] << 16);
                        dst[2 * q + 1] = __uint_as_float(wv[q] & 0xFFFF0000u);
                    }
                }
            } else {
#pragma unroll
                for (int q = 0; q < VL; ++q) dst[q] = padv;
            }
        } else {
            LT val = padv;
            if (row_in && (unsigned)iw < (unsigned)a.w) {
                if constexpr (sizeof(T) == 2) val = bf16_to_f32(xp[(int64_t)ih * a.w + iw]);
                else val = (LT)xp[(int64_t)ih * a.w + iw];
            }
            *dst = val;
        }
    }

    // Filter taps of this channel (OIHW with one input channel per group).
    const int khw = kh * kw;
    constexpr int KMAX = (KH && KW) ? KH * KW : 25;
    using AT = typename std::conditional<sizeof(T) == 1, int32_t, float>::type;
    AT wt[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
        if (i < khw) {
            if constexpr (sizeof(T) == 2) wt[i] = bf16_to_f32(((const T*)a.wptr)[(int64_t)c * khw + i]);
            else wt[i] = (AT)((const T*)a.wptr)[(int64_t)c * khw + i];
        } else {
            wt[i] = 0;
        }
    }
    __syncthreads();

    // Outputs: each thread makes VO consecutive outputs of one row.
    const int uw = (tw_n + VO - 1) / VO;
    const int units = th_n * uw;
    const int64_t oplane = (int64_t)a.ho * a.wo;
    T* __restrict__ yp = (T*)a.yptr + ((int64_t)n * a.out_total + a.out_off + c) * oplane;
    const bool relu8 = a.act == CONV_ACT_RELU;
    for (int u = threadIdx.x; u < units; u += kThreads) {
        const int th = u / uw;
        const int q0 = (u - th * uw) * VO;
        AT acc[VO];
#pragma unroll
        for (int q = 0; q < VO; ++q) acc[q] = 0;
        for (int r = 0; r < kh; ++r) {
            const LT* row = tile + (th * sh + r * dh) * lw + shift;
#pragma unroll
            for (int s = 0; s < KMAX; ++s) {
                if (!(KH && KW) && s >= kw) break;
                if ((KH && KW) && s >= KW) break;
#pragma unroll
                for (int q = 0; q < VO; ++q) {
                    const int col = (q0 + q) * sw + s * dwl;
                    const AT xv = (AT)row[col < lw - shift ? col : 0];
                    if constexpr (sizeof(T) == 1) acc[q] += xv * wt[r * kw + s];
                    else acc[q] = fmaf(xv, wt[r * kw + s], acc[q]);
                }
            }
        }
        const int ho = ho0 + th;
        const int wo = wo0 + q0;
        T outv[VO];
#pragma unroll
        for (int q = 0; q < VO; ++q) {
            if constexpr (sizeof(T) == 1) {
                const int32_t v = acc[q] + (a.qbias ? a.qbias[c] : 0);
                outv[q] = requant(v, a.composite, a.rounding, a.y_zp, relu8);
            } else if constexpr (sizeof(T) == 2) {
                outv[q] = f32_to_bf16(bias_act(a, acc[q], c));
            } else {
                outv[q] = bias_act(a, acc[q], c);
            }
        }
        T* dst = yp + (int64_t)ho * a.wo + wo;
        const bool full = q0 + VO <= tw_n;
        if (VEC && full && (a.wo % VO) == 0) {
            if constexpr (sizeof(T) == 4) {
                *(float4*)dst = make_float4(outv[0], outv[1], outv[2], outv[3]);
            } else if constexpr (sizeof(T) == 1) {
                const uint32_t packed = (uint32_t)(uint8_t)outv[0] | ((uint32_t)(uint8_t)outv[1] << 8) |
                                        ((uint32_t)(uint8_t)outv[2] << 16) | ((uint32_t)(uint8_t)outv[3] << 24);
                *(uint32_t*)dst = packed;
            } else {
                uint2 packed;
                packed.x = (uint32_t)__bfloat16_as_ushort(outv[0]) | ((uint32_t)__bfloat16_as_ushort(outv[1]) << 16);
                packed.y = (uint32_t)__bfloat16_as_ushort(outv[2]) | ((uint32_t)__bfloat16_as_ushort(outv[3]) << 16);
                *(uint2*)dst = packed;
            }
        } else {
#pragma unroll
            for (int q = 0; q < VO; ++q)
                if (q0 + q < tw_n) dst[q] = outv[q];
        }
    }
}

template <typename T>
size_t window_bytes(const conv2d_params_t& p, int tile_h, int tile_w, int ho, int wo) {
    using LT = typename Elem<T>::lds_t;
    const int VL = Elem<T>::VL;
    const int th = tile_h < ho ? tile_h : ho;
    const int tw = tile_w < wo ? tile_w : wo;
    const int rows = (th - 1) * p.stride_h + (p.k_h - 1) * p.dilation_h + 1;
    const int span = (tw - 1) * p.stride_w + (p.k_w - 1) * p.dilation_w + 1;
    const int lw = (span + 2 * VL - 2 + VL - 1) / VL * VL;   // worst-case alignment slack
    return (size_t)rows * lw * sizeof(LT);
}

template <typename T>
bool plan_dw_t(Desc& d) {
    const conv2d_params_t& p = d.p;
    if (p.k_h * p.k_w > 25) return false;
    // Whole rows when they fit; otherwise 256-wide column strips.
    int tw = d.wo <= 512 ? d.wo : 256;
    const int uw = (tw + VO - 1) / VO;
    // About four output vectors per thread.
    int th = (4 * kThreads) / uw;
    if (th < 1) th = 1;
    if (th > d.ho) th = d.ho;
    while (th > 1 && window_bytes<T>(p, th, tw, d.ho, d.wo) > 32 * 1024) th = (th + 1) / 2;
    if (window_bytes<T>(p, th, tw, d.ho, d.wo) > 48 * 1024) return false;
    d.tile_h = th;
    d.tile_w = tw;
    d.lds_bytes = (int)window_bytes<T>(p, th, tw, d.ho, d.wo);
    return true;
}

template <typename T, bool VEC>
const void* pick(const conv2d_params_t& p) {
    if (p.k_h == 3 && p.k_w == 3 && p.stride_h == 1 && p.stride_w == 1)
        return (const void*)dw_kernel<T, VEC, 3, 3, 1, 1>;
    if (p.k_h == 3 && p.k_w == 3 && p.stride_h == 2 && p.stride_w == 2)
        return (const void*)dw_kernel<T, VEC, 3, 3, 2, 2>;
    return (const void*)dw_kernel<T, VEC, 0, 0, 0, 0>;
}

template <typename T>
hipError_t launch_t(const Desc& d, ConvArgs a, hipStream_t s) {
    a.tile_h = d.tile_h;
    a.tile_w = d.tile_w;
    a.tiles_h = (d.ho + d.tile_h - 1) / d.tile_h;
    a.tiles_w = (d.wo + d.tile_w - 1) / d.tile_w;
    const uint64_t blocks = (uint64_t)a.tiles_w * a.tiles_h * a.c_out * a.n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0xFFFFFFFFull) return hipErrorInvalidConfiguration;
    const bool vec = (d.p.w % Elem<T>::VL) == 0 && ((uintptr_t)a.xptr % 16) == 0 && ((uintptr_t)a.yptr % 16) == 0;
    const void* fn = vec ? pick<T, true>(d.p) : pick<T, false>(d.p);
    void* args[] = {&a};
    return hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(kThreads), args, d.lds_bytes, s);
}

}  // namespace

bool plan_dw(Desc& d) {
    return d.p.dtype == CONV_DTYPE_BF16 ? plan_dw_t<__hip_bfloat16>(d) : plan_dw_t<float>(d);
}

bool plan_qdw(Desc& d) { return plan_dw_t<int8_t>(d); }

hipError_t launch_dw(const Desc& d, ConvArgs a, hipStream_t s) {
    return d.p.dtype == CONV_DTYPE_BF16 ? launch_t<__hip_bfloat16>(d, a, s) : launch_t<float>(d, a, s);
}

hipError_t launch_qdw(const Desc& d, ConvArgs a, hipStream_t s) { return launch_t<int8_t>(d, a, s); }

}  // namespace conv2d
