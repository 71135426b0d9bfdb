// Direct convolution: one thread per output element, reading x and w from
// global memory.  It covers every shape and dtype the descriptor accepts
// that the tiled kernels do not (large kernels, int8 dense convolutions),
// following the ncnn "convolution" definition term by term: pad_value (or
// the zero point, for int8) for taps outside the image, then + bias, then the
// activation or the requant.  Not a fast path.
#include "device_common.h"

namespace conv2d {

namespace {

template <typename T>
__device__ __forceinline__ float load_f(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_f<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_f<__hip_bfloat16>(const __hip_bfloat16* p, int64_t i) {
    return bf16_to_f32(p[i]);
}

template <typename T>
__global__ __launch_bounds__(256) void direct_float_kernel(ConvArgs a, int64_t total, float pad_v) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    int64_t t = idx;
    const int wo = (int)(t % a.wo); t /= a.wo;
    const int ho = (int)(t % a.ho); t /= a.ho;
    const int co = (int)(t % a.c_out); t /= a.c_out;
    const int n = (int)t;
    const int g = co / a.cout_g;
    const T* x = (const T*)a.xptr;
    const T* w = (const T*)a.wptr;
    const int64_t HW = (int64_t)a.h * a.w;
    float acc = 0.0f;
    for (int ci = 0; ci < a.cin_g; ++ci) {
        const int64_t xbase = ((int64_t)n * a.in_total + a.in_off + (int64_t)g * a.cin_g + ci) * HW;
        const int64_t wbase = ((int64_t)co * a.cin_g + ci) * a.k_h * a.k_w;
        for (int r = 0; r < a.k_h; ++r) {
            const int ih = ho * a.stride_h - a.pad_top + r * a.dilation_h;
            for (int s = 0; s < a.k_w; ++s) {
                const int iw = wo * a.stride_w - a.pad_left + s * a.dilation_w;
                const float xv = ((unsigned)ih < (unsigned)a.h && (unsigned)iw < (unsigned)a.w)
                                     ? load_f<T>(x, xbase + (int64_t)ih * a.w + iw)
                                     : pad_v;
                acc = fmaf(xv, load_f<T>(w, wbase + r * a.k_w + s), acc);
            }
        }
    }
    const float v = bias_act(a, acc, co);
    const int64_t o = (((int64_t)n * a.out_total + a.out_off + co) * a.ho + ho) * a.wo + wo;
    if constexpr (sizeof(T) == 4)
        ((float*)a.yptr)[o] = v;
    else
        ((__hip_bfloat16*)a.yptr)[o] = f32_to_bf16(v);
}

__global__ __launch_bounds__(256) void direct_int8_kernel(ConvArgs a, int64_t total) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    int64_t t = idx;
    const int wo = (int)(t % a.wo); t /= a.wo;
    const int ho = (int)(t % a.ho); t /= a.ho;
    const int co = (int)(t % a.c_out); t /= a.c_out;
    const int n = (int)t;
    const int g = co / a.cout_g;
    const int8_t* x = (const int8_t*)a.xptr;
    const int8_t* w = (const int8_t*)a.wptr;
    const int64_t HW = (int64_t)a.h * a.w;
    int32_t acc = 0;
    for (int ci = 0; ci < a.cin_g; ++ci) {
        const int64_t xbase = ((int64_t)n * a.in_total + a.in_off + (int64_t)g * a.cin_g + ci) * HW;
        const int64_t wbase = ((int64_t)co * a.cin_g + ci) * a.k_h * a.k_w;
        for (int r = 0; r < a.k_h; ++r) {
            const int ih = ho * a.stride_h - a.pad_top + r * a.dilation_h;
            for (int s = 0; s < a.k_w; ++s) {
                const int iw = wo * a.stride_w - a.pad_left + s * a.dilation_w;
                // Symmetric scheme: the input zero point, and so the pad, is 0.
                const int32_t xv = ((unsigned)ih < (unsigned)a.h && (unsigned)iw < (unsigned)a.w)
                                       ? (int32_t)x[xbase + (int64_t)ih * a.w + iw]
                                       : 0;
                acc += xv * (int32_t)w[wbase + r * a.k_w + s];
            }
        }
    }
    if (a.qbias) acc += a.qbias[co];
    const int64_t o = (((int64_t)n * a.out_total + a.out_off + co) * a.ho + ho) * a.wo + wo;
    ((int8_t*)a.yptr)[o] = requant(acc, a.composite, a.rounding, a.y_zp, a.act == CONV_ACT_RELU);
}

}  // namespace

hipError_t launch_direct(const Desc& d, ConvArgs a, hipStream_t s) {
    const int64_t total = (int64_t)a.n * a.c_out * a.ho * a.wo;
    if (total == 0) return hipSuccess;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const void* fn;
    float pv = a.pad_value;
    switch (d.p.dtype) {
    case CONV_DTYPE_F32: fn = (const void*)direct_float_kernel<float>; break;
    case CONV_DTYPE_BF16:
        // The pad enters the same storage type as the input (bf16).
        fn = (const void*)direct_float_kernel<__hip_bfloat16>;
        pv = bf16_to_f32(f32_to_bf16(a.pad_value));
        break;
    default: fn = (const void*)direct_int8_kernel; break;
    }
    // hipLaunchKernel reports this launch's own status (hipGetLastError would
    // also return, and clear, an earlier call's error).
    void* fargs[] = {&a, (void*)&total, &pv};
    void* iargs[] = {&a, (void*)&total};
    return hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(256), d.p.dtype == CONV_DTYPE_I8 ? iargs : fargs, 0, s);
}

}  // namespace conv2d
