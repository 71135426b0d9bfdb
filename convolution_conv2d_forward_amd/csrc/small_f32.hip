// Small fp32 3x3 convolutions on the vector units: ncnn "convolution" (pad
// with pad_value, correlate under stride and dilation, + bias, activation)
// term by term, for layers whose whole output is a few hundred waves of work
// (the single 16 -> 32 conv on a 32 x 32 image is 9.4 MFLOP).  At that size
// a layer's time is launch, the first memory round trip and one workgroup's
// serial chain, so the kernel keeps the chain short: a workgroup owns 128
// output pixels and CO output channels, and each pixel's input channels are
// split between two threads (waves 0-1 and 2-3), whose sums meet in LDS.  A
// thread computes its nine tap offsets and in-image tests once, then
// requests all taps of 8 channels before the first multiply (unconditional
// loads: taps outside the image read the channel's first element and are
// replaced by pad_value), with the weights at wave-uniform addresses read
// through the scalar cache.
#include "device_common.h"

namespace conv2d {

namespace {

constexpr int UCH = 8;                 // channels whose 9 taps each are loaded together

struct SmallArgs {
    ConvArgs a;
    uint32_t npix;          // n * ho * wo
    uint32_t pxblocks;      // workgroups of 128 pixels
    DivU32 dv_pxb, dv_wo, dv_ho;
};

template <int CO>
__global__ __launch_bounds__(256) void small3x3_f32_kernel(SmallArgs sa) {
    const ConvArgs& a = sa.a;
    const uint32_t bid = blockIdx.x;
    const uint32_t cog = divu(bid, sa.dv_pxb);                 // output-channel group (wave-uniform)
    const uint32_t pb = bid - cog * sa.pxblocks;
    const int ks = threadIdx.x >> 7;                           // half of the input channels (wave-uniform)
    const uint32_t p = pb * 128 + (threadIdx.x & 127);
    const bool live = p < sa.npix;
    const uint32_t pc = live ? p : 0;
    const uint32_t q1 = divu(pc, sa.dv_wo);
    const int ox = (int)(pc - q1 * (uint32_t)a.wo);
    const uint32_t n = divu(q1, sa.dv_ho);
    const int oy = (int)(q1 - n * (uint32_t)a.ho);
    const int co0 = (int)cog * CO;

    const int64_t HW = (int64_t)a.h * a.w;
    const float* __restrict__ xn = (const float*)a.xptr + ((int64_t)n * a.in_total + a.in_off) * HW;
    const float* __restrict__ wg = (const float*)a.wptr + (int64_t)co0 * a.c_in * 9;
    const float pv = a.pad_value;

    int off[9];
    uint32_t valid = 0;
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        const int ih = oy * a.stride_h - a.pad_top + r * a.dilation_h;
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            const int iw = ox * a.stride_w - a.pad_left + s * a.dilation_w;
            const bool ok = (unsigned)ih < (unsigned)a.h && (unsigned)iw < (unsigned)a.w;
            off[3 * r + s] = ok ? ih * a.w + iw : 0;
            valid |= (ok ? 1u : 0u) << (3 * r + s);
        }
    }

    float acc[CO];
#pragma unroll
    for (int j = 0; j < CO; ++j) acc[j] = 0.0f;
    const int C = a.c_in;
    const int ch = (C + 1) >> 1;
    const int cbeg = ks * ch, cend = min(C, cbeg + ch);
    for (int c0 = cbeg; c0 < cend; c0 += UCH) {
        // all taps of UCH channels requested before the first multiply
        float xv[UCH][9];
#pragma unroll
        for (int u = 0; u < UCH; ++u) {
            const float* __restrict__ xc = xn + (int64_t)min(c0 + u, cend - 1) * HW;
#pragma unroll
            for (int t = 0; t < 9; ++t) {
                const float v = xc[off[t]];
                xv[u][t] = ((valid >> t) & 1u) ? v : pv;
            }
        }
#pragma unroll
        for (int u = 0; u < UCH; ++u) {
            if (c0 + u < cend) {
#pragma unroll
                for (int j = 0; j < CO; ++j) {
                    if (co0 + j < a.c_out) {
                        const float* __restrict__ wj = wg + ((int64_t)j * C + c0 + u) * 9;
#pragma unroll
                        for (int t = 0; t < 9; ++t) acc[j] = fmaf(xv[u][t], wj[t], acc[j]);
                    }
                }
            }
        }
    }

    // the second half's partial sums join the first half's through LDS
    __shared__ float part[CO][128];
    if (ks == 1) {
#pragma unroll
        for (int j = 0; j < CO; ++j) part[j][threadIdx.x & 127] = acc[j];
    }
    __syncthreads();
    if (ks == 1 || !live) return;
#pragma unroll
    for (int j = 0; j < CO; ++j) acc[j] += part[j][threadIdx.x];
    const int64_t plane = (int64_t)a.ho * a.wo;
    float* __restrict__ yb = (float*)a.yptr + ((int64_t)n * a.out_total + a.out_off) * plane + (int64_t)oy * a.wo + ox;
    ChanEpi ce[CO];   // every channel's bias and slope before the first store
#pragma unroll
    for (int j = 0; j < CO; ++j) ce[j] = chan_epi(a, co0 + j < a.c_out ? co0 + j : 0);
#pragma unroll
    for (int j = 0; j < CO; ++j) {
        const int co = co0 + j;
        if (co < a.c_out) yb[(int64_t)co * plane] = bias_act_pre(a, acc[j], ce[j]);
    }
}

}  // namespace

// fp32, one group, 3x3 window, at most 64 input channels, and an output of
// at most 64K elements: the layers where one short chain per output beats the
// tiled classes' set-up (input patch copies, split-K reduction).
bool plan_small_f32(const Desc& d) {
    const conv2d_params_t& p = d.p;
    if (p.dtype != CONV_DTYPE_F32 || p.groups != 1 || p.k_h != 3 || p.k_w != 3) return false;
    if (p.c_in > 64) return false;
    const int64_t outs = (int64_t)p.n * p.c_out * d.ho * d.wo;
    if (outs == 0 || outs > 65536) return false;
    // 32-bit offsets within a plane and pixel indices
    return (int64_t)p.h * p.w < (1 << 30) && (int64_t)p.n * d.ho * d.wo < (1ll << 31);
}

hipError_t launch_small_f32(const Desc& d, ConvArgs a, hipStream_t s) {
    SmallArgs sa;
    sa.a = a;
    const int64_t pix = (int64_t)a.n * a.ho * a.wo;
    if (pix == 0 || a.c_out == 0) return hipSuccess;
    sa.npix = (uint32_t)pix;
    sa.pxblocks = (uint32_t)((pix + 127) / 128);
    // Output channels per thread: one while the grid stays within four
    // workgroups per CU, else more (fewer, longer chains).
    int co = 1;
    while (co < 4 && (int64_t)sa.pxblocks * ((a.c_out + co - 1) / co) > 1024) co *= 2;
    const int64_t blocks = (int64_t)sa.pxblocks * ((a.c_out + co - 1) / co);
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    sa.dv_pxb = make_divu32(sa.pxblocks);
    sa.dv_wo = make_divu32((uint32_t)a.wo);
    sa.dv_ho = make_divu32((uint32_t)a.ho);
    void* args[] = {&sa};
    const void* fn = co == 1 ? (const void*)small3x3_f32_kernel<1>
                   : co == 2 ? (const void*)small3x3_f32_kernel<2>
                             : (const void*)small3x3_f32_kernel<4>;
    return hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(256), args, 0, s);
}

}  // namespace conv2d
