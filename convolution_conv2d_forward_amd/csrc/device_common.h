// Device helpers shared by the gfx950 kernels: bias + activation epilogue,
// requant epilogue, XCD-aware block remap, fast division.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

#include "conv2d_internal.h"

namespace conv2d {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fdiv(uint32_t x, FastDiv f) {
    return f.d == 1 ? x : __umulhi(x, f.m);
}

__device__ __forceinline__ uint32_t divu(uint32_t x, DivU32 f) {
    if (f.d == 1) return x;
    const uint32_t t = __umulhi(x, f.m);
    return (t + ((x - t) >> 1)) >> f.s;
}

// MI355X has 8 XCDs and the dispatcher hands consecutive workgroups to
// consecutive XCDs.  Remap so that consecutive logical tiles (which share
// input patches) land on the same XCD and hit its L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t nblocks) {
    const uint32_t full = nblocks & ~7u;
    if (b >= full) return b;
    const uint32_t per = full >> 3;
    return (b & 7u) * per + (b >> 3);
}

// The five activations as one branch-free form, y = min(max(v >= 0 ? v : s*v,
// lo), hi), with (s, lo, hi) = (1, -inf, inf) for none, (1, 0, inf) for ReLU,
// (alpha, -inf, inf) for LeakyReLU, (slope[c], -inf, inf) for PReLU and
// (1, lo, hi) for Clip: the same value as each activation's own formula for
// finite v (ReLU may keep the sign of a zero).  Chosen once per kernel (s per
// channel for PReLU), it keeps the per-value epilogues free of branches; the
// fused kernels, whose epilogues the compiler did not unswitch, use it.
struct ActP {
    float s, lo, hi;
};

__device__ __forceinline__ ActP act_params(const ConvArgs& a) {
    ActP p{1.0f, -INFINITY, INFINITY};
    if (a.act == CONV_ACT_RELU) {
        p.lo = 0.0f;
    } else if (a.act == CONV_ACT_LEAKY_RELU) {
        p.s = a.act_a;
    } else if (a.act == CONV_ACT_CLIP) {
        p.lo = a.act_a;
        p.hi = a.act_b;
    }
    return p;
}

__device__ __forceinline__ float act_apply(float v, float s, float lo, float hi) {
    return fminf(fmaxf(v >= 0.0f ? v : s * v, lo), hi);
}

// Slope of channel c: the PReLU slope, else the kernel-wide one.
__device__ __forceinline__ float act_slope(const ConvArgs& a, const ActP& p, int c) {
    return a.act == CONV_ACT_PRELU ? a.slope[a.slope_count == 1 ? 0 : c] : p.s;
}

// Bias add then the fused activation (ncnn convolution: y = act(conv + bias);
// Go ops ConvLeakyReluOp / ConvPReluOp fuse them into the GEMM write).  The
// switch on the kernel-wide activation is left to the compiler to hoist out
// of the callers' loops (measured faster here than the branch-free form for
// the implicit GEMMs and the depthwise kernels).
__device__ __forceinline__ float bias_act(const ConvArgs& a, float v, int co) {
    if (a.bias) v += a.bias[co];
    switch (a.act) {
    case CONV_ACT_RELU:
        v = v > 0.0f ? v : 0.0f;
        break;
    case CONV_ACT_LEAKY_RELU:
        v = v >= 0.0f ? v : a.act_a * v;
        break;
    case CONV_ACT_PRELU: {
        const float s = a.slope[a.slope_count == 1 ? 0 : co];
        v = v >= 0.0f ? v : s * v;
        break;
    }
    case CONV_ACT_CLIP:
        v = fminf(fmaxf(v, a.act_a), a.act_b);
        break;
    default:
        break;
    }
    return v;
}

// A channel's bias and PReLU slope, read before an epilogue's first store.
// bias_act re-reads them for every value, and since a store may alias them
// the compiler keeps each read after the stores before it: every read then
// waits for all earlier stores to be acknowledged.  bias_act_pre computes
// exactly what bias_act does from the preloaded pair.
struct ChanEpi {
    float b, s;
};

__device__ __forceinline__ ChanEpi chan_epi(const ConvArgs& a, int co) {
    ChanEpi e;
    e.b = a.bias ? a.bias[co] : 0.0f;
    e.s = a.act == CONV_ACT_PRELU ? a.slope[a.slope_count == 1 ? 0 : co] : 0.0f;
    return e;
}

__device__ __forceinline__ float bias_act_pre(const ConvArgs& a, float v, ChanEpi e) {
    if (a.bias) v += e.b;
    switch (a.act) {
    case CONV_ACT_RELU:
        v = v > 0.0f ? v : 0.0f;
        break;
    case CONV_ACT_LEAKY_RELU:
        v = v >= 0.0f ? v : a.act_a * v;
        break;
    case CONV_ACT_PRELU:
        v = v >= 0.0f ? v : e.s * v;
        break;
    case CONV_ACT_CLIP:
        v = fminf(fmaxf(v, a.act_a), a.act_b);
        break;
    default:
        break;
    }
    return v;
}

// The activation alone, with the channel's PReLU slope already loaded.
__device__ __forceinline__ float apply_act(const ConvArgs& a, float v, float slope) {
    switch (a.act) {
    case CONV_ACT_RELU:
        return v > 0.0f ? v : 0.0f;
    case CONV_ACT_LEAKY_RELU:
        return v >= 0.0f ? v : a.act_a * v;
    case CONV_ACT_PRELU:
        return v >= 0.0f ? v : slope * v;
    case CONV_ACT_CLIP:
        return fminf(fmaxf(v, a.act_a), a.act_b);
    default:
        return v;
    }
}

// int8 requant: q = sat8(round(f32(acc) * composite) + y_zp), ReLU as
// max(q, y_zp) (yscv requant epilogue).  The product is a plain f32 multiply
// (no contraction); rintf rounds ties to even, roundf away from zero.
__device__ __forceinline__ int8_t requant(int32_t acc, float composite, int rounding, int y_zp,
                                          bool relu) {
    float yf = __fmul_rn((float)acc, composite);
    // Materialise the rounded f32 product: under -ffp-contract=fast the
    // compiler would otherwise fuse it into roundf's own subtraction of the
    // truncated value (one fma, no intermediate rounding), and a product
    // that rounds to an exact tie (25.4999994 -> 25.5) would then round
    // toward zero.
    asm volatile("" : "+v"(yf));
    const float r = rounding == CONV_ROUND_HALF_AWAY ? roundf(yf) : rintf(yf);
    // Saturate on the rounded float before the conversion: clamp(r + y_zp,
    // -128, 127) is clamp(r, -128 - y_zp, 127 - y_zp) + y_zp for integer r,
    // and ReLU (q >= y_zp) raises the lower bound to 0.  The float is then at
    // most 255 in magnitude, so the conversion is exact for any product
    // (an infinite one included).
    const float lo = relu ? 0.0f : (float)(-128 - y_zp), hi = (float)(127 - y_zp);
    return (int8_t)((int)__builtin_amdgcn_fmed3f(r, lo, hi) + y_zp);
}

__host__ __device__ __forceinline__ float bf16_to_f32(__hip_bfloat16 v) {
    return __bfloat162float(v);
}

__host__ __device__ __forceinline__ __hip_bfloat16 f32_to_bf16(float v) {
    return __float2bfloat16(v);   // round to nearest even
}

}  // namespace conv2d
