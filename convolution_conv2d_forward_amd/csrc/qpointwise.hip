// int8 pointwise (1x1, stride 1, no pad, groups 1) QLinearConv on the i8
// matrix cores of gfx950: v_mfma_i32_16x16x64_i8, int32 accumulation, then
// + int32 bias and the requant epilogue (yscv "ONNX CPU Kernels" page, fused
// INT8 chains: (acc + bias) as f32 times the composite scale, rounded,
// + y_zp, clamped to int8, optional Relu).
//
// Per image the product is Y[co, p] = sum_k W[co, k] X[k, p].  The MFMA wants
// each lane to hold 16 consecutive k of one row (A) or one column (B).  The
// weights are already k-contiguous (OIHW, 1x1), so A fragments come straight
// from global memory (they stay in L1/L2: 7 KB for 144 -> 48).  The input is
// NCHW (pixels contiguous), so each thread loads a 4-channel x 4-pixel block
// with four 4-byte loads, transposes it in registers with byte permutes, and
// stores four 4-byte words pixel-major into LDS; B fragments are then one
// 16-byte LDS read.  The pairing of k inside one MFMA only has to agree
// between A and B, which both use k = 16*(lane/16) + byte.
#include "device_common.h"

namespace conv2d {

namespace {

constexpr int kThreads = 256;
constexpr int BN = 64;         // pixels per tile: one 16-pixel fragment per wave
constexpr int KC = 64;         // channels per chunk (one MFMA K step)
constexpr int XROW = KC + 16;  // LDS bytes per pixel row (padding spreads banks)

// Transpose a 4x4 byte block: in[c] holds pixels 0..3 of channel c; out[p]
// holds channels 0..3 of pixel p.
__device__ __forceinline__ void transpose4x4(const uint32_t in[4], uint32_t out[4]) {
    // Interleave bytes of channel pairs, then 16-bit halves.
    const uint32_t t0 = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);  // c0p0 c1p0 c0p1 c1p1
    const uint32_t t1 = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);  // c0p2 c1p2 c0p3 c1p3
    const uint32_t t2 = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);  // c2p0 c3p0 c2p1 c3p1
    const uint32_t t3 = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);  // c2p2 c3p2 c2p3 c3p3
    out[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);  // c0p0 c1p0 c2p0 c3p0
    out[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);  // c0p1 c1p1 c2p1 c3p1
    out[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
    out[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

template <int MI>
__global__ __launch_bounds__(kThreads) void qpw_kernel(ConvArgs a) {
    __shared__ __align__(16) uint8_t xs[BN * XROW];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int K = a.c_in;
    const int HW = a.h * a.w;

    uint32_t L = blockIdx.x;
    const int cot = L % a.co_tiles;  L /= a.co_tiles;
    const int pt = L % a.tiles_w;    L /= a.tiles_w;
    const int n = L;
    const int co0 = cot * MI * 16;
    const int p0 = pt * BN;

    const int8_t* __restrict__ xg = (const int8_t*)a.xptr + ((int64_t)n * a.in_total + a.in_off) * HW;
    const int8_t* __restrict__ wg = (const int8_t*)a.wptr;
    const bool vec_x = (HW % 4) == 0 && (((uintptr_t)a.xptr) % 4) == 0 && (((int64_t)a.in_total * HW) % 4) == 0;
    const bool vec_w = (K % 16) == 0 && (((uintptr_t)a.wptr) % 16) == 0;

    // This thread's 4x4 block of the input tile: channels 4*kq.., pixels 4*pq..
    const int kq = tid >> 4;   // 0..15
    const int pq = tid & 15;   // 0..15

    i32x4 acc[MI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) acc[mi] = i32x4{0, 0, 0, 0};

    for (int c0 = 0; c0 < K; c0 += KC) {
        // Input block -> registers (zero outside the channel range / image).
        uint32_t in[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const int ch = c0 + 4 * kq + cc;
            const int p = p0 + 4 * pq;
            uint32_t v = 0;
            if (ch < K) {
                const int8_t* src = xg + (int64_t)ch * HW + p;
                if (vec_x && p + 4 <= HW) {
                    v = *(const uint32_t*)src;
                } else {
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        if (p + b < HW) v |= (uint32_t)(uint8_t)src[b] << (8 * b);
                }
            }
            in[cc] = v;
        }
        uint32_t outw[4];
        transpose4x4(in, outw);
        __syncthreads();   // previous chunk's B reads are done
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) *(uint32_t*)&xs[(4 * pq + pp) * XROW + 4 * kq] = outw[pp];
        __syncthreads();

        // B fragment: pixel (wave*16 + lane%16), k = 16*(lane/16) .. +15.
        const i32x4 bfrag = *(const i32x4*)&xs[(wave * 16 + (lane & 15)) * XROW + 16 * (lane >> 4)];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const int co = co0 + mi * 16 + (lane & 15);
            const int k = c0 + 16 * (lane >> 4);
            i32x4 afrag = i32x4{0, 0, 0, 0};
            if (co < a.c_out) {
                const int8_t* src = wg + (int64_t)co * K + k;
                if (vec_w && k + 16 <= K) {
                    afrag = *(const i32x4*)src;
                } else {
                    uint32_t w4[4] = {0, 0, 0, 0};
                    for (int b = 0; b < 16; ++b)
                        if (k + b < K) w4[b >> 2] |= (uint32_t)(uint8_t)src[b] << (8 * (b & 3));
                    afrag = i32x4{(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]};
                }
            }
            acc[mi] = __builtin_amdgcn_mfma_i32_16x16x64_i8(afrag, bfrag, acc[mi], 0, 0, 0);
        }
    }

    // Epilogue: lane holds rows 4*(lane/16)+v of column lane%16.
    const int p = p0 + wave * 16 + (lane & 15);
    if (p < HW) {
        int8_t* __restrict__ yg = (int8_t*)a.yptr;
        const bool relu = a.act == CONV_ACT_RELU;
        // Biases read before the first store (a read behind a store waits
        // for every earlier store).
        int32_t bias[MI][4];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int co = co0 + mi * 16 + (lane >> 4) * 4 + v;
                bias[mi][v] = (a.qbias && co < a.c_out) ? a.qbias[co] : 0;
            }
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int co = co0 + mi * 16 + (lane >> 4) * 4 + v;
                if (co < a.c_out) {
                    const int32_t val = acc[mi][v] + bias[mi][v];
                    yg[((int64_t)n * a.out_total + a.out_off + co) * HW + p] =
                        requant(val, a.composite, a.rounding, a.y_zp, relu);
                }
            }
    }
}


// Fast path for K <= 256 with 4-byte input rows: every chunk's input words
// and weight fragments are requested up front (loads unconditional, a slot
// past the channels reads channel 0 and its bytes are zeroed when stored),
// all chunks are transposed into LDS behind one barrier, then the MFMAs run
// with the pixel fragment as the first operand, so a lane holds 4
// consecutive pixels of one output channel and stores them as one word.
template <int MI, int NCH>
__global__ __launch_bounds__(kThreads) void qpw_fast_kernel(ConvArgs a) {
    __shared__ __align__(16) uint8_t xs[NCH][BN * XROW];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int K = a.c_in;
    const int HW = a.h * a.w;

    uint32_t L = blockIdx.x;
    const int cot = L % a.co_tiles;  L /= a.co_tiles;
    const int pt = L % a.tiles_w;    L /= a.tiles_w;
    const int n = L;
    const int co0 = cot * MI * 16;
    const int p0 = pt * BN;

    const int8_t* __restrict__ xg = (const int8_t*)a.xptr + ((int64_t)n * a.in_total + a.in_off) * HW;
    const int8_t* __restrict__ wg = (const int8_t*)a.wptr;
    const int kq = tid >> 4;   // this thread's 4 channels of a chunk: 4*kq ..
    const int pq = tid & 15;   // and 4 pixels: p0 + 4*pq ..
    const int p = p0 + 4 * pq;
    const bool pok = p < HW;   // HW % 4 == 0: a word is all in or all out

    uint32_t in[NCH][4];
    i32x4 wf[NCH][MI];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const int ch = 64 * c + 4 * kq + cc;
            in[c][cc] = *(const uint32_t*)(xg + (ch < K && pok ? (int64_t)ch * HW + p : 0));
        }
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const int co = co0 + mi * 16 + (lane & 15);
            const int k = 64 * c + 16 * (lane >> 4);
            const bool ok = co < a.c_out && k < K;
            wf[c][mi] = *(const i32x4*)(wg + (ok ? (int64_t)co * K + k : 0));
        }
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        uint32_t v[4], outw[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) v[cc] = 64 * c + 4 * kq + cc < K && pok ? in[c][cc] : 0u;
        transpose4x4(v, outw);
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) *(uint32_t*)&xs[c][(4 * pq + pp) * XROW + 4 * kq] = outw[pp];
    }
    __syncthreads();

    i32x4 acc[MI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) acc[mi] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const i32x4 pf = *(const i32x4*)&xs[c][(wave * 16 + (lane & 15)) * XROW + 16 * (lane >> 4)];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const int k = 64 * c + 16 * (lane >> 4);
            const i32x4 w = co0 + mi * 16 + (lane & 15) < a.c_out && k < K ? wf[c][mi] : i32x4{0, 0, 0, 0};
            acc[mi] = __builtin_amdgcn_mfma_i32_16x16x64_i8(pf, w, acc[mi], 0, 0, 0);
        }
    }

    // Lane: pixels 4*(lane/16) .. +3 of the wave's fragment, channel lane%16.
    const int px = p0 + wave * 16 + 4 * (lane >> 4);
    if (px < HW) {
        int8_t* __restrict__ yg = (int8_t*)a.yptr;
        const bool relu = a.act == CONV_ACT_RELU;
        int32_t bias[MI];   // read before the first store
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const int co = co0 + mi * 16 + (lane & 15);
            bias[mi] = (a.qbias && co < a.c_out) ? a.qbias[co] : 0;
        }
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const int co = co0 + mi * 16 + (lane & 15);
            if (co >= a.c_out) continue;
            const int32_t b = bias[mi];
            uint32_t word = 0;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                word |= (uint32_t)(uint8_t)requant(acc[mi][v] + b, a.composite, a.rounding, a.y_zp, relu) << (8 * v);
            *(uint32_t*)(yg + ((int64_t)n * a.out_total + a.out_off + co) * HW + px) = word;
        }
    }
}

template <int MI>
const void* pick_fast_nch(int nch) {
    switch (nch) {
    case 1: return (const void*)qpw_fast_kernel<MI, 1>;
    case 2: return (const void*)qpw_fast_kernel<MI, 2>;
    case 3: return (const void*)qpw_fast_kernel<MI, 3>;
    default: return (const void*)qpw_fast_kernel<MI, 4>;
    }
}

}  // namespace

bool plan_qpw(Desc& d) {
    const conv2d_params_t& p = d.p;
    if (!(p.k_h == 1 && p.k_w == 1 && p.stride_h == 1 && p.stride_w == 1 && p.groups == 1 &&
          p.pad_top == 0 && p.pad_left == 0 && p.pad_bottom == 0 && p.pad_right == 0))
        return false;
    if ((int64_t)p.h * p.w > INT32_MAX / 2) return false;
    d.tile_h = 1;
    d.tile_w = BN;
    d.lds_bytes = 0;
    return true;
}

hipError_t launch_qpw(const Desc& d, ConvArgs a, hipStream_t s) {
    const int hw = d.p.h * d.p.w;
    const int mi = d.p.c_out <= 16 ? 1 : d.p.c_out <= 32 ? 2 : d.p.c_out <= 48 ? 3 : 4;
    a.co_tiles = (d.p.c_out + mi * 16 - 1) / (mi * 16);
    a.tiles_w = (hw + BN - 1) / BN;
    const uint64_t blocks = (uint64_t)a.co_tiles * a.tiles_w * a.n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0xFFFFFFFFull) return hipErrorInvalidConfiguration;
    const dim3 grid((uint32_t)blocks), block(kThreads);
    // Fast path: whole 4-byte words of pixels in and out (plane sizes, channel
    // offsets and the pointers 4-byte aligned) and K <= 256.
    const int64_t ihw = (int64_t)hw;
    const bool words = hw % 4 == 0 && (uintptr_t)a.xptr % 4 == 0 && (uintptr_t)a.yptr % 4 == 0 &&
                       ((int64_t)a.in_total * ihw) % 4 == 0 && ((int64_t)a.out_total * ihw) % 4 == 0 &&
                       ((int64_t)a.in_off * ihw) % 4 == 0 && ((int64_t)a.out_off * ihw) % 4 == 0;
    const bool wvec = d.p.c_in % 16 == 0 && (uintptr_t)a.wptr % 16 == 0;
    if (words && wvec && d.p.c_in <= 4 * KC) {
        const int nch = (d.p.c_in + KC - 1) / KC;
        const void* fn = mi == 1 ? pick_fast_nch<1>(nch) : mi == 2 ? pick_fast_nch<2>(nch)
                         : mi == 3 ? pick_fast_nch<3>(nch) : pick_fast_nch<4>(nch);
        void* args[] = {&a};
        return hipLaunchKernel(fn, grid, block, args, 0, s);
    }
    const void* fn = mi == 1 ? (const void*)qpw_kernel<1> : mi == 2 ? (const void*)qpw_kernel<2>
                     : mi == 3 ? (const void*)qpw_kernel<3> : (const void*)qpw_kernel<4>;
    void* args[] = {&a};
    return hipLaunchKernel(fn, grid, block, args, 0, s);
}

}  // namespace conv2d
