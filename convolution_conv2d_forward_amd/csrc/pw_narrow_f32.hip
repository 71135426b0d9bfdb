// fp32 pointwise 1x1 convolution (stride 1, no pads, one group) that narrows
// a deep input to few channels: Y[co, p] = act(sum_k W[co, k] X[k, p] +
// b[co]) with 64 < K <= 256 and at most 32 output channels (ncnn
// convolution with a 1x1 kernel; the inverted bottleneck's linear
// projection, 192 -> 32).
//
// Such a layer moves K floats in per 32 floats out per pixel and does little
// arithmetic per byte, so it is set by how many input bytes are in flight.
// A workgroup owns 32 pixels of one image:
//   1. every thread issues all of its 16-byte loads of the [K][32] input
//      tile (up to 8) and of its weight operands before the first wait; the
//      tile goes to LDS (row stride 36 floats, so the four lane groups of an
//      operand fetch start 16 banks apart);
//   2. four waves split the 16-channel chunks (wave w takes chunks w, w + 4,
//      ...) over the 2 x 2 fragments of 16 pixels x 16 channels on
//      v_mfma_f32_16x16x4f32, pixels as the first operand; step s of lane
//      group q takes input channel 4q + s of the chunk, so a lane's weight
//      operands of a chunk are one 16-byte load;
//   3. the four partial tiles meet in LDS; each thread adds bias, applies
//      the activation and stores 4 pixels of one channel (16 bytes).
// The grid has one workgroup per 32 pixels (784 on the bottleneck), all
// resident at once.
#include "device_common.h"

namespace conv2d {

namespace {

constexpr int kT = 256;
constexpr int TP = 32;           // pixels per workgroup
constexpr int KMAX = 256;
constexpr int XST = TP + 4;      // LDS row stride of the input tile
constexpr int CPW = KMAX / 16 / 4;   // chunks per wave at most

__global__ __launch_bounds__(kT) void pw_narrow_f32_kernel(ConvArgs a) {
    __shared__ __align__(16) float xs[KMAX * XST];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 4, r = lane & 15;
    const int K = a.c_in, M = a.c_out, HW = a.w;
    const int tiles = a.tiles_w;
    const int pt = blockIdx.x % tiles, n = blockIdx.x / tiles;
    const int p0 = pt * TP;
    const int nch = (K + 15) / 16;
    const float* __restrict__ xg = (const float*)a.xptr + ((int64_t)n * a.in_total + a.in_off) * HW;
    const float* __restrict__ wg = (const float*)a.wptr;

    // ---- 1. loads: input units (channel u >> 3, pixels 4 (u & 7) ..) for
    // the chunks' rows, zero past K and past the image; weight operands of
    // this wave's chunks ----
    f32x4 v[KMAX * TP / 4 / kT];
#pragma unroll
    for (int i = 0; i < KMAX * TP / 4 / kT; ++i) {
        const int u = tid + kT * i;
        const int k = u >> 3, px = p0 + 4 * (u & 7);
        v[i] = (k < K && px < HW) ? *(const f32x4*)(xg + (int64_t)k * HW + px) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    f32x4 wv[CPW][2];
#pragma unroll
    for (int t = 0; t < CPW; ++t) {
        const int c = wave + 4 * t;
        const int k = 16 * c + 4 * q;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int co = 16 * j + r;
            wv[t][j] = (c < nch && k < K && co < M) ? *(const f32x4*)(wg + (int64_t)co * K + k)
                                                    : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }
#pragma unroll
    for (int i = 0; i < KMAX * TP / 4 / kT; ++i) {
        const int u = tid + kT * i;
        if ((u >> 3) < 16 * nch) *(f32x4*)(xs + (u >> 3) * XST + 4 * (u & 7)) = v[i];
    }
    __syncthreads();

    // ---- 2. this wave's chunks on the matrix cores ----
    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < CPW; ++t) {
        const int c = wave + 4 * t;
        if (c >= nch) break;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float x0 = xs[(16 * c + 4 * q + s) * XST + r];
            const float x1 = xs[(16 * c + 4 * q + s) * XST + 16 + r];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(x0, wv[t][j][s], acc[0][j], 0, 0, 0);
                acc[1][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(x1, wv[t][j][s], acc[1][j], 0, 0, 0);
            }
        }
    }
    __syncthreads();

    // ---- 3. partial tiles [wave][co][pixel] in LDS, summed per 4 pixels ----
    // Lane (q, r) of fragment (i, j) holds pixels 16 i + 4 q .. + 3 of
    // channel 16 j + r.
    float* red = xs;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            *(f32x4*)(red + (wave * 32 + 16 * j + r) * XST + 16 * i + 4 * q) = acc[i][j];
    __syncthreads();
    const int co = tid >> 3, px = 4 * (tid & 7);
    if (co < M && p0 + px < HW) {
        f32x4 sum = *(const f32x4*)(red + co * XST + px);
#pragma unroll
        for (int w = 1; w < 4; ++w) sum += *(const f32x4*)(red + (w * 32 + co) * XST + px);
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = bias_act(a, sum[e], co);
        float* __restrict__ yg = (float*)a.yptr + ((int64_t)n * a.out_total + a.out_off) * HW;
        *(f32x4*)(yg + (int64_t)co * HW + p0 + px) = o;
    }
}

}  // namespace

bool plan_pw_narrow_f32(const Desc& d) {
    const conv2d_params_t& p = d.p;
    if (p.dtype != CONV_DTYPE_F32 || p.k_h != 1 || p.k_w != 1 || p.stride_h != 1 || p.stride_w != 1) return false;
    if (p.pad_top || p.pad_left || p.pad_bottom || p.pad_right || p.groups != 1) return false;
    if (p.c_in <= 64 || p.c_in > KMAX || p.c_in % 4 != 0 || p.c_out > 32) return false;
    const int64_t hw = (int64_t)p.h * p.w;
    return hw % 4 == 0 && (int64_t)p.c_in * hw < INT32_MAX && (int64_t)p.c_out * hw < INT32_MAX;
}

hipError_t launch_pw_narrow_f32(const Desc& d, ConvArgs a, hipStream_t s) {
    if (!pointwise_f32_fits(d, a)) return hipErrorInvalidValue;
    const int64_t hw = (int64_t)d.p.h * d.p.w;
    a.h = 1;
    a.w = (int32_t)hw;
    a.tiles_w = (int32_t)((hw + TP - 1) / TP);
    const uint64_t blocks = (uint64_t)a.tiles_w * a.n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
    void* args[] = {&a};
    return hipLaunchKernel((const void*)pw_narrow_f32_kernel, dim3((uint32_t)blocks), dim3(kT), args, 0, s);
}

}  // namespace conv2d
