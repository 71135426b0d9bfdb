// fp32 pointwise 1x1 convolution (stride 1, no pads, one group) for shallow
// reductions: Y[co, p] = act(sum_k W[co, k] X[k, p] + b[co]) (ncnn
// convolution with a 1x1 kernel; the inverted bottleneck's expansion and
// projection layers).
//
// With K <= 64 the implicit GEMM's K-split pipeline has little to pipeline,
// and its 32-channel tiles re-read the input once per tile.  Here a
// workgroup owns 64 pixels of one image and every output channel (measured
// on the inverted bottleneck: 32 -> 192 runs ~10% faster this way, while
// 192 -> 32, whose 48 KB input tile leaves one workgroup per CU, runs 1.7x
// slower, so deeper reductions stay with the implicit GEMM):
//   1. the 64-pixel input tile (K rows) and the whole weight matrix
//      (Cout x K) are copied into LDS once, all 16-byte loads issued before
//      the first LDS write;
//   2. eight waves: wave w multiplies pixel fragment w % 4 (16 pixels) with
//      every other block of 32 output channels on the fp32 matrix cores
//      (v_mfma_f32_16x16x4f32, pixels as the first operand, so a lane ends
//      up holding 4 consecutive pixels of one output channel); the pixel
//      operands are read from LDS once, a block's weight operands before its
//      first MFMA;
//   3. bias + activation, one 16-byte store per lane and channel
//      (ConcatFusedTail offsets included).
#include "device_common.h"

namespace conv2d {

namespace {

constexpr int kT = 512;          // 8 waves: 4 pixel fragments x 2 halves of the channel blocks
constexpr int PT = 64;           // pixels per workgroup
constexpr int XS = PT + 16;      // LDS row stride of the input tile (= 16 mod 32)
constexpr int KMAX = 64;
constexpr int WMAX = 16384;      // weight floats staged in LDS (64 KB)

// LDS row stride of the weight matrix: >= k, a multiple of 4, = 4 mod 64 (the
// 16 rows x 4 k of an operand fetch then hit 64 different banks).
__host__ __device__ inline int w_stride(int k) {
    int s = (k + 3) / 4 * 4;
    while (s % 64 != 4) s += 4;
    return s;
}

__global__ __launch_bounds__(kT) void pointwise_f32_kernel(ConvArgs a, int ws) {
    extern __shared__ __align__(16) float lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = tid >> 6;
    const int K = a.c_in, M = a.c_out;
    const int HW = a.w;                                 // flattened: one row of h*w pixels
    const int tiles = a.tiles_w;
    const int pt = blockIdx.x % tiles, n = blockIdx.x / tiles;
    const int p0 = pt * PT;
    const int K4 = (K + 3) & ~3;

    float* xs = lds;                                    // [K4][XS]
    float* wsm = lds + K4 * XS;                         // [M][ws]
    const float* __restrict__ xg = (const float*)a.xptr + ((int64_t)n * a.in_total + a.in_off) * HW;
    const float* __restrict__ wg = (const float*)a.wptr;

    // ---- 1. input tile and weights -> LDS ----
    // Input: 16 four-pixel units per channel row; weights: K/4 units per row
    // (K % 4 == 0 on this path).  Rows past K and pixels past the image are
    // zero.
    const int xunits = K4 * (PT / 4);
    const int wunits = M * (K / 4);
    for (int base = 0; base < xunits + wunits; base += 8 * kT) {
        f32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int u = base + tid + i * kT;
            f32x4 r = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (u < xunits) {
                const int k = u >> 4, q = u & 15;
                const int p = p0 + 4 * q;
                if (k < K && p < HW) r = *(const f32x4*)(xg + (int64_t)k * HW + p);
            } else if (u < xunits + wunits) {
                const int e = u - xunits;
                r = *(const f32x4*)(wg + 4 * (int64_t)e);
            }
            v[i] = r;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int u = base + tid + i * kT;
            if (u < xunits) {
                *(f32x4*)(xs + (u >> 4) * XS + 4 * (u & 15)) = v[i];
            } else if (u < xunits + wunits) {
                const int e = u - xunits;
                const int row = e / (K / 4), c4 = e - row * (K / 4);
                *(f32x4*)(wsm + row * ws + 4 * c4) = v[i];
            }
        }
    }
    __syncthreads();

    // ---- 2./3. per 32-channel block: MFMAs, bias + activation, store ----
    // Wave w multiplies pixel fragment w % 4 with every other 32-channel
    // block (those of parity w / 4).  Its pixel operands are the same for
    // every block and are read once; a block's weight operands are all read
    // before its first MFMA.
    const int kq = lane >> 4, l16 = lane & 15;
    const int frag = wave & 3, half = wave >> 2;
    const int px = p0 + frag * 16 + 4 * kq;             // this lane's 4 output pixels
    float* __restrict__ yg = (float*)a.yptr;
    const int64_t ybase = ((int64_t)n * a.out_total + a.out_off) * HW;
    const int ksteps = K4 >> 2;
    float xa[KMAX / 4];
#pragma unroll
    for (int s = 0; s < KMAX / 4; ++s) xa[s] = s < ksteps ? xs[(4 * s + kq) * XS + frag * 16 + l16] : 0.0f;
    for (int cb = 32 * half; cb < M; cb += 64) {
        f32x4 acc[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
        const int co_a = cb + l16, co_b = cb + 16 + l16;
        const float* wa = wsm + min(co_a, M - 1) * ws;
        const float* wb = wsm + min(co_b, M - 1) * ws;
        float fa[KMAX / 4], fb[KMAX / 4];
#pragma unroll
        for (int s = 0; s < KMAX / 4; ++s) {
            fa[s] = s < ksteps ? wa[4 * s + kq] : 0.0f;
            fb[s] = s < ksteps ? wb[4 * s + kq] : 0.0f;
        }
#pragma unroll
        for (int s = 0; s < KMAX / 4; ++s) {
            if (s < ksteps) {
                acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[s], fa[s], acc[0], 0, 0, 0);
                acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[s], fb[s], acc[1], 0, 0, 0);
            }
        }
        if (px < HW) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int co = cb + 16 * m + l16;
                if (co >= M) continue;
                f32x4 o;
#pragma unroll
                for (int v = 0; v < 4; ++v) o[v] = bias_act(a, acc[m][v], co);
                *(f32x4*)(yg + ybase + (int64_t)co * HW + px) = o;
            }
        }
    }
}

}  // namespace

bool plan_pointwise_f32(const Desc& d) {
    const conv2d_params_t& p = d.p;
    if (p.dtype != CONV_DTYPE_F32 || p.k_h != 1 || p.k_w != 1 || p.stride_h != 1 || p.stride_w != 1) return false;
    if (p.pad_top || p.pad_left || p.pad_bottom || p.pad_right || p.groups != 1) return false;
    if (p.c_in > KMAX || p.c_in % 4 != 0 || (int64_t)p.c_out * w_stride(p.c_in) > WMAX) return false;
    const int64_t hw = (int64_t)p.h * p.w;
    if (hw % 4 != 0 || hw >= INT32_MAX / 2) return false;
    return true;
}

// 16-byte loads and stores: the pointers, the planes and the channel offsets
// must keep every pixel row 16-byte aligned.
bool pointwise_f32_fits(const Desc& d, const ConvArgs& a) {
    const int64_t hw = (int64_t)d.p.h * d.p.w;
    return (uintptr_t)a.xptr % 16 == 0 && (uintptr_t)a.yptr % 16 == 0 && (uintptr_t)a.wptr % 16 == 0 &&
           (a.in_total * hw) % 4 == 0 && (a.out_total * hw) % 4 == 0 && (a.in_off * hw) % 4 == 0 &&
           (a.out_off * hw) % 4 == 0;
}

hipError_t launch_pointwise_f32(const Desc& d, ConvArgs a, hipStream_t s) {
    const int hw = d.p.h * d.p.w;
    if (!pointwise_f32_fits(d, a)) return hipErrorInvalidValue;
    a.h = 1;
    a.w = hw;
    a.tiles_w = (hw + PT - 1) / PT;
    const uint64_t blocks = (uint64_t)a.tiles_w * a.n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
    const int ws = w_stride(d.p.c_in);
    const int k4 = (d.p.c_in + 3) & ~3;
    const int lds = 4 * (k4 * XS + d.p.c_out * ws);
    const void* fn = (const void*)pointwise_f32_kernel;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
    }
    void* args[] = {&a, (void*)&ws};
    return hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(kT), args, lds, s);
}

}  // namespace conv2d
