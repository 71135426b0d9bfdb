// Depthwise convolution (groups == c_in == c_out): ncnn
// "convolutiondepthwise" with one filter per channel, and the yscv int8
// depthwise QLinearConv (3x3 s1 / s2, int32 accumulate, requant).
//
// There is about one multiply-add per byte moved, so the kernel is bound by
// HBM and is built to keep HBM busy: a workgroup owns a tile of one (n, c)
// plane, every thread first issues all of its 16-byte loads of the input
// window (pad_value, or the zero point for int8, outside the image) and only
// then writes them to LDS, so a plane's worth of reads is in flight at once.
// Each thread then computes an R x VO block of outputs from a register
// window read out of LDS (R rows share their input rows, VO columns share
// their columns) and writes each output row with one vector store.  No MFMA:
// there is no reduction dimension to feed it.
#include "device_common.h"

#include <type_traits>

namespace conv2d {

namespace {

constexpr int kThreads = 256;
constexpr int VO = 4;        // consecutive outputs per thread and row
constexpr int NVMAX = 8;     // 16-byte input vectors per thread (window <= 2048 vectors)

template <typename T> struct Elem;
template <> struct Elem<float> { using lds_t = float; using acc_t = float; static constexpr int VL = 4; };
template <> struct Elem<__hip_bfloat16> { using lds_t = float; using acc_t = float; static constexpr int VL = 8; };
template <> struct Elem<int8_t> { using lds_t = int32_t; using acc_t = int32_t; static constexpr int VL = 16; };

// Convert one 16-byte input vector to VL LDS values.
template <typename T>
__device__ __forceinline__ void widen(uint4 raw, typename Elem<T>::lds_t* out) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    if constexpr (std::is_same<T, float>::value) {
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = __uint_as_float(w[q]);
    } else if constexpr (std::is_same<T, int8_t>::value) {
#pragma unroll
        for (int q = 0; q < 16; ++q) out[q] = (int32_t)(int8_t)(w[q >> 2] >> (8 * (q & 3)));
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            out[2 * q] = __uint_as_float(w[q] << 16);
            out[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
        }
    }
}

template <typename T>
__device__ __forceinline__ typename Elem<T>::lds_t load_scalar(const T* p, int64_t i) {
    if constexpr (std::is_same<T, __hip_bfloat16>::value) return bf16_to_f32(p[i]);
    else return (typename Elem<T>::lds_t)p[i];
}

// VEC: rows move as 16-byte vectors (w % VL == 0, 16-byte aligned x).
// KH/KW/SH/SW: compile-time kernel and stride with dilation 1 (0 = runtime
// kernel, stride and dilation, one output row per thread).  R: output rows
// per thread.
template <typename T, bool VEC, int KH, int KW, int SH, int SW, int R>
__global__ __launch_bounds__(kThreads) void dw_kernel(ConvArgs a) {
    using LT = typename Elem<T>::lds_t;
    using AT = typename Elem<T>::acc_t;
    constexpr int VL = VEC ? Elem<T>::VL : 1;
    constexpr bool FIXED = KH > 0;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    LT* tile = (LT*)lds_raw;

    const int kh = FIXED ? KH : a.k_h, kw = FIXED ? KW : a.k_w;
    const int sh = FIXED ? SH : a.stride_h, sw = FIXED ? SW : a.stride_w;
    const int dh = FIXED ? 1 : a.dilation_h, dwl = FIXED ? 1 : a.dilation_w;

    // block -> (tile col, tile row, channel, image)
    uint32_t L = blockIdx.x;
    uint32_t Q = divu(L, a.dv_tiles_w);
    const int twi = L - Q * a.tiles_w;
    L = Q; Q = divu(L, a.dv_tiles_h);
    const int thi = L - Q * a.tiles_h;
    L = Q; Q = divu(L, a.dv_co_tiles);       // co_tiles holds c_out here
    const int c = L - Q * a.c_out;
    const int n = Q;

    const int ho0 = thi * a.tile_h, wo0 = twi * a.tile_w;
    const int th_n = min(a.tile_h, a.ho - ho0);
    const int tw_n = min(a.tile_w, a.wo - wo0);
    const int ih_lo = ho0 * sh - a.pad_top;
    const int iw_lo = wo0 * sw - a.pad_left;
    // First LDS column: iw_lo rounded down to a multiple of VL.
    const int iw_a = VL > 1 ? (iw_lo >= 0 ? iw_lo / VL * VL : -((-iw_lo + VL - 1) / VL) * VL) : iw_lo;
    const int rows = (th_n - 1) * sh + (kh - 1) * dh + 1;
    const int iw_hi = (wo0 + tw_n - 1) * sw - a.pad_left + (kw - 1) * dwl;
    const int lw = (iw_hi + 1 - iw_a + VL - 1) / VL * VL;   // LDS row length (elements)
    const int lwv = lw / VL;
    const int shift = iw_lo - iw_a;

    const int64_t HW = (int64_t)a.h * a.w;
    const T* __restrict__ xp = (const T*)a.xptr + ((int64_t)n * a.in_total + a.in_off + c) * HW;

    LT padv;
    if constexpr (std::is_same<T, int8_t>::value) padv = 0;   // symmetric int8: the pad is the zero point
    else padv = (LT)a.pad_value;

    // ---- input window -> LDS: all loads first, then the LDS writes ----
    const int nvec = rows * lwv;
    if constexpr (VL > 1) {
        uint4 buf[NVMAX];
        bool inb[NVMAX];
#pragma unroll
        for (int i = 0; i < NVMAX; ++i) {
            const int v = threadIdx.x + i * kThreads;
            const int r = v / lwv;
            const int iw = iw_a + (v - r * lwv) * VL;
            const int ih = ih_lo + r;
            // Vectors never straddle the image edge: w % VL == 0 and iw % VL == 0.
            inb[i] = v < nvec && (unsigned)ih < (unsigned)a.h && iw >= 0 && iw < a.w;
            buf[i] = inb[i] ? *(const uint4*)(xp + (int64_t)ih * a.w + iw) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NVMAX; ++i) {
            const int v = threadIdx.x + i * kThreads;
            if (v < nvec) {
                LT vals[VL];
                widen<T>(buf[i], vals);
                LT* dst = tile + v * VL;
#pragma unroll
                for (int q = 0; q < VL; ++q) dst[q] = inb[i] ? vals[q] : padv;
            }
        }
    } else {
        for (int v = threadIdx.x; v < nvec; v += kThreads) {
            const int r = v / lwv;
            const int iw = iw_a + (v - r * lwv);
            const int ih = ih_lo + r;
            tile[v] = ((unsigned)ih < (unsigned)a.h && (unsigned)iw < (unsigned)a.w)
                          ? load_scalar<T>(xp, (int64_t)ih * a.w + iw)
                          : padv;
        }
    }

    // Filter taps of this channel (OIHW with one input channel per group).
    const int khw = kh * kw;
    constexpr int KMAX = FIXED ? KH * KW : 25;
    AT wt[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) wt[i] = i < khw ? (AT)load_scalar<T>((const T*)a.wptr, (int64_t)c * khw + i) : (AT)0;
    AT bias = 0;
    if constexpr (std::is_same<T, int8_t>::value) {
        if (a.qbias) bias = a.qbias[c];
    }
    __syncthreads();

    // ---- outputs: R rows x VO columns per thread ----
    const int uw = (tw_n + VO - 1) / VO;
    const int uh = (th_n + R - 1) / R;
    const int units = uh * uw;
    const int64_t oplane = (int64_t)a.ho * a.wo;
    T* __restrict__ yp = (T*)a.yptr + ((int64_t)n * a.out_total + a.out_off + c) * oplane;
    const bool relu8 = a.act == CONV_ACT_RELU;
    for (int u = threadIdx.x; u < units; u += kThreads) {
        const int rr = u / uw;
        const int q0 = (u - rr * uw) * VO;
        const int r0 = rr * R;
        AT acc[R][VO];
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int q = 0; q < VO; ++q) acc[i][q] = 0;
        if constexpr (FIXED) {
            // Register window: RIN rows x CIN columns of the LDS tile.
            constexpr int RIN = (R - 1) * SH + KH;
            constexpr int CIN = (VO - 1) * SW + KW;
            const int cmax = lw - shift - 1;     // last readable column of the window
#pragma unroll
            for (int i = 0; i < RIN; ++i) {
                const int row = r0 * SH + i;
                if (row >= rows) break;
                const LT* src = tile + row * lw + shift + q0 * SW;
                LT win[CIN];
#pragma unroll
                for (int j = 0; j < CIN; ++j) win[j] = src[q0 * SW + j <= cmax ? j : 0];
#pragma unroll
                for (int orow = 0; orow < R; ++orow) {
                    const int r = i - orow * SH;       // filter row this input row feeds
                    if (r < 0 || r >= KH) continue;
#pragma unroll
                    for (int s = 0; s < KW; ++s)
#pragma unroll
                        for (int q = 0; q < VO; ++q) {
                            if constexpr (std::is_same<AT, int32_t>::value) acc[orow][q] += win[q * SW + s] * wt[r * KW + s];
                            else acc[orow][q] = fmaf(win[q * SW + s], wt[r * KW + s], acc[orow][q]);
                        }
                }
            }
        } else {
            for (int r = 0; r < kh; ++r) {
                const LT* row = tile + (r0 * sh + r * dh) * lw + shift;
                for (int s = 0; s < kw; ++s) {
#pragma unroll
                    for (int q = 0; q < VO; ++q) {
                        const int col = (q0 + q) * sw + s * dwl;
                        const AT xv = (AT)row[col < lw - shift ? col : 0];
                        if constexpr (std::is_same<AT, int32_t>::value) acc[0][q] += xv * wt[r * kw + s];
                        else acc[0][q] = fmaf(xv, wt[r * kw + s], acc[0][q]);
                    }
                }
            }
        }
#pragma unroll
        for (int orow = 0; orow < R; ++orow) {
            const int th = r0 + orow;
            if (th >= th_n) break;
            const int ho = ho0 + th;
            const int wo = wo0 + q0;
            T outv[VO];
#pragma unroll
            for (int q = 0; q < VO; ++q) {
                if constexpr (std::is_same<T, int8_t>::value) {
                    outv[q] = requant(acc[orow][q] + bias, a.composite, a.rounding, a.y_zp, relu8);
                } else if constexpr (std::is_same<T, __hip_bfloat16>::value) {
                    outv[q] = f32_to_bf16(bias_act(a, acc[orow][q], c));
                } else {
                    outv[q] = bias_act(a, acc[orow][q], c);
                }
            }
            T* dst = yp + (int64_t)ho * a.wo + wo;
            if (a.vec_store && q0 + VO <= tw_n) {
                if constexpr (sizeof(T) == 4) {
                    *(float4*)dst = make_float4(outv[0], outv[1], outv[2], outv[3]);
                } else if constexpr (sizeof(T) == 1) {
                    *(uint32_t*)dst = (uint32_t)(uint8_t)outv[0] | ((uint32_t)(uint8_t)outv[1] << 8) |
                                      ((uint32_t)(uint8_t)outv[2] << 16) | ((uint32_t)(uint8_t)outv[3] << 24);
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
}

// fp32 3x3 stride-1 depthwise over whole planes (ncnn "convolutiondepthwise",
// one filter per channel).  The tile kernel above gives every (n, c) plane a
// workgroup of its own: all of a launch's reads are in flight together, then
// all of its writes, so reads and writes barely overlap.  Here a smaller grid
// of persistent workgroups walks the planes (plane p, p + grid, ...) through
// two LDS buffers: the next plane's 16-byte loads are issued before the
// current plane's taps, so its reads run under the current plane's stores.
// LDS column pad_left + iw holds input column iw, so output column wo reads
// columns wo .. wo + 2 and four outputs read one float4 and one float2 per
// row; pad cells never change from plane to plane and are written once.
constexpr int PNV = 4;          // 16-byte input vectors per thread and plane (planes <= 4096 elements)
constexpr int kPlaneWgPerCu = 3;  // persistent workgroups per compute unit

__global__ __launch_bounds__(kThreads) void dw3s1_planes_kernel(ConvArgs a) {
    extern __shared__ __align__(16) unsigned char lds_raw[];
    float* lds = (float*)lds_raw;
    const int tid = threadIdx.x;
    const int H = a.h, W = a.w, Ho = a.ho, Wo = a.wo;
    const int pt = a.pad_top, pl = a.pad_left;
    const int LW = a.patch_w, RHA = a.patch_h;   // LDS row stride, rows per buffer
    const int bufsz = RHA * LW;
    const int C = a.c_out;
    const int P = a.n * C;
    const int G = gridDim.x;
    const int64_t HW = (int64_t)H * W;
    const int64_t oplane = (int64_t)Ho * Wo;

    // This thread's input vectors: the same plane-relative offsets for every plane.
    const int wv = W >> 2;
    const int nvec = H * wv;
    int goff[PNV], loff[PNV];
    bool ok[PNV];
#pragma unroll
    for (int i = 0; i < PNV; ++i) {
        const int v = tid + i * kThreads;
        const int r = v / wv;
        const int cq = v - r * wv;
        ok[i] = v < nvec;
        goff[i] = ok[i] ? r * W + 4 * cq : 0;   // spare lanes reload the first vector
        loff[i] = (r + pt) * LW + pl + 4 * cq;
    }

    // The next plane in flight: its 16-byte vectors, taps, bias and PReLU
    // slope, copied out at the top of its plane after the one wait for the
    // vectors, so the taps and the stores never wait for a load still in
    // flight.
    const ActP ap = act_params(a);
    uint4 buf[PNV];
    float wn[9], bn, sn;
    auto issue = [&](int pp) {
        const int nn = (int)divu((uint32_t)pp, a.dv_co_tiles);
        const int cc = pp - nn * C;
        const float* xp = (const float*)a.xptr + ((int64_t)nn * a.in_total + a.in_off + cc) * HW;
#pragma unroll
        for (int i = 0; i < PNV; ++i) buf[i] = *(const uint4*)(xp + goff[i]);
        const float* wq = (const float*)a.wptr + (int64_t)cc * 9;
#pragma unroll
        for (int k = 0; k < 9; ++k) wn[k] = wq[k];
        bn = a.bias ? a.bias[cc] : 0.0f;
        sn = act_slope(a, ap, cc);
    };

    int p = blockIdx.x;
    if (p < P) issue(p);

    // Pad cells of both buffers: whole rows above and below the image, then
    // the columns left and right of it on the image rows.
    const float padv = a.pad_value;
    const int prow = RHA - H;
    for (int idx = tid; idx < 2 * prow * LW; idx += kThreads) {
        const int b = idx >= prow * LW;
        const int j = idx - b * prow * LW;
        const int rr = j / LW;
        const int col = j - rr * LW;
        lds[b * bufsz + (rr < pt ? rr : rr + H) * LW + col] = padv;
    }
    const int pc = LW - W;
    for (int idx = tid; idx < 2 * H * pc; idx += kThreads) {
        const int b = idx >= H * pc;
        const int j = idx - b * H * pc;
        const int rr = j / pc;
        const int k = j - rr * pc;
        lds[b * bufsz + (rr + pt) * LW + (k < pl ? k : k + W)] = padv;
    }

    const int gw = Wo >> 2;
    const int units = ((Ho + 3) >> 2) * gw;
    for (int it = 0; p < P; ++it, p += G) {
        float* T = lds + (it & 1) * bufsz;
#pragma unroll
        for (int i = 0; i < PNV; ++i) {
            if (!ok[i]) continue;
            float* dst = T + loff[i];
            if ((pl & 3) == 0) {
                *(uint4*)dst = buf[i];
            } else if ((pl & 1) == 0) {
                *(uint2*)dst = make_uint2(buf[i].x, buf[i].y);
                *(uint2*)(dst + 2) = make_uint2(buf[i].z, buf[i].w);
            } else {
                dst[0] = __uint_as_float(buf[i].x);
                dst[1] = __uint_as_float(buf[i].y);
                dst[2] = __uint_as_float(buf[i].z);
                dst[3] = __uint_as_float(buf[i].w);
            }
        }
        float wt[9];
#pragma unroll
        for (int k = 0; k < 9; ++k) wt[k] = wn[k];
        const float bv = bn, slope = sn;
        const int n = (int)divu((uint32_t)p, a.dv_co_tiles);
        const int c = p - n * C;
        float* yp = (float*)a.yptr + ((int64_t)n * a.out_total + a.out_off + c) * oplane;
        if (p + G < P) issue(p + G);
        __syncthreads();

        for (int u = tid; u < units; u += kThreads) {
            const int rb = (int)fdiv((uint32_t)u, a.div_tile_w);
            const int r0 = rb * 4;
            const int wo0 = (u - rb * gw) * 4;
            float acc[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[i][q] = 0.0f;
            const float* src = T + r0 * LW + wo0;
#pragma unroll
            for (int i = 0; i < 6; ++i) {
                const float4 lo = *(const float4*)(src + i * LW);
                const float2 hi = *(const float2*)(src + i * LW + 4);
                const float win[6] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y};
#pragma unroll
                for (int orow = 0; orow < 4; ++orow) {
                    const int r = i - orow;
                    if (r < 0 || r > 2) continue;
#pragma unroll
                    for (int s = 0; s < 3; ++s)
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[orow][q] = fmaf(win[q + s], wt[r * 3 + s], acc[orow][q]);
                }
            }
#pragma unroll
            for (int orow = 0; orow < 4; ++orow) {
                const int ho = r0 + orow;
                if (ho >= Ho) break;
                float4 o;
                o.x = act_apply(acc[orow][0] + bv, slope, ap.lo, ap.hi);
                o.y = act_apply(acc[orow][1] + bv, slope, ap.lo, ap.hi);
                o.z = act_apply(acc[orow][2] + bv, slope, ap.lo, ap.hi);
                o.w = act_apply(acc[orow][3] + bv, slope, ap.lo, ap.hi);
                *(float4*)(yp + (int64_t)ho * Wo + wo0) = o;
            }
        }
    }
}

// Shapes the plane kernel takes (fp32, 3x3, stride 1, dilation 1, rows of
// whole 16-byte vectors in and out, a plane of at most PNV * 256 vectors and
// two plane buffers in 64 KB of LDS); the call also needs 16-byte aligned x
// and y.
bool dw_planes_fit(const Desc& d, int* lds_bytes) {
    const conv2d_params_t& p = d.p;
    if (p.dtype != CONV_DTYPE_F32 || p.k_h != 3 || p.k_w != 3 || p.stride_h != 1 || p.stride_w != 1 ||
        p.dilation_h != 1 || p.dilation_w != 1)
        return false;
    if (p.w % 4 != 0 || d.wo % 4 != 0 || d.ho < 1 || (int64_t)p.h * p.w > (int64_t)PNV * kThreads * 4)
        return false;
    const int64_t bytes = 2 * (int64_t)((d.ho + 3) / 4 * 4 + 2) * (d.wo + 4) * 4;
    if (bytes > 64 * 1024) return false;
    *lds_bytes = (int)bytes;
    return true;
}

hipError_t launch_dw_planes(const Desc& d, ConvArgs a, hipStream_t s) {
    const int64_t planes = (int64_t)a.n * a.c_out;
    if (planes == 0) return hipSuccess;
    if (planes > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    a.patch_w = d.wo + 4;
    a.patch_h = (d.ho + 3) / 4 * 4 + 2;
    a.div_tile_w = make_fastdiv((uint32_t)(d.wo / 4));
    a.dv_co_tiles = make_divu32((uint32_t)a.c_out);
    const int64_t cap = (int64_t)kPlaneWgPerCu * device_cu_count();
    const uint32_t grid = (uint32_t)(planes < cap ? planes : cap);
    const size_t lds = (size_t)2 * a.patch_h * a.patch_w * sizeof(float);
    void* args[] = {&a};
    return hipLaunchKernel((const void*)dw3s1_planes_kernel, dim3(grid), dim3(kThreads), args, lds, s);
}

// LDS bytes of the window of a tile (worst-case alignment slack).
template <typename T>
size_t window_bytes(const conv2d_params_t& p, int tile_h, int tile_w, int ho, int wo) {
    using LT = typename Elem<T>::lds_t;
    const int VL = Elem<T>::VL;
    const int th = tile_h < ho ? tile_h : ho;
    const int tw = tile_w < wo ? tile_w : wo;
    const int rows = (th - 1) * p.stride_h + (p.k_h - 1) * p.dilation_h + 1;
    const int span = (tw - 1) * p.stride_w + (p.k_w - 1) * p.dilation_w + 1;
    const int lw = (span + 2 * VL - 2 + VL - 1) / VL * VL;
    return (size_t)rows * lw * sizeof(LT);
}

// Input vectors of the window (for the NVMAX bound of the vector path).
template <typename T>
int window_vectors(const conv2d_params_t& p, int tile_h, int tile_w, int ho, int wo) {
    return (int)(window_bytes<T>(p, tile_h, tile_w, ho, wo) / sizeof(typename Elem<T>::lds_t) / Elem<T>::VL);
}

template <typename T>
bool plan_dw_t(Desc& d) {
    const conv2d_params_t& p = d.p;
    if (p.k_h * p.k_w > 25) return false;
    // Whole rows when they fit; otherwise 256-wide column strips.  Halve the
    // rows until the window fits both LDS and the per-thread load budget.
    const int tw = d.wo <= 256 ? d.wo : 256;
    int th = d.ho;
    while (th > 1 && (window_bytes<T>(p, th, tw, d.ho, d.wo) > 32 * 1024 ||
                      window_vectors<T>(p, th, tw, d.ho, d.wo) > NVMAX * kThreads))
        th = (th + 1) / 2;
    if (window_bytes<T>(p, th, tw, d.ho, d.wo) > 48 * 1024 ||
        window_vectors<T>(p, th, tw, d.ho, d.wo) > NVMAX * kThreads)
        return false;
    d.tile_h = th;
    d.tile_w = tw;
    d.lds_bytes = (int)window_bytes<T>(p, th, tw, d.ho, d.wo);
    return true;
}

template <typename T, bool VEC>
const void* pick(const conv2d_params_t& p) {
    const bool d1 = p.dilation_h == 1 && p.dilation_w == 1;
    if (d1 && p.k_h == 3 && p.k_w == 3 && p.stride_h == 1 && p.stride_w == 1)
        return (const void*)dw_kernel<T, VEC, 3, 3, 1, 1, 4>;
    if (d1 && p.k_h == 3 && p.k_w == 3 && p.stride_h == 2 && p.stride_w == 2)
        return (const void*)dw_kernel<T, VEC, 3, 3, 2, 2, 2>;
    if (d1 && p.k_h == 5 && p.k_w == 5 && p.stride_h == 1 && p.stride_w == 1)
        return (const void*)dw_kernel<T, VEC, 5, 5, 1, 1, 4>;
    return (const void*)dw_kernel<T, VEC, 0, 0, 0, 0, 1>;
}

template <typename T>
hipError_t launch_t(const Desc& d, ConvArgs a, hipStream_t s) {
    // The pad enters the input's storage type, as every other bf16 kernel
    // takes it: padded taps read the bf16 value nearest pad_value.
    if constexpr (std::is_same<T, __hip_bfloat16>::value) a.pad_value = bf16_to_f32(f32_to_bf16(a.pad_value));
    a.tile_h = d.tile_h;
    a.tile_w = d.tile_w;
    a.tiles_h = (d.ho + d.tile_h - 1) / d.tile_h;
    a.tiles_w = (d.wo + d.tile_w - 1) / d.tile_w;
    const uint64_t blocks = (uint64_t)a.tiles_w * a.tiles_h * a.c_out * a.n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0xFFFFFFFFull) return hipErrorInvalidConfiguration;
    a.dv_tiles_w = make_divu32((uint32_t)a.tiles_w);
    a.dv_tiles_h = make_divu32((uint32_t)a.tiles_h);
    a.dv_co_tiles = make_divu32((uint32_t)a.c_out);
    const bool vec = (d.p.w % Elem<T>::VL) == 0 && ((uintptr_t)a.xptr % 16) == 0;
    // Output rows move as one VO-element vector when every row start keeps
    // the vector alignment.
    a.vec_store = (d.wo % VO) == 0 && ((uintptr_t)a.yptr % (VO * sizeof(T))) == 0;
    const void* fn = vec ? pick<T, true>(d.p) : pick<T, false>(d.p);
    void* args[] = {&a};
    return hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(kThreads), args, d.lds_bytes, s);
}

}  // namespace

// cfg 1: the shape also fits the fp32 plane kernel (launch_dw takes it when
// x and y are 16-byte aligned); the tile kernel is planned in every case.
bool plan_dw(Desc& d) {
    if (d.p.dtype == CONV_DTYPE_BF16) return plan_dw_t<__hip_bfloat16>(d);
    if (!plan_dw_t<float>(d)) return false;
    int lds = 0;
    d.cfg = dw_planes_fit(d, &lds) ? 1 : 0;
    return true;
}

// int8: the byte-plane dot-product kernel for 3x3 s1/s2 (cfg 1), else the
// generic one (cfg 0).
bool plan_qdw(Desc& d) {
    if (plan_qdw3(d)) {
        d.cfg = 1;
        return true;
    }
    d.cfg = 0;
    return plan_dw_t<int8_t>(d);
}

hipError_t launch_dw(const Desc& d, ConvArgs a, hipStream_t s) {
    if (d.p.dtype == CONV_DTYPE_F32 && d.cfg == 1 && ((uintptr_t)a.xptr % 16) == 0 && ((uintptr_t)a.yptr % 16) == 0)
        return launch_dw_planes(d, a, s);
    return d.p.dtype == CONV_DTYPE_BF16 ? launch_t<__hip_bfloat16>(d, a, s) : launch_t<float>(d, a, s);
}

hipError_t launch_qdw(const Desc& d, ConvArgs a, hipStream_t s) {
    return d.cfg == 1 ? launch_qdw3(d, a, s) : launch_t<int8_t>(d, a, s);
}

}  // namespace conv2d
