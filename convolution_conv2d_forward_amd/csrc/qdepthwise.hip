// int8 depthwise 3x3 (stride 1 or 2, dilation 1): the yscv int8 depthwise
// QLinearConv (int32 accumulation, + int32 bias, requant) on the VALU
// dot-product unit.
//
//   * A workgroup owns P whole (n, c) planes, P sized for three workgroups
//     per compute unit.  They are staged in LDS one at a time as int8 (not
//     widened), one 16-byte chunk per global load (8-byte chunks for widths
//     that are multiples of 8 but not of 16), through two buffers so that
//     plane p+1's copy runs under plane p's outputs:
//     chunks inside the image are copied, the margins and the rows outside it
//     are the zero point (0), so no tap needs a bounds check.
//   * A thread computes 4 consecutive outputs of one row (one 32-bit store of
//     4 requantized bytes).  For each filter row it reads the covering LDS
//     dwords once; the 3 input bytes under output j are cut out with
//     v_alignbyte and multiplied by the packed (w0, w1, w2, 0) with one
//     v_dot4_i32_i8, exact in int32 like the oracle's sum.
//   * The byte offset of the first tap inside its dword depends only on
//     pad_left, so it is a template parameter and every byte select is a
//     fixed instruction.
#include "device_common.h"

namespace conv2d {

namespace {

constexpr int kQT = 256;
constexpr int kMarg = 16;    // zero bytes left of input column 0 in every LDS row
constexpr int kNQ = 16;      // max 16-byte chunks per thread and plane (bound checked when planning)

// LDS geometry of a plane for stride ss, pad_left pl, input width w, output width wo.
struct QGeom {
    int rows, row_bytes, plane_bytes, planes;
};

__host__ __device__ inline int qdw_q0(int k, int ss, int pl) { return ss * k + ((kMarg - pl) >> 2); }

// Requant with the rounding mode fixed at compile time (same arithmetic as
// the shared requant(): f32 product, then ties-to-even or ties-away).
template <int RND>
__device__ __forceinline__ uint32_t rq(int32_t acc, float comp, int y_zp, bool relu) {
    float yf = __fmul_rn((float)acc, comp);
    // Materialise the rounded f32 product: under -ffp-contract=fast the
    // compiler would otherwise fuse it into roundf's own subtraction of the
    // truncated value (one fma, no intermediate rounding), and a product
    // that rounds to an exact tie (25.4999994 -> 25.5) would then round
    // toward zero.
    asm volatile("" : "+v"(yf));
    const float r = RND == CONV_ROUND_HALF_AWAY ? roundf(yf) : rintf(yf);
    // Saturation (and ReLU) on the rounded float, as in requant(): the
    // conversion then sees at most 255 in magnitude.
    const float lo = relu ? 0.0f : (float)(-128 - y_zp), hi = (float)(127 - y_zp);
    return (uint32_t)(uint8_t)(int8_t)((int)__builtin_amdgcn_fmed3f(r, lo, hi) + y_zp);
}

// The same requant with the saturation (and ReLU) done on the f32 product:
// lo = max(-128, relu ? y_zp : -128) - y_zp and hi = 127 - y_zp are integers,
// and rounding is monotone with integers as fixed points, so clamping before
// rounding gives the same byte as clamping the rounded value (ReLU after the
// clamp is the raised lower bound, y_zp <= 127).  One v_med3_f32 replaces the
// integer clamp, the compare and the select.
template <int RND>
__device__ __forceinline__ uint32_t rq_clamped(int32_t acc, float comp, float lo, float hi, int y_zp) {
    float yf = __fmul_rn((float)acc, comp);
    asm volatile("" : "+v"(yf));   // as in rq(): no contraction into the rounding
    yf = __builtin_amdgcn_fmed3f(yf, lo, hi);
    const float r = RND == CONV_ROUND_HALF_AWAY ? roundf(yf) : rintf(yf);
    return (uint32_t)(uint8_t)(int8_t)((int)r + y_zp);
}

// NQ: copy chunks per thread and plane (4, 8 or 16; the chunks of the next
// plane stay in registers while the current one is computed).  CB: bytes per
// copy chunk, 16, or 8 for images whose width is a multiple of 8 but not of
// 16 (their rows start 8-byte aligned).
template <int CB>
struct QChunk;
template <>
struct QChunk<16> { using T = uint4; static __device__ T zero() { return make_uint4(0, 0, 0, 0); } };
template <>
struct QChunk<8> { using T = uint2; static __device__ T zero() { return make_uint2(0, 0); } };

template <int SS, int OFF, int RND, int NQ, int CB>
__global__ __launch_bounds__(kQT) void qdw3_kernel(ConvArgs a, int rows, int row_bytes, int P) {
    using CT = typename QChunk<CB>::T;
    extern __shared__ __align__(16) uint8_t lds8[];
    const int plane_bytes = rows * row_bytes;
    int32_t* wpk = (int32_t*)(lds8 + 2 * plane_bytes);     // [P][3] packed filter rows
    int32_t* bsh = wpk + 3 * P;                             // [P] bias

    const int cblocks = (a.c_out + P - 1) / P;
    const int n = blockIdx.x / cblocks;
    const int c0 = (blockIdx.x - n * cblocks) * P;
    const int np = min(P, a.c_out - c0);
    const int64_t HW = (int64_t)a.h * a.w;
    const int8_t* __restrict__ xp = (const int8_t*)a.xptr + ((int64_t)n * a.in_total + a.in_off + c0) * HW;

    // One plane at a time through two LDS buffers: the 16-byte chunks of
    // plane p+1 are requested before plane p's outputs are computed and are
    // written to the other buffer after them, so their latency runs under
    // the arithmetic.  Chunks inside the image are copied; the margins and
    // the rows outside it are the zero point (0), so no tap needs a bounds check.
    const int cpr = row_bytes / CB;                        // chunks per LDS row
    const int nchunks = rows * cpr;                        // chunks per plane (<= NQ * kQT)
    CT buf[NQ];
    auto load_plane = [&](int p) __attribute__((always_inline)) {
        const int8_t* __restrict__ xq = xp + p * HW;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int e = threadIdx.x + i * kQT;
            buf[i] = QChunk<CB>::zero();
            if (e < nchunks) {
                const int r = e / cpr, j = e - r * cpr;
                const int ih = r - a.pad_top, iw = CB * j - kMarg;
                if ((unsigned)ih < (unsigned)a.h && iw >= 0 && iw < a.w)
                    buf[i] = *(const CT*)(xq + (int64_t)ih * a.w + iw);
            }
        }
    };
    auto store_plane = [&](uint8_t* dst) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int e = threadIdx.x + i * kQT;
            if (e < nchunks) *(CT*)(dst + e * CB) = buf[i];
        }
    };
    load_plane(0);
    if (threadIdx.x < np * 3) {
        const int p = threadIdx.x / 3, r = threadIdx.x - p * 3;
        const int8_t* w = (const int8_t*)a.wptr + (int64_t)(c0 + p) * 9 + 3 * r;
        wpk[threadIdx.x] = (int32_t)((uint32_t)(uint8_t)w[0] | ((uint32_t)(uint8_t)w[1] << 8) |
                                     ((uint32_t)(uint8_t)w[2] << 16));
    }
    if (threadIdx.x < np) bsh[threadIdx.x] = a.qbias ? a.qbias[c0 + threadIdx.x] : 0;
    store_plane(lds8);
    __syncthreads();

    // ---- outputs: 4 consecutive columns of one row per unit ----
    // A thread keeps one column group k and walks down rows t0, t0 + rpi, ...
    // of each plane, its LDS and output pointers stepping by constants.
    constexpr int ND = SS == 1 ? 3 : 4;                    // dwords covering the taps of 4 outputs
    const int wq = a.wo / 4;
    const int rpi = kQT / wq;                              // rows covered by one pass of the workgroup
    const int t0 = divu((uint32_t)threadIdx.x, a.dv_tiles_w);
    const bool active = t0 < rpi;
    const int k = threadIdx.x - t0 * wq;
    const int64_t oplane = (int64_t)a.ho * a.wo;
    const int q0 = qdw_q0(k, SS, a.pad_left);
    const bool relu = a.act == CONV_ACT_RELU;
    const float qlo = (float)((relu ? max(-128, a.y_zp) : -128) - a.y_zp), qhi = (float)(127 - a.y_zp);
    const int lstep = rpi * SS * row_bytes;               // LDS bytes per pass down a plane
    const int64_t ystep = (int64_t)rpi * a.wo;            // output bytes per pass
    int8_t* const ybase = (int8_t*)a.yptr + ((int64_t)n * a.out_total + a.out_off + c0) * oplane + 4 * k;
    for (int p = 0; p < np; ++p) {
        const bool more = p + 1 < np;
        if (more) load_plane(p + 1);
        if (active) {
            const int32_t b = bsh[p];
            const int32_t wrow[3] = {wpk[3 * p], wpk[3 * p + 1], wpk[3 * p + 2]};
            const uint8_t* prow = lds8 + (p & 1) * plane_bytes + t0 * SS * row_bytes + 4 * q0;
            int8_t* yrow = ybase + (int64_t)p * oplane + (int64_t)t0 * a.wo;
            for (int ho = t0; ho < a.ho; ho += rpi, prow += lstep, yrow += ystep) {
                int32_t acc[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] = b;
#pragma unroll
                for (int r = 0; r < 3; ++r) {
                    const uint32_t* src = (const uint32_t*)(prow + r * row_bytes);
                    uint32_t d[ND];
#pragma unroll
                    for (int t = 0; t < ND; ++t) d[t] = src[t];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int idx = OFF + SS * j;      // byte of the first tap, from dword q0
                        const uint32_t lo = d[idx >> 2], hi = d[(idx >> 2) + 1 < ND ? (idx >> 2) + 1 : ND - 1];
                        const uint32_t win = (idx & 3) ? __builtin_amdgcn_alignbyte(hi, lo, idx & 3) : lo;
                        acc[j] = __builtin_amdgcn_sdot4((int)win, wrow[r], acc[j], false);
                    }
                }
                uint32_t packed = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    packed |= rq_clamped<RND>(acc[j], a.composite, qlo, qhi, a.y_zp) << (8 * j);
                *(uint32_t*)yrow = packed;
            }
        }
        if (more) {
            // Buffer (p+1)&1 was last read by plane p-1's outputs, which every
            // thread finished before the previous barrier.
            store_plane(lds8 + ((p + 1) & 1) * plane_bytes);
            __syncthreads();
        }
    }
}

// Byte offset of output 0's first tap inside dword q0: (kMarg - pad_left) & 3.
template <int SS, int RND, int NQ, int CB>
const void* pick_off(int off) {
    switch (off) {
    case 0: return (const void*)qdw3_kernel<SS, 0, RND, NQ, CB>;
    case 1: return (const void*)qdw3_kernel<SS, 1, RND, NQ, CB>;
    case 2: return (const void*)qdw3_kernel<SS, 2, RND, NQ, CB>;
    default: return (const void*)qdw3_kernel<SS, 3, RND, NQ, CB>;
    }
}

template <int SS, int NQ, int CB>
const void* pick_rnd(int off, int rounding) {
    return rounding == CONV_ROUND_HALF_AWAY ? pick_off<SS, CONV_ROUND_HALF_AWAY, NQ, CB>(off)
                                            : pick_off<SS, CONV_ROUND_HALF_EVEN, NQ, CB>(off);
}

// 16-byte chunks: up to 16 per thread; 8-byte chunks (planned only for
// planes of at most 8 * kQT of them): 4 or 8.
template <int SS>
const void* pick_nq(int nchunks, int off, int rounding, int cb) {
    if (cb == 8) return nchunks <= 4 * kQT ? pick_rnd<SS, 4, 8>(off, rounding) : pick_rnd<SS, 8, 8>(off, rounding);
    if (nchunks <= 4 * kQT) return pick_rnd<SS, 4, 16>(off, rounding);
    if (nchunks <= 8 * kQT) return pick_rnd<SS, 8, 16>(off, rounding);
    return pick_rnd<SS, 16, 16>(off, rounding);
}

// Copy chunk bytes for an image width: 16 where rows are 16-byte multiples.
int qdw_cb(int w) { return w % 16 == 0 ? 16 : 8; }

bool qgeom(const Desc& d, QGeom& G) {
    const conv2d_params_t& p = d.p;
    const int ss = p.stride_h;
    const int pl = p.pad_left;
    const int wq = d.wo / 4;
    // Last byte a unit reads in a row: dwords q0 .. q0 + ND - 1 of the last column group.
    const int nd = ss == 1 ? 3 : 4;
    const int last = 4 * (qdw_q0(wq - 1, ss, pl) + nd) - 1;
    int rb = kMarg + p.w + 16;
    if (last + 1 > rb) rb = last + 1;
    G.row_bytes = (rb + 15) / 16 * 16;
    G.rows = (d.ho - 1) * ss + 3;
    G.plane_bytes = G.rows * G.row_bytes;
    // Planes per workgroup: enough for three workgroups per compute unit
    // (at most 8).  Each streams its planes through two buffers, so fewer,
    // longer workgroups hide the latency of each plane's copy behind the
    // previous plane's outputs, while three per CU keep every CU busy with
    // independent copies; measured on 56x56 and 80x80 planes (s1 and s2),
    // three per CU beat one, two, or five to eight planes per workgroup.
    const int64_t planes = (int64_t)p.n * p.c_out;
    const int64_t slots = 3 * (int64_t)device_cu_count();
    int64_t P = (planes + slots - 1) / slots;
    if (P > 8) P = 8;
    if (P < 1) P = 1;
    G.planes = (int)P;
    const int cb = qdw_cb(p.w);
    return G.rows * (G.row_bytes / cb) <= (cb == 16 ? kNQ : 8) * kQT && 2 * G.plane_bytes + 16 * P <= 160 * 1024;
}

}  // namespace

bool plan_qdw3(const Desc& d) {
    const conv2d_params_t& p = d.p;
    if (p.k_h != 3 || p.k_w != 3 || p.dilation_h != 1 || p.dilation_w != 1) return false;
    if (p.stride_h != p.stride_w || (p.stride_h != 1 && p.stride_h != 2)) return false;
    if (p.w % 8 != 0 || d.wo % 4 != 0 || p.pad_left > kMarg) return false;
    if (d.wo / 4 > kQT) return false;   // a row's column groups must fit one workgroup pass
    if ((int64_t)p.h * p.w >= INT32_MAX / 16) return false;
    QGeom G;
    return qgeom(d, G);
}

hipError_t launch_qdw3(const Desc& d, ConvArgs a, hipStream_t s) {
    const int cb = qdw_cb(d.p.w);
    if ((uintptr_t)a.xptr % cb != 0 || (uintptr_t)a.yptr % 4 != 0) return launch_direct(d, a, s);
    QGeom G;
    if (!qgeom(d, G)) return hipErrorInvalidConfiguration;
    const int64_t blocks = (int64_t)a.n * ((a.c_out + G.planes - 1) / G.planes);
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const int off = (kMarg - d.p.pad_left) & 3;
    a.dv_tiles_h = make_divu32((uint32_t)(a.ho * (a.wo / 4)));
    a.dv_tiles_w = make_divu32((uint32_t)(a.wo / 4));
    const int nchunks = G.rows * (G.row_bytes / cb);
    const void* fn = d.p.stride_h == 1 ? pick_nq<1>(nchunks, off, a.rounding, cb)
                                       : pick_nq<2>(nchunks, off, a.rounding, cb);
    int rows = G.rows, rb = G.row_bytes, P = G.planes;
    void* args[] = {&a, &rows, &rb, &P};
    const size_t lds = 2 * (size_t)G.plane_bytes + 16 * P;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    return hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(kQT), args, lds, s);
}

}  // namespace conv2d
