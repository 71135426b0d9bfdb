// Implicit-GEMM convolution with bfloat16 operands on the gfx950 matrix
// cores (v_mfma_f32_16x16x32_bf16), fp32 accumulation, fp32 bias and
// activation, bf16 output rounded to nearest even.
//
// Same GEMM view as the fp32 kernel (M = output channels, N = output pixels,
// K = input channels x taps), but one MFMA step consumes 32 K values and each
// lane supplies 8 consecutive ones, so the LDS tiles are laid out with K
// innermost:
//   input patch   [patch position][channel]    (CKP bf16 per position)
//   weights       [output channel][tap*CK + channel]
// and a fragment is a single 16-byte LDS read.  Inside a channel chunk of CK
// channels the K order is tap-major, channel-minor (k = rs*CK + ci); a step
// of 32 K values covers 32/CK taps when CK < 32, and K is zero-padded to a
// multiple of 32 (zero weights).  Which lane slot carries which K value only
// has to agree between A and B; both use k = 8*(lane/16) + element.
#include "device_common.h"

namespace conv2d {

namespace {

constexpr int kThreads = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int CK_, int KH_, int KW_, int XU_, int WU_>
struct Bf16Cfg {
    static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int CK = CK_, KH = KH_, KW = KW_, KHW = KH_ * KW_;
    static constexpr int XU = XU_;   // input units (8 channels x 1 position) per thread, max
    static constexpr int WU = WU_;   // weight units (1 output channel x 8 channels) per thread, max
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int MI = WM / 16, NI = WN / 16;
    static constexpr int KREAL = KHW * CK;
    static constexpr int KP = (KREAL + 31) / 32 * 32;
    static constexpr int KSTEPS = KP / 32;
    static constexpr int CKP = CK + 8;        // bf16 per patch position (16-byte aligned rows)
    static constexpr int WROW = KP + 8;       // bf16 per weight row
    static_assert(WAVES_M * WAVES_N == 4, "4 waves");
    static_assert(CK % 8 == 0 && (CK >= 32 ? CK % 32 == 0 : 32 % CK == 0), "CK must tile 32-wide K steps");
    static_assert(WM % 16 == 0 && WN % 16 == 0, "whole fragments");
};

__device__ __forceinline__ uint16_t bf_bits(const __hip_bfloat16* p, int64_t i) {
    return ((const uint16_t*)p)[i];
}

template <class C>
__global__ __launch_bounds__(kThreads) void igemm_bf16_kernel(ConvArgs a) {
    extern __shared__ __align__(16) uint16_t lds16[];
    constexpr int BM = C::BM, CK = C::CK, CKP = C::CKP, WROW = C::WROW, MI = C::MI, NI = C::NI;
    constexpr int KHW = C::KHW, KW = C::KW;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % C::WAVES_M, wn = wave / C::WAVES_M;

    uint32_t L = xcd_remap(blockIdx.x, a.num_blocks);
    const int cot = L % a.co_tiles;  L /= a.co_tiles;
    const int g = L % a.groups;      L /= a.groups;
    const int twi = L % a.tiles_w;   L /= a.tiles_w;
    const int thi = L % a.tiles_h;   L /= a.tiles_h;
    const int n = L;

    const int co0 = cot * BM;
    const int ho0 = thi * a.tile_h, wo0 = twi * a.tile_w;
    const int ih0 = ho0 * a.stride_h - a.pad_top;
    const int iw0 = wo0 * a.stride_w - a.pad_left;
    const int PW = a.patch_w;
    const int PHW = a.patch_h * PW;
    const int64_t HW = (int64_t)a.h * a.w;
    const int xs_elems = PHW * CKP;
    const int stage = xs_elems + BM * WROW;      // uint16 per stage

    const __hip_bfloat16* __restrict__ xg =
        (const __hip_bfloat16*)a.xptr + ((int64_t)n * a.in_total + a.in_off + (int64_t)g * a.cin_g) * HW;
    const __hip_bfloat16* __restrict__ wg =
        (const __hip_bfloat16*)a.wptr + ((int64_t)g * a.cout_g + co0) * a.cin_g * KHW;
    const int co_valid = min(BM, a.cout_g - co0);
    // pad_value in the input's storage type
    const uint16_t padb = __bfloat16_as_ushort(f32_to_bf16(a.pad_value));
    const bool w_vec = (a.cin_g % 8) == 0 && (((uintptr_t)a.wptr) % 16) == 0;

    const int x_units = PHW * (CK / 8);          // (position, 8-channel group)
    const int w_units = BM * (CK / 8);           // (output channel, 8-channel group)

    uint4 xr[C::XU];
    uint4 wr[C::WU][KHW];

    auto load_chunk = [&](int c0) {
#pragma unroll
        for (int i = 0; i < C::XU; ++i) {
            const int u = tid + i * kThreads;
            uint32_t v[4] = {0, 0, 0, 0};
            if (u < x_units) {
                const int grp = (int)fdiv(u, a.div_patch_hw);  // channel group (slowest: coalesced positions)
                const int pos = u - grp * PHW;
                const int pr = (int)fdiv(pos, a.div_patch_w);
                const int pc = pos - pr * PW;
                const int ih = ih0 + pr, iw = iw0 + pc;
                const bool inside = (unsigned)ih < (unsigned)a.h && (unsigned)iw < (unsigned)a.w;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int ch = c0 + grp * 8 + e;
                    uint32_t b = 0;
                    if (ch < a.cin_g) b = inside ? bf_bits(xg, (int64_t)ch * HW + (int64_t)ih * a.w + iw) : padb;
                    v[e >> 1] |= b << (16 * (e & 1));
                }
            }
            xr[i] = make_uint4(v[0], v[1], v[2], v[3]);
        }
#pragma unroll
        for (int i = 0; i < C::WU; ++i) {
            const int u = tid + i * kThreads;
            const int co = u % BM;
            const int grp = u / BM;
            const int ch0 = c0 + grp * 8;
            const bool ok = u < w_units && co < co_valid;
            const __hip_bfloat16* src = wg + (int64_t)co * a.cin_g * KHW + (int64_t)ch0 * KHW;
            if (ok && w_vec && ch0 + 8 <= a.cin_g) {
                // 8 channels x KHW taps are contiguous in OIHW: KHW 16-byte loads.
#pragma unroll
                for (int t = 0; t < KHW; ++t) wr[i][t] = ((const uint4*)src)[t];
            } else {
                uint32_t tmp[KHW * 4];
#pragma unroll
                for (int t = 0; t < KHW * 4; ++t) tmp[t] = 0;
                if (ok) {
#pragma unroll
                    for (int e = 0; e < 8 * KHW; ++e)
                        if (ch0 + e / KHW < a.cin_g) tmp[e >> 1] |= (uint32_t)bf_bits(src, e) << (16 * (e & 1));
                }
#pragma unroll
                for (int t = 0; t < KHW; ++t)
                    wr[i][t] = make_uint4(tmp[4 * t], tmp[4 * t + 1], tmp[4 * t + 2], tmp[4 * t + 3]);
            }
        }
    };

    auto store_chunk = [&](int s) {
        uint16_t* xs = lds16 + s * stage;
        uint16_t* ws = xs + xs_elems;
#pragma unroll
        for (int i = 0; i < C::XU; ++i) {
            const int u = tid + i * kThreads;
            if (u < x_units) {
                const int grp = (int)fdiv(u, a.div_patch_hw);
                const int pos = u - grp * PHW;
                *(uint4*)&xs[pos * CKP + grp * 8] = xr[i];
            }
        }
#pragma unroll
        for (int i = 0; i < C::WU; ++i) {
            const int u = tid + i * kThreads;
            if (u < w_units) {
                const int co = u % BM;
                const int grp = u / BM;
                // wr holds element (c, t) of the 8 channels at flat c*KHW + t; write
                // tap t's 8 channels to [co][t*CK + grp*8].
                const uint32_t* src = (const uint32_t*)wr[i];
#pragma unroll
                for (int t = 0; t < KHW; ++t) {
                    uint32_t o[4];
#pragma unroll
                    for (int c2 = 0; c2 < 4; ++c2) {
                        const int e0 = (2 * c2) * KHW + t, e1 = (2 * c2 + 1) * KHW + t;
                        const uint32_t lo = (src[e0 >> 1] >> (16 * (e0 & 1))) & 0xFFFFu;
                        const uint32_t hi = (src[e1 >> 1] >> (16 * (e1 & 1))) & 0xFFFFu;
                        o[c2] = lo | (hi << 16);
                    }
                    *(uint4*)&ws[co * WROW + t * CK + grp * 8] = make_uint4(o[0], o[1], o[2], o[3]);
                }
            }
        }
        // Zero the K padding columns (tap-major K beyond KHW*CK) once per stage.
        if constexpr (C::KP > C::KREAL) {
            for (int e = tid; e < BM * (C::KP - C::KREAL); e += kThreads) {
                const int co = e / (C::KP - C::KREAL);
                const int k = C::KREAL + e % (C::KP - C::KREAL);
                ws[co * WROW + k] = 0;
            }
        }
    };

    // Per-lane fragment bases.
    int b_pos[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
        const int j = wn * C::WN + ni * 16 + (lane & 15);
        const int th = (int)fdiv(j, a.div_tile_w);
        const int tw = j - th * a.tile_w;
        b_pos[ni] = th * a.stride_h * PW + tw * a.stride_w;
    }
    const int q = lane >> 4;

    f32x4 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](int s) {
        const uint16_t* xs = lds16 + s * stage;
        const uint16_t* ws = xs + xs_elems;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
            const int k0 = ks * 32 + 8 * q;           // this lane's first K of the step
            int rs = k0 / CK;
            const int ci = k0 - rs * CK;
            if (rs >= KHW) rs = 0;                    // K padding: zero weights, any finite input
            const int r = rs / KW, sc = rs - (rs / KW) * KW;
            const int tap = r * a.dilation_h * PW + sc * a.dilation_w;
            bf16x8 av[MI], bv[NI];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                av[mi] = *(const bf16x8*)&ws[(wm * C::WM + mi * 16 + (lane & 15)) * WROW + k0];
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) bv[ni] = *(const bf16x8*)&xs[(b_pos[ni] + tap) * CKP + ci];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mi], bv[ni], acc[mi][ni], 0, 0, 0);
        }
    };

    // Two LDS stages when they fit (one barrier per chunk), else one stage
    // with the next chunk still prefetched into registers.
    load_chunk(0);
    store_chunk(0);
    __syncthreads();
    for (int kc = 0; kc < a.chunks; ++kc) {
        const bool more = kc + 1 < a.chunks;
        if (more) load_chunk((kc + 1) * CK);
        if (a.stages == 2) {
            const int s = kc & 1;
            compute(s);
            if (more) store_chunk(s ^ 1);
            __syncthreads();
        } else {
            compute(0);
            __syncthreads();
            if (more) {
                store_chunk(0);
                __syncthreads();
            }
        }
    }

    __hip_bfloat16* __restrict__ yg = (__hip_bfloat16*)a.yptr;
    const int64_t out_plane = (int64_t)a.ho * a.wo;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            const int j = wn * C::WN + ni * 16 + (lane & 15);
            const int th = (int)fdiv(j, a.div_tile_w);
            const int tw = j - th * a.tile_w;
            const int ho = ho0 + th, wo = wo0 + tw;
            if (ho >= a.ho || wo >= a.wo) continue;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int co = co0 + wm * C::WM + mi * 16 + q * 4 + v;
                if (co < a.cout_g) {
                    const int cg = g * a.cout_g + co;
                    yg[((int64_t)n * a.out_total + a.out_off + cg) * out_plane + (int64_t)ho * a.wo + wo] =
                        f32_to_bf16(bias_act(a, acc[mi][ni][v], cg));
                }
            }
        }
}

struct CfgInfo {
    int bm, bn, ck, kh, kw, xu, wu, kp;
    const void* fn;
    int stage_u16(int phw) const { return phw * (ck + 8) + bm * (kp + 8); }
};

template <class C>
CfgInfo info() {
    return CfgInfo{C::BM, C::BN, C::CK, C::KH, C::KW, C::XU, C::WU, C::KP, (const void*)igemm_bf16_kernel<C>};
}

//                      BM  BN  WM WN CK KH KW XU WU
using B3_M64  = Bf16Cfg<64, 64, 2, 2, 16, 3, 3, 3, 1>;
using B3_M128 = Bf16Cfg<128, 64, 2, 2, 16, 3, 3, 3, 1>;
using B3_M16  = Bf16Cfg<16, 128, 1, 4, 8, 3, 3, 3, 1>;
using B1_M64  = Bf16Cfg<64, 128, 1, 4, 32, 1, 1, 2, 1>;
using B1_M128 = Bf16Cfg<128, 128, 2, 2, 32, 1, 1, 2, 2>;

const CfgInfo& cfg(int i) {
    static const CfgInfo t[] = {info<B3_M64>(), info<B3_M128>(), info<B3_M16>(), info<B1_M64>(), info<B1_M128>()};
    return t[i];
}


int patch_stride_for(int phw) {
    // Smallest stride >= phw with stride % 64 == 16: the four channel planes
    // read by one MFMA operand fetch then start 16 banks apart.
    int s = ((phw + 63 - 16) / 64) * 64 + 16;
    if (s < phw) s += 64;
    return s;
}

}  // namespace

void fill_tiling(const Desc& d, ConvArgs& a) {
    // Per-tile geometry of the bf16 implicit GEMM.
    const conv2d_params_t& p = d.p;
    if (d.flatten_1x1) {
        a.h = 1; a.w = p.h * p.w; a.ho = 1; a.wo = d.ho * d.wo;
    }
    a.tile_h = d.tile_h;
    a.tile_w = d.tile_w;
    a.tiles_h = (a.ho + d.tile_h - 1) / d.tile_h;
    a.tiles_w = (a.wo + d.tile_w - 1) / d.tile_w;
    a.patch_h = (d.tile_h - 1) * p.stride_h + (p.k_h - 1) * p.dilation_h + 1;
    a.patch_w = (d.tile_w - 1) * p.stride_w + (p.k_w - 1) * p.dilation_w + 1;
    a.patch_stride = patch_stride_for(a.patch_h * a.patch_w);
    a.div_patch_hw = make_fastdiv((uint32_t)(a.patch_h * a.patch_w));
    a.div_patch_w = make_fastdiv((uint32_t)a.patch_w);
    a.div_tile_w = make_fastdiv((uint32_t)d.tile_w);
}

bool plan_igemm_bf16(Desc& d) {
    const conv2d_params_t& p = d.p;
    const bool is3 = p.k_h == 3 && p.k_w == 3;
    const bool is1 = p.k_h == 1 && p.k_w == 1;
    d.flatten_1x1 = is1 && p.stride_h == 1 && p.stride_w == 1 && p.pad_top == 0 && p.pad_left == 0 &&
                    p.pad_bottom == 0 && p.pad_right == 0;
    if (d.flatten_1x1 && (int64_t)p.h * p.w > INT32_MAX / 2) return false;
    const int m = d.cout_g;
    int ci;
    if (is3) ci = m <= 16 ? 2 : (m % 128 == 0 ? 1 : 0);
    else if (d.flatten_1x1) ci = (m % 128 == 0) ? 4 : 3;
    else return false;
    const CfgInfo& c = cfg(ci);
    int best_tw = 0, best_th = 0;
    long best_waste = -1;
    const int ho_eff = d.flatten_1x1 ? 1 : d.ho;
    const int wo_eff = d.flatten_1x1 ? d.ho * d.wo : d.wo;
    for (int tw = 8; tw <= c.bn; tw *= 2) {
        if (d.flatten_1x1 && tw != c.bn) continue;
        const int th = c.bn / tw;
        const int ph = d.flatten_1x1 ? 1 : (th - 1) * p.stride_h + (p.k_h - 1) * p.dilation_h + 1;
        const int pw = d.flatten_1x1 ? tw : (tw - 1) * p.stride_w + (p.k_w - 1) * p.dilation_w + 1;
        if (ph * pw >= 65536) continue;
        if (ph * pw * (c.ck / 8) > kThreads * c.xu) continue;
        if (c.bm * (c.ck / 8) > kThreads * c.wu) continue;
        if (c.stage_u16(ph * pw) * 2 > 64 * 1024) continue;
        const long tiles = (long)((ho_eff + th - 1) / th) * ((wo_eff + tw - 1) / tw);
        const long waste = tiles * c.bn - (long)ho_eff * wo_eff;
        if (best_waste < 0 || waste < best_waste || (waste == best_waste && tw > best_tw)) {
            best_waste = waste; best_tw = tw; best_th = th;
        }
    }
    if (best_waste < 0) return false;
    d.cfg = ci;
    d.tile_h = best_th;
    d.tile_w = best_tw;
    const int ph = d.flatten_1x1 ? 1 : (best_th - 1) * p.stride_h + (p.k_h - 1) * p.dilation_h + 1;
    const int pw = d.flatten_1x1 ? best_tw : (best_tw - 1) * p.stride_w + (p.k_w - 1) * p.dilation_w + 1;
    const int one = c.stage_u16(ph * pw) * 2;
    d.stages = 2 * one <= 64 * 1024 ? 2 : 1;
    d.lds_bytes = d.stages * one;
    return true;
}

hipError_t launch_igemm_bf16(const Desc& d, ConvArgs a, hipStream_t s) {
    const CfgInfo& c = cfg(d.cfg);
    fill_tiling(d, a);
    a.co_tiles = (d.cout_g + c.bm - 1) / c.bm;
    a.chunks = (d.cin_g + c.ck - 1) / c.ck;
    const uint64_t blocks = (uint64_t)a.co_tiles * a.groups * a.tiles_h * a.tiles_w * a.n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0xFFFFFFFFull) return hipErrorInvalidConfiguration;
    a.num_blocks = (uint32_t)blocks;
    a.stages = d.stages;
    void* args[] = {&a};
    return hipLaunchKernel(c.fn, dim3((uint32_t)blocks), dim3(kThreads), args, d.lds_bytes, s);
}

}  // namespace conv2d
