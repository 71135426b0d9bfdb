// Implicit-GEMM convolution with bfloat16 operands on the gfx950 matrix
// cores (v_mfma_f32_16x16x32_bf16), fp32 accumulation, fp32 bias and
// activation, bf16 output rounded to nearest even.
//
// The GEMM view is the one of the fp32 kernel (M = output channels, N =
// output pixels, K = input channels x taps; ncnn "convolution": pad with
// pad_value, correlate, + bias, activation), but a bf16 MFMA step takes 32
// K values and each lane supplies 8 consecutive ones, and at bf16 rates the
// LDS bandwidth is the first limit.  So:
//   * the tiles are shared by the whole workgroup and every wave owns a
//     WR x 64 output tile (WR/16 x 4 MFMA fragments; WR = 64 in the wide
//     configurations), which keeps LDS reads at one 16-byte read per two
//     MFMAs;
//   * inside a chunk of CC input channels, K runs tap-major and channel-minor,
//     and both LDS tiles keep the channels innermost:
//       weights  [tap][output channel][CC + 8]
//       patch    [patch position][CC + 8]
//     so an MFMA operand is one 16-byte LDS read, and the row strides (80 or
//     144 bytes) put 16 consecutive rows on 16 distinct 16-byte bank groups;
//   * the copy from global memory (16-byte loads of OIHW weights and of NCHW
//     rows) transposes into that layout with 2-byte LDS writes, the lanes of
//     a write walking along output channels (weights) or input channels
//     (patch) so that the writes spread over the banks.  The next chunk's
//     loads are in flight while the current one is multiplied out.
// The epilogue adds the bias, applies the activation, rounds to bf16 and
// writes channel out_off + g*cout_g + co of a buffer with out_total channels
// (ConcatFusedTail).
#include "device_common.h"

namespace conv2d {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int BM_, int WM_, int WN_, int NI_, int TW_, int CC_, int KH_, int KW_, int XS_>
struct BCfg {
    static constexpr int BM = BM_, WM = WM_, WN = WN_, TW = TW_, CC = CC_, KH = KH_, KW = KW_;
    static constexpr int KHW = KH_ * KW_;
    static constexpr int NW = WM * WN, NT = 64 * NW;   // waves, threads
    static constexpr int WR = BM / WM;                 // rows of a wave tile
    static constexpr int MI = WR / 16, NI = NI_;       // MFMA fragments of a wave tile
    static constexpr int WC = 16 * NI;                 // pixels of a wave tile
    static constexpr int BN = WC * WN;                 // pixels of the workgroup tile
    static constexpr int TH = BN / TW;
    static constexpr int CCP = CC + 8;                 // bf16 per LDS row
    static constexpr int STEPS = (KHW * CC + 31) / 32; // K steps of 32 per chunk
    static constexpr int KHWP = STEPS * 32 / CC;       // taps incl. the zero padding of the last step
    static constexpr int RV = CC * KHW / 8;            // 16-byte vectors per weight row and chunk
    static constexpr int AV = BM * RV;                 // 16-byte weight vectors per chunk
    static constexpr int AS = (AV + NT - 1) / NT;      // per thread
    static constexpr int XS = XS_;                     // 16-byte input vectors per thread (upper bound)
    static constexpr int ALDS = KHWP * BM * CCP;       // bf16 of the weight tile
    static_assert(CC % 16 == 0 && (CC >= 32 ? CC % 32 == 0 : 32 % CC == 0), "K steps of 32 tile the chunk");
    static_assert((CC * KHW) % 8 == 0, "whole 16-byte weight vectors");
    static_assert(WR % 16 == 0 && BN % TW == 0 && TW % 16 == 0, "whole fragments");
};

template <class C>
__global__ __launch_bounds__(C::NT) void igemm_bf16_kernel(ConvArgs a) {
    extern __shared__ __align__(16) uint16_t lds16[];
    constexpr int BM = C::BM, TW = C::TW, TH = C::TH, CC = C::CC, CCP = C::CCP;
    constexpr int KHW = C::KHW, KW = C::KW, MI = C::MI, NI = C::NI, RV = C::RV;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % C::WM, wn = wave / C::WM;

    uint32_t L = xcd_remap(blockIdx.x, a.num_blocks);
    uint32_t Q = divu(L, a.dv_co_tiles);
    const int cot = L - Q * a.co_tiles;
    L = Q; Q = divu(L, a.dv_groups);
    const int g = L - Q * a.groups;
    L = Q; Q = divu(L, a.dv_tiles_w);
    const int twi = L - Q * a.tiles_w;
    L = Q; Q = divu(L, a.dv_tiles_h);
    const int thi = L - Q * a.tiles_h;
    const int n = Q;

    const int co0 = cot * BM;
    const int ho0 = thi * TH, wo0 = twi * TW;
    const int ih0 = ho0 * a.stride_h - a.pad_top;
    const int iw_lo = wo0 * a.stride_w - a.pad_left;      // input column of patch column 0
    const int span = a.patch_w;                           // patch columns kept in LDS
    const int PH = a.patch_h;
    const int shift = a.patch_shift;                      // iw_lo minus its 8-aligned floor
    const int nvr = a.patch_stride;                       // 8-pixel vectors per patch row
    const int xv = CC * PH * nvr;                         // input vectors per chunk
    const int HW = a.h * a.w;

    const uint16_t* __restrict__ xg = (const uint16_t*)a.xptr +
                                      ((int64_t)n * a.in_total + a.in_off + (int64_t)g * a.cin_g) * HW;
    const uint16_t* __restrict__ wg = (const uint16_t*)a.wptr + ((int64_t)g * a.cout_g + co0) * a.cin_g * KHW;
    const bool vx = a.w % 8 == 0 && ((uintptr_t)a.xptr % 16) == 0;
    const bool vw = (a.cin_g * KHW) % 8 == 0 && ((uintptr_t)a.wptr % 16) == 0;
    const uint32_t padb = __bfloat16_as_ushort(f32_to_bf16(a.pad_value));
    const uint32_t pad2 = padb | (padb << 16);

    uint16_t* As = lds16;                 // [tap][BM][CCP]
    uint16_t* Bs = lds16 + C::ALDS;       // [pos][CCP]

    // ---- per-lane input plan: vector i = 8 pixels of one row of one channel,
    // channels fastest across the lanes ----
    int xgo[C::XS];    // element offset from the chunk's first channel plane, -1 = outside the image
    int xpk[C::XS];    // packed (row << 20) | ((patch column of the first pixel + 8) << 8) | channel; -1 = none
#pragma unroll
    for (int i = 0; i < C::XS; ++i) {
        const int v = tid + C::NT * i;
        xgo[i] = -1; xpk[i] = -1;
        if (v < xv) {
            const int ci = v % CC;
            const int rest = v / CC;
            const int row = rest / nvr;
            const int vc = rest - row * nvr;
            const int ih = ih0 + row, iw = iw_lo - shift + 8 * vc;
            xpk[i] = (row << 20) | ((8 * vc - shift + 8) << 8) | ci;
            if ((unsigned)ih < (unsigned)a.h && iw >= 0 && iw < a.w) xgo[i] = ci * HW + ih * a.w + iw;
        }
    }
    auto pk_ci = [](int pk) { return pk & 255; };
    auto pk_pc = [](int pk) { return ((pk >> 8) & 4095) - 8; };
    auto pk_row = [](int pk) { return pk >> 20; };
    // Zero the padding taps of the weight tile once (K steps past the last tap).
    if constexpr (C::KHWP > KHW) {
        for (int e = tid; e < (C::KHWP - KHW) * BM * CCP; e += C::NT) As[KHW * BM * CCP + e] = 0;
    }

    uint4 ar[C::AS];
    uint4 xr[C::XS];

    // Global -> registers for the channels [c0, c0 + CC) of the group.
    // Weight vector i: output channel v % BM (fastest), 8 elements 8*(v / BM)..
    // of the channel chunk's OIHW row.
    auto load = [&](int c0) __attribute__((always_inline)) {
        const int cl = a.cin_g - c0;
        const uint16_t* __restrict__ wc = wg + (int64_t)c0 * KHW;
#pragma unroll
        for (int i = 0; i < C::AS; ++i) {
            const int v = tid + C::NT * i;
            const int co = v % BM, j = v / BM;
            uint4 r = make_uint4(0, 0, 0, 0);
            if (v < C::AV && co0 + co < a.cout_g) {
                const uint16_t* src = wc + (int64_t)co * a.cin_g * KHW + 8 * j;
                if (vw && cl >= CC) {
                    r = *(const uint4*)src;
                } else {
                    uint32_t e[8];
#pragma unroll
                    for (int t = 0; t < 8; ++t) e[t] = (8 * j + t) / KHW < cl ? src[t] : 0u;
                    r = make_uint4(e[0] | e[1] << 16, e[2] | e[3] << 16, e[4] | e[5] << 16, e[6] | e[7] << 16);
                }
            }
            ar[i] = r;
        }
        const uint16_t* __restrict__ xc = xg + (int64_t)c0 * HW;
#pragma unroll
        for (int i = 0; i < C::XS; ++i) {
            uint4 r = make_uint4(0, 0, 0, 0);
            if (xpk[i] >= 0 && pk_ci(xpk[i]) < cl) {
                if (vx) {
                    r = xgo[i] >= 0 ? *(const uint4*)(xc + xgo[i]) : make_uint4(pad2, pad2, pad2, pad2);
                } else {
                    const int ih = ih0 + pk_row(xpk[i]);
                    const int iw0 = iw_lo + pk_pc(xpk[i]);
                    uint32_t e[8];
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const int iw = iw0 + t;
                        e[t] = ((unsigned)ih < (unsigned)a.h && (unsigned)iw < (unsigned)a.w)
                                   ? (uint32_t)xc[pk_ci(xpk[i]) * HW + ih * a.w + iw]
                                   : padb;
                    }
                    r = make_uint4(e[0] | e[1] << 16, e[2] | e[3] << 16, e[4] | e[5] << 16, e[6] | e[7] << 16);
                }
            }
            xr[i] = r;
        }
    };

    // Registers -> LDS, transposing to channel-innermost rows.
    auto store = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < C::AS; ++i) {
            const int v = tid + C::NT * i;
            if (v < C::AV) {
                const int co = v % BM, j = v / BM;
                if constexpr (KHW == 1) {
                    *(uint4*)(As + co * CCP + 8 * j) = ar[i];
                } else {
                    const uint32_t w4[4] = {ar[i].x, ar[i].y, ar[i].z, ar[i].w};
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const int e = 8 * j + t;          // OIHW order within the row: e = ci*KHW + rs
                        const int ci = e / KHW, rs = e - (e / KHW) * KHW;
                        As[(rs * BM + co) * CCP + ci] = (uint16_t)(w4[t >> 1] >> (16 * (t & 1)));
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < C::XS; ++i) {
            if (xpk[i] >= 0) {
                const uint32_t w4[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
                const int pc0 = pk_pc(xpk[i]);
                uint16_t* dst = Bs + (pk_row(xpk[i]) * span + pc0) * CCP + pk_ci(xpk[i]);
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int pc = pc0 + t;
                    if (pc >= 0 && pc < span) dst[t * CCP] = (uint16_t)(w4[t >> 1] >> (16 * (t & 1)));
                }
            }
        }
    };

    // Operand addresses.  Chunk K index k = tap*CC + channel; step s takes
    // k in [32s, 32s + 32) and lane group q = lane/16 supplies k = 32s + 8q..+7,
    // i.e. tap (32s + 8q) / CC, channels (32s + 8q) % CC.. of that tap.
    // A: row co = wm*WR + mi*16 + lane%16.  B: pixel j = wn*WC + ni*16 + lane%16.
    const int a_lane = (wm * C::WR + (lane & 15)) * CCP;
    int b_lane[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
        const int j = wn * C::WC + ni * 16 + (lane & 15);
        b_lane[ni] = ((j / TW) * a.stride_h * span + (j % TW) * a.stride_w) * CCP;
    }

    f32x4 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    auto fetch = [&](int s, int al, const int (&bl)[NI], bf16x8 (&av)[MI], bf16x8 (&bv)[NI])
                     __attribute__((always_inline)) {
        const int k = 32 * s + 8 * (lane >> 4);
        const int rs = k / CC, kc = k % CC;
        // Padding taps (rs >= KHW) have zero weights; read tap 0's finite inputs.
        const int rv = rs < KHW ? rs : 0;
        const int r = rv / KW, sc = rv % KW;
        const int boff = (r * a.dilation_h * span + sc * a.dilation_w) * CCP + kc;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) av[mi] = *(const bf16x8*)(As + (rs * BM) * CCP + al + mi * 16 * CCP + kc);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) bv[ni] = *(const bf16x8*)(Bs + bl[ni] + boff);
    };
    auto mfmas = [&](const bf16x8 (&av)[MI], const bf16x8 (&bv)[NI]) __attribute__((always_inline)) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mi], bv[ni], acc[mi][ni], 0, 0, 0);
    };

    // ---- main loop: one LDS stage, next chunk prefetched into registers ----
    const int nch = a.chunks;
    load(0);
    store();
    __syncthreads();
    for (int kc = 0; kc < nch; ++kc) {
        if (kc + 1 < nch) load((kc + 1) * CC);
        // Operand offsets are re-derived every chunk from copies the compiler
        // cannot see through, so it does not keep all the steps' addresses
        // live across the loop.
        int al = a_lane, bl[NI];
        asm volatile("" : "+v"(al));
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            bl[ni] = b_lane[ni];
            asm volatile("" : "+v"(bl[ni]));
        }
        bf16x8 a0[MI], b0[NI], a1[MI], b1[NI];
        fetch(0, al, bl, a0, b0);
#pragma unroll
        for (int s = 0; s < C::STEPS; ++s) {
            if (s + 1 < C::STEPS) {
                if (s & 1) fetch(s + 1, al, bl, a0, b0);
                else fetch(s + 1, al, bl, a1, b1);
            }
            // Keep the fetches of step s+1 ahead of the MFMAs of step s.
            __builtin_amdgcn_sched_barrier(0);
            if (s & 1) mfmas(a1, b1);
            else mfmas(a0, b0);
        }
        __syncthreads();
        if (kc + 1 < nch) {
            store();
            __syncthreads();
        }
    }

    // ---- epilogue: bias, activation, bf16, store ----
    __hip_bfloat16* __restrict__ yg = (__hip_bfloat16*)a.yptr;
    const int64_t out_plane = (int64_t)a.ho * a.wo;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            const int j = wn * C::WC + ni * 16 + (lane & 15);
            const int ho = ho0 + j / TW, wo = wo0 + j % TW;
            if (ho < a.ho && wo < a.wo) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int co = co0 + wm * C::WR + mi * 16 + (lane >> 4) * 4 + v;
                    if (co < a.cout_g) {
                        const int cg = g * a.cout_g + co;
                        yg[((int64_t)n * a.out_total + a.out_off + cg) * out_plane + (int64_t)ho * a.wo + wo] =
                            f32_to_bf16(bias_act(a, acc[mi][ni][v], cg));
                    }
                }
            }
        }
}

// ------------------------------------------------------------ configs ---

struct CfgInfo {
    int bm, bn, tw, cc, kh, kw, xs, nt, alds;
    const void* fn;
};

template <class C>
CfgInfo info() {
    return CfgInfo{C::BM, C::BN, C::TW, C::CC, C::KH, C::KW, C::XS, C::NT, C::ALDS,
                   (const void*)igemm_bf16_kernel<C>};
}

// Four waves (one per SIMD, up to 512 registers each) in a 2 x 2 grid of
// 64 x 128 or 64 x 64 wave tiles.
//                      BM WM WN NI   TW  CC KH KW  XS
using B3_128x128 = BCfg<128, 2, 2, 4,  16, 16, 3, 3,  6>;   // 3x3 any stride: 8 x 16 output pixels
using B3_32x256  = BCfg<32,  1, 4, 4,  16, 16, 3, 3,  6>;   // few output channels per group
using B1_128x256 = BCfg<128, 2, 2, 8, 256, 64, 1, 1,  8>;   // flattened 1x1
using B1_32x256  = BCfg<32,  1, 4, 4, 256, 64, 1, 1,  8>;

enum { C3_128x128, C3_32x256, C1_128x256, C1_32x256, NCFG };

const CfgInfo& cfg(int i) {
    static const CfgInfo t[NCFG] = {info<B3_128x128>(), info<B3_32x256>(), info<B1_128x256>(),
                                    info<B1_32x256>()};
    return t[i];
}

struct Geom {
    int ph, span, shift, nvr;
};

Geom geom(const conv2d_params_t& p, const CfgInfo& c, bool flat) {
    Geom G;
    const int th = c.bn / c.tw;
    if (flat) {
        G.ph = 1; G.span = c.tw; G.shift = 0; G.nvr = c.tw / 8;
    } else {
        G.ph = (th - 1) * p.stride_h + (p.k_h - 1) * p.dilation_h + 1;
        G.span = (c.tw - 1) * p.stride_w + (p.k_w - 1) * p.dilation_w + 1;
        G.shift = ((-p.pad_left) % 8 + 8) % 8;
        G.nvr = (G.shift + G.span + 7) / 8;
    }
    return G;
}

}  // namespace

bool plan_igemm_bf16(Desc& d) {
    const conv2d_params_t& p = d.p;
    const bool is3 = p.k_h == 3 && p.k_w == 3;
    const bool flat = p.k_h == 1 && p.k_w == 1 && p.stride_h == 1 && p.stride_w == 1 && p.pad_top == 0 &&
                      p.pad_left == 0 && p.pad_bottom == 0 && p.pad_right == 0;
    int cands[3];
    int nc = 0;
    const bool small_m = d.cout_g <= 32;
    if (is3) {
        if (small_m) cands[nc++] = C3_32x256;
        cands[nc++] = C3_128x128;
    } else if (flat) {
        cands[nc++] = small_m ? C1_32x256 : C1_128x256;
    }
    for (int k = 0; k < nc; ++k) {
        const CfgInfo& c = cfg(cands[k]);
        const Geom G = geom(p, c, flat);
        if (c.cc * G.ph * G.nvr > c.xs * c.nt) continue;                    // input vectors per thread
        if (G.ph >= 2048 || 8 * G.nvr + 8 >= 4096 || c.cc > 256) continue;  // packed vector plan fields
        const int lds = 2 * (c.alds + G.ph * G.span * (c.cc + 8));
        if (lds > 160 * 1024) continue;
        if ((int64_t)c.cc * p.h * p.w >= INT32_MAX / 2) continue;
        if ((int64_t)c.bm * d.cin_g * p.k_h * p.k_w >= INT32_MAX / 2) continue;
        d.cfg = cands[k];
        d.flatten_1x1 = flat;
        d.tile_w = c.tw;
        d.tile_h = c.bn / c.tw;
        d.lds_bytes = lds;
        return true;
    }
    return false;
}

hipError_t launch_igemm_bf16(const Desc& d, ConvArgs a, hipStream_t s) {
    const CfgInfo& c = cfg(d.cfg);
    const conv2d_params_t& p = d.p;
    const Geom G = geom(p, c, d.flatten_1x1);
    if (d.flatten_1x1) {
        a.h = 1; a.w = p.h * p.w; a.ho = 1; a.wo = d.ho * d.wo;
    }
    a.tiles_h = (a.ho + d.tile_h - 1) / d.tile_h;
    a.tiles_w = (a.wo + d.tile_w - 1) / d.tile_w;
    a.patch_h = G.ph;
    a.patch_w = G.span;
    a.patch_shift = G.shift;
    a.patch_stride = G.nvr;
    a.co_tiles = (d.cout_g + c.bm - 1) / c.bm;
    a.chunks = (d.cin_g + c.cc - 1) / c.cc;
    a.dv_co_tiles = make_divu32((uint32_t)a.co_tiles);
    a.dv_groups = make_divu32((uint32_t)a.groups);
    a.dv_tiles_w = make_divu32((uint32_t)a.tiles_w);
    a.dv_tiles_h = make_divu32((uint32_t)a.tiles_h);
    const uint64_t blocks = (uint64_t)a.co_tiles * a.groups * a.tiles_h * a.tiles_w * a.n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0xFFFFFFFFull) return hipErrorInvalidConfiguration;
    a.num_blocks = (uint32_t)blocks;
    if (d.lds_bytes > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(c.fn, hipFuncAttributeMaxDynamicSharedMemorySize, d.lds_bytes);
        if (e != hipSuccess) return e;
    }
    void* args[] = {&a};
    return hipLaunchKernel(c.fn, dim3((uint32_t)blocks), dim3(c.nt), args, d.lds_bytes, s);
}

}  // namespace conv2d
