// Implicit-GEMM convolution with bfloat16 operands on the gfx950 matrix
// cores (v_mfma_f32_16x16x32_bf16), fp32 accumulation, fp32 bias and
// activation, bf16 output rounded to nearest even.
//
// GEMM view (ncnn "convolution": pad with pad_value, correlate, + bias,
// activation): M = output channels of a group, N = output pixels, K = input
// channels x taps.  A bf16 MFMA step takes 32 K values and every lane
// supplies 8 consecutive ones, so both operands are kept in LDS as 16-byte
// cells of 8 consecutive input channels:
//   weights  [tap*G + group-of-8][output channel]      (one cell each)
//   patch    [group-of-8][patch position]              (one cell each)
// K runs tap-major inside a chunk of CC = 8*G input channels; an MFMA operand
// is one 16-byte LDS read and 16 lanes of a read touch 16 consecutive cells.
//
// Copy path.  The weights are re-laid once per call (pack kernel below) into
// exactly the LDS image of each (output-channel tile, channel chunk), so a
// chunk's weights move with direct global->LDS loads (no registers, no
// transposition).  The NCHW input is transposed on the fly: a lane loads 8
// channels x 8 pixels (eight 16-byte row loads), permutes them in registers
// and writes eight 16-byte cells.  Stride-2 patches keep even and odd columns
// in separate halves of a row, so a stride-2 read of 16 output pixels is
// still 16 consecutive cells.  The row and plane strides of the patch are
// chosen on the host to spread those cell writes over the LDS banks.
//
// Pipeline: two LDS stages; the copy instructions of chunk c+1 (DMA and row
// loads) are interleaved with the MFMAs of chunk c, then its rows are
// transposed into the free stage; one workgroup barrier per chunk.
// The epilogue adds the bias, applies the activation, rounds to bf16 and
// writes channel out_off + g*cout_g + co of a buffer with out_total channels
// (ConcatFusedTail), 4 pixels of a row per 8-byte store.
#include "device_common.h"

namespace conv2d {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int BM_, int WM_, int WN_, int NI_, int TW_, int CC_, int KH_, int KW_, int SD_, int XS_>
struct BCfg {
    static constexpr int BM = BM_, WM = WM_, WN = WN_, NI = NI_, TW = TW_, CC = CC_, KH = KH_, KW = KW_;
    static constexpr bool SD = SD_ != 0;               // stride-2 column split
    static constexpr int XS = XS_;                     // input tasks per thread (upper bound)
    static constexpr int KHW = KH * KW;
    static constexpr int NW = WM * WN, NT = 64 * NW;   // waves, threads
    static constexpr int WR = BM / WM, MI = WR / 16;   // rows / row fragments of a wave tile
    static constexpr int WC = 16 * NI, BN = WC * WN;   // pixels of a wave tile / of the workgroup tile
    static constexpr int TH = BN / TW;
    static constexpr int G = CC / 8;                   // 8-channel groups per chunk
    static constexpr int STEPS = (KHW * CC + 31) / 32; // K steps of 32 per chunk
    static constexpr int TGP = 4 * STEPS;              // (tap, group) slots incl. the zero K padding
    static constexpr int ACELLS = TGP * BM;            // 16-byte cells of a chunk's weight image
    static constexpr int DMAR = ACELLS / 64;           // 1 KB wave copies per weight image
    // One wave per SIMD: double-buffer the MFMA operands and spread the copy
    // instructions over the MFMAs.  Two waves per SIMD: the other wave covers
    // those stalls, and the registers are needed elsewhere.
    static constexpr bool PIPE = NW <= 4;
    static_assert(CC % 8 == 0 && TGP % G == 0, "K steps tile whole (tap, group) slots");
    static_assert(ACELLS % 64 == 0, "weight image in whole 1 KB pieces");
    static_assert(WR % 16 == 0 && TW % 16 == 0 && BN % TW == 0, "whole fragments");
};

// Input task v of a chunk: 8 channels (group g) x 8 pixels (vector vc) of
// patch row `row`.  Vectors run fastest, then rows, then groups.
__host__ __device__ inline void input_task(int v, int nvr, int ph, int& vc, int& row, int& g) {
    vc = v % nvr;
    const int rest = v / nvr;
    row = rest % ph;
    g = rest / ph;
}

// Cell of patch column pc inside its row (stride-2 patches: evens, then odds).
__host__ __device__ inline int col_cell(int pc, int half, bool split) {
    return split ? (pc & 1) * half + (pc >> 1) : pc;
}

__device__ __forceinline__ void copy16_to_lds(const uint4* src, uint4* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds((const float*)src, (float*)lds_base, 16, 0, 0);
#endif
}

template <class C>
__global__ __launch_bounds__(C::NT) void igemm_bf16_kernel(ConvArgs a) {
    extern __shared__ __align__(16) uint4 lds[];
    constexpr int BM = C::BM, TW = C::TW, TH = C::TH, G = C::G;
    constexpr int KHW = C::KHW, KW = C::KW, MI = C::MI, NI = C::NI, STEPS = C::STEPS;

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
    const int PH = a.patch_h, span = a.patch_w;
    const int shift = a.patch_shift;                      // iw_lo minus its 8-aligned floor
    const int nvr = a.patch_stride;                       // 8-pixel vectors per patch row
    const int RS = a.lds_rs, PL = a.lds_plane, HALF = a.col_half;
    const int scells = C::ACELLS + G * PL;                // cells per stage
    const int HW = a.h * a.w;

    const uint16_t* __restrict__ xg = (const uint16_t*)a.xptr +
                                      ((int64_t)n * a.in_total + a.in_off + (int64_t)g * a.cin_g) * HW;
    const uint4* __restrict__ wp = (const uint4*)a.wptr + (int64_t)(g * a.co_tiles + cot) * a.chunks * C::ACELLS;
    const bool vx = a.w % 8 == 0 && ((uintptr_t)a.xptr % 16) == 0;
    const uint32_t padb = __bfloat16_as_ushort(f32_to_bf16(a.pad_value));
    const uint32_t pad2 = padb | (padb << 16);

    // ---- per-thread input tasks ----
    int tcell[C::XS];   // cell (in the patch part of a stage) of the task's row start; -1 = no task
    int tpc[C::XS];     // patch column of the vector's first pixel
    int tg8[C::XS];     // first channel of the task's group
    int trow[C::XS];    // patch row
    int txo[C::XS];     // offset of the vector's first pixel in a channel plane; -1 = outside the image
#pragma unroll
    for (int i = 0; i < C::XS; ++i) {
        const int v = tid + C::NT * i;
        tcell[i] = -1; tpc[i] = 0; tg8[i] = 0; trow[i] = 0; txo[i] = -1;
        if (v < G * PH * nvr) {
            int vc, row, gg;
            input_task(v, nvr, PH, vc, row, gg);
            const int ih = ih0 + row, iw = iw_lo - shift + 8 * vc;
            tcell[i] = gg * PL + row * RS;
            tpc[i] = 8 * vc - shift;
            tg8[i] = 8 * gg;
            trow[i] = row;
            if ((unsigned)ih < (unsigned)a.h && iw >= 0 && iw < a.w) txo[i] = ih * a.w + iw;
        }
    }

    uint4 xr[C::XS][8];
    // Global -> register: channel c0 + tg8 + t of input task i (8 pixels).
    auto load_op = [&](int i, int t, int c0) __attribute__((always_inline)) {
        if (tcell[i] < 0) return;
        uint4 r = make_uint4(0, 0, 0, 0);
        if (tg8[i] + t < a.cin_g - c0) {
            const uint16_t* __restrict__ plane = xg + (int64_t)(c0 + tg8[i] + t) * HW;
            if (vx) {
                r = txo[i] >= 0 ? *(const uint4*)(plane + txo[i]) : make_uint4(pad2, pad2, pad2, pad2);
            } else {
                const int ih = ih0 + trow[i];
                const int iw0 = iw_lo + tpc[i];
                uint32_t e[8];
#pragma unroll
                for (int p = 0; p < 8; ++p) {
                    const int iw = iw0 + p;
                    e[p] = ((unsigned)ih < (unsigned)a.h && (unsigned)iw < (unsigned)a.w)
                               ? (uint32_t)plane[ih * a.w + iw]
                               : padb;
                }
                r = make_uint4(e[0] | e[1] << 16, e[2] | e[3] << 16, e[4] | e[5] << 16, e[6] | e[7] << 16);
            }
        }
        xr[i][t] = r;
    };
    // Registers -> LDS: 8 channels x 8 pixels become 8 cells of 8 channels.
    auto store_x = [&](uint4* bst) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < C::XS; ++i) {
            if (tcell[i] < 0) continue;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const int pc = tpc[i] + p;
                uint32_t d[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint4 lo = xr[i][2 * k], hi = xr[i][2 * k + 1];
                    const uint32_t wl = (p >> 1) == 0 ? lo.x : (p >> 1) == 1 ? lo.y : (p >> 1) == 2 ? lo.z : lo.w;
                    const uint32_t wh = (p >> 1) == 0 ? hi.x : (p >> 1) == 1 ? hi.y : (p >> 1) == 2 ? hi.z : hi.w;
                    d[k] = (p & 1) ? ((wl >> 16) | (wh & 0xffff0000u)) : ((wl & 0xffffu) | (wh << 16));
                }
                if (pc >= 0 && pc < span) bst[tcell[i] + col_cell(pc, HALF, C::SD)] = make_uint4(d[0], d[1], d[2], d[3]);
            }
        }
    };
    // Weight image of chunk kc -> LDS: the wave's k-th 1 KB piece.
    constexpr int ND = (C::DMAR + C::NW - 1) / C::NW;    // DMA pieces per wave
    constexpr int NOPS = ND + C::XS * 8;                  // copy instructions per wave and chunk
    auto dma_op = [&](int k, int kc, uint4* ast) __attribute__((always_inline)) {
        const int r = wave + C::NW * k;
        if (r < C::DMAR) copy16_to_lds(wp + (int64_t)kc * C::ACELLS + r * 64 + lane, ast + r * 64);
    };
    // Copy instruction k of chunk kc: DMA pieces first, then the input loads.
    auto copy_op = [&](int k, int kc, uint4* ast) __attribute__((always_inline)) {
        if (k < ND) dma_op(k, kc, ast);
        else load_op((k - ND) / 8, (k - ND) % 8, kc * C::CC);
    };

    // ---- operand offsets (cells) ----
    // Step s, lane group q = lane/16 supplies K slot tg = 4s + q: tap tg / G,
    // channel group tg % G.  A row co = wm*WR + mi*16 + lane%16; B pixel
    // j = wn*WC + ni*16 + lane%16.
    const int q = lane >> 4, l16 = lane & 15;
    const int a_lane = q * BM + wm * C::WR + l16;
    int b_lane[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
        const int j = wn * C::WC + ni * 16 + l16;
        const int jr = j / TW, jc = j % TW;
        b_lane[ni] = C::SD ? jr * a.stride_h * RS + jc : jr * a.stride_h * RS + jc * a.stride_w;
    }
    int b_step[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        const int tg = 4 * s + q;
        int tap = tg / G;
        const int gg = tg - (tg / G) * G;
        if (tap >= KHW) tap = 0;     // K padding: zero weights, finite inputs of tap 0
        const int r = tap / KW, sc = tap - (tap / KW) * KW;
        const int cdx = sc * a.dilation_w;
        b_step[s] = gg * PL + r * a.dilation_h * RS + (C::SD ? (cdx & 1) * HALF + (cdx >> 1) : cdx);
    }

    f32x4 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    auto fetch = [&](const uint4* st, int s, bf16x8 (&av)[MI], bf16x8 (&bv)[NI]) __attribute__((always_inline)) {
        const uint4* as = st + a_lane + 4 * s * BM;
        const uint4* bs = st + C::ACELLS + b_step[s];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) av[mi] = __builtin_bit_cast(bf16x8, as[16 * mi]);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) bv[ni] = __builtin_bit_cast(bf16x8, bs[b_lane[ni]]);
    };
    // Chunk from stage st.  With `copy`, the copy instructions of chunk kn
    // (DMA into stage nst, input rows into registers) are spread over the
    // MFMAs of the first half of the steps, so the memory pipe drains while
    // the matrix cores run.
    auto compute = [&](const uint4* st, bool copy, int kn, uint4* nst) __attribute__((always_inline)) {
        constexpr int SP = STEPS > 1 ? (STEPS + 1) / 2 : 1;
        constexpr int SLOTS = SP * MI * NI;                      // MFMAs that may carry copy instructions
        constexpr int PER = (NOPS + SLOTS - 1) / SLOTS;          // copy instructions per carrying MFMA
        constexpr int NGRP = (NOPS + PER - 1) / PER;
        constexpr int STRIDE = SLOTS / NGRP;
        if constexpr (!C::PIPE) {
            if (copy) {
#pragma unroll
                for (int k = 0; k < NOPS; ++k) copy_op(k, kn, nst);
            }
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                bf16x8 av[MI], bv[NI];
                fetch(st, s, av, bv);
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv[ni], av[mi], acc[mi][ni], 0, 0, 0);
            }
            return;
        }
        bf16x8 a0[MI], b0[NI], a1[MI], b1[NI];
        fetch(st, 0, a0, b0);
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            if (s + 1 < STEPS) {
                if (s & 1) fetch(st, s + 1, a0, b0);
                else fetch(st, s + 1, a1, b1);
            }
            // Keep the fetches of step s+1 ahead of the MFMAs of step s.
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) {
                    if (s & 1)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b1[ni], a1[mi], acc[mi][ni], 0, 0, 0);
                    else
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0[ni], a0[mi], acc[mi][ni], 0, 0, 0);
                    const int gm = (s * MI + mi) * NI + ni;
                    if (copy && gm % STRIDE == 0 && gm / STRIDE < NGRP) {
#pragma unroll
                        for (int u = 0; u < PER; ++u)
                            if ((gm / STRIDE) * PER + u < NOPS) copy_op((gm / STRIDE) * PER + u, kn, nst);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
        }
    };

    // ---- main loop: two stages, chunk c+1 copied while chunk c computes ----
    const int nch = a.chunks;
    uint4* const st0 = lds;
    uint4* const st1 = lds + scells;
#pragma unroll
    for (int k = 0; k < NOPS; ++k) copy_op(k, 0, st0);
    __builtin_amdgcn_s_waitcnt(0);
    store_x(st0 + C::ACELLS);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        uint4* cur = (c & 1) ? st1 : st0;
        uint4* nxt = (c & 1) ? st0 : st1;
        if (c + 1 < nch) {
            compute(cur, true, c + 1, nxt);
            __builtin_amdgcn_s_waitcnt(0);   // chunk c+1: weight image and input rows have landed
            store_x(nxt + C::ACELLS);
        } else {
            compute(cur, false, 0, nxt);
        }
        __syncthreads();                     // stage cur is free, stage nxt is complete
    }

    // ---- epilogue: bias, activation, bf16, store ----
    // The workgroup's BM biases and PReLU slopes go through LDS (free after
    // the last barrier), one global load per channel instead of one per output.
    float* eb = (float*)lds;
    float* es = eb + BM;
    for (int i = tid; i < BM; i += C::NT) {
        const int co = co0 + i;
        const int cg = g * a.cout_g + (co < a.cout_g ? co : a.cout_g - 1);
        eb[i] = a.bias ? a.bias[cg] : 0.0f;
        es[i] = a.act == CONV_ACT_PRELU ? a.slope[a.slope_count == 1 ? 0 : cg] : 0.0f;
    }
    __syncthreads();
    // The MFMA's first operand is the pixel fragment, so lane (q, l16) holds
    // output channel mi*16 + l16 at the 4 consecutive pixels ni*16 + 4q ..+3
    // of one output row: one 8-byte store where the row allows it.
    uint16_t* __restrict__ yg = (uint16_t*)a.yptr;
    const int64_t out_plane = (int64_t)a.ho * a.wo;
    const bool vy = a.wo % 4 == 0 && ((uintptr_t)a.yptr % 8) == 0;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
        const int col = wm * C::WR + mi * 16 + l16;
        const int co = co0 + col;
        if (co >= a.cout_g) continue;
        const int cg = g * a.cout_g + co;
        const float bb = eb[col], ss = es[col];
        uint16_t* yc = yg + ((int64_t)n * a.out_total + a.out_off + cg) * out_plane;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            const int j = wn * C::WC + ni * 16 + 4 * q;
            const int ho = ho0 + j / TW, wo = wo0 + j % TW;
            if (ho >= a.ho) continue;
            uint32_t h[4];
#pragma unroll
            for (int v = 0; v < 4; ++v)
                h[v] = __bfloat16_as_ushort(f32_to_bf16(apply_act(a, acc[mi][ni][v] + bb, ss)));
            uint16_t* dst = yc + (int64_t)ho * a.wo + wo;
            if (vy && wo + 3 < a.wo) {
                *(uint2*)dst = make_uint2(h[0] | h[1] << 16, h[2] | h[3] << 16);
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (wo + v < a.wo) dst[v] = (uint16_t)h[v];
            }
        }
    }
}

// Weight re-layout: OIHW bf16 -> per (group, output-channel tile, chunk) the
// LDS image [tap*G + group-of-8][BM][8 channels], zero where the tap, the
// output channel or the input channel lies past the filter.
__global__ __launch_bounds__(256) void pack_weights_bf16(const uint16_t* __restrict__ w, uint4* __restrict__ out,
                                                         int64_t total, int bm, int tgp, int gq, int cc, int khw,
                                                         int chunks, int co_tiles, int cin_g, int cout_g) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    int64_t rest = idx;
    const int co = rest % bm; rest /= bm;
    const int tg = rest % tgp; rest /= tgp;
    const int kc = rest % chunks; rest /= chunks;
    const int cot = rest % co_tiles;
    const int grp = rest / co_tiles;
    const int tap = tg / gq, g8 = tg % gq;
    const int cog = cot * bm + co;
    uint32_t e[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int ci = kc * cc + g8 * 8 + t;
        e[t] = (tap < khw && cog < cout_g && ci < cin_g)
                   ? (uint32_t)w[(((int64_t)grp * cout_g + cog) * cin_g + ci) * khw + tap]
                   : 0u;
    }
    out[idx] = make_uint4(e[0] | e[1] << 16, e[2] | e[3] << 16, e[4] | e[5] << 16, e[6] | e[7] << 16);
}

// ------------------------------------------------------------ configs ---

struct CfgInfo {
    int bm, bn, tw, cc, kh, kw, sd, xs, nt, tgp;
    const void* fn;
};

template <class C>
CfgInfo info() {
    return CfgInfo{C::BM, C::BN, C::TW, C::CC, C::KH, C::KW, C::SD ? 1 : 0, C::XS, C::NT, C::TGP,
                   (const void*)igemm_bf16_kernel<C>};
}

// Eight waves (two per SIMD, so one wave's memory or barrier stalls are
// covered by the other's MFMAs) in a 2 x 4 grid of 64 x 64 wave tiles; the
// small-channel variants use four waves.
//                   BM WM WN NI   TW  CC KH KW SD XS
using B3_128 = BCfg<128, 2, 4, 4,  16, 16, 3, 3, 0, 2>;   // 3x3 stride 1: 16 x 16 output pixels
using B3_128s = BCfg<128, 2, 4, 4, 16, 16, 3, 3, 0, 1>;   // the same for patches of <= 512 input tasks
using B3S_128 = BCfg<128, 2, 4, 4, 16, 16, 3, 3, 1, 1>;   // 3x3 stride 2 (column split)
using B3_32 = BCfg<32, 1, 4, 4,  16, 16, 3, 3, 0, 2>;     // 3x3, few output channels per group
using B3_16 = BCfg<16, 1, 4, 4,  16, 8, 3, 3, 0, 2>;      // 3x3, <= 16 output and <= 8 input channels per group
using B1_128 = BCfg<128, 2, 4, 4, 256, 64, 1, 1, 0, 1>;   // flattened 1x1
using B1_32 = BCfg<32, 1, 4, 4, 256, 64, 1, 1, 0, 1>;

enum { C3_128, C3_128s, C3S_128, C3_32, C3_16, C1_128, C1_32, NCFG };

const CfgInfo& cfg(int i) {
    static const CfgInfo t[NCFG] = {info<B3_128>(), info<B3_128s>(), info<B3S_128>(), info<B3_32>(),
                                    info<B3_16>(),  info<B1_128>(),   info<B1_32>()};
    return t[i];
}

struct Geom {
    int ph, span, shift, nvr, half, rs, plane;
};

// LDS cell-write cost of one chunk's input tasks for row stride rs and
// plane stride pl: per 16-lane pass of a 16-byte write, the largest number
// of lanes that fall on the same 16-byte bank group.
int64_t write_cost(const Geom& G, const CfgInfo& c, int rs, int pl) {
    const int tasks = (c.cc / 8) * G.ph * G.nvr;
    int64_t cost = 0;
    for (int base = 0; base < tasks; base += 16) {
        for (int p = 0; p < 8; ++p) {
            int hits[16] = {0};
            int worst = 0;
            for (int l = 0; l < 16 && base + l < tasks; ++l) {
                int vc, row, gg;
                input_task(base + l, G.nvr, G.ph, vc, row, gg);
                const int pc = 8 * vc - G.shift + p;
                if (pc < 0 || pc >= G.span) continue;
                const int cell = gg * pl + row * rs + col_cell(pc, G.half, c.sd != 0);
                const int h = ++hits[cell & 15];
                worst = h > worst ? h : worst;
            }
            cost += worst;
        }
    }
    return cost;
}

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
    G.half = (G.span + 1) / 2;
    const int rs0 = c.sd ? 2 * G.half : G.span;
    // Smallest write cost over row strides rs0..rs0+15 and plane padding 0..15.
    int64_t best = -1;
    G.rs = rs0;
    G.plane = G.ph * rs0;
    for (int rs = rs0; rs < rs0 + 16; ++rs)
        for (int pad = 0; pad < (c.cc > 8 ? 16 : 1); ++pad) {
            const int pl = G.ph * rs + pad;
            const int64_t cost = write_cost(G, c, rs, pl);
            if (best < 0 || cost < best || (cost == best && pl < G.plane)) {
                best = cost; G.rs = rs; G.plane = pl;
            }
        }
    return G;
}

int64_t wpack_cells(const Desc& d, const CfgInfo& c) {
    const int64_t co_tiles = (d.cout_g + c.bm - 1) / c.bm;
    const int64_t chunks = (d.cin_g + c.cc - 1) / c.cc;
    return (int64_t)d.p.groups * co_tiles * chunks * c.tgp * c.bm;
}

}  // namespace

bool plan_igemm_bf16(Desc& d) {
    const conv2d_params_t& p = d.p;
    const bool is3 = p.k_h == 3 && p.k_w == 3;
    const bool flat = p.k_h == 1 && p.k_w == 1 && p.stride_h == 1 && p.stride_w == 1 && p.pad_top == 0 &&
                      p.pad_left == 0 && p.pad_bottom == 0 && p.pad_right == 0;
    int cands[4];
    int nc = 0;
    if (is3 && p.stride_h == p.stride_w) {
        if (p.stride_w == 2) {
            cands[nc++] = C3S_128;
        } else if (p.stride_w == 1) {
            if (d.cout_g <= 16 && d.cin_g <= 8) cands[nc++] = C3_16;
            if (d.cout_g <= 32) cands[nc++] = C3_32;
            cands[nc++] = C3_128s;
            cands[nc++] = C3_128;
        }
    } else if (flat) {
        cands[nc++] = d.cout_g <= 32 ? C1_32 : C1_128;
    }
    for (int k = 0; k < nc; ++k) {
        const CfgInfo& c = cfg(cands[k]);
        const Geom G = geom(p, c, flat);
        if ((c.cc / 8) * G.ph * G.nvr > c.xs * c.nt) continue;         // input tasks per thread
        const int64_t stage = 16 * ((int64_t)c.tgp * c.bm + (int64_t)(c.cc / 8) * G.plane);
        if (2 * stage > 160 * 1024) continue;
        if ((int64_t)c.cc * p.h * p.w >= INT32_MAX / 2) continue;
        if (wpack_cells(d, c) * 16 >= ((int64_t)1 << 40)) continue;
        d.cfg = cands[k];
        d.flatten_1x1 = flat;
        d.tile_w = c.tw;
        d.tile_h = c.bn / c.tw;
        d.lds_bytes = (int32_t)(2 * stage);
        d.wpack_bytes = wpack_cells(d, c) * 16;
        d.g_ph = G.ph; d.g_span = G.span; d.g_shift = G.shift; d.g_nvr = G.nvr;
        d.g_rs = G.rs; d.g_plane = G.plane; d.g_half = G.half;
        return true;
    }
    return false;
}

hipError_t launch_igemm_bf16(const Desc& d, ConvArgs a, hipStream_t s) {
    const CfgInfo& c = cfg(d.cfg);
    const conv2d_params_t& p = d.p;
    if (d.flatten_1x1) {
        a.h = 1; a.w = p.h * p.w; a.ho = 1; a.wo = d.ho * d.wo;
    }
    a.tiles_h = (a.ho + d.tile_h - 1) / d.tile_h;
    a.tiles_w = (a.wo + d.tile_w - 1) / d.tile_w;
    a.patch_h = d.g_ph;
    a.patch_w = d.g_span;
    a.patch_shift = d.g_shift;
    a.patch_stride = d.g_nvr;
    a.lds_rs = d.g_rs;
    a.lds_plane = d.g_plane;
    a.col_half = d.g_half;
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
    if (!d.wpack || d.wpack_bytes != wpack_cells(d, c) * 16) return hipErrorInvalidValue;

    // 1) weights -> per-chunk LDS images
    const int64_t total = d.wpack_bytes / 16;
    const void* w_src = a.wptr;
    uint4* pk = (uint4*)d.wpack;
    int64_t tot = total;
    int bm = c.bm, tgp = c.tgp, gq = c.cc / 8, cc = c.cc, khw = p.k_h * p.k_w, chunks = a.chunks,
        co_tiles = a.co_tiles, cin_g = d.cin_g, cout_g = d.cout_g;
    void* pargs[] = {&w_src, &pk, &tot, &bm, &tgp, &gq, &cc, &khw, &chunks, &co_tiles, &cin_g, &cout_g};
    hipError_t e = hipLaunchKernel((const void*)pack_weights_bf16, dim3((uint32_t)((total + 255) / 256)), dim3(256),
                                   pargs, 0, s);
    if (e != hipSuccess) return e;

    // 2) the convolution
    a.wptr = d.wpack;
    if (d.lds_bytes > 64 * 1024) {
        e = hipFuncSetAttribute(c.fn, hipFuncAttributeMaxDynamicSharedMemorySize, d.lds_bytes);
        if (e != hipSuccess) return e;
    }
    void* args[] = {&a};
    return hipLaunchKernel(c.fn, dim3((uint32_t)blocks), dim3(c.nt), args, d.lds_bytes, s);
}

}  // namespace conv2d
