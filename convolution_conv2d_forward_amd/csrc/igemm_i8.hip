// int8 dense and grouped convolution (symmetric QLinearConv: int32
// accumulation, + int32 bias, requant) as an implicit GEMM on the gfx950 i8
// matrix cores (v_mfma_i32_16x16x64_i8), for the windows the depthwise and
// pointwise kernels do not take.  The requant follows the yscv "ONNX CPU
// Kernels (Conv/MatMul) -- Runtime Map" page (section "Hot kernel paths",
// fused INT8 chains); the convolution is ncnn's "convolution" definition
// with the zero point as the pad.
//
// GEMM per group: Y[co, p] = sum_k W[co, k] X^[k, p].  K runs over chunks
// of up to 64 input channels; within a chunk it is a list of items, item i =
// (tap i / ncg, 16-channel group i % ncg), ncg = 1, 2 or 4 groups of 16
// channels (enough for the group's channels), and an MFMA K step is four
// consecutive items: a 3x3 window over 64 channels is one tap per step,
// over 8 channels four taps per step (instead of a step of 64 channels of
// which 56 are padding).  A lane's 16 consecutive k are 16 channels at one
// tap.  The input patch of the tile is staged in LDS pixel-major, [pixel][16
// * ncg channels] (4 channels x 4 pixels per unit: four 4-byte loads,
// transposed with v_perm), so the pixel operand is one 16-byte LDS read at
// the item's patch pixel and channel group.  Pixels are the first MFMA
// operand, so a lane's result is 4 consecutive output columns of one
// channel: + bias, requant, one packed 4-byte store where the row allows it.
//
// Two kernels:
//   - igemm_i8_fast_kernel, 3x3 windows over word-aligned input rows: the
//     weights are re-laid once (at bind, or by a pack kernel before the
//     call) into per-chunk LDS images, [K step][co][64 bytes] with the four
//     16-byte pieces of a row rotated by (co / 4) % 4 so that the 16 rows a
//     B-operand read touches fall on distinct banks; a chunk's image reaches
//     LDS by direct global->LDS copies, 1 KB per wave instruction.  A
//     thread holds its share of the next chunk's patch in registers: those
//     loads are issued as soon as the current chunk is in LDS and land while
//     its MFMAs run.  The K steps are unrolled (per-lane patch offsets
//     computed once), and the four waves split the tile 2 x 2 (output
//     channel halves x output row halves) where it has two or more channel
//     tiles, so each operand read feeds more MFMAs.
//   - igemm_i8_kernel, every other window: weights re-laid per chunk from
//     OIHW by the workgroup ([K step][co][80 bytes], 16 pad bytes per row),
//     the patch staged in passes, each chunk in turn.
#include <algorithm>

#include "device_common.h"

namespace conv2d {

namespace {

constexpr int kT = 256;
constexpr int WR = 80;          // igemm_i8_kernel: LDS bytes per weight row (64 + 16 pad bytes)
constexpr int TW = 16;          // output columns per tile (one MFMA fragment)
constexpr int QV = 4;           // igemm_i8_kernel: staged 4x4 blocks per thread and pass

struct I8Args {
    ConvArgs a;
    int32_t khw;            // taps
    int32_t th;             // output rows per tile (4 * NFW)
    int32_t ph, pw;         // patch rows, patch columns (a multiple of 4)
    int32_t pw4;            // pw / 4
    int32_t ncg, lg_nq;     // 16-channel groups per chunk (its 16 * ncg input channels); log2 of its channel quads
    int32_t xr;             // LDS bytes per staged patch pixel (16 * ncg + 16)
    int32_t qs;             // patch slots per quarter (see the patch layout)
    int32_t items, steps;   // (tap, channel group) items per chunk; MFMA K steps, items / 4 rounded up
    int32_t co_tiles, tiles_h, tiles_w, chunks;
    int32_t xs_bytes, ws_bytes;
    int32_t vec_x;          // patch rows move as 4-byte words
    int32_t vec_w;          // filter blocks move as 4-byte words
    int32_t away;           // requant ties away from zero
    uint32_t num_blocks;
    DivU32 dv_co_tiles, dv_groups, dv_tiles_w, dv_tiles_h;
    DivU32 dv_pw4;          // staging unit -> (quad, patch row)
    DivU32 dv_ppix;         // staging unit / 4 -> channel quad group (patch words per quad)
    DivU32 dv_kw;           // tap -> (r, s)
    DivU32 dv_ncg;          // item -> (tap, channel group)
};

__device__ __forceinline__ void tr4x4(const uint32_t in[4], uint32_t out[4]) {
    const uint32_t t0 = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);
    const uint32_t t1 = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);
    const uint32_t t2 = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);
    const uint32_t t3 = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);
    out[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
    out[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
    out[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
    out[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// Requant, ties to even or (AWAY) away from zero, branch-free; the clamp to
// [lo, hi] (the int8 range shifted by the zero point, raised to 0 under
// ReLU) runs on the rounded value.
template <bool AWAY>
__device__ __forceinline__ int rq8(int32_t acc, float comp, float lo, float hi, int zp) {
    float yf = __fmul_rn((float)acc, comp);
    asm volatile("" : "+v"(yf));   // the rounded f32 product decides ties (no fma into the rounding)
    float r;
    if constexpr (AWAY) {
        const float t = truncf(yf);
        r = fabsf(yf - t) == 0.5f ? t + copysignf(1.0f, yf) : rintf(yf);
    } else {
        r = rintf(yf);
    }
    return (int)__builtin_amdgcn_fmed3f(r, lo, hi) + zp;
}

// Four requantised values (each in [-128, 127]) as the bytes of one word.
template <bool AWAY>
__device__ __forceinline__ uint32_t rq8x4(i32x4 acc, int32_t bb, float comp, float lo, float hi, int zp) {
    const uint32_t b0 = (uint32_t)rq8<AWAY>(acc[0] + bb, comp, lo, hi, zp);
    const uint32_t b1 = (uint32_t)rq8<AWAY>(acc[1] + bb, comp, lo, hi, zp);
    const uint32_t b2 = (uint32_t)rq8<AWAY>(acc[2] + bb, comp, lo, hi, zp);
    const uint32_t b3 = (uint32_t)rq8<AWAY>(acc[3] + bb, comp, lo, hi, zp);
    // low bytes of b0, b1 -> bytes 0, 1; of b2, b3 -> bytes 2, 3
    const uint32_t lo01 = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
    const uint32_t hi23 = __builtin_amdgcn_perm(b3, b2, 0x04000c0cu);
    return lo01 | hi23;
}

// Block index -> (output-channel tile, group, column tile, row tile, image).
struct I8Tile {
    int cot, g, twi, thi, n;
};

__device__ __forceinline__ I8Tile i8_tile(const I8Args& f) {
    I8Tile t;
    uint32_t L = xcd_remap(blockIdx.x, f.num_blocks);
    uint32_t Q = divu(L, f.dv_co_tiles);
    t.cot = L - Q * f.co_tiles;
    L = Q; Q = divu(L, f.dv_groups);
    t.g = L - Q * f.a.groups;
    L = Q; Q = divu(L, f.dv_tiles_w);
    t.twi = L - Q * f.tiles_w;
    L = Q; Q = divu(L, f.dv_tiles_h);
    t.thi = L - Q * f.tiles_h;
    t.n = Q;
    return t;
}

// + bias, requant, 4 consecutive columns per lane.  acc[j][m] holds output
// row ho0 + rbase + rstep * j of channel tile mbase + m.
template <bool AWAY, int NR, int NM>
__device__ __forceinline__ void i8_epilogue_r(const I8Args& f, const I8Tile& t, const i32x4 (&acc)[NR][NM], int rbase,
                                              int rstep, int mbase, int co0, int ho0, int wo0, int lane) {
    const ConvArgs& a = f.a;
    const bool relu = a.act == CONV_ACT_RELU;
    const float lo = relu ? 0.0f : (float)(-128 - a.y_zp), hi = (float)(127 - a.y_zp);
    int8_t* __restrict__ yg = (int8_t*)a.yptr;
    const int64_t oplane = (int64_t)a.ho * a.wo;
    const bool vec_y = (a.wo % 4) == 0 && ((uintptr_t)a.yptr % 4) == 0;
    const int wo = wo0 + 4 * (lane >> 4);
    // Every channel's bias before the first store: a read behind a store
    // waits for all earlier memory operations, the next tile's loads included.
    int32_t bias[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int co = co0 + 16 * (mbase + m) + (lane & 15);
        bias[m] = (a.qbias && co < a.cout_g) ? a.qbias[t.g * a.cout_g + co] : 0;
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int co = co0 + 16 * (mbase + m) + (lane & 15);
        if (co >= a.cout_g) continue;
        const int cg = t.g * a.cout_g + co;
        const int32_t bb = bias[m];
        int8_t* yc = yg + ((int64_t)t.n * a.out_total + a.out_off + cg) * oplane;
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            const int ho = ho0 + rbase + rstep * j;
            if (ho >= a.ho || wo >= a.wo) continue;
            const uint32_t word = rq8x4<AWAY>(acc[j][m], bb, a.composite, lo, hi, a.y_zp);
            int8_t* dst = yc + (int64_t)ho * a.wo + wo;
            if (vec_y && wo + 4 <= a.wo) {
                *(uint32_t*)dst = word;
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (wo + v < a.wo) dst[v] = (int8_t)(word >> (8 * v));
            }
        }
    }
}

template <int NR, int NM>
__device__ __forceinline__ void i8_epilogue(const I8Args& f, const I8Tile& t, const i32x4 (&acc)[NR][NM], int rbase,
                                            int rstep, int mbase, int co0, int ho0, int wo0, int lane) {
    if (f.away)
        i8_epilogue_r<true>(f, t, acc, rbase, rstep, mbase, co0, ho0, wo0, lane);
    else
        i8_epilogue_r<false>(f, t, acc, rbase, rstep, mbase, co0, ho0, wo0, lane);
}

// Direct global->LDS copy of 16 bytes per lane: lane l writes lds_base + 16*l
// (lds_base wave-uniform).  Inline assembly, so that the compiler does not
// order the workgroup's later LDS reads behind it; the kernel's own
// s_waitcnt before the barrier is what orders the copy.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(const void* src, const void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m)
                 : "memory", "m0");
#endif
}
#pragma clang diagnostic pop

// ---------------------------------------------------------------------------
// 3x3 windows over word-aligned rows, weights pre-packed.
//
// Packed weights: for each (group, channel tile, chunk) an image of STEPS x
// BM rows x 64 bytes; row (s, co) holds the four items 4s .. 4s+3, item i =
// (tap i / ncg, channel group i % ncg) as W[co][16 * cg .. +15][tap], piece
// kq stored at position kq ^ ((co / 4) % 4).  Items past the last, channels
// past the group and channels past cout_g are zero.
// The kernel is persistent: workgroup b takes tiles b', b' + G, b' + 2G, ...
// (G workgroups, b' its XCD-grouped index), and the pipeline runs across
// tile boundaries, so the first chunk of the next tile is in flight during
// the last chunk's MFMAs and the epilogue.
struct I8TileGeo {
    int g, co0, ho0, wo0, ih0, iw_a, n;
};

__device__ __forceinline__ I8TileGeo i8_geo(const I8Args& f, uint32_t L, int BM) {
    const ConvArgs& a = f.a;
    I8TileGeo t;
    uint32_t Q = divu(L, f.dv_co_tiles);
    t.co0 = (int)(L - Q * f.co_tiles) * BM;
    L = Q; Q = divu(L, f.dv_groups);
    t.g = (int)(L - Q * a.groups);
    L = Q; Q = divu(L, f.dv_tiles_w);
    t.wo0 = (int)(L - Q * f.tiles_w) * TW;
    L = Q; Q = divu(L, f.dv_tiles_h);
    t.ho0 = (int)(L - Q * f.tiles_h) * f.th;
    t.n = (int)Q;
    t.ih0 = t.ho0 * a.stride_h - a.pad_top;
    const int iw_lo = t.wo0 * a.stride_w - a.pad_left;
    t.iw_a = iw_lo >= 0 ? iw_lo & ~3 : -((-iw_lo + 3) & ~3);   // patch column 0, a multiple of 4
    return t;
}

// 16 bytes per lane from global memory straight into LDS: lane l reads
// base + off and writes lds_base + 16*l (base and lds_base wave-uniform).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16s_to_lds(const uint8_t* base, uint32_t off, const void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(m)
                 : "memory", "m0");
#endif
}
#pragma clang diagnostic pop

template <int NFW, int MB, int NCG>
__global__ __launch_bounds__(kT, 2) void igemm_i8_fast_kernel(I8Args f, const uint8_t* __restrict__ wpk) {
    extern __shared__ __align__(16) uint8_t lds[];
    const ConvArgs& a = f.a;
    constexpr int BM = 16 * MB;
    constexpr int WM = MB >= 2 ? 2 : 1;         // waves across the channel tiles
    constexpr int MBW = MB / WM;                // channel tiles per wave
    constexpr int NFR = NFW * WM;               // output-row fragments per wave
    constexpr int STEPS = (9 * NCG + 3) / 4;
    constexpr int XR = 16 * NCG + 16;           // LDS bytes per patch pixel
    constexpr int NQ = 4 * NCG;                 // channel quads per chunk
    constexpr int CKC = 16 * NCG;               // input channels per chunk
    constexpr int UQ = 3 * NCG;                 // patch units per thread held in registers
    constexpr int WIMG = STEPS * BM * 64;       // bytes of a chunk's weight image
    constexpr int PIECES = WIMG / 1024;         // 1 KB copies per chunk image
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wr = wave / WM;
    const int kq = lane >> 4;

    const int H = a.h, W = a.w;
    const int64_t HW = (int64_t)H * W;
    const uint32_t HW32 = (uint32_t)HW;
    const int cin_g = a.cin_g;
    const int PW = f.pw;
    const int pq_n = f.ph * f.pw4;       // 4-pixel words of the patch per channel quad
    const int QS = f.qs;                 // slots per quarter of the patch (>= pq_n)
    const int chunks = f.chunks;
    // The patch starts 0-3 columns left of the first input column a tile
    // reads; tiles start at multiples of 16 output columns, so this shift is
    // the same for every tile.
    const int shift = (((-a.pad_left) % 4) + 4) % 4;

    uint8_t* xs = lds;                   // [4 * QS][XR]; pixel p at slot (p % 4) * QS + p / 4
    uint8_t* ws = lds + f.xs_bytes;      // two buffers of [STEPS][BM][64]

    // Per lane, the same for every tile: the LDS address of its pixel
    // operand for each K step (item 4s + kq) and fragment, and of its weight
    // operand (row s * BM + 16 * m + lane % 16, piece kq at its rotated place).
    int aoff[STEPS][NFR];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        const int i = 4 * s + kq;
        const int tap = i / NCG, cg = i % NCG;
        const int r = (tap * 11) >> 5;   // tap / 3 for tap < 12
        const bool live = i < 9 * NCG;
        const int toff = live ? r * a.dilation_h * PW + (tap - 3 * r) * a.dilation_w : 0;
        const int cgo = live ? 16 * cg : 0;
#pragma unroll
        for (int j = 0; j < NFR; ++j) {
            const int pp = (wr * NFR + j) * a.stride_h * PW + (lane & 15) * a.stride_w + shift + toff;
            aoff[s][j] = ((pp & 3) * QS + (pp >> 2)) * XR + cgo;
        }
    }
    const int boff = (16 * wm * MBW + (lane & 15)) * 64 + 16 * (kq ^ ((lane >> 2) & 3));

    // Patch unit u: channel quad 4 * (u / (4 * pq_n)) + u % 4 and word rem =
    // (u / 4) % pq_n (patch row rem / pw4, columns 4 * (rem % pw4) ..+3).
    // Four consecutive lanes take four channel quads of one word, so a
    // wave's transposed words fill 16 bytes of each of 16 consecutive slots
    // (every bank once).  Per unit, the same for every tile: patch row and
    // column, the offset of its first channel, and its LDS place.
    const int units0 = ((min(NQ, (cin_g + 3) >> 2) + 3) & ~3) * pq_n;   // units of a full chunk
    int upr[UQ], upc[UQ], ucq[UQ], sbase[UQ];
#pragma unroll
    for (int i = 0; i < UQ; ++i) {
        const int u = tid + i * kT;
        const int hi = (int)divu((uint32_t)(u >> 2), f.dv_ppix);
        const int cq = 4 * hi + (u & 3);
        const int rem = (u >> 2) - hi * pq_n;
        const int pr = (int)divu((uint32_t)rem, f.dv_pw4);
        upr[i] = u < units0 ? pr : -(1 << 20);   // units past the chunk: never inside the image
        upc[i] = 4 * (rem - pr * f.pw4);
        ucq[i] = 4 * cq;
        // byte b of the word is patch pixel 4 * rem + b, at slot b * QS + rem;
        // units past the chunk store their zeros to slot pq_n of each
        // quarter, which no pixel uses
        sbase[i] = u < units0 ? rem * XR + 4 * cq : pq_n * XR;
    }

    // A tile's patch offsets: channel 4 * cq's word inside the image, or an
    // offset past every buffer range (the buffer load then returns zero).
    uint32_t goff[UQ];
    auto set_units = [&](const I8TileGeo& t) {
#pragma unroll
        for (int i = 0; i < UQ; ++i) {
            const int ih = t.ih0 + upr[i], iw = t.iw_a + upc[i];
            // W % 4 == 0 and iw % 4 == 0: the word is inside the row or outside it.
            const bool in = (unsigned)ih < (unsigned)H && (unsigned)iw < (unsigned)W;
            goff[i] = in ? (uint32_t)(ih * W + iw) + (uint32_t)ucq[i] * HW32 : 0x80000000u;
        }
    };
    uint32_t pv[UQ][4];
    // Chunk kc of tile t: the patch words through four buffer resources,
    // resource cc starting at the chunk's channel cc and ending at its last
    // channel (channels past cin_g and units outside the image read as
    // zero), the weight image into LDS buffer wb.
    auto issue = [&](const I8TileGeo& t, int kc, int wb) {
        const int cleft = min(CKC, cin_g - kc * CKC);
        const int8_t* xc = (const int8_t*)a.xptr +
                           ((int64_t)t.n * a.in_total + a.in_off + (int64_t)t.g * cin_g + (int64_t)kc * CKC) * HW;
        __amdgpu_buffer_rsrc_t rs[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
            rs[cc] = __builtin_amdgcn_make_buffer_rsrc((void*)(xc + cc * HW), (short)0,
                                                       (int)((uint32_t)max(cleft - cc, 0) * HW32), 0x00020000);
        const uint8_t* wsrc = wpk + ((int64_t)(t.g * f.co_tiles + t.co0 / BM) * chunks + kc) * WIMG;
        uint8_t* wdst = ws + wb * WIMG;
#pragma unroll
        for (int p = 0; p < (PIECES + 3) / 4; ++p) {
            const int piece = wave + 4 * p;
            // (every wave copies PIECES / 4 pieces when 4 divides PIECES)
            if (PIECES % 4 == 0 || piece < PIECES)
                copy16s_to_lds(wsrc + 4096 * p, (uint32_t)(wave * 1024 + 16 * lane), wdst + piece * 1024);
        }
#pragma unroll
        for (int i = 0; i < UQ; ++i) {
            if (i * kT >= units0) break;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc)
                pv[i][cc] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs[cc], (int)goff[i], 0, 0);
        }
    };
    auto store_patch = [&]() {
#pragma unroll
        for (int i = 0; i < UQ; ++i) {
            if (i * kT >= units0) break;
            uint32_t outw[4];
            tr4x4(pv[i], outw);
#pragma unroll
            for (int b = 0; b < 4; ++b) *(uint32_t*)&xs[b * QS * XR + sbase[i]] = outw[b];
        }
    };

    i32x4 acc[NFR][MBW];
#pragma unroll
    for (int j = 0; j < NFR; ++j)
#pragma unroll
        for (int m = 0; m < MBW; ++m) acc[j][m] = i32x4{0, 0, 0, 0};

    const uint32_t ntiles = f.num_blocks, G = gridDim.x;
    uint32_t tl = xcd_remap(blockIdx.x, G);
    I8TileGeo cur = i8_geo(f, tl, BM);
    set_units(cur);
    issue(cur, 0, 0);
    int kc = 0, wb = 0;
    for (;;) {
        store_patch();
        __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0): this thread's copies of the chunk have landed
        __syncthreads();                      // ... and every thread's; the previous chunk's MFMAs are done
        // the next chunk: of this tile, or the first of the next one
        const bool last = kc + 1 == chunks;
        const uint32_t tn = last ? tl + G : tl;
        const bool more = tn < ntiles;
        I8TileGeo nxt = cur;
        if (more) {
            if (last) {
                nxt = i8_geo(f, tn, BM);
                set_units(nxt);
            }
            issue(nxt, last ? 0 : kc + 1, wb ^ 1);
        }
        const uint8_t* wsc = ws + wb * WIMG;
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            i32x4 bw[MBW];
#pragma unroll
            for (int m = 0; m < MBW; ++m) bw[m] = *(const i32x4*)&wsc[s * BM * 64 + m * 1024 + boff];
#pragma unroll
            for (int j = 0; j < NFR; ++j) {
                const i32x4 av = *(const i32x4*)&xs[aoff[s][j]];
#pragma unroll
                for (int m = 0; m < MBW; ++m)
                    acc[j][m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bw[m], acc[j][m], 0, 0, 0);
            }
        }
        if (last) {
            I8Tile t;
            t.g = cur.g;
            t.n = cur.n;
            i8_epilogue<NFR, MBW>(f, t, acc, wr * NFR, 1, wm * MBW, cur.co0, cur.ho0, cur.wo0, lane);
#pragma unroll
            for (int j = 0; j < NFR; ++j)
#pragma unroll
                for (int m = 0; m < MBW; ++m) acc[j][m] = i32x4{0, 0, 0, 0};
        }
        __syncthreads();
        if (!more) break;
        cur = nxt;
        tl = tn;
        kc = last ? 0 : kc + 1;
        wb ^= 1;
    }
}

// OIHW int8 -> the fast kernel's per-chunk weight images, one thread per
// 16-byte piece of the output (16 channels of one item).
struct I8PackArgs {
    int32_t cin_g, cout_g, bm, ncg, steps, co_tiles, chunks;
    int64_t words;
};

__global__ __launch_bounds__(256) void pack_i8_kernel(const int8_t* __restrict__ w, uint4* __restrict__ dst,
                                                      I8PackArgs p) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;     // 16-byte piece of the output
    if (q >= p.words / 4) return;
    const int img_pieces = p.steps * p.bm * 4;
    const int64_t img = q / img_pieces;
    const int r = (int)(q - img * img_pieces);
    const int kc = (int)(img % p.chunks);
    const int64_t gt = img / p.chunks;
    const int cot = (int)(gt % p.co_tiles);
    const int g = (int)(gt / p.co_tiles);
    const int s = r / (p.bm * 4);
    const int row = (r >> 2) % p.bm;
    const int kq = (r & 3) ^ ((row >> 2) & 3);          // the item stored at this position
    const int i = 4 * s + kq;
    const int co = cot * p.bm + row;
    uint32_t v[4] = {0u, 0u, 0u, 0u};
    if (i < 9 * p.ncg && co < p.cout_g) {
        const int tap = i / p.ncg, cg = i % p.ncg;
        const int c0 = kc * 16 * p.ncg + 16 * cg;
        const int8_t* wc = w + (((int64_t)g * p.cout_g + co) * p.cin_g + c0) * 9 + tap;
#pragma unroll
        for (int b = 0; b < 16; ++b)
            if (c0 + b < p.cin_g) v[b >> 2] |= (uint32_t)(uint8_t)wc[b * 9] << (8 * (b & 3));
    }
    dst[q] = uint4{v[0], v[1], v[2], v[3]};
}

// ---------------------------------------------------------------------------
// Every other window: weights re-laid per chunk by the workgroup from OIHW,
// each chunk staged in turn.  Wave w owns output rows w, w+4, ...
template <int NFW, int MB>
__global__ __launch_bounds__(kT) void igemm_i8_kernel(I8Args f) {
    extern __shared__ __align__(16) uint8_t lds[];
    const ConvArgs& a = f.a;
    constexpr int BM = 16 * MB;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const I8Tile tl = i8_tile(f);
    const int co0 = tl.cot * BM;
    const int ho0 = tl.thi * f.th, wo0 = tl.twi * TW;
    const int ih0 = ho0 * a.stride_h - a.pad_top;
    const int iw_lo = wo0 * a.stride_w - a.pad_left;
    const int iw_a = iw_lo >= 0 ? iw_lo & ~3 : -((-iw_lo + 3) & ~3);   // patch column 0, a multiple of 4
    const int shift = iw_lo - iw_a;
    const int H = a.h, W = a.w;
    const int64_t HW = (int64_t)H * W;
    const int cin_g = a.cin_g;
    const int khw = f.khw;
    const int PW = f.pw;
    const int XR = f.xr;
    const int ncg = f.ncg;
    const int nq = 4 * ncg;               // channel quads per chunk

    const int8_t* __restrict__ xg = (const int8_t*)a.xptr + ((int64_t)tl.n * a.in_total + a.in_off + (int64_t)tl.g * cin_g) * HW;
    const int8_t* __restrict__ wg = (const int8_t*)a.wptr + (int64_t)(tl.g * a.cout_g + co0) * cin_g * khw;

    uint8_t* xs = lds;                                  // [4 * QS][XR]
    uint8_t* ws = lds + f.xs_bytes;                     // [steps][BM][WR]
    int* itab = (int*)(lds + f.xs_bytes + f.ws_bytes);  // [4 * steps]: (tap's patch offset << 2) | channel group
    const int pq_n = f.ph * f.pw4;        // 4-pixel words of the patch per channel quad
    const int QS = f.qs;                  // slots per quarter of the patch (>= pq_n)

    // Item table; weight rows of the items past the last one (the last K
    // step's padding) stay zero for the whole kernel.
    for (int i = tid; i < 4 * f.steps; i += kT) {
        int e = 0;
        if (i < f.items) {
            const int tap = (int)divu((uint32_t)i, f.dv_ncg);
            const int cg = i - tap * ncg;
            const int r = (int)divu((uint32_t)tap, f.dv_kw);
            const int s = tap - r * a.k_w;
            e = ((r * a.dilation_h * PW + s * a.dilation_w) << 2) | cg;
        }
        itab[i] = e;
    }
    for (int v = tid; v < (4 * f.steps - f.items) * BM; v += kT) {
        const int i = f.items + v / BM, co = v % BM;
        *(i32x4*)&ws[((i >> 2) * BM + co) * WR + 16 * (i & 3)] = i32x4{0, 0, 0, 0};
    }

    // This lane's pixel in each of its fragments: patch pixel of tap (0, 0).
    int pbase[NFW];
#pragma unroll
    for (int j = 0; j < NFW; ++j) pbase[j] = (wave + 4 * j) * a.stride_h * PW + (lane & 15) * a.stride_w + shift;

    i32x4 acc[NFW][MB];
#pragma unroll
    for (int j = 0; j < NFW; ++j)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[j][m] = i32x4{0, 0, 0, 0};

    const int kq = lane >> 4;
    for (int kc = 0; kc < f.chunks; ++kc) {
        const int c0 = kc * 16 * ncg;
        const int kq_n = min(nq, (cin_g - c0 + 3) >> 2);
        // ---- patch -> LDS (pixel-major) in passes; quads past cin_g are
        // left as they are: their weights are staged as zero.  Unit u: channel
        // quad 4 * (u / (4 * pq_n)) + u % 4 and word rem = (u / 4) % pq_n. ----
        const int units = ((kq_n + 3) & ~3) * pq_n;
        for (int u0 = 0; u0 < units; u0 += QV * kT) {
            uint32_t in[QV][4];
#pragma unroll
            for (int i = 0; i < QV; ++i) {
                const int u = u0 + tid + i * kT;
                const int hi = (int)divu((uint32_t)(u >> 2), f.dv_ppix);
                const int cq = 4 * hi + (u & 3);
                const int rem = (u >> 2) - hi * pq_n;
                const int pr = (int)divu((uint32_t)rem, f.dv_pw4);
                const int ih = ih0 + pr, iw = iw_a + 4 * (rem - pr * f.pw4);
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    const int ch = c0 + 4 * cq + cc;
                    uint32_t v = 0;
                    if (u < units && cq < kq_n && ch < cin_g && (unsigned)ih < (unsigned)H) {
                        const int8_t* src = xg + (int64_t)ch * HW + (int64_t)ih * W;
                        if (f.vec_x) {
                            // W % 4 == 0 and iw % 4 == 0: the word is inside the row or outside it.
                            if (iw >= 0 && iw < W) v = *(const uint32_t*)(src + iw);
                        } else {
#pragma unroll
                            for (int b = 0; b < 4; ++b)
                                if ((unsigned)(iw + b) < (unsigned)W) v |= (uint32_t)(uint8_t)src[iw + b] << (8 * b);
                        }
                    }
                    in[i][cc] = v;
                }
            }
#pragma unroll
            for (int i = 0; i < QV; ++i) {
                const int u = u0 + tid + i * kT;
                const int hi = (int)divu((uint32_t)(u >> 2), f.dv_ppix);
                const int cq = 4 * hi + (u & 3);
                if (u >= units || cq >= kq_n) continue;
                const int rem = (u >> 2) - hi * pq_n;
                uint32_t outw[4];
                tr4x4(in[i], outw);
                // byte b of the word is patch pixel 4 * rem + b, at slot b * QS + rem
#pragma unroll
                for (int b = 0; b < 4; ++b) *(uint32_t*)&xs[(b * QS + rem) * XR + 4 * cq] = outw[b];
            }
        }
        // ---- weights: unit (co, cq) = one output channel's 4 input channels
        // x all taps; word t (4 channels at tap t) belongs to item t * ncg +
        // cq / 4, bytes 4 * (cq % 4) ..+3 of its 16 ----
        auto w_slot = [&](int tap, int co, int cq) {
            const int i = tap * ncg + (cq >> 2);
            return &ws[((i >> 2) * BM + co) * WR + 16 * (i & 3) + 4 * (cq & 3)];
        };
        for (int u = tid; u < BM * nq; u += kT) {
            const int co = u >> f.lg_nq, cq = u & (nq - 1);
            const int ci = c0 + 4 * cq;
            const bool live = co0 + co < a.cout_g && ci < cin_g;
            const int8_t* src = wg + ((int64_t)co * cin_g + ci) * khw;
            if (live && f.vec_w && ci + 4 <= cin_g) {
                // cin_g % 4 == 0 and an aligned base: the 4 channels x khw taps
                // are 4 * khw contiguous bytes starting on a word.
                const uint32_t* src32 = (const uint32_t*)src;
                for (int t0 = 0; t0 < khw; t0 += 4) {
                    // Taps t0 .. t0+3 of channels ci .. ci+3 sit at bytes
                    // c * khw + t.  Bytes past the block (taps past the window
                    // of the last channel) are never stored below.
                    uint32_t wv4[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int b0 = c * khw + t0;
                        const int wi = b0 >> 2;
                        const uint32_t lo = wi < khw ? src32[wi] : 0u;
                        const uint32_t hi = ((b0 & 3) && wi + 1 < khw) ? src32[wi + 1] : 0u;
                        wv4[c] = __builtin_amdgcn_alignbyte(hi, lo, b0 & 3);
                    }
                    uint32_t outw[4];
                    tr4x4(wv4, outw);      // outw[t] = channels 0..3 at tap t0 + t
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (t0 + t < khw) *(uint32_t*)w_slot(t0 + t, co, cq) = outw[t];
                }
            } else {
                for (int t = 0; t < khw; ++t) {
                    uint32_t v = 0;
                    if (live) {
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            if (ci + c < cin_g) v |= (uint32_t)(uint8_t)src[c * khw + t] << (8 * c);
                    }
                    *(uint32_t*)w_slot(t, co, cq) = v;
                }
            }
        }
        __syncthreads();
        // ---- MFMAs: four items per K step ----
        for (int s = 0; s < f.steps; ++s) {
            const int e = itab[4 * s + kq];
            const int toff = e >> 2, cgo = (e & 3) << 4;
            i32x4 bw[MB];
#pragma unroll
            for (int m = 0; m < MB; ++m)
                bw[m] = *(const i32x4*)&ws[((s * BM) + 16 * m + (lane & 15)) * WR + 16 * kq];
#pragma unroll
            for (int j = 0; j < NFW; ++j) {
                const int pp = pbase[j] + toff;
                const i32x4 av = *(const i32x4*)&xs[((pp & 3) * QS + (pp >> 2)) * XR + cgo];
#pragma unroll
                for (int m = 0; m < MB; ++m)
                    acc[j][m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bw[m], acc[j][m], 0, 0, 0);
            }
        }
        __syncthreads();
    }
    i8_epilogue<NFW, MB>(f, tl, acc, wave, 4, 0, co0, ho0, wo0, lane);
}

struct I8Plan {
    int nfw, mb, ncg, xr, qs, items, steps, th, ph, pw, xs_bytes, ws_bytes, lds;
};

// Slots per quarter of the patch: pixel p lives at slot (p % 4) * qs + p / 4
// (a unit's four pixels in four quarters, so its transposed words go to
// consecutive slots).  A pixel operand read takes 16 bytes at 16 pixels p0 +
// l * stride; qs is padded so that any 8 of them (stride 1 or 2) fall on 8
// distinct 16-byte bank groups of a 256-byte bank line: qs = 4 (mod 16)
// when the slot size in 16-byte units (ncg + 1) is odd, qs = 2 (mod 8) when
// it is even.
int i8_qs(int words, int ncg) {
    const int m = (ncg + 1) % 2 ? 16 : 8, r = (ncg + 1) % 2 ? 4 : 2;
    return words + ((r - words % m) % m + m) % m;
}

constexpr int kLdsMax = 160 * 1024;

// Output channels per workgroup: 64 for windows of up to 9 taps, 32 for
// larger ones, and no more than the group has.  Chunks of 16 * ncg input
// channels: for the generic kernel enough for the group (at most 64); for
// the 3x3 kernel 16 or 32, which keeps a workgroup's LDS small enough for
// three or four per CU (a 3x3 step then holds two taps of 32 channels; the
// last of a chunk's five steps is half padding).  The tallest tile whose
// LDS allows two workgroups per CU (and, for the 3x3 kernel, whose patch
// fits the prefetch registers): 16 output rows (3x3 kernel only), 8 or 4.
bool i8_plan(const Desc& d, bool fast, I8Plan* out) {
    const conv2d_params_t& p = d.p;
    const int khw = p.k_h * p.k_w;
    if (fast && !(p.k_h == 3 && p.k_w == 3 && p.w % 4 == 0)) return false;
    const int mb = d.cout_g <= 16 ? 1 : (d.cout_g <= 32 || khw > 9) ? 2 : 4;
    const int ncg = fast ? (d.cin_g > 16 ? 2 : 1) : d.cin_g > 32 ? 4 : d.cin_g > 16 ? 2 : 1;
    const int xr = 16 * ncg + 16;
    const int items = khw * ncg, steps = (items + 3) / 4;
    // channel quads of the first chunk, rounded up to 4 (a unit group)
    const int quads = (std::min(4 * ncg, (d.cin_g + 3) / 4) + 3) / 4 * 4;
    // the 3x3 kernel also has 16-row tiles (four fragments per wave)
    for (int nfw = fast ? 4 : 2; nfw >= 1; nfw /= 2) {
        const int th = 4 * nfw;
        const int ph = (th - 1) * p.stride_h + (p.k_h - 1) * p.dilation_h + 1;
        const int pw = ((3 + (TW - 1) * p.stride_w + (p.k_w - 1) * p.dilation_w + 1) + 3) / 4 * 4;
        const int qs = i8_qs(ph * pw / 4 + 1, ncg);   // + a slot no pixel uses
        const int xs = 4 * qs * xr;
        // the 3x3 kernel: 64-byte weight rows in two buffers, no item table,
        // 3 * ncg patch units per thread, 32-bit offsets within the chunk
        const int wsb = fast ? steps * 16 * mb * 64 : steps * 16 * mb * WR;
        const int lds = xs + (fast ? 2 * wsb : wsb + 16 * steps);
        const bool fits = !fast || ((int64_t)quads * (ph * pw / 4) <= 3 * ncg * kT &&
                                    (int64_t)16 * ncg * p.h * p.w < (1ll << 31));
        if (fits && lds <= (nfw >= 2 ? 80 * 1024 : kLdsMax)) {
            *out = I8Plan{nfw, mb, ncg, xr, qs, items, steps, th, ph, pw, xs, wsb, lds};
            return true;
        }
    }
    return false;
}

template <int NFW, int MB>
const void* i8_fast_fn(int ncg) {
    return ncg == 2 ? (const void*)igemm_i8_fast_kernel<NFW, MB, 2> : (const void*)igemm_i8_fast_kernel<NFW, MB, 1>;
}

template <int NFW>
const void* i8_fn(const I8Plan& ip, bool fast) {
    if (fast) return ip.mb == 4 ? i8_fast_fn<NFW, 4>(ip.ncg) : ip.mb == 2 ? i8_fast_fn<NFW, 2>(ip.ncg) : i8_fast_fn<NFW, 1>(ip.ncg);
    return ip.mb == 4 ? (const void*)igemm_i8_kernel<NFW, 4>
         : ip.mb == 2 ? (const void*)igemm_i8_kernel<NFW, 2>
                      : (const void*)igemm_i8_kernel<NFW, 1>;
}

const void* i8_fast_nfw4(const I8Plan& ip) {
    return ip.mb == 4 ? i8_fast_fn<4, 4>(ip.ncg) : ip.mb == 2 ? i8_fast_fn<4, 2>(ip.ncg) : i8_fast_fn<4, 1>(ip.ncg);
}

int64_t i8_co_tiles(const Desc& d, const I8Plan& ip) { return (d.cout_g + 16 * ip.mb - 1) / (16 * ip.mb); }
int64_t i8_chunks(const Desc& d, const I8Plan& ip) { return (d.cin_g + 16 * ip.ncg - 1) / (16 * ip.ncg); }

}  // namespace

bool plan_igemm_i8(const Desc& d) {
    const conv2d_params_t& p = d.p;
    if (p.dtype != CONV_DTYPE_I8) return false;
    if ((int64_t)d.cin_g * p.k_h * p.k_w > (1 << 24)) return false;
    I8Plan ip{};
    return i8_plan(d, false, &ip);
}

int64_t igemm_i8_pack_bytes(const Desc& d) {
    I8Plan ip{};
    if (!i8_plan(d, true, &ip)) return 0;
    return (int64_t)d.p.groups * i8_co_tiles(d, ip) * i8_chunks(d, ip) * ip.ws_bytes;
}

bool igemm_i8_fast(const Desc& d, const void* x) {
    return igemm_i8_pack_bytes(d) > 0 && ((uintptr_t)x % 4) == 0;
}

hipError_t pack_igemm_i8_weights(const Desc& d, const void* w, void* dst, hipStream_t s) {
    I8Plan ip{};
    if (!i8_plan(d, true, &ip)) return hipErrorInvalidConfiguration;
    I8PackArgs p;
    p.cin_g = d.cin_g;
    p.cout_g = d.cout_g;
    p.bm = 16 * ip.mb;
    p.ncg = ip.ncg;
    p.steps = ip.steps;
    p.co_tiles = (int32_t)i8_co_tiles(d, ip);
    p.chunks = (int32_t)i8_chunks(d, ip);
    p.words = igemm_i8_pack_bytes(d) / 4;
    if (p.words == 0) return hipSuccess;
    const int64_t blocks = (p.words / 4 + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    void* args[] = {(void*)&w, &dst, &p};
    return hipLaunchKernel((const void*)pack_i8_kernel, dim3((uint32_t)blocks), dim3(256), args, 0, s);
}

hipError_t launch_igemm_i8(const Desc& d, ConvArgs a, hipStream_t s, const void* wpacked) {
    const conv2d_params_t& p = d.p;
    const bool vec_x = p.w % 4 == 0 && ((uintptr_t)a.xptr % 4) == 0;
    // The 3x3 kernel needs the packed image and word-aligned input rows.
    I8Plan ip{};
    const bool fast = wpacked && vec_x && i8_plan(d, true, &ip);
    if (!fast && !i8_plan(d, false, &ip)) return hipErrorInvalidConfiguration;
    I8Args f;
    f.a = a;
    f.khw = p.k_h * p.k_w;
    f.th = ip.th;
    f.ph = ip.ph;
    f.pw = ip.pw;
    f.pw4 = ip.pw / 4;
    f.ncg = ip.ncg;
    f.lg_nq = ip.ncg == 1 ? 2 : ip.ncg == 2 ? 3 : 4;
    f.xr = ip.xr;
    f.qs = ip.qs;
    f.items = ip.items;
    f.steps = ip.steps;
    f.co_tiles = (int32_t)i8_co_tiles(d, ip);
    f.tiles_h = (d.ho + ip.th - 1) / ip.th;
    f.tiles_w = (d.wo + TW - 1) / TW;
    f.chunks = (int32_t)i8_chunks(d, ip);
    f.xs_bytes = ip.xs_bytes;
    f.ws_bytes = ip.ws_bytes;
    f.vec_x = vec_x;
    f.vec_w = d.cin_g % 4 == 0 && ((uintptr_t)a.wptr % 4) == 0;
    f.away = p.int8_rounding == CONV_ROUND_HALF_AWAY;
    f.dv_co_tiles = make_divu32((uint32_t)f.co_tiles);
    f.dv_groups = make_divu32((uint32_t)p.groups);
    f.dv_tiles_w = make_divu32((uint32_t)f.tiles_w);
    f.dv_tiles_h = make_divu32((uint32_t)f.tiles_h);
    f.dv_pw4 = make_divu32((uint32_t)f.pw4);
    f.dv_ppix = make_divu32((uint32_t)(ip.ph * f.pw4));
    f.dv_kw = make_divu32((uint32_t)p.k_w);
    f.dv_ncg = make_divu32((uint32_t)ip.ncg);
    const uint64_t blocks = (uint64_t)f.co_tiles * p.groups * f.tiles_w * f.tiles_h * p.n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0xFFFFFFFFull) return hipErrorInvalidConfiguration;
    f.num_blocks = (uint32_t)blocks;
    const void* fn = ip.nfw == 4 ? i8_fast_nfw4(ip) : ip.nfw == 2 ? i8_fn<2>(ip, fast) : i8_fn<1>(ip, fast);
    if (ip.lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, ip.lds);
        if (e != hipSuccess) return e;
    }
    if (fast) {
        // persistent: as many workgroups as fit on the device at once (each
        // then takes every G-th tile), a multiple of 8 for the XCD grouping
        int per_cu = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kT, ip.lds);
        if (e != hipSuccess) return e;
        uint64_t g = (uint64_t)std::max(per_cu, 1) * device_cu_count();
        g = std::min<uint64_t>(g, blocks);
        if (g > 8) g &= ~7ull;
        void* args[] = {&f, (void*)&wpacked};
        return hipLaunchKernel(fn, dim3((uint32_t)g), dim3(kT), args, ip.lds, s);
    }
    void* args[] = {&f};
    return hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(kT), args, ip.lds, s);
}

}  // namespace conv2d
