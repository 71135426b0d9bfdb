// Implicit-GEMM convolution on the fp32 matrix cores of gfx950.
//
// The Go "ops" page (section ConvOp) runs Conv as im2col + GEMM and fuses the
// bias and activation into the GEMM write (ConvLeakyReluOp, ConvPReluOp).
// Here the im2col matrix is never built.  Per group g the GEMM is
//   Y_g[co, pixel] = sum_k W_g[co, k] * Xhat_g[k, pixel],  k = (ci, r, s),
// with M = output channels, N = output pixels, K = input channels x taps, and
// Xhat read out of an input patch staged in LDS: the B operand of tap (r, s)
// is the patch shifted by (r*dilation_h, s*dilation_w), and patch positions
// outside the image hold pad_value (ncnn "convolution": pad, then correlate).
//
// Work split.  A workgroup owns BM output channels x PT pixel sub-tiles of
// TH x TW outputs; its waves are WM row halves x KS-way split-K x PT pixel sub-tiles.
// Each wave streams its own slice of the input channels, CW channels at a
// time, through a private double-buffered LDS stage:
//   weights  [co][ci*KHW + rs]     (OIHW order, row stride KP)
//   patch    [ci][row][col]        (channel stride PS)
// so the main loop has no workgroup barrier at all; the waves only meet in
// the epilogue, where the split-K partial sums are added through LDS.
// One MFMA step (v_mfma_f32_16x16x4f32) takes four channels at one tap: lane
// group q = lane/16 supplies channel 4*step+q of both operands.  The strides
// are chosen so that every operand fetch hits 64 distinct LDS banks:
// KP is a multiple of 4 with KP/4 odd (16 rows x 4 k-slots), PS = 16 mod 64
// (4 channel planes x 16 consecutive pixels).
//
// Global traffic per chunk is a few 16-byte loads per lane at offsets
// computed once per workgroup (the patch geometry does not change from one
// chunk to the next); the loads of chunk c+1 are in flight while chunk c is
// multiplied out of LDS.
//
// The epilogue adds the bias, applies the activation and writes channel
// out_off + g*cout_g + co of a buffer with out_total channels (the
// ConcatFusedTail store of the Go "ops" page, any batch size), four
// consecutive pixels per lane so that a row of 16 lanes writes 256 bytes.
#include "device_common.h"

namespace conv2d {

namespace {


// LDS row stride of the weight tile: >= k, a multiple of 4, stride/4 odd.
__host__ __device__ constexpr int a_stride(int k) {
    return ((k + 3) / 4) % 2 ? (k + 3) / 4 * 4 : (k + 3) / 4 * 4 + 4;
}

template <int BM_, int BN_, int TW_, int CW_, int KH_, int KW_, int NW_, int WM_, int KS_, int ST_, int XS_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, TW = TW_, TH = BN_ / TW_, CW = CW_;
    static constexpr int KH = KH_, KW = KW_, KHW = KH_ * KW_;
    static constexpr int NW = NW_, NT = 64 * NW_;  // waves and threads per workgroup
    static constexpr int WM = WM_;                 // waves splitting the BM rows
    static constexpr int KS = KS_;                 // waves splitting K
    static constexpr int PT = NW_ / (WM_ * KS_);   // pixel sub-tiles per workgroup
    static constexpr int ST = ST_;                 // LDS stages per wave (1 or 2)
    static constexpr int WR = BM / WM;             // rows of one wave tile
    static constexpr int MI = WR / 16, NI = BN / 16;
    static constexpr int K = CW * KHW;            // K values of one wave chunk
    static constexpr int KP = a_stride(K);        // weight row stride in LDS
    static constexpr int AF4 = WR * K / 4;        // 16-byte weight units per wave chunk
    static constexpr int AS = (AF4 + 63) / 64;    // weight units per lane
    static constexpr int XS = XS_;                // patch units per lane (upper bound)
    static constexpr int ASZ = WR * KP;           // LDS floats of the weight tile
    static constexpr int STEPS = KHW * (CW / 4);  // MFMA steps of one chunk
    static constexpr int AU = (MI * STEPS + 3) / 4;   // packed weights: 16-byte units per lane and chunk
    static constexpr int RS = BN + 4;             // row stride of the reduction tile
    // Packed weights: the partial tiles sit behind the (patch-only) pipeline
    // when both fit beside each other.
    static constexpr bool RBEHIND = NW * WR * RS * 4 <= 96 * 1024;
    static_assert(WR % 16 == 0 && BN % 16 == 0, "whole 16x16 fragments");
    static_assert(NW % (WM * KS) == 0, "waves split into row halves, K slices and pixel sub-tiles");
    static_assert(TW % 16 == 0 && BN % TW == 0, "a fragment is 16 pixels of one row");
    static_assert(CW % 4 == 0, "a wave chunk is whole 4-channel MFMA steps");
    static_assert((PT * BM * BN / 4) % 64 == 0, "epilogue units fill whole waves");
    static_assert(ST == 1 || ST == 2, "one or two LDS stages");
};

// 16 bytes per lane from global memory straight into LDS (gfx950
// global_load_lds_dwordx4): lane l reads base + off (bytes) and writes
// lds_base + 16*l; completion is counted by vmcnt.  The address is given as
// a wave-uniform 64-bit base in scalar registers plus a 32-bit per-lane
// offset, which halves the address data each copy sends to the memory unit
// compared with a 64-bit address per lane (measured: the main loop ran ~6%
// faster).  The compiler does not pick that form for the builtin, hence the
// inline assembly; the "memory" clobber and the kernel's own s_waitcnt order
// it against the LDS reads.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(const float* base, uint32_t off, float* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(m)
                 : "memory", "m0");
#endif
}
#pragma clang diagnostic pop

__device__ __forceinline__ void wave_lds_sync() {
    // The LDS stage is private to the wave; order its writes before the reads
    // of other lanes of the same wave.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// AP (packed weights): a.wptr holds the weights in fragment order, as
// pack_igemm_f32_weights lays them out: for each group, tile of WR output
// channels and chunk, AU 16-byte units per lane, unit-major, so that each
// unit is one coalesced 1 KB load per wave.  The A operands then go from
// global memory straight into registers, one chunk ahead, and the LDS stages
// hold the input patch only (a third fewer LDS reads per MFMA step).  Only
// the two-stage direct-copy pipeline has this form.
template <class C, bool AP>
__global__ __launch_bounds__(C::NT) void igemm_f32_kernel(ConvArgs a) {
    extern __shared__ __align__(16) float lds[];
    constexpr int BM = C::BM, BN = C::BN, TW = C::TW, TH = C::TH, CW = C::CW;
    constexpr int KW = C::KW, KHW = C::KHW, KP = C::KP;
    constexpr int MI = C::MI, NI = C::NI;

    const int lane = threadIdx.x & 63;
    // The wave index is uniform across the wave; saying so keeps the loop
    // bounds and chunk offsets derived from it in scalar registers.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wk = wave % C::KS;                  // K slice of this wave
    const int wm = (wave / C::KS) % C::WM;        // row slice of this wave
    const int pt = wave / (C::KS * C::WM);        // pixel sub-tile of this wave

    // Block -> (co tile, group, column block, row block, image); output-channel
    // tiles fastest so that blocks reading the same patch are neighbours.
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

    const int co0 = cot * BM + wm * C::WR;        // first output channel of this wave
    const int ho0 = a.pt_vertical ? (thi * C::PT + pt) * TH : thi * TH;
    const int wo0 = a.pt_vertical ? twi * TW : (twi * C::PT + pt) * TW;
    const int ih0 = ho0 * a.stride_h - a.pad_top;
    const int ca = wo0 * a.stride_w - a.pad_left - a.patch_shift;   // multiple of 4
    const int PWA = a.patch_w, PS = a.patch_stride;
    const int xf4 = CW * a.patch_h * (PWA >> 2);
    const int HW = a.h * a.w;
    constexpr int XO = AP ? 0 : C::ASZ;   // patch offset in an LDS stage
    const int SF = XO + CW * PS;          // floats of one LDS stage
    // LDS: the per-wave stages, later reused for the split-K reduction.
    float* pipe = lds;

    const float* __restrict__ xg =
        (const float*)a.xptr + ((int64_t)n * a.in_total + a.in_off + (int64_t)g * a.cin_g) * HW;
    const float* __restrict__ wg = (const float*)a.wptr + ((int64_t)g * a.cout_g + co0) * a.cin_g * KHW;
    const bool vx = a.w % 4 == 0 && ((uintptr_t)a.xptr % 16) == 0;
    const bool vw = (a.cin_g * KHW) % 4 == 0 && ((uintptr_t)a.wptr % 16) == 0;

    // Patch unit e of this wave's chunk: channel, row and 4-column group.
    // (Numerators stay below 2^16, so the host-made magic divisions are exact.)
    struct XPos { int ci, ih, iw, lo; };
    auto xpos = [&](int e) __attribute__((always_inline)) {
        XPos q;
        q.ci = (int)fdiv(e, a.div_patch_hw);
        const int rem = e - q.ci * (int)a.div_patch_hw.d;
        const int row = (int)fdiv(rem, a.div_patch_w);
        const int cv = rem - row * (int)a.div_patch_w.d;
        q.ih = ih0 + row;
        q.iw = ca + 4 * cv;
        q.lo = q.ci * PS + row * PWA + 4 * cv;
        return q;
    };

    // ---- per-lane load plan, fixed for all chunks ----
    int xgo[C::XS];    // patch unit: element offset from the chunk's first channel, -1 = padding
    int xlo[C::XS];    // its LDS offset in the patch tile, -1 = no unit
#pragma unroll
    for (int i = 0; i < C::XS; ++i) {
        const int e = lane + 64 * i;
        xgo[i] = -1; xlo[i] = -1;
        if (e < xf4) {
            const XPos q = xpos(e);
            xlo[i] = q.lo;
            if ((unsigned)q.ih < (unsigned)a.h && q.iw >= 0 && q.iw < a.w) xgo[i] = q.ci * HW + q.ih * a.w + q.iw;
        }
    }
    constexpr int K4 = C::K / 4;
    int wgo[C::AS];    // weight unit: offset within the co tile at the chunk's first channel, -1 = none
#pragma unroll
    for (int i = 0; i < (AP ? 0 : C::AS); ++i) {
        const int e = lane + 64 * i;
        const int co = e / K4, j4 = e - (e / K4) * K4;
        wgo[i] = (e < C::AF4 && co0 + co < a.cout_g) ? co * a.cin_g * KHW + 4 * j4 : -1;
    }

    const float pv = a.pad_value;
    float4 xr[C::XS];
    float4 wr[C::AS];

    // Global -> registers for the channels [c0, c0 + CW) of the group.
    auto load = [&](int c0) __attribute__((always_inline)) {
        const float* __restrict__ xc = xg + (int64_t)c0 * HW;
        const float* __restrict__ wc = wg + (int64_t)c0 * KHW;
        const int cl = a.cin_g - c0;          // channels of the group left
        if (cl >= CW && vx) {
#pragma unroll
            for (int i = 0; i < C::XS; ++i)
                xr[i] = xgo[i] >= 0 ? *(const float4*)(xc + xgo[i]) : make_float4(pv, pv, pv, pv);
        } else {
            // Last, partial chunk or unaligned rows: element by element; channels
            // past the group read zero (their weights are zero too).
#pragma unroll
            for (int i = 0; i < C::XS; ++i) {
                const int e = lane + 64 * i;
                float v[4] = {0.f, 0.f, 0.f, 0.f};
                if (e < xf4) {
                    const XPos q = xpos(e);
                    const bool row_in = (unsigned)q.ih < (unsigned)a.h;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int col = q.iw + t;
                        if (q.ci < cl)
                            v[t] = (row_in && (unsigned)col < (unsigned)a.w) ? xc[q.ci * HW + q.ih * a.w + col] : pv;
                    }
                }
                xr[i] = make_float4(v[0], v[1], v[2], v[3]);
            }
        }
        if constexpr (AP) {
            // Packed weights go to registers separately.
        } else if (cl >= CW && vw) {
#pragma unroll
            for (int i = 0; i < C::AS; ++i)
                wr[i] = wgo[i] >= 0 ? *(const float4*)(wc + wgo[i]) : make_float4(0.f, 0.f, 0.f, 0.f);
        } else {
            const int kl = (cl < CW ? cl : CW) * KHW;   // valid k of this chunk
#pragma unroll
            for (int i = 0; i < C::AS; ++i) {
                const int k0 = 4 * ((lane + 64 * i) % K4);
                float v[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = (wgo[i] >= 0 && k0 + t < kl) ? wc[wgo[i] + t] : 0.0f;
                wr[i] = make_float4(v[0], v[1], v[2], v[3]);
            }
        }
    };

    auto store = [&](float* st) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < (AP ? 0 : C::AS); ++i) {
            const int e = lane + 64 * i;
            if (e < C::AF4) *(float4*)(st + (e / K4) * KP + 4 * (e % K4)) = wr[i];
        }
#pragma unroll
        for (int i = 0; i < C::XS; ++i)
            if (xlo[i] >= 0) *(float4*)(st + XO + xlo[i]) = xr[i];
    };

    // Operand addresses: A lane reads row co = lane%16 at k = (4*step + lane/16)*KHW + rs;
    // B lane reads channel plane 4*step + lane/16 at pixel j = ni*16 + lane%16.
    const int a_lane = (lane & 15) * KP + (lane >> 4) * KHW;
    int b_lane[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
        const int j = ni * 16 + (lane & 15);
        b_lane[ni] = (lane >> 4) * PS + (j / TW) * a.stride_h * PWA + (j % TW) * a.stride_w + a.patch_shift;
    }
    const int rstep = a.dilation_h * PWA, sstep = a.dilation_w;

    f32x4 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // One MFMA step: tap rs, channels 4q..4q+3 of the chunk.  Operands of
    // step t+1 are fetched from LDS while the MFMAs of step t run.
    constexpr int STEPS = C::STEPS;
    auto fetch = [&](const float* st, int t, float (&av)[MI], float (&bv)[NI]) __attribute__((always_inline)) {
        const int rs = t / (CW / 4), q = t % (CW / 4);
        const int boff = (rs / KW) * rstep + (rs % KW) * sstep;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) av[mi] = st[a_lane + mi * 16 * KP + q * 4 * KHW + rs];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) bv[ni] = st[XO + b_lane[ni] + q * 4 * PS + boff];
    };
    auto mfmas = [&](const float (&av)[MI], const float (&bv)[NI]) __attribute__((always_inline)) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mi], bv[ni], acc[mi][ni], 0, 0, 0);
    };

    // ---- main loop over this wave's chunks [kb, ke) ----
    const int nch = a.chunks;
    const int kb = (nch * wk) / C::KS, ke = (nch * (wk + 1)) / C::KS;
    float* st0 = pipe + wave * C::ST * SF;
    float* st1 = st0 + (C::ST - 1) * SF;
    // One chunk of MFMAs out of LDS stage cur.  With copy_mid, halfway
    // through the registers are written to stage nxt and, if load_next, chunk
    // kn's copy is loaded into them.
    auto run_chunk = [&](const float* cur, bool copy_mid, float* nxt, bool load_next, int kn) __attribute__((always_inline)) {
        float a0[MI], b0[NI], a1[MI], b1[NI];
        fetch(cur, 0, a0, b0);
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
            if (t + 1 < STEPS) {
                if (t & 1) fetch(cur, t + 1, a0, b0);
                else fetch(cur, t + 1, a1, b1);
            }
            // Keep the fetches of step t+1 ahead of the MFMAs of step t.
            __builtin_amdgcn_sched_barrier(0);
            if (t & 1) mfmas(a1, b1);
            else mfmas(a0, b0);
            if (t == STEPS / 2 && copy_mid) {
                store(nxt);
                if (load_next) load(kn * CW);
            }
        }
    };
    if constexpr (AP) {
        static_assert(C::ST == 2, "packed weights ride the two-stage copy pipeline");
        // Patch: direct global->LDS copies as below, padding written once per
        // stage; partial chunks through registers.  Weights: chunk kc's AU
        // units of this wave's tile, loaded into registers while chunk kc-1
        // is multiplied out; the wait at the chunk boundary covers both.
        const int tiles_g = a.co_tiles * C::WM;
        const f32x4* __restrict__ wp = (const f32x4*)a.wptr +
            (int64_t)(g * tiles_g + cot * C::WM + wm) * a.chunks * (C::AU * 64) + lane;
        auto aload = [&](int kc, f32x4 (&dst)[C::AU]) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < C::AU; ++u) dst[u] = wp[((int64_t)kc * C::AU + u) * 64];
        };
        auto copy_x = [&](int kc, float* st) __attribute__((always_inline)) {
            if (a.cin_g - kc * CW >= CW) {
                const float* __restrict__ xc = xg + (int64_t)kc * CW * HW;
#pragma unroll
                for (int i = 0; i < C::XS; ++i)
                    if (xgo[i] >= 0) copy16_to_lds(xc, 4u * (uint32_t)xgo[i], st + 256 * i);
            } else {
                load(kc * CW);
                store(st);
            }
        };
        auto fetch_b = [&](const float* st, int t, float (&bv)[NI]) __attribute__((always_inline)) {
            const int rs = t / (CW / 4), q = t % (CW / 4);
            const int boff = (rs / KW) * rstep + (rs % KW) * sstep;
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) bv[ni] = st[b_lane[ni] + q * 4 * PS + boff];
        };
        if (kb < ke) {
#pragma unroll
            for (int i = 0; i < C::XS; ++i)
                if (xlo[i] >= 0 && xgo[i] < 0) {
                    *(float4*)(st0 + xlo[i]) = make_float4(pv, pv, pv, pv);
                    *(float4*)(st1 + xlo[i]) = make_float4(pv, pv, pv, pv);
                }
            f32x4 acur[C::AU], anx[C::AU];
            aload(kb, acur);
            copy_x(kb, st0);
            __builtin_amdgcn_s_waitcnt(0);          // chunk kb has landed
            wave_lds_sync();
            float b0[NI], b1[NI];
            fetch_b(st0, 0, b0);
            for (int kc = kb; kc < ke; ++kc) {
                const bool odd = (kc - kb) & 1;
                const float* cur = odd ? st1 : st0;
                float* nxt = odd ? st0 : st1;
                const bool more = kc + 1 < ke;
                if (more) {
                    copy_x(kc + 1, nxt);
                    aload(kc + 1, anx);
                }
#pragma unroll
                for (int t = 0; t < STEPS; ++t) {
                    if (t + 1 < STEPS) {
                        if (t & 1) fetch_b(cur, t + 1, b0);
                        else fetch_b(cur, t + 1, b1);
                    } else if (more) {
                        __builtin_amdgcn_s_waitcnt(0);   // chunk kc+1 (patch and weights) has landed
                        wave_lds_sync();
                        if (t & 1) fetch_b(nxt, 0, b0);
                        else fetch_b(nxt, 0, b1);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    float av[MI];
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi) av[mi] = acur[(mi * STEPS + t) >> 2][(mi * STEPS + t) & 3];
                    if (t & 1) mfmas(av, b1);
                    else mfmas(av, b0);
                }
                if (STEPS & 1) {
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni) b0[ni] = b1[ni];
                }
                if (more) {
#pragma unroll
                    for (int u = 0; u < C::AU; ++u) acur[u] = anx[u];
                }
            }
        }
    } else if (C::ST == 2 && a.dma) {
        // Direct global->LDS copies (global_load_lds_dwordx4): lane l of copy
        // unit i writes 16 bytes at stage + 1024*i + 16*l, which is exactly the
        // unit-major layout of both tiles here (weight rows of K = KP floats,
        // patch planes of PS = patch_h*patch_w floats).  Padding positions are
        // the same for every chunk, so they are written once per stage and the
        // copies skip them.  Chunk kc+1 is issued right after chunk kc's copy
        // has landed and runs under chunk kc's MFMAs.
        auto pad_fill = [&](float* st) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < C::XS; ++i)
                if (xlo[i] >= 0 && xgo[i] < 0) *(float4*)(st + XO + xlo[i]) = make_float4(pv, pv, pv, pv);
        };
        auto dma = [&](int c0, float* st) __attribute__((always_inline)) {
            const float* __restrict__ wc = wg + (int64_t)c0 * KHW;
            const float* __restrict__ xc = xg + (int64_t)c0 * HW;
#pragma unroll
            for (int i = 0; i < (AP ? 0 : C::AS); ++i)
                if (wgo[i] >= 0) copy16_to_lds(wc, 4u * (uint32_t)wgo[i], st + 256 * i);
#pragma unroll
            for (int i = 0; i < C::XS; ++i)
                if (xgo[i] >= 0) copy16_to_lds(xc, 4u * (uint32_t)xgo[i], st + XO + 256 * i);
        };
        // Chunks that are not whole (the last one when CW does not divide the
        // group's channels) go through registers.
        auto copy_chunk = [&](int kc, float* st) __attribute__((always_inline)) {
            if (a.cin_g - kc * CW >= CW) {
                dma(kc * CW, st);
            } else {
                load(kc * CW);
                store(st);
            }
        };
        if (kb < ke) {
            pad_fill(st0);
            pad_fill(st1);
            copy_chunk(kb, st0);
            __builtin_amdgcn_s_waitcnt(0);          // chunk kb has landed
            wave_lds_sync();
            // The chunk boundary is pipelined like the steps inside a chunk:
            // during the last step of chunk kc the wave waits for chunk kc+1
            // (issued when chunk kc began) and fetches its first operands, so
            // the MFMAs run on without an LDS round trip between chunks.
            float a0[MI], b0[NI], a1[MI], b1[NI];
            fetch(st0, 0, a0, b0);
            for (int kc = kb; kc < ke; ++kc) {
                const bool odd = (kc - kb) & 1;
                const float* cur = odd ? st1 : st0;
                float* nxt = odd ? st0 : st1;
                const bool more = kc + 1 < ke;
                // Stage nxt held chunk kc-1, whose operands are all in registers by now.
                if (more) copy_chunk(kc + 1, nxt);
#pragma unroll
                for (int t = 0; t < STEPS; ++t) {
                    if (t + 1 < STEPS) {
                        if (t & 1) fetch(cur, t + 1, a0, b0);
                        else fetch(cur, t + 1, a1, b1);
                    } else if (more) {
                        __builtin_amdgcn_s_waitcnt(0);   // chunk kc+1 has landed
                        wave_lds_sync();
                        if (t & 1) fetch(nxt, 0, a0, b0);
                        else fetch(nxt, 0, a1, b1);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    if (t & 1) mfmas(a1, b1);
                    else mfmas(a0, b0);
                }
                // The next chunk's first operands are in set STEPS % 2.
                if (STEPS & 1) {
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi) a0[mi] = a1[mi];
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni) b0[ni] = b1[ni];
                }
            }
        }
    } else if (kb < ke) {
        // Register copies.  Registers hold chunk kc+1 (loaded one chunk
        // ahead).  With two LDS stages it is written to the other stage
        // halfway through chunk kc's MFMAs and chunk kc+2 is loaded right
        // after; with one stage the writes follow the last reads of chunk kc
        // (the LDS executes a wave's accesses in order).
        load(kb * CW);
        store(st0);
        if (kb + 1 < ke) load((kb + 1) * CW);
        for (int kc = kb; kc < ke; ++kc) {
            const bool odd = (kc - kb) & 1;
            const float* cur = odd ? st1 : st0;
            float* nxt = odd ? st0 : st1;
            const bool more = kc + 1 < ke;
            wave_lds_sync();
            run_chunk(cur, C::ST == 2 && more, nxt, kc + 2 < ke, kc + 2);
            if (C::ST == 1 && more) {
                wave_lds_sync();
                store(nxt);
                if (kc + 2 < ke) load((kc + 2) * CW);
            }
        }
    }
    // The static chunk split keeps the summation order, and so the result,
    // identical from run to run.

    // ---- epilogue: split-K sum through LDS, bias, activation, store ----
    // Wave w parks its WR x BN partial tile at red[w]; wave index is
    // ((pt * WM) + wm) * KS + wk.  The packed-weight kernel's pipeline is
    // small enough for the partial tiles to sit behind it, so a wave parks
    // its tile as soon as it is done; otherwise they reuse the pipeline
    // stages once every wave has left them.
    constexpr bool BEHIND = AP && C::RBEHIND;
    float* const redb = BEHIND ? pipe + C::NW * C::ST * SF : pipe;
    if constexpr (!BEHIND) __syncthreads();
    {
        float* red = redb + wave * C::WR * C::RS;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    red[(mi * 16 + (lane >> 4) * 4 + v) * C::RS + ni * 16 + (lane & 15)] = acc[mi][ni][v];
    }
    __syncthreads();

    float* __restrict__ yg = (float*)a.yptr;
    const int64_t out_plane = (int64_t)a.ho * a.wo;
    constexpr int UNITS = C::PT * BM * BN / 4;
    constexpr int ROW4 = BN / 4;
    constexpr int ITERS = (UNITS + C::NT - 1) / C::NT;
    constexpr int CH = ITERS < 8 ? ITERS : 8;   // units whose bias and slope are read at once
#pragma unroll
    for (int i0 = 0; i0 < ITERS; i0 += CH) {
        // Bias and slope of the next CH units before their stores (one wait
        // for earlier stores per CH units instead of one per unit).
        ChanEpi ce[CH];
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int u = (i0 + k) * C::NT + threadIdx.x;
            const int rem = u % (BM * ROW4);
            const int cog = cot * BM + rem / ROW4;
            ce[k] = chan_epi(a, (u < UNITS && cog < a.cout_g) ? g * a.cout_g + cog : 0);
        }
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            if (i0 + k >= ITERS) break;
            const int u = (i0 + k) * C::NT + threadIdx.x;
            if (UNITS % C::NT != 0 && u >= UNITS) break;
            const int p = u / (BM * ROW4);
            const int rem = u - p * (BM * ROW4);
            const int co = rem / ROW4;                // row within the workgroup's BM
            const int j = 4 * (rem - co * ROW4);
            const int w0 = (p * C::WM + co / C::WR) * C::KS;
            const float* src = redb + (co % C::WR) * C::RS + j;
            float4 s = *(const float4*)(src + w0 * C::WR * C::RS);
#pragma unroll
            for (int kk = 1; kk < C::KS; ++kk) {
                const float4 t = *(const float4*)(src + (w0 + kk) * C::WR * C::RS);
                s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
            }
            const int cog = cot * BM + co;
            const int pho = a.pt_vertical ? (thi * C::PT + p) * TH : thi * TH;
            const int pwo = a.pt_vertical ? twi * TW : (twi * C::PT + p) * TW;
            const int ho = pho + j / TW, wo = pwo + (j % TW);
            if (cog < a.cout_g && ho < a.ho) {
                const int cg = g * a.cout_g + cog;
                float v[4] = {bias_act_pre(a, s.x, ce[k]), bias_act_pre(a, s.y, ce[k]), bias_act_pre(a, s.z, ce[k]),
                              bias_act_pre(a, s.w, ce[k])};
                float* dst = yg + ((int64_t)n * a.out_total + a.out_off + cg) * out_plane + (int64_t)ho * a.wo + wo;
                if (a.vec_store && wo + 3 < a.wo) {
                    *(float4*)dst = make_float4(v[0], v[1], v[2], v[3]);
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (wo + t < a.wo) dst[t] = v[t];
                }
            }
        }
    }
}

// ------------------------------------------------------------ configs ---

struct CfgInfo {
    int bm, bn, tw, cw, kh, kw, nw, wm, ks, st, xs, asz, mi, steps, au;
    const void* fn;
    const void* fn_ap;   // packed-weight variant, or null
    int stage_floats(int ps, bool ap) const { return (ap ? 0 : asz) + cw * ps; }
    bool rbehind;
    int lds_floats(int ps, bool ap = false) const {
        const int pipe = nw * st * stage_floats(ps, ap);
        const int red = nw * (bm / wm) * (bn + 4);
        if (ap && rbehind) return pipe + red;   // the partial tiles sit behind the pipeline
        return pipe > red ? pipe : red;
    }
};

// AP: also the packed-weight kernel; AP_ONLY: only that one (the weight
// tiles of the OIHW kernel would not fit in LDS).
template <class C, bool AP = false, bool AP_ONLY = false>
CfgInfo info() {
    const void* ap = nullptr;
    const void* fn = nullptr;
    if constexpr (AP) ap = (const void*)igemm_f32_kernel<C, true>;
    if constexpr (!AP_ONLY) fn = (const void*)igemm_f32_kernel<C, false>;
    return CfgInfo{C::BM, C::BN, C::TW, C::CW, C::KH, C::KW, C::NW, C::WM, C::KS, C::ST, C::XS, C::ASZ,
                   C::MI, C::STEPS, C::AU, fn, ap, C::RBEHIND};
}

// Eight waves (two per SIMD) split K eight ways for the common case, or
// split the rows in two and K four ways for the wider tiles; four waves split
// over pixels when the group has too few input channels.
//                      BM  BN  TW  CW KH KW NW WM KS ST XS
using K3_M16   = Cfg<16,  64, 16,  4, 3, 3, 8, 1, 8, 2, 3>;
using K3_M32   = Cfg<32,  64, 16,  4, 3, 3, 8, 1, 8, 2, 3>;
using K3_M64   = Cfg<64,  64, 16,  4, 3, 3, 8, 2, 4, 2, 3>;
using K3W_M16  = Cfg<16,  64, 16,  4, 3, 3, 8, 1, 8, 2, 6>;   // wider patches (stride 2)
using K3W_M32  = Cfg<32,  64, 16,  4, 3, 3, 8, 1, 8, 2, 6>;
using K3W_M64  = Cfg<64,  64, 16,  4, 3, 3, 8, 2, 4, 1, 6>;
using K3P_M16  = Cfg<16,  64, 16,  4, 3, 3, 4, 1, 1, 2, 6>;   // few input channels: waves split pixels
using K3P_M32  = Cfg<32,  64, 16,  4, 3, 3, 4, 1, 1, 2, 6>;
using K1F_M32  = Cfg<32,  64, 64, 16, 1, 1, 8, 1, 8, 2, 4>;   // flattened 1x1: one row of h*w pixels
using K1F_M64  = Cfg<64,  64, 64, 16, 1, 1, 8, 2, 4, 2, 4>;
using K1F_M128 = Cfg<128, 64, 64, 16, 1, 1, 8, 2, 4, 1, 4>;
using K1FP_M16 = Cfg<16,  64, 64, 16, 1, 1, 4, 1, 1, 2, 4>;
using K1FP_M32 = Cfg<32,  64, 64, 16, 1, 1, 4, 1, 1, 2, 4>;
using K1_M32   = Cfg<32,  64, 16,  8, 1, 1, 8, 1, 8, 2, 8>;   // 1x1 with stride or padding
using K1_M64   = Cfg<64,  64, 16,  8, 1, 1, 8, 2, 4, 2, 8>;
using K5_M16   = Cfg<16,  64, 16,  4, 5, 5, 8, 1, 8, 1, 4>;
// Packed weights only: a wave owns all 64 output channels (4 row blocks per
// patch operand read, K split 8 ways); the OIHW form of its weight tiles
// would not fit in LDS.
using K3A_M64  = Cfg<64,  64, 16,  4, 3, 3, 8, 1, 8, 2, 3>;
// Few input channels on a small image: the four waves split K instead of
// the pixels, so a workgroup owns one 64-pixel tile and the grid has four
// times as many workgroups (a 32x32 image: 16 instead of 4).
using K3S_M16  = Cfg<16,  64, 16,  4, 3, 3, 4, 1, 4, 2, 6>;
using K3S_M32  = Cfg<32,  64, 16,  4, 3, 3, 4, 1, 4, 2, 6>;
// Large grids (at least two workgroups per compute unit with these): the
// waves split K fewer ways and cover more pixel sub-tiles instead, so each
// wave runs a longer K loop and the split-K reduction shrinks or vanishes.
// Measured on the batch-32 sweep: 3x3 d2 494 -> 453 us, 3x3 s2 255 -> 241
// us, 1x1 256 -> 512 148 -> 127 us; on small grids they leave CUs idle.
using K3L_M64   = Cfg<64,  64, 16,  4, 3, 3, 8, 2, 1, 2, 3>;
using K3WL_M64  = Cfg<64,  64, 16,  4, 3, 3, 8, 2, 2, 1, 6>;
using K1FL_M128 = Cfg<128, 64, 64, 16, 1, 1, 8, 2, 1, 1, 4>;

enum {
    C3_M16, C3_M32, C3_M64, C3W_M16, C3W_M32, C3W_M64, C3P_M16, C3P_M32,
    C1F_M32, C1F_M64, C1F_M128, C1FP_M16, C1FP_M32, C1_M32, C1_M64, C5_M16, C3A_M64, C3S_M16, C3S_M32,
    C3L_M64, C3WL_M64, C1FL_M128, NCFG
};

const CfgInfo& cfg(int i) {
    static const CfgInfo table[NCFG] = {
        info<K3_M16, true>(), info<K3_M32, true>(), info<K3_M64, true>(), info<K3W_M16>(), info<K3W_M32>(),
        info<K3W_M64>(),  info<K3P_M16>(),  info<K3P_M32>(),   info<K1F_M32>(),  info<K1F_M64>(),
        info<K1F_M128>(), info<K1FP_M16>(), info<K1FP_M32>(),  info<K1_M32>(),   info<K1_M64>(),
        info<K5_M16>(),   info<K3A_M64, true, true>(), info<K3S_M16>(), info<K3S_M32>(),
        info<K3L_M64>(),  info<K3WL_M64>(), info<K1FL_M128>(),
    };
    return table[i];
}

int patch_stride(int phw) {
    // Smallest stride >= phw with stride % 64 == 16: the four channel planes
    // of one operand fetch then start 16 banks apart.
    int s = ((phw + 63 - 16) / 64) * 64 + 16;
    if (s < phw) s += 64;
    return s;
}

struct Geom {
    int tw, th, ph, pwa, ps, shift;
};

// Patch geometry of a TH x TW output sub-tile (columns aligned down to 4).
Geom geom(const conv2d_params_t& p, const CfgInfo& c, bool flat) {
    Geom G;
    G.tw = c.tw;
    G.th = c.bn / c.tw;
    if (flat) {
        G.ph = 1; G.pwa = c.tw; G.shift = 0;
    } else {
        G.ph = (G.th - 1) * p.stride_h + (p.k_h - 1) * p.dilation_h + 1;
        const int span = (G.tw - 1) * p.stride_w + (p.k_w - 1) * p.dilation_w + 1;
        G.shift = ((-p.pad_left) % 4 + 4) % 4;
        G.pwa = (G.shift + span + 3) / 4 * 4;
    }
    G.ps = patch_stride(G.ph * G.pwa);
    return G;
}

// Workgroups of a launch with config c (pixel sub-tiles stacked the cheaper
// way, as the planner below picks).
int64_t grid_blocks(const Desc& d, const CfgInfo& c, bool flat) {
    const conv2d_params_t& p = d.p;
    const int pt = c.nw / (c.wm * c.ks);
    const int64_t co = p.n * (int64_t)p.groups * ((d.cout_g + c.bm - 1) / c.bm);
    if (flat) return co * ((d.ho * d.wo + c.tw * pt - 1) / (c.tw * pt));
    const int th = c.bn / c.tw;
    const int64_t v = (int64_t)((d.ho + th * pt - 1) / (th * pt)) * ((d.wo + c.tw - 1) / c.tw);
    const int64_t h = (int64_t)((d.ho + th - 1) / th) * ((d.wo + c.tw * pt - 1) / (c.tw * pt));
    return co * (v < h ? v : h);
}

}  // namespace

bool plan_igemm_f32(Desc& d) {
    const conv2d_params_t& p = d.p;
    const bool is3 = p.k_h == 3 && p.k_w == 3;
    const bool is1 = p.k_h == 1 && p.k_w == 1;
    const bool is5 = p.k_h == 5 && p.k_w == 5;
    const bool flat = is1 && p.stride_h == 1 && p.stride_w == 1 && p.pad_top == 0 && p.pad_left == 0 &&
                      p.pad_bottom == 0 && p.pad_right == 0;
    const int m = d.cout_g;
    int cands[6];
    int nc = 0;
    if (is3) {
        if (d.cin_g < 32) {
            // 64-pixel tiles of the whole batch and all groups; with few of
            // them the pixel-splitting tiles would leave most CUs idle.
            const long tiles = (long)p.n * p.groups * ((d.ho + 3) / 4) * ((d.wo + 15) / 16);
            if (tiles <= 256 && m <= 32) cands[nc++] = m <= 16 ? C3S_M16 : C3S_M32;
            cands[nc++] = m <= 16 ? C3P_M16 : C3P_M32;
        } else {
            cands[nc++] = m <= 16 ? C3_M16 : (m <= 32 ? C3_M32 : C3_M64);
            cands[nc++] = m <= 16 ? C3W_M16 : (m <= 32 ? C3W_M32 : C3W_M64);
        }
    } else if (flat) {
        if (d.cin_g < 128) cands[nc++] = m <= 16 ? C1FP_M16 : C1FP_M32;
        if (d.cin_g >= 64 || m > 32) cands[nc++] = m <= 32 ? C1F_M32 : (m <= 64 || m % 128 ? C1F_M64 : C1F_M128);
    } else if (is1) {
        cands[nc++] = m <= 32 ? C1_M32 : C1_M64;
    } else if (is5) {
        cands[nc++] = C5_M16;
    }
    // Large grids try the variant with fewer K slices first.
    for (int k = 0; k < nc; ++k) {
        const int l = cands[k] == C3_M64 ? C3L_M64 : cands[k] == C3W_M64 ? C3WL_M64
                      : cands[k] == C1F_M128 ? C1FL_M128 : -1;
        if (l < 0 || grid_blocks(d, cfg(l), flat) < 2 * (int64_t)device_cu_count()) continue;
        for (int j = nc; j > k; --j) cands[j] = cands[j - 1];
        cands[k] = l;
        ++nc;
        ++k;
    }
    for (int k = 0; k < nc; ++k) {
        const CfgInfo& c = cfg(cands[k]);
        const Geom G = geom(p, c, flat);
        // Where the packed-weight variant applies (same geometry as C3_M64),
        // keep the config that has it.
        if (cands[k] == C3L_M64 && G.ph * G.pwa == G.ps && p.w % 4 == 0) continue;
        if (c.cw * G.ph * G.pwa / 4 > 64 * c.xs) continue;            // patch units per lane
        if (c.cw * G.ph * G.pwa / 4 >= 65536 || G.ph * G.pwa >= 65536) continue;   // magic division range
        if ((int64_t)c.cw * p.h * p.w >= INT32_MAX / 2) continue;      // 32-bit patch offsets
        if ((int64_t)c.bm * d.cin_g * c.kh * c.kw >= INT32_MAX / 2) continue;
        const int lds = 4 * c.lds_floats(G.ps);
        if (lds > 160 * 1024) continue;
        d.cfg = cands[k];
        d.flatten_1x1 = flat;
        // Packed weights (bound weights only): the patch must have the
        // unit-major layout of the direct copies.
        // The 64-channel tiles have a packed-only variant in which a wave owns
        // all 64 rows (same tile and patch geometry, so the same launch grid).
        d.apack_bytes = 0;
        d.cfg_ap = -1;
        const int ca = cands[k] == C3_M64 ? C3A_M64 : cands[k];
        const CfgInfo& cp = cfg(ca);
        if (cp.fn_ap && !flat && G.ph * G.pwa == G.ps && p.w % 4 == 0 &&
            4 * cp.lds_floats(G.ps, true) <= 160 * 1024) {
            const int64_t co_tiles = (d.cout_g + cp.bm - 1) / cp.bm, chunks = (d.cin_g + cp.cw - 1) / cp.cw;
            d.cfg_ap = ca;
            d.apack_bytes = 4 * (int64_t)p.groups * co_tiles * cp.wm * chunks * cp.au * 256;
        }
        d.tile_h = G.th;
        d.tile_w = G.tw;
        d.lds_bytes = lds;
        // Stack a block's pixel sub-tiles along rows unless that wastes more.
        const int pt = c.nw / (c.wm * c.ks);
        if (flat || pt == 1) {
            d.pt_vertical = 0;
        } else {
            const long v = (long)((d.ho + G.th * pt - 1) / (G.th * pt)) * ((d.wo + G.tw - 1) / G.tw);
            const long h = (long)((d.ho + G.th - 1) / G.th) * ((d.wo + G.tw * pt - 1) / (G.tw * pt));
            d.pt_vertical = v <= h;
        }
        return true;
    }
    return false;
}

hipError_t launch_igemm_f32(const Desc& d, ConvArgs a, hipStream_t s, const void* wpacked) {
    const bool ap = wpacked && d.apack_bytes > 0 && d.cfg_ap >= 0 && (uintptr_t)a.xptr % 16 == 0 &&
                    (uintptr_t)wpacked % 16 == 0;
    const CfgInfo& c = cfg(ap ? d.cfg_ap : d.cfg);
    const conv2d_params_t& p = d.p;
    const Geom G = geom(p, c, d.flatten_1x1);
    if (d.flatten_1x1) {
        a.h = 1; a.w = p.h * p.w; a.ho = 1; a.wo = d.ho * d.wo;
    }
    const int pt = c.nw / (c.wm * c.ks);
    const int bth = d.pt_vertical ? G.th * pt : G.th;
    const int btw = d.pt_vertical ? G.tw : G.tw * pt;
    a.tiles_h = (a.ho + bth - 1) / bth;
    a.tiles_w = (a.wo + btw - 1) / btw;
    a.patch_h = G.ph;
    a.patch_w = G.pwa;
    a.patch_stride = G.ps;
    a.patch_shift = G.shift;
    a.div_patch_hw = make_fastdiv((uint32_t)(G.ph * G.pwa / 4));   // patch units per channel
    a.div_patch_w = make_fastdiv((uint32_t)(G.pwa / 4));           // patch units per row
    a.pt_vertical = d.pt_vertical;
    a.co_tiles = (d.cout_g + c.bm - 1) / c.bm;
    a.chunks = (d.cin_g + c.cw - 1) / c.cw;
    a.vec_store = (a.wo % 4 == 0) && ((uintptr_t)a.yptr % 16 == 0);
    // Direct global->LDS copies need the unit-major layout to be the tile
    // layout (weight row stride K, patch plane stride patch_h*patch_w, which
    // must keep the four planes of an operand fetch 16 banks apart) and
    // 16-byte aligned sources.
    const int kdma = c.cw * c.kh * c.kw;
    a.dma = c.st == 2 && !d.flatten_1x1 && kdma % 4 == 0 && a_stride(kdma) == kdma &&
            G.ph * G.pwa == G.ps && p.w % 4 == 0 && (d.cin_g * c.kh * c.kw) % 4 == 0 &&
            (uintptr_t)a.xptr % 16 == 0 && (uintptr_t)a.wptr % 16 == 0;
    if (ap) {
        a.wptr = wpacked;
        a.dma = 1;
    }
    a.dv_co_tiles = make_divu32((uint32_t)a.co_tiles);
    a.dv_groups = make_divu32((uint32_t)a.groups);
    a.dv_tiles_w = make_divu32((uint32_t)a.tiles_w);
    a.dv_tiles_h = make_divu32((uint32_t)a.tiles_h);
    const uint64_t blocks = (uint64_t)a.co_tiles * a.groups * a.tiles_h * a.tiles_w * a.n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0xFFFFFFFFull) return hipErrorInvalidConfiguration;
    a.num_blocks = (uint32_t)blocks;
    const void* fn = ap ? c.fn_ap : c.fn;
    const int lds = ap ? 4 * c.lds_floats(G.ps, true) : d.lds_bytes;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
    }
    void* args[] = {&a};
    return hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(c.nw * 64), args, lds, s);
}

namespace {

// Fragment-order weights: element i of dst is, with i = ((((g * T + tile) *
// chunks + kc) * AU + u) * 64 + lane) * 4 + e and f = 4u + e, the A operand of
// MFMA step t = f % STEPS of row block mi = f / STEPS that lane `lane` feeds
// for chunk kc of output tile `tile` (WR channels) of group g: output channel
// tile*WR + 16*mi + lane%16, input channel kc*CW + 4*(t % (CW/4)) + lane/16,
// tap t / (CW/4); zero past the group's channels and for f >= MI*STEPS.
__global__ __launch_bounds__(256) void pack_igemm_f32_kernel(const float* __restrict__ w, float* __restrict__ dst,
                                                             int64_t total, int cin_g, int cout_g, int khw, int cw,
                                                             int wr, int mi_n, int steps, int au, int chunks,
                                                             int tiles_g) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int e = (int)(i & 3), lane = (int)((i >> 2) & 63);
    int64_t r = i >> 8;
    const int u = (int)(r % au);
    r /= au;
    const int kc = (int)(r % chunks);
    r /= chunks;
    const int tile = (int)(r % tiles_g);
    const int g = (int)(r / tiles_g);
    const int f = 4 * u + e;
    float v = 0.0f;
    if (f < mi_n * steps) {
        const int mi = f / steps, t = f % steps;
        const int rs = t / (cw / 4), q = t % (cw / 4);
        const int row = tile * wr + mi * 16 + (lane & 15);
        const int ch = kc * cw + 4 * q + (lane >> 4);
        if (row < cout_g && ch < cin_g) v = w[((int64_t)(g * cout_g + row) * cin_g + ch) * khw + rs];
    }
    dst[i] = v;
}

}  // namespace

hipError_t pack_igemm_f32_weights(const Desc& d, const void* w, void* dst, hipStream_t s) {
    if (d.apack_bytes <= 0 || d.cfg_ap < 0) return hipErrorInvalidValue;
    const CfgInfo& c = cfg(d.cfg_ap);
    const int co_tiles = (d.cout_g + c.bm - 1) / c.bm, chunks = (d.cin_g + c.cw - 1) / c.cw;
    const int64_t total = d.apack_bytes / 4;
    const uint64_t blocks = (uint64_t)(total + 255) / 256;
    if (blocks > 0x7FFFFFFFull) return hipErrorInvalidConfiguration;
    const float* src = (const float*)w;
    float* out = (float*)dst;
    int64_t tot = total;
    int cin_g = d.cin_g, cout_g = d.cout_g, khw = d.p.k_h * d.p.k_w, cw = c.cw, wr = c.bm / c.wm, mi = c.mi,
        steps = c.steps, au = c.au, nch = chunks, tiles_g = co_tiles * c.wm;
    void* args[] = {&src, &out, &tot, &cin_g, &cout_g, &khw, &cw, &wr, &mi, &steps, &au, &nch, &tiles_g};
    return hipLaunchKernel((const void*)pack_igemm_f32_kernel, dim3((uint32_t)blocks), dim3(256), args, 0, s);
}

}  // namespace conv2d
