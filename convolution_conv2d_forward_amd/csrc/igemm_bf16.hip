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
//   patch    [group-of-8][patch row][patch column]    (one cell each)
// K runs tap-major inside a chunk of CC = 8*G input channels; an MFMA operand
// is one 16-byte LDS read and 16 lanes of a read touch 16 consecutive cells.
// K slots past the last tap (when taps*G is not a multiple of 4) read a
// block of zero cells instead of stored zeros.
//
// Copy path.  The weights are re-laid once per call (pack kernel below) into
// exactly the LDS image of each (output-channel tile, channel chunk), so a
// chunk's weights move with direct global->LDS loads (no registers, no
// transposition).  The NCHW input is transposed on the fly: a lane loads 8
// channels x 8 pixels (eight 16-byte row loads from wave-uniform plane
// pointers), permutes them in registers and writes eight 16-byte cells.
// Patch rows hold whole 8-pixel vectors (the row starts at the 8-aligned
// input column below the tile's first one), so no cell write needs a range
// check; vectors entirely outside the image are pad cells written once per
// stage.  Stride-2 patches keep even and odd columns in separate halves of a
// row, so a stride-2 read of 16 output pixels is still 16 consecutive cells.
// The row and plane strides are chosen on the host to spread the cell writes
// over the LDS banks.
//
// Pipeline: eight waves, two per SIMD, 64 x 64 wave tiles; two LDS stages,
// the copy of chunk c+1 issued at the start of chunk c, its rows transposed
// into the free stage after chunk c's MFMAs; one barrier per chunk.
// The epilogue adds the bias, applies the activation, rounds to bf16 and
// writes channel out_off + g*cout_g + co of a buffer with out_total channels
// (ConcatFusedTail), 4 pixels of a row per 8-byte store.
#include "device_common.h"

namespace conv2d {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int cgcd(int a, int b) { return b == 0 ? a : cgcd(b, a % b); }

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
    // Stored (tap, group) slots: taps*G rounded up so the image is whole 1 KB pieces.
    static constexpr int SQ = 64 / cgcd(BM, 64);
    static constexpr int TGA = (KHW * G + SQ - 1) / SQ * SQ;
    static constexpr int ACELLS = TGA * BM;            // 16-byte cells of a chunk's weight image
    static constexpr int DMAR = ACELLS / 64;           // 1 KB wave copies per weight image
    static constexpr int ZCELLS = 16 * MI;             // zero cells read by K slots past TGA
    static_assert(CC % 8 == 0 && TGA <= 4 * STEPS, "K steps cover the stored slots");
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

// Input task of lane slot u (= lane + 64*i) of wave w: the tasks of a chunk
// are dealt to the waves in equal contiguous runs.  -1 = none.
__host__ __device__ inline int task_of(int w, int u, int tasks, int nw) {
    const int per = (tasks + nw - 1) / nw;
    const int v = w * per + u;
    return (u < per && v < tasks) ? v : -1;
}

// Cell of patch column pc inside its row (stride-2 patches: evens, then odds).
__host__ __device__ inline int col_cell(int pc, int half, bool split) {
    return split ? (pc & 1) * half + (pc >> 1) : pc;
}

// Direct global->LDS copy of 16 bytes per lane: lane l writes lds_base + 16*l
// (lds_base wave-uniform).  Issued as inline assembly so that the compiler
// does not order every later LDS read of the workgroup behind it (it cannot
// tell that the reads go to the other stage); the kernel's own s_waitcnt
// before the barrier is what orders the copy.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(const void* src, const uint4* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m)
                 : "memory", "m0");
#endif
}
#pragma clang diagnostic pop

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
    const int shift = a.patch_shift;                         // 8-aligned patch start: iw_lo - shift
    const int iw8 = wo0 * a.stride_w - a.pad_left - shift;  // input column of patch column 0
    const int PH = a.patch_h;
    const int nvr = a.patch_stride;                          // 8-pixel vectors per patch row
    const int RS = a.lds_rs, PL = a.lds_plane, HALF = a.col_half;
    const int scells = C::ACELLS + G * PL;                   // cells per stage
    const int HW = a.h * a.w;

    uint4* const st0 = lds;
    uint4* const st1 = lds + scells;
    uint4* const zero = lds + 2 * scells;                    // C::ZCELLS zero cells

    const char* __restrict__ xg = (const char*)a.xptr +
                                  2 * ((int64_t)n * a.in_total + a.in_off + (int64_t)g * a.cin_g) * HW;
    const char* __restrict__ wp =
        (const char*)a.wptr + 16 * (int64_t)(g * a.co_tiles + cot) * a.chunks * C::ACELLS;
    const uint32_t padb = __bfloat16_as_ushort(f32_to_bf16(a.pad_value));
    const uint32_t pad2 = padb | (padb << 16);

    // ---- per-thread input tasks ----
    int tcell[C::XS];   // cell (in the patch part of a stage) of the vector's first pixel; -1 = no task
    int toff[C::XS];    // byte offset of the vector in the task's first channel plane; -1 = outside the image
#pragma unroll
    for (int i = 0; i < C::XS; ++i) {
        const int v = task_of(wave, lane + 64 * i, G * PH * nvr, C::NW);
        tcell[i] = -1; toff[i] = -1;
        if (v >= 0) {
            int vc, row, gg;
            input_task(v, nvr, PH, vc, row, gg);
            const int ih = ih0 + row, iw = iw8 + 8 * vc;
            tcell[i] = gg * PL + row * RS + (C::SD ? 4 * vc : 8 * vc);
            if ((unsigned)ih < (unsigned)a.h && iw >= 0 && iw < a.w) toff[i] = 2 * (8 * gg * HW + ih * a.w + iw);
        }
    }
    // Buffer over the group's input channels (byte size < 2^31, checked when
    // planning).  tvo = per-lane byte offset; 2^31 for lanes that load
    // nothing, so that offset + channel offset stays past the buffer.
    const __amdgpu_buffer_rsrc_t xrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)xg, (short)0, 2 * a.cin_g * HW, 0x00020000);
    int tvo[C::XS];
#pragma unroll
    for (int i = 0; i < C::XS; ++i) tvo[i] = toff[i] >= 0 ? toff[i] : INT32_MIN;
    // Cell of pixel p of a task's vector, relative to tcell.
    auto pcell = [&](int p) __attribute__((always_inline)) { return C::SD ? (p & 1) * HALF + (p >> 1) : p; };

    // Zero cells, and pad cells of vectors outside the image in both stages
    // (no chunk writes them again).
    for (int e = tid; e < C::ZCELLS; e += C::NT) zero[e] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < C::XS; ++i)
        if (tcell[i] >= 0 && toff[i] < 0) {
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                st0[C::ACELLS + tcell[i] + pcell(p)] = make_uint4(pad2, pad2, pad2, pad2);
                st1[C::ACELLS + tcell[i] + pcell(p)] = make_uint4(pad2, pad2, pad2, pad2);
            }
        }

    // Chunk kc's weight image -> stage ast (direct to LDS).
    auto dma_w = [&](int kc, uint4* ast) __attribute__((always_inline)) {
        const char* src = wp + 16 * ((int64_t)kc * C::ACELLS + lane);
#pragma unroll
        for (int k = 0; k < (C::DMAR + C::NW - 1) / C::NW; ++k) {
            const int r = wave + C::NW * k;
            if (r < C::DMAR) copy16_to_lds(src + 1024 * r, ast + 64 * r);
        }
    };
    // Chunk kc's input rows -> registers xr.  Unconditional buffer loads:
    // lanes without an in-image vector, and channels past the group's last
    // one, read beyond the buffer and get zeros without touching memory (no
    // per-lane branches, so no register merges that would make the compiler
    // hold later LDS reads behind these loads).
    auto load_row = [&](int kc, uint4 (&xr)[C::XS][8], int j) __attribute__((always_inline)) {
        const int i = j / 8, t = j % 8;
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xrs, tvo[i] + 2 * (kc * C::CC + t) * HW, 0, 0);
        xr[i][t] = make_uint4(v.x, v.y, v.z, v.w);
    };
    auto load_x = [&](int kc, uint4 (&xr)[C::XS][8]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 8 * C::XS; ++j) load_row(kc, xr, j);
    };
    // Registers -> LDS: 8 channels x 8 pixels of task i become 8 cells of 8 channels.
    auto store_task = [&](const uint4 (&xr)[C::XS][8], uint4* bst, int i) __attribute__((always_inline)) {
        if (toff[i] >= 0) {
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                uint32_t d[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint4 lo = xr[i][2 * k], hi = xr[i][2 * k + 1];
                    const uint32_t wl = (p >> 1) == 0 ? lo.x : (p >> 1) == 1 ? lo.y : (p >> 1) == 2 ? lo.z : lo.w;
                    const uint32_t wh = (p >> 1) == 0 ? hi.x : (p >> 1) == 1 ? hi.y : (p >> 1) == 2 ? hi.z : hi.w;
                    d[k] = (p & 1) ? ((wl >> 16) | (wh & 0xffff0000u)) : ((wl & 0xffffu) | (wh << 16));
                }
                bst[tcell[i] + pcell(p)] = make_uint4(d[0], d[1], d[2], d[3]);
            }
        }
    };
    auto store_x = [&](const uint4 (&xr)[C::XS][8], uint4* bst) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < C::XS; ++i) store_task(xr, bst, i);
    };

    // ---- operand offsets (cells) ----
    // Step s, lane group q = lane/16 supplies K slot tg = 4s + q: tap tg / G,
    // channel group tg % G.  A row co = wm*WR + mi*16 + lane%16; B pixel
    // j = wn*WC + ni*16 + lane%16.
    const int q = lane >> 4, l16 = lane & 15;
    int b_lane[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
        const int j = wn * C::WC + ni * 16 + l16;
        const int jr = j / TW, jc = j % TW;
        b_lane[ni] = jr * a.stride_h * RS + (C::SD ? jc : jc * a.stride_w);
    }
    int b_step[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        const int tg = 4 * s + q;
        int tap = tg / G;
        const int gg = tg - (tg / G) * G;
        if (tap >= KHW) tap = 0;     // K padding: zero weights, finite inputs of tap 0
        const int r = tap / KW, sc = tap - (tap / KW) * KW;
        const int cdx = shift + sc * a.dilation_w;
        b_step[s] = C::ACELLS + gg * PL + r * a.dilation_h * RS + (C::SD ? (cdx & 1) * HALF + (cdx >> 1) : cdx);
    }

    f32x4 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // The MFMAs of one chunk; after step s, between(s) runs (the
    // transposition of the next chunk's rows goes there, so that its VALU and
    // LDS writes issue while the matrix core works).
    auto compute = [&](const uint4* st, auto&& between) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            const int tg = 4 * s + q;
            const uint4* as = (4 * s + 3 < C::TGA || tg < C::TGA) ? st + tg * BM + wm * C::WR + l16 : zero + l16;
            const uint4* bs = st + b_step[s];
            bf16x8 av[MI], bv[NI];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) av[mi] = __builtin_bit_cast(bf16x8, as[16 * mi]);
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) bv[ni] = __builtin_bit_cast(bf16x8, bs[b_lane[ni]]);
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv[ni], av[mi], acc[mi][ni], 0, 0, 0);
            between(s);
        }
    };
    auto nothing = [](int) {};

    // ---- main loop ----
    // Two LDS stages: chunk c computes from stage c%2 while chunk c+1's
    // weight image lands in the other one and its rows (loaded into
    // registers one step earlier) are transposed into it between chunk c's
    // MFMA steps.  Input rows are loaded two chunks ahead into two register
    // sets: rows of chunk k live in R[k%2].  Steady-state steps load and wait
    // unconditionally, so the compiler sees nothing outstanding at the top of
    // a step.  Loads complete in issue order, so a wait for "at most n
    // outstanding" leaves exactly the newest n in flight: right after a
    // step's copies are issued, waiting down to (this step's weight copies +
    // row loads) means the previous step's row loads have landed.  A wave
    // issues DMAR/NW or one more weight copies; the wait counts the smaller
    // number, which at worst also waits for one of this step's copies.
    constexpr int VMX = 8 * C::XS;                 // row loads per chunk and thread
    constexpr int DMA_LO = C::DMAR / C::NW;        // fewest weight copies per wave and chunk
    static_assert(VMX + DMA_LO < 64, "vmcnt field");
    auto vm_wait = [](auto n) __attribute__((always_inline)) {
        constexpr int N = decltype(n)::value;
        __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));   // vmcnt(N) only
    };
    using vm_rows_prev = std::integral_constant<int, VMX + DMA_LO>;
    using vm_rows_new = std::integral_constant<int, VMX>;
    using vm_copies = std::integral_constant<int, DMA_LO>;
    using vm_none = std::integral_constant<int, 0>;
    const int nch = a.chunks;
    uint4 R0[C::XS][8], R1[C::XS][8];
    auto stage = [&](int k) __attribute__((always_inline)) { return (k & 1) ? st1 : st0; };
    // Between the MFMA steps of chunk c: the row loads of chunk c+2 are
    // issued a few at a time over steps 0..S_ROWS (issued all at once, they
    // fill the memory unit's queue and stall the wave, MFMAs included), and
    // after step S_ROWS the rows of chunk c+1, loaded during the previous
    // chunk, are waited for and transposed into the free stage.
    constexpr int S_ROWS = STEPS >= 3 ? STEPS - 2 : STEPS - 1;
    auto interleave = [&](const uint4 (&rs)[C::XS][8], uint4* bst, int kl, uint4 (*rl)[C::XS][8], auto n)
        __attribute__((always_inline)) {
        return [&rs, bst, kl, rl, &store_task, &load_row, &vm_wait, n](int s) __attribute__((always_inline)) {
            if (rl) {
#pragma unroll
                for (int j = 0; j < VMX; ++j)
                    if (j * (S_ROWS + 1) / VMX == s) load_row(kl, *rl, j);
            }
            if (s == S_ROWS) {
                vm_wait(n);
#pragma unroll
                for (int i = 0; i < C::XS; ++i) store_task(rs, bst, i);
            }
        };
    };
    // Step c with chunk c+2 to prefetch: rows of c+1 are in rs, rows of c+2 go to rl.
    auto step_full = [&](int c, uint4 (&rl)[C::XS][8], const uint4 (&rs)[C::XS][8]) __attribute__((always_inline)) {
        dma_w(c + 1, stage(c + 1));
        compute(stage(c), interleave(rs, stage(c + 1) + C::ACELLS, c + 2, &rl, vm_rows_prev{}));   // rows of c+1 landed
        vm_wait(vm_rows_new{});                  // chunk c+1's weight image has landed
        __syncthreads();
    };
    // Step c, c+1 being the last chunk.
    auto step_last = [&](int c, const uint4 (&rs)[C::XS][8]) __attribute__((always_inline)) {
        dma_w(c + 1, stage(c + 1));
        compute(stage(c), interleave(rs, stage(c + 1) + C::ACELLS, 0, nullptr, vm_copies{}));   // rows of c+1 landed
        vm_wait(vm_none{});
        __syncthreads();
    };
    dma_w(0, st0);
    load_x(0, R0);
    __builtin_amdgcn_s_waitcnt(0);
    store_x(R0, st0 + C::ACELLS);
    if (nch > 1) load_x(1, R1);
    __syncthreads();
    int c = 0;
    for (; c + 3 < nch; c += 2) {
        step_full(c, R0, R1);
        step_full(c + 1, R1, R0);
    }
    // c is even: rows of chunk c+1 (if any) are in R1.
    if (c + 2 < nch) {           // three chunks left
        step_full(c, R0, R1);
        step_last(c + 1, R0);
        c += 2;
    } else if (c + 1 < nch) {    // two chunks left
        step_last(c, R1);
        c += 1;
    }
    compute(stage(c), nothing);
    __syncthreads();

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
// LDS image [tap*G + group-of-8][BM][8 channels] with tga slots, zero where
// the tap, the output channel or the input channel lies past the filter.
__global__ __launch_bounds__(256) void pack_weights_bf16(const uint16_t* __restrict__ w, uint4* __restrict__ out,
                                                         int64_t total, int bm, int tga, int gq, int cc, int khw,
                                                         int chunks, int co_tiles, int cin_g, int cout_g) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    int64_t rest = idx;
    const int co = rest % bm; rest /= bm;
    const int tg = rest % tga; rest /= tga;
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
    int bm, bn, tw, cc, kh, kw, sd, xs, nt, nw, tga, acells, zcells;
    const void* fn;
};

template <class C>
CfgInfo info() {
    return CfgInfo{C::BM, C::BN, C::TW, C::CC, C::KH, C::KW, C::SD ? 1 : 0, C::XS, C::NT, C::NW, C::TGA,
                   C::ACELLS, C::ZCELLS, (const void*)igemm_bf16_kernel<C>};
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
    int ph, shift, nvr, half, rs, plane;
};

// LDS cell-write cost of one chunk's input tasks for row stride rs and
// plane stride pl: per 16-lane pass of a 16-byte write, the largest number
// of lanes that fall on the same 16-byte bank group.
int64_t write_cost(const Geom& G, const CfgInfo& c, int rs, int pl) {
    const int tasks = (c.cc / 8) * G.ph * G.nvr;
    const int per = (tasks + c.nw - 1) / c.nw;
    int64_t cost = 0;
    for (int w = 0; w < c.nw; ++w)
        for (int base = 0; base < per; base += 16)
            for (int p = 0; p < 8; ++p) {
                int hits[16] = {0};
                int worst = 0;
                for (int l = 0; l < 16; ++l) {
                    const int v = task_of(w, base + l, tasks, c.nw);
                    if (v < 0) continue;
                    int vc, row, gg;
                    input_task(v, G.nvr, G.ph, vc, row, gg);
                    const int cell = gg * pl + row * rs + col_cell(8 * vc + p, G.half, c.sd != 0);
                    const int h = ++hits[cell & 15];
                    worst = h > worst ? h : worst;
                }
                cost += worst;
            }
    return cost;
}

// Patch geometry; the plane stride is kept <= max_plane.  Returns false if
// even the densest layout does not fit.
bool geom(const conv2d_params_t& p, const CfgInfo& c, bool flat, int max_plane, Geom& G) {
    const int th = c.bn / c.tw;
    int span;
    if (flat) {
        G.ph = 1; G.shift = 0; span = c.tw;
    } else {
        G.ph = (th - 1) * p.stride_h + (p.k_h - 1) * p.dilation_h + 1;
        span = (c.tw - 1) * p.stride_w + (p.k_w - 1) * p.dilation_w + 1;
        G.shift = ((-p.pad_left) % 8 + 8) % 8;
    }
    G.nvr = (G.shift + span + 7) / 8;
    G.half = 4 * G.nvr;
    const int rs0 = 8 * G.nvr;
    if ((int64_t)G.ph * rs0 > max_plane) return false;
    // Smallest write cost over row strides rs0..rs0+15 and plane padding 0..15.
    int64_t best = -1;
    G.rs = rs0;
    G.plane = G.ph * rs0;
    for (int rs = rs0; rs < rs0 + 16; ++rs)
        for (int pad = 0; pad < (c.cc > 8 ? 16 : 1); ++pad) {
            const int pl = G.ph * rs + pad;
            if (pl > max_plane) continue;
            const int64_t cost = write_cost(G, c, rs, pl);
            if (best < 0 || cost < best || (cost == best && pl < G.plane)) {
                best = cost; G.rs = rs; G.plane = pl;
            }
        }
    return true;
}

int64_t wpack_cells(const Desc& d, const CfgInfo& c) {
    const int64_t co_tiles = (d.cout_g + c.bm - 1) / c.bm;
    const int64_t chunks = (d.cin_g + c.cc - 1) / c.cc;
    return (int64_t)d.p.groups * co_tiles * chunks * c.acells;
}

constexpr int kLdsMax = 160 * 1024;

}  // namespace

bool plan_igemm_bf16(Desc& d) {
    const conv2d_params_t& p = d.p;
    const bool is3 = p.k_h == 3 && p.k_w == 3;
    const bool flat = p.k_h == 1 && p.k_w == 1 && p.stride_h == 1 && p.stride_w == 1 && p.pad_top == 0 &&
                      p.pad_left == 0 && p.pad_bottom == 0 && p.pad_right == 0;
    // Input rows are read as 16-byte vectors of 8 pixels.
    if ((flat ? (int64_t)p.h * p.w : p.w) % 8 != 0) return false;
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
        const int gq = c.cc / 8;
        const int max_plane = (kLdsMax - 16 * c.zcells - 2 * 16 * c.acells) / (2 * 16 * gq);
        Geom G;
        if (max_plane <= 0 || !geom(p, c, flat, max_plane, G)) continue;
        if (gq * G.ph * G.nvr > c.xs * c.nt) continue;                  // input tasks per thread
        if (2 * (int64_t)d.cin_g * p.h * p.w >= INT32_MAX) continue;      // 32-bit byte offsets in a group
        if (wpack_cells(d, c) * 16 >= ((int64_t)1 << 40)) continue;
        d.cfg = cands[k];
        d.flatten_1x1 = flat;
        d.tile_w = c.tw;
        d.tile_h = c.bn / c.tw;
        d.lds_bytes = 16 * (2 * (c.acells + gq * G.plane) + c.zcells);
        d.wpack_bytes = wpack_cells(d, c) * 16;
        d.g_ph = G.ph; d.g_span = 8 * G.nvr; d.g_shift = G.shift; d.g_nvr = G.nvr;
        d.g_rs = G.rs; d.g_plane = G.plane; d.g_half = G.half;
        return true;
    }
    return false;
}

hipError_t pack_igemm_bf16_weights(const Desc& d, const void* w, void* dst, hipStream_t s) {
    const CfgInfo& c = cfg(d.cfg);
    const conv2d_params_t& p = d.p;
    const int64_t total = d.wpack_bytes / 16;
    if (total == 0) return hipSuccess;
    const void* w_src = w;
    uint4* pk = (uint4*)dst;
    int64_t tot = total;
    int bm = c.bm, tga = c.tga, gq = c.cc / 8, cc = c.cc, khw = p.k_h * p.k_w,
        chunks = (d.cin_g + c.cc - 1) / c.cc, co_tiles = (d.cout_g + c.bm - 1) / c.bm, cin_g = d.cin_g,
        cout_g = d.cout_g;
    void* pargs[] = {&w_src, &pk, &tot, &bm, &tga, &gq, &cc, &khw, &chunks, &co_tiles, &cin_g, &cout_g};
    return hipLaunchKernel((const void*)pack_weights_bf16, dim3((uint32_t)((total + 255) / 256)), dim3(256), pargs,
                           0, s);
}

hipError_t launch_igemm_bf16(const Desc& d, ConvArgs a, hipStream_t s, const void* packed, void* pack_buf) {
    // The kernel reads input rows as 16-byte vectors.
    if ((uintptr_t)a.xptr % 16 != 0) return launch_direct(d, a, s);
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
    if (d.wpack_bytes != wpack_cells(d, c) * 16) return hipErrorInvalidValue;
    // 1) weights -> per-chunk LDS images (unless they are bound, packed once)
    if (!packed) {
        if (!pack_buf) return hipErrorInvalidValue;
        const hipError_t e = pack_igemm_bf16_weights(d, a.wptr, pack_buf, s);
        if (e != hipSuccess) return e;
        packed = pack_buf;
    }

    // 2) the convolution
    a.wptr = packed;
    if (d.lds_bytes > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(c.fn, hipFuncAttributeMaxDynamicSharedMemorySize, d.lds_bytes);
        if (e != hipSuccess) return e;
    }
    void* args[] = {&a};
    return hipLaunchKernel(c.fn, dim3((uint32_t)blocks), dim3(c.nt), args, d.lds_bytes, s);
}

}  // namespace conv2d
