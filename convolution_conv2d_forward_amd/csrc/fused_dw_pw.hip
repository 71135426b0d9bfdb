// Fused depthwise kxk -> pointwise 1x1 (the FusedDwPw step of the yscv
// "ONNX CPU Kernels" page, section "Hot kernel paths": the depthwise rows
// feed the pointwise GEMM from on-chip memory, so the depthwise output is
// never written to main memory).
//
// Workgroup tile: one image, TH output rows of full width, COT (32 or 64)
// pointwise output channels.  The depthwise channels (= the pointwise K) are
// walked in chunks of KC = 32:
//   1. the chunk's input rows (TH rows of output need IR input rows, halo
//      included) are loaded into registers one chunk ahead and written to an
//      LDS tile whose pad rows and columns hold the depthwise pad_value
//      (written once: they are the same for every chunk); the chunk's
//      pointwise weights go to LDS as [k][co] at the same time;
//   2. the depthwise conv reads that tile (lane l of a 16-lane unit computes
//      columns l, l+16, l+32, l+48 of one output row, so the lanes of a read
//      touch consecutive LDS words), adds its bias, applies its activation and
//      writes the result to LDS as the GEMM's A operand, [k][pixel];
//   3. Y[co, pixel] += W_pw[co, k] * D[k, pixel] runs on the fp32 matrix
//      cores (v_mfma_f32_16x16x4f32, the pixel fragment as first operand so a
//      lane ends up holding 4 consecutive pixels of one output channel).
// The depthwise result and the pointwise weights are double-buffered, so a
// chunk costs two workgroup barriers.  The epilogue adds the pointwise bias,
// applies its activation and stores 16-byte vectors into channel
// out_off + co of a buffer with out_total channels (ConcatFusedTail).
// With more output channels than one tile holds, each channel tile redoes the
// depthwise conv of its pixels (the planner counts that).
#include "device_common.h"

namespace conv2d {

namespace {

constexpr int kT = 512;
constexpr int kWaves = kT / 64;
constexpr int KC = 32;        // depthwise channels per chunk
constexpr int NPW = KC * 64 / kT;   // pointwise weights per thread and chunk (KC x up to 64 channels)
constexpr int KHW_MAX = 25;   // depthwise windows up to 5x5
constexpr int NDW = (KC * KHW_MAX + kT - 1) / kT;   // depthwise weights per thread and chunk
constexpr int DWP = KC * KHW_MAX + 2 * KC;          // LDS floats of a chunk's depthwise weights, bias, slopes

struct DwPwArgs {
    ConvArgs dw, pw;
    int32_t th, tiles_h, co_tiles, cot;
    int32_t ir;            // input rows per tile
    int32_t xoff;          // LDS column of image column 0 (a multiple of 4, >= pad_left)
    int32_t xw;            // LDS row stride of the input tile
    int32_t xs_plane;      // LDS floats per channel of the input tile
    int32_t npx, nf;       // pixels of a tile (th * wo) and 16-pixel fragments
    int32_t es_stride;     // LDS floats per channel of the depthwise result (= 16 mod 32)
    int32_t cop;           // LDS row stride of the pointwise weight chunk (= 16 mod 32)
    uint32_t num_blocks;
    DivU32 dv_co_tiles, dv_tiles_h;
    FastDiv div_cg, div_th;   // 64-column groups per row; output rows per tile
    FastDiv div_q4, div_rp;   // 4-column groups per output row; output row pairs per tile
};

// Smallest s >= n with s % 32 == 16: four rows s apart start 16 or 48 banks
// apart, so a 4 x 16 operand fetch hits 64 distinct banks.
__host__ __device__ inline int stride16(int n) {
    const int s = n / 32 * 32 + 16;
    return s < n ? s + 32 : s;
}

// One chunk's global data, held in registers between its loads and its LDS
// writes (loaded two chunks ahead).  VEC: the input moves as 16-byte vectors.
template <bool VEC, int NX>
struct ChunkRegs {
    typename std::conditional<VEC, f32x4, float>::type x[NX];
    float pw[NPW];
    float dwt[NDW];
    float bias, slope;
};

// KH/KW/SS > 0: fixed 3x3 window with stride SS and dilation 1 (the reads are
// constant offsets); 0: any window up to 5x5 with the descriptor's stride and
// dilation.  MI: 16-channel output fragments (COT / 16).  NJ: pixel fragments
// per wave.  VEC/NX: input loads per thread and chunk (16-byte vectors or
// single floats).
template <int KH, int KW, int SS, int MI, int NJ, bool VEC, int NX>
__global__ __launch_bounds__(kT) void fused_dw_pw_kernel(DwPwArgs f) {
    extern __shared__ __align__(16) float lds[];
    const ConvArgs& D = f.dw;
    const ConvArgs& P = f.pw;
    constexpr bool FIXED = KH > 0;
    const int kh = FIXED ? KH : D.k_h, kw = FIXED ? KW : D.k_w;
    const int khw = kh * kw;
    const int sh = FIXED ? SS : D.stride_h, sw = FIXED ? SS : D.stride_w;
    const int dh = FIXED ? 1 : D.dilation_h, dwl = FIXED ? 1 : D.dilation_w;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, l16 = lane & 15;

    uint32_t L = xcd_remap(blockIdx.x, f.num_blocks);
    uint32_t Q = divu(L, f.dv_co_tiles);
    const int cot = L - Q * f.co_tiles;
    L = Q; Q = divu(L, f.dv_tiles_h);
    const int tht = L - Q * f.tiles_h;
    const int n = Q;
    const int co0 = cot * f.cot;
    const int ho0 = tht * f.th;
    const int th_n = min(f.th, D.ho - ho0);                 // output rows of this tile
    const int ih0 = ho0 * sh - D.pad_top;                   // image row of tile input row 0
    const int C = D.c_out, W = D.w, H = D.h, WO = D.wo;
    const int64_t HW = (int64_t)H * W;
    const int nch = (C + KC - 1) / KC;

    float* xs = lds;                                        // [KC][ir][xw]
    float* es0 = xs + KC * f.xs_plane;                      // [KC][es_stride] x 2
    float* ws0 = es0 + 2 * KC * f.es_stride;                // [KC][cop] x 2
    float* dp0 = ws0 + 2 * KC * f.cop;                      // [KC][khw], bias[KC], slope[KC] x 2
    const float* __restrict__ xg = (const float*)D.xptr + ((int64_t)n * D.in_total + D.in_off) * HW;
    const float* __restrict__ wdw = (const float*)D.wptr;
    const float* __restrict__ wpw = (const float*)P.wptr;
    const float pv = D.pad_value;

    // Pad rows (outside the image) and pad columns of the input tile: the
    // same for every chunk, written once, one LDS row per thread.
    for (int rr = tid; rr < KC * f.ir; rr += kT) {
        const int row = rr % f.ir;
        float* dst = xs + rr * f.xw;
        if ((unsigned)(ih0 + row) >= (unsigned)H) {
            for (int col = 0; col < f.xw; ++col) dst[col] = pv;
        } else {
            for (int col = 0; col < f.xoff; ++col) dst[col] = pv;
            for (int col = f.xoff + W; col < f.xw; ++col) dst[col] = pv;
        }
    }

    // ---- chunk loads ----
    // Every load is issued unconditionally (elements outside the tile read a
    // valid address and are dropped when written to LDS), so each wave issues
    // the same loads in the same order for every chunk and the compiler's
    // waits before the LDS writes leave the next chunk's loads in flight.
    const int per_ch = VEC ? f.ir * (W >> 2) : f.ir * W;    // load units per channel
    const int units_x = KC * per_ch;
    using Regs = ChunkRegs<VEC, NX>;
    // Load unit u = tid + i*kT is the same (channel, row, column) of every
    // chunk: its offset in the chunk's first plane (ch*HW + row*W + col,
    // < KC*HW < 2^31) and its LDS offset are worked out once; -1 marks units
    // past the tile or on rows outside the image.  A unit's channel exists
    // when its offset is below (C - c0)*HW.
    int xoff_g[NX], xoff_l[NX];
#pragma unroll
    for (int i = 0; i < NX; ++i) {
        const int u = tid + i * kT;
        const int ch = u / per_ch, rem = u - ch * per_ch;
        int row, col;
        if (VEC) { row = rem / (W >> 2); col = 4 * (rem - row * (W >> 2)); }
        else { row = rem / W; col = rem - row * W; }
        const bool ok = u < units_x && (unsigned)(ih0 + row) < (unsigned)H;
        xoff_g[i] = ok ? ch * (int)HW + (ih0 + row) * W + col : -1;
        xoff_l[i] = ok ? ch * f.xs_plane + row * f.xw + f.xoff + col : -1;
    }
    auto load_x = [&](int c, Regs& R) __attribute__((always_inline)) {
        const int c0 = c * KC;
        // A chunk past the last channel (the loop's padding step) reads
        // element 0 of the first plane for every unit.
        const float* __restrict__ xc = xg + (c0 < C ? (int64_t)c0 * HW : 0);
        const int64_t lim = c0 < C ? (int64_t)(C - c0) * HW : 0;
        const int lim32 = lim < INT32_MAX ? (int)lim : INT32_MAX;
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int off = (unsigned)xoff_g[i] < (unsigned)lim32 ? xoff_g[i] : 0;
            if constexpr (VEC) R.x[i] = *(const f32x4*)(xc + off);
            else R.x[i] = xc[off];
        }
    };
    // The chunk's pointwise and depthwise weights, depthwise bias and slope.
    // The loaded values are not touched here: masking them now would make
    // the compiler wait for every load in flight, the next chunk's included.
    auto load_w = [&](int c, Regs& R) __attribute__((always_inline)) {
        const int c0 = c * KC;
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
            const int e = tid + i * kT;                     // k-major: e = k * 64 + co
            const int k = e >> 6, co = e & 63;
            const bool ok = co < f.cot && co0 + co < P.c_out && c0 + k < C;
            R.pw[i] = wpw[ok ? (int64_t)(co0 + co) * C + c0 + k : 0];
        }
#pragma unroll
        for (int i = 0; i < NDW; ++i) {
            const int e = tid + i * kT;                     // e = ch * khw + tap
            const bool ok = e < KC * khw && c0 * khw + e < C * khw;
            R.dwt[i] = wdw[ok ? (int64_t)c0 * khw + e : 0];
        }
        const bool okc = tid < KC && c0 + tid < C;
        const float* bsrc = D.bias ? D.bias : wdw;
        const float* ssrc = D.act == CONV_ACT_PRELU ? D.slope : wdw;
        R.bias = bsrc[okc && D.bias ? c0 + tid : 0];
        R.slope = ssrc[okc && D.act == CONV_ACT_PRELU ? (D.slope_count == 1 ? 0 : c0 + tid) : 0];
    };
    auto store_chunk = [&](int c, const Regs& R, float* ws, float* dp) __attribute__((always_inline)) {
        const int c0 = c * KC;
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            if (xoff_l[i] >= 0) {
                float* dst = xs + xoff_l[i];
                if constexpr (VEC) *(f32x4*)dst = R.x[i];
                else *dst = R.x[i];
            }
        }
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
            const int e = tid + i * kT;
            const int k = e >> 6, co = e & 63;
            const bool ok = co0 + co < P.c_out && c0 + k < C;
            if (co < f.cot) ws[k * f.cop + co] = ok ? R.pw[i] : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < NDW; ++i) {
            const int e = tid + i * kT;
            if (e < KC * khw) dp[e] = c0 * khw + e < C * khw ? R.dwt[i] : 0.0f;
        }
        if (tid < KC) {
            const bool okc = c0 + tid < C;
            dp[KC * KHW_MAX + tid] = okc && D.bias ? R.bias : 0.0f;
            dp[KC * KHW_MAX + KC + tid] = okc ? R.slope : 0.0f;
        }
    };

    f32x4 acc[MI][NJ];
#pragma unroll
    for (int m = 0; m < MI; ++m)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[m][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // ---- 2. depthwise into the GEMM operand ----
    // A thread unit is 16 lanes' worth of one (channel, output row, 64-column
    // group): lane l computes columns g*64 + l + 16v (v < 4), so the lanes of a
    // window read touch consecutive LDS words (no bank conflicts at stride 1).
    const int cgroups = (WO + 63) / 64;
    const int units = KC * f.th * cgroups * 16;
    const ActP da = act_params(D);
    // 3x3 stride 1 with pad_left 1 and whole 4-column groups: a unit is one
    // (channel, output row pair, 4 columns); each of its four input rows is
    // read once as float2 + float4 + float2 (the LDS column of output column
    // 4l sits at xoff + 4l, a multiple of 4) into a 6-column register window.
    const bool quad = FIXED && SS == 1 && KH == 3 && KW == 3 && D.pad_left == 1 && WO % 4 == 0;
    const int nq = WO >> 2, nrp = (f.th + 1) >> 1;
    const int units_q = KC * nrp * nq;
    auto depthwise_quad = [&](int c, float* es, const float* dp) __attribute__((always_inline)) {
        const int c0 = c * KC;
        for (int u = tid; u < units_q; u += kT) {
            const int rest = (int)fdiv((uint32_t)u, f.div_q4);      // ch * nrp + row pair
            const int l = u - rest * nq;
            const int ch = (int)fdiv((uint32_t)rest, f.div_rp);
            const int r0 = 2 * (rest - ch * nrp);
            if (r0 >= th_n) continue;
            const bool two = r0 + 1 < th_n;
            float o[2][4];
            if (c0 + ch < C) {
                float wv[9];
#pragma unroll
                for (int t = 0; t < 9; ++t) wv[t] = dp[ch * 9 + t];
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int v = 0; v < 4; ++v) o[m][v] = 0.0f;
                const float* base = xs + ch * f.xs_plane + r0 * f.xw + f.xoff + 4 * l;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (i == 3 && !two) break;
                    const float* rp = base + i * f.xw;
                    const float2 lo = *(const float2*)(rp - 2);
                    const float4 mid = *(const float4*)rp;
                    const float2 hi = *(const float2*)(rp + 4);
                    const float win[6] = {lo.y, mid.x, mid.y, mid.z, mid.w, hi.x};
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        const int r = i - m;                       // filter row feeding output row r0+m
                        if (r < 0 || r > 2) continue;
#pragma unroll
                        for (int s2 = 0; s2 < 3; ++s2)
#pragma unroll
                            for (int v = 0; v < 4; ++v) o[m][v] = fmaf(win[v + s2], wv[3 * r + s2], o[m][v]);
                    }
                }
                const float bb = dp[KC * KHW_MAX + ch];
                const float sl = D.act == CONV_ACT_PRELU ? dp[KC * KHW_MAX + KC + ch] : da.s;
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int v = 0; v < 4; ++v) o[m][v] = act_apply(o[m][v] + bb, sl, da.lo, da.hi);
            } else {
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int v = 0; v < 4; ++v) o[m][v] = 0.0f;   // past the last channel: zero weights too
            }
            float* dst = es + ch * f.es_stride + r0 * WO + 4 * l;
            *(float4*)dst = make_float4(o[0][0], o[0][1], o[0][2], o[0][3]);
            if (two) *(float4*)(dst + WO) = make_float4(o[1][0], o[1][1], o[1][2], o[1][3]);
        }
    };
    auto depthwise = [&](int c, float* es, const float* dp) __attribute__((always_inline)) {
        if (quad) {
            depthwise_quad(c, es, dp);
            return;
        }
        const int c0 = c * KC;
        for (int u = tid; u < units; u += kT) {
            const int l = u & 15;
            const int rest = u >> 4;
            const int rg = (int)fdiv((uint32_t)rest, f.div_cg);        // ch * th + r
            const int g = rest - rg * cgroups;
            const int ch = (int)fdiv((uint32_t)rg, f.div_th);
            const int r = rg - ch * f.th;
            if (r >= th_n) continue;
            const int col0 = g * 64 + l;
            float outv[4];
            if (c0 + ch < C) {
                float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                const float* base = xs + ch * f.xs_plane + r * sh * f.xw + f.xoff - D.pad_left + col0 * sw;
                const float* wch = dp + ch * khw;
                if constexpr (FIXED) {
#pragma unroll
                    for (int i = 0; i < KH; ++i)
#pragma unroll
                        for (int s2 = 0; s2 < KW; ++s2) {
                            const float wv = wch[i * KW + s2];
#pragma unroll
                            for (int v = 0; v < 4; ++v) a[v] = fmaf(base[i * f.xw + 16 * v * SS + s2], wv, a[v]);
                        }
                } else {
                    for (int i = 0; i < kh; ++i)
                        for (int s2 = 0; s2 < kw; ++s2) {
                            const float wv = wch[i * kw + s2];
                            const float* rp = base + i * dh * f.xw + s2 * dwl;
#pragma unroll
                            for (int v = 0; v < 4; ++v) a[v] = fmaf(rp[16 * v * sw], wv, a[v]);
                        }
                }
                const float bb = dp[KC * KHW_MAX + ch];
                const float sl = D.act == CONV_ACT_PRELU ? dp[KC * KHW_MAX + KC + ch] : da.s;
#pragma unroll
                for (int v = 0; v < 4; ++v) outv[v] = act_apply(a[v] + bb, sl, da.lo, da.hi);
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v) outv[v] = 0.0f;   // past the last channel: zero weights too
            }
            float* dst = es + ch * f.es_stride + r * WO;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (col0 + 16 * v < WO) dst[col0 + 16 * v] = outv[v];
        }
    };

    // ---- 3. pointwise on the matrix cores ----
    // The operands of k step t+1 are read from LDS while the MFMAs of step t run.
    // between(t) runs after the MFMAs of k step t are issued (the next
    // chunk's loads go there, so their address work and issue overlap the
    // matrix cores).
    auto pointwise = [&](const float* es, const float* ws, auto&& between) __attribute__((always_inline)) {
        float bv[2][MI], av[2][NJ];
        auto fetch = [&](int kq, int set) __attribute__((always_inline)) {
            const int kr = kq + q;
#pragma unroll
            for (int m = 0; m < MI; ++m) bv[set][m] = ws[kr * f.cop + m * 16 + l16];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int fj = wave + kWaves * j;
                av[set][j] = fj < f.nf ? es[kr * f.es_stride + fj * 16 + l16] : 0.0f;
            }
        };
        fetch(0, 0);
#pragma unroll
        for (int t = 0; t < KC / 4; ++t) {
            if (t + 1 < KC / 4) fetch(4 * (t + 1), (t + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                if (wave + kWaves * j < f.nf) {
#pragma unroll
                    for (int m = 0; m < MI; ++m)
                        acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[t & 1][j], bv[t & 1][m], acc[m][j], 0, 0, 0);
                }
            }
            between(t);
        }
    };

    // Chunk c: its registers -> LDS (the input tile is free: the depthwise of
    // chunk c-1 finished before the last barrier; the weight and result
    // buffers c%2 were last read by chunk c-2's MFMAs), barrier, depthwise,
    // barrier, MFMAs with the loads of chunk cn (two ahead) into the same
    // registers issued between them.
    auto step = [&](int c, Regs& R, int cn) __attribute__((always_inline)) {
        float* es = es0 + (c & 1) * KC * f.es_stride;
        float* ws = ws0 + (c & 1) * KC * f.cop;
        float* dp = dp0 + (c & 1) * DWP;
        store_chunk(c, R, ws, dp);
        __syncthreads();
        depthwise(c, es, dp);
        __syncthreads();
        pointwise(es, ws, [&](int t) __attribute__((always_inline)) {
            if (t == 0) load_x(cn, R);
            if (t == 2) load_w(cn, R);
        });
    };
    // An even number of steps, two per iteration with fixed register sets, and
    // loads in every step (the last two reload the last chunk; with an odd
    // chunk count the extra chunk lies past the channels and adds zeros): no
    // load sits behind a condition, so the waits stay exact.
    const int nch2 = (nch + 1) & ~1;
    Regs R0, R1;
    load_x(0, R0);
    load_w(0, R0);
    load_x(1, R1);
    load_w(1, R1);
    for (int c = 0; c < nch2; c += 2) {
        step(c, R0, min(c + 2, nch2 - 1));
        step(c + 1, R1, min(c + 3, nch2 - 1));
    }

    // ---- epilogue: lane (q, l16) of fragment (m, j) holds output channel
    // co0 + m*16 + l16 at the 4 pixels j*16 + 4q .. +3 of the tile ----
    const int64_t oplane = (int64_t)P.ho * P.wo;
    float* __restrict__ yg = (float*)P.yptr;
    const bool vec_out = WO % 4 == 0 && ((uintptr_t)P.yptr % 16) == 0;
    const int npx_n = th_n * WO;
    const ActP pa = act_params(P);
#pragma unroll
    for (int m = 0; m < MI; ++m) {
        const int co = co0 + m * 16 + l16;
        if (m * 16 + l16 >= f.cot || co >= P.c_out) continue;
        float* yc = yg + ((int64_t)n * P.out_total + P.out_off + co) * oplane + (int64_t)ho0 * WO;
        const float bb = P.bias ? P.bias[co] : 0.0f;
        const float sl = act_slope(P, pa, co);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int fj = wave + kWaves * j;
            const int px = fj * 16 + 4 * q;
            if (fj >= f.nf || px >= npx_n) continue;
            float v4[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) v4[v] = act_apply(acc[m][j][v] + bb, sl, pa.lo, pa.hi);
            if (vec_out) {
                *(float4*)(yc + px) = make_float4(v4[0], v4[1], v4[2], v4[3]);
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (px + v < npx_n) yc[px + v] = v4[v];
            }
        }
    }
}

struct Plan {
    int th, ir, xoff, xw, xs_plane, npx, nf, nj, nx, es_stride, cot, cop, lds_floats;
};

// vec: the input moves as 16-byte vectors (row width and pointer allow it).
bool plan(const Desc& dw, const Desc& pw, bool vec, Plan* out, int cot = 0) {
    const conv2d_params_t& d = dw.p;
    const int W = d.w, WO = dw.wo;
    if (cot == 0) {
        // 64 output channels per tile; 32 when there are few or the 64-wide
        // variant does not fit the rows (each tile then redoes the depthwise).
        if (pw.p.c_out > 32 && plan(dw, pw, vec, out, 64)) return true;
        return plan(dw, pw, vec, out, 32);
    }
    const int co_tiles = (pw.p.c_out + cot - 1) / cot;
    const int xoff = (d.pad_left + 3) / 4 * 4;
    // Columns a tile reads (outputs padded to whole 64-column groups):
    // up to xoff - pad_left + (wo_padded-1)*sw + (kw-1)*dw + 1.
    const int wo_pad = (WO + 63) / 64 * 64;
    const int need = xoff - d.pad_left + (wo_pad - 1) * d.stride_w + (d.k_w - 1) * d.dilation_w + 1;
    int xw = xoff + W + d.pad_right;
    if (xw < need) xw = need;
    xw = (xw + 3) / 4 * 4;
    bool ok = false;
    long best = 0;
    for (int th = 1; th <= dw.ho; ++th) {
        const int ir = (th - 1) * d.stride_h + (d.k_h - 1) * d.dilation_h + 1;
        const int npx = th * WO;
        const int nf = (npx + 15) / 16;
        const int nj = (nf + kWaves - 1) / kWaves;
        if (nj > 4) break;
        const int units = vec ? KC * ir * (W / 4) : KC * ir * W;
        const int nx = (units + kT - 1) / kT;
        const int nxt = vec ? (nx <= 2 ? 2 : (nx <= 4 ? 4 : 8)) : 8;
        const int njt = nj <= 2 ? 2 : 4;
        // Variants that keep within 256 registers (larger ones spill).
        const bool fits = (vec ? (nxt == 8 ? cot == 32 && njt == 2 : njt == 2 || (nxt == 2 && cot == 32)) : njt == 2);
        if (nx > 8 || !fits) break;
        const int xs_plane = ir * xw;
        const int es_stride = stride16(nf * 16);
        const int cop = stride16(cot);
        const int lds = KC * xs_plane + 2 * KC * es_stride + 2 * KC * cop + 2 * DWP;
        if (lds * 4 > 160 * 1024) break;
        // One workgroup per compute unit: 8 waves of up to 256 registers.
        const long blocks = (long)d.n * ((dw.ho + th - 1) / th) * co_tiles;
        const long rounds = (blocks + device_cu_count() - 1) / device_cu_count();
        // Time ~ rounds x input rows a workgroup stages (halo included).
        const long cost = rounds * ir;
        if (!ok || cost < best) {
            *out = Plan{th, ir, xoff, xw, xs_plane, npx, nf, njt, nxt, es_stride, cot, cop, lds};
            best = cost;
            ok = true;
        }
    }
    return ok;
}

// The instantiations the planner may pick (see `fits` there).
template <int KH, int KW, int SS>
const void* pick_x(bool vec, int nx, int mi, int nj) {
#define K_(MI, NJ, V, NX) (const void*)fused_dw_pw_kernel<KH, KW, SS, MI, NJ, V, NX>
    if (!vec) return mi == 2 ? K_(2, 2, false, 8) : K_(4, 2, false, 8);
    if (nx == 8) return K_(2, 2, true, 8);
    if (nx == 4) return mi == 2 ? K_(2, 2, true, 4) : K_(4, 2, true, 4);
    if (mi == 2) return nj == 2 ? K_(2, 2, true, 2) : K_(2, 4, true, 2);
    return K_(4, 2, true, 2);
#undef K_
}

bool vec_ok(const Desc& dw, const void* x) {
    const conv2d_params_t& d = dw.p;
    const int64_t hw = (int64_t)d.h * d.w;
    return d.w % 4 == 0 && ((uintptr_t)x % 16) == 0 && ((int64_t)d.in_channel_offset * hw) % 4 == 0 &&
           ((int64_t)dw.in_total * hw) % 4 == 0;
}

}  // namespace

bool plan_fused_dw_pw(const Desc& dw, const Desc& pw, const void* x) {
    if (dw.p.k_h > 5 || dw.p.k_w > 5) return false;
    if ((int64_t)KC * dw.p.h * dw.p.w >= INT32_MAX || (int64_t)dw.ho * dw.wo >= INT32_MAX / 2) return false;
    Plan pl{};
    return plan(dw, pw, vec_ok(dw, x), &pl);
}

hipError_t launch_fused_dw_pw(const Desc& dw, const Desc& pw, ConvArgs adw, ConvArgs apw, hipStream_t s) {
    const bool vec = vec_ok(dw, adw.xptr);
    Plan pl{};
    if (!plan(dw, pw, vec, &pl)) return hipErrorInvalidConfiguration;
    DwPwArgs f;
    f.dw = adw;
    f.pw = apw;
    f.th = pl.th;
    f.tiles_h = (dw.ho + pl.th - 1) / pl.th;
    f.cot = pl.cot;
    f.co_tiles = (pw.p.c_out + pl.cot - 1) / pl.cot;
    f.ir = pl.ir;
    f.xoff = pl.xoff;
    f.xw = pl.xw;
    f.xs_plane = pl.xs_plane;
    f.npx = pl.npx;
    f.nf = pl.nf;
    f.es_stride = pl.es_stride;
    f.cop = pl.cop;
    f.dv_co_tiles = make_divu32((uint32_t)f.co_tiles);
    f.dv_tiles_h = make_divu32((uint32_t)f.tiles_h);
    f.div_cg = make_fastdiv((uint32_t)((dw.wo + 63) / 64));
    f.div_th = make_fastdiv((uint32_t)pl.th);
    f.div_q4 = make_fastdiv((uint32_t)(dw.wo >= 4 ? dw.wo / 4 : 1));
    f.div_rp = make_fastdiv((uint32_t)((pl.th + 1) / 2));
    const uint64_t blocks = (uint64_t)f.co_tiles * f.tiles_h * adw.n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0xFFFFFFFFull) return hipErrorInvalidConfiguration;
    f.num_blocks = (uint32_t)blocks;
    const conv2d_params_t& d = dw.p;
    const bool k3 = d.k_h == 3 && d.k_w == 3 && d.dilation_h == 1 && d.dilation_w == 1 && d.stride_h == d.stride_w &&
                    (d.stride_h == 1 || d.stride_h == 2);
    const int mi = pl.cot / 16;
    const void* fn = !k3 ? pick_x<0, 0, 0>(vec, pl.nx, mi, pl.nj)
                         : (d.stride_h == 1 ? pick_x<3, 3, 1>(vec, pl.nx, mi, pl.nj)
                                            : pick_x<3, 3, 2>(vec, pl.nx, mi, pl.nj));
    const int lds = pl.lds_floats * 4;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
    }
    void* args[] = {&f};
    return hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(kT), args, lds, s);
}

}  // namespace conv2d
