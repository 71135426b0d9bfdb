// Implicit-GEMM convolution on the fp32 matrix cores of gfx950.
//
// The Go "ops" page (section ConvOp) runs Conv as im2col + GEMM and fuses the
// bias and activation into the GEMM write (ConvLeakyReluOp, ConvPReluOp).
// Here the im2col matrix is never built: per output tile the kernel stages a
// halo patch of the input (pad_value outside the image, ncnn "convolution")
// and a slice of the OIHW weights in LDS, then feeds v_mfma_f32_16x16x4f32
// straight from those tiles.  Per group g the GEMM is
//   Y_g[co, pixel] = sum_k W_g[co, k] * Xhat_g[k, pixel],  k = (ci, r, s),
// with M = output channels (rows of the MFMA), N = output pixels (columns:
// consecutive pixels of a row give coalesced stores), K = input channels x
// kernel taps.  Inside a channel chunk the K order is (r, s) outer, ci inner,
// so four consecutive K of one MFMA step are four channels at the same tap.
//
// Tile: BM output channels x BN output pixels (tile_h rows x tile_w cols of
// one image), 4 waves arranged WAVES_M x WAVES_N x WAVES_K; waves that share
// an output sub-tile split the channel chunk and are summed through LDS at
// the end.  The epilogue adds the bias, applies the activation and writes
// channel out_off + g*cout_g + co of a buffer with out_total channels (the
// ConcatFusedTail store of the Go "ops" page, for any batch size).
#include "device_common.h"

namespace conv2d {

namespace {

constexpr int kThreads = 256;

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int WAVES_K_, int CK_, int KH_, int KW_,
          int XPT_, int WPT_>
struct IgemmF32Cfg {
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, WAVES_K = WAVES_K_;
    static constexpr int CK = CK_, KH = KH_, KW = KW_;
    static constexpr int XPT = XPT_, WPT = WPT_;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int MI = WM / 16, NI = WN / 16;
    static constexpr int CKW = CK / WAVES_K;            // channels of a chunk per wave
    static constexpr int BMP = BM == 16 ? 16 : BM + 16; // LDS row stride of the weight tile
    static_assert(WAVES_M * WAVES_N * WAVES_K == 4, "4 waves per workgroup");
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be whole 16x16 fragments");
    static_assert(CKW % 4 == 0, "each wave needs whole 4-channel MFMA steps");
};

// Floats of LDS one pipeline stage needs.
template <class C>
__host__ __device__ inline int stage_floats(int patch_stride, int khw) {
    return C::CK * patch_stride + khw * C::CK * C::BMP;
}

template <class C>
__global__ __launch_bounds__(kThreads) void igemm_f32_kernel(ConvArgs a) {
    extern __shared__ float lds[];
    constexpr int BM = C::BM, CK = C::CK, BMP = C::BMP, MI = C::MI, NI = C::NI;
    const int kh = C::KH > 0 ? C::KH : a.k_h;
    const int kw = C::KW > 0 ? C::KW : a.k_w;
    const int khw = kh * kw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wk = wave % C::WAVES_K;
    const int wmn = wave / C::WAVES_K;
    const int wm = wmn % C::WAVES_M;
    const int wn = wmn / C::WAVES_M;

    // Block -> (co tile, group, pixel tile, image), output-channel tiles fastest
    // so that blocks reading the same input patch are neighbours on one XCD.
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
    const int PS = a.patch_stride, PW = a.patch_w;
    const int PHW = a.patch_h * PW;
    const int x_total = CK * PHW;
    const int w_row = CK * khw;                 // weight floats per output channel per chunk
    const int w_total = BM * w_row;
    const int stage = stage_floats<C>(PS, khw);
    const int64_t HW = (int64_t)a.h * a.w;

    const float* __restrict__ xg =
        (const float*)a.xptr + ((int64_t)n * a.in_total + a.in_off + (int64_t)g * a.cin_g) * HW;
    const float* __restrict__ wg =
        (const float*)a.wptr + ((int64_t)g * a.cout_g + co0) * a.cin_g * khw;
    const int co_valid = min(BM, a.cout_g - co0);

    float xr[C::XPT];
    float wr[C::WPT];

    // Global -> registers for the channel chunk starting at c0.
    auto load_chunk = [&](int c0) {
#pragma unroll
        for (int i = 0; i < C::XPT; ++i) {
            const int e = tid + i * kThreads;
            float v = 0.0f;
            if (e < x_total) {
                const int ci = (int)fdiv(e, a.div_patch_hw);
                const int rem = e - ci * PHW;
                const int pr = (int)fdiv(rem, a.div_patch_w);
                const int pc = rem - pr * PW;
                const int ih = ih0 + pr, iw = iw0 + pc;
                if (c0 + ci < a.cin_g) {
                    if ((unsigned)ih < (unsigned)a.h && (unsigned)iw < (unsigned)a.w)
                        v = xg[(int64_t)(c0 + ci) * HW + (int64_t)ih * a.w + iw];
                    else
                        v = a.pad_value;
                }
            }
            xr[i] = v;
        }
#pragma unroll
        for (int i = 0; i < C::WPT; ++i) {
            const int e = tid + i * kThreads;
            float v = 0.0f;
            if (e < w_total) {
                const int co = e % BM;          // output channel fastest: conflict-free LDS rows
                const int j = e / BM;           // (ci, r, s) within the chunk, OIHW order
                const int ci = j / khw;
                if (co < co_valid && c0 + ci < a.cin_g)
                    v = wg[(int64_t)co * a.cin_g * khw + (int64_t)c0 * khw + j];
            }
            wr[i] = v;
        }
    };

    // Registers -> LDS stage.  Input plane ci at [ci*PS], weights at
    // [(rs*CK + ci)*BMP + co] after the input planes.
    auto store_chunk = [&](int s) {
        float* xs = lds + s * stage;
        float* ws = xs + CK * PS;
#pragma unroll
        for (int i = 0; i < C::XPT; ++i) {
            const int e = tid + i * kThreads;
            if (e < x_total) {
                const int ci = (int)fdiv(e, a.div_patch_hw);
                xs[ci * PS + (e - ci * PHW)] = xr[i];
            }
        }
#pragma unroll
        for (int i = 0; i < C::WPT; ++i) {
            const int e = tid + i * kThreads;
            if (e < w_total) {
                const int co = e % BM;
                const int j = e / BM;
                const int ci = j / khw;
                const int rs = j - ci * khw;
                ws[(rs * CK + ci) * BMP + co] = wr[i];
            }
        }
    };

    // Per-lane LDS bases of the MFMA operands.  A (weights): lane holds
    // row co = lane%16 at k = lane/16.  B (input): lane holds pixel lane%16
    // at k = lane/16, i.e. channel plane lane/16 of the current 4-channel step.
    const int a_base = (lane >> 4) * BMP + wm * C::WM + (lane & 15);
    int b_base[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
        const int j = wn * C::WN + ni * 16 + (lane & 15);
        const int th = (int)fdiv(j, a.div_tile_w);
        const int tw = j - th * a.tile_w;
        b_base[ni] = (lane >> 4) * PS + th * a.stride_h * PW + tw * a.stride_w;
    }

    f32x4 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](int s) {
        const float* xs = lds + s * stage;
        const float* ws = xs + CK * PS;
        for (int rs = 0; rs < khw; ++rs) {
            const int r = rs / kw;
            const int sc = rs - r * kw;
            const int uoff = r * a.dilation_h * PW + sc * a.dilation_w;
#pragma unroll
            for (int cq = 0; cq < C::CKW / 4; ++cq) {
                const int ci = wk * C::CKW + cq * 4;
                float av[MI], bv[NI];
#pragma unroll
                for (int mi = 0; mi < MI; ++mi) av[mi] = ws[(rs * CK + ci) * BMP + a_base + mi * 16];
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) bv[ni] = xs[ci * PS + uoff + b_base[ni]];
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mi], bv[ni], acc[mi][ni],
                                                                           0, 0, 0);
            }
        }
    };

    // Two-stage pipeline: the next chunk's global loads are in flight while
    // the current chunk is multiplied out of LDS.
    load_chunk(0);
    store_chunk(0);
    __syncthreads();
    for (int kc = 0; kc < a.chunks; ++kc) {
        const int s = kc & 1;
        const bool more = kc + 1 < a.chunks;
        if (more) load_chunk((kc + 1) * CK);
        compute(s);
        if (more) store_chunk(s ^ 1);
        __syncthreads();
    }

    // Epilogue.  D layout of the 16x16 MFMA: lane holds rows 4*(lane/16)+v
    // (v = 0..3) of column lane%16.
    float* __restrict__ yg = (float*)a.yptr;
    const int64_t out_plane = (int64_t)a.ho * a.wo;
    auto emit = [&](int mi, int ni, int v, float val) {
        const int co = co0 + wm * C::WM + mi * 16 + (lane >> 4) * 4 + v;
        const int j = wn * C::WN + ni * 16 + (lane & 15);
        const int th = (int)fdiv(j, a.div_tile_w);
        const int tw = j - th * a.tile_w;
        const int ho = ho0 + th, wo = wo0 + tw;
        if (co < a.cout_g && ho < a.ho && wo < a.wo) {
            const int cg = g * a.cout_g + co;
            yg[((int64_t)n * a.out_total + a.out_off + cg) * out_plane + (int64_t)ho * a.wo + wo] =
                bias_act(a, val, cg);
        }
    };

    if constexpr (C::WAVES_K == 1) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                for (int v = 0; v < 4; ++v) emit(mi, ni, v, acc[mi][ni][v]);
    } else {
        // Waves that split K park their partial sums in LDS (the pipeline
        // buffers are free after the last barrier); each then finishes the
        // fragments f with f % WAVES_K == wk.
        constexpr int FR = MI * NI * 4;
        float* red = lds;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    red[((wmn * C::WAVES_K + wk) * FR + (mi * NI + ni) * 4 + v) * 64 + lane] =
                        acc[mi][ni][v];
        __syncthreads();
#pragma unroll
        for (int f = 0; f < FR; ++f) {
            if (f % C::WAVES_K != wk) continue;
            float sum = 0.0f;
#pragma unroll
            for (int k2 = 0; k2 < C::WAVES_K; ++k2) sum += red[((wmn * C::WAVES_K + k2) * FR + f) * 64 + lane];
            emit(f / (NI * 4), (f / 4) % NI, f % 4, sum);
        }
    }
}

// ------------------------------------------------------------ configs ---

struct CfgInfo {
    int bm, bn, waves_k, ck, kh, kw, xpt, wpt;
    int red_floats;   // LDS floats of the split-K reduction (0 if none)
    const void* fn;
    int stage_floats(int ps, int khw) const {
        const int bmp = bm == 16 ? 16 : bm + 16;
        return ck * ps + khw * ck * bmp;
    }
};

template <class C>
CfgInfo info() {
    CfgInfo i;
    i.bm = C::BM; i.bn = C::BN; i.waves_k = C::WAVES_K; i.ck = C::CK; i.kh = C::KH; i.kw = C::KW;
    i.xpt = C::XPT; i.wpt = C::WPT;
    i.red_floats = C::WAVES_K > 1 ? 4 * C::MI * C::NI * 4 * 64 : 0;
    i.fn = (const void*)igemm_f32_kernel<C>;
    return i;
}

//                       BM  BN  WM WN WK  CK KH KW XPT WPT
using K3_M32  = IgemmF32Cfg<32,  64, 1, 2, 2,  8, 3, 3, 8, 9>;
using K3_M64  = IgemmF32Cfg<64,  64, 2, 2, 1,  8, 3, 3, 8, 18>;
using K3_M128 = IgemmF32Cfg<128, 128, 2, 2, 1, 4, 3, 3, 12, 18>;
using K3_M16  = IgemmF32Cfg<16,  64, 1, 4, 1,  8, 3, 3, 8, 5>;
using K1_M32  = IgemmF32Cfg<32,  128, 1, 4, 1, 16, 1, 1, 8, 2>;
using K1_M64  = IgemmF32Cfg<64,  128, 1, 4, 1, 16, 1, 1, 8, 4>;
using K1_M128 = IgemmF32Cfg<128, 128, 2, 2, 1, 16, 1, 1, 8, 8>;
using KG_M32  = IgemmF32Cfg<32,  64, 1, 4, 1,  4, 0, 0, 16, 16>;
using KG_M16  = IgemmF32Cfg<16,  64, 1, 4, 1,  4, 0, 0, 16, 16>;

const CfgInfo& cfg(int i) {
    static const CfgInfo table[] = {
        info<K3_M32>(), info<K3_M64>(), info<K3_M128>(), info<K3_M16>(),
        info<K1_M32>(), info<K1_M64>(), info<K1_M128>(),
        info<KG_M32>(), info<KG_M16>(),
    };
    return table[i];
}

int patch_stride_for(int phw) {
    // Smallest stride >= phw with stride % 64 == 16: the four channel planes
    // read by one MFMA operand fetch then start 16 banks apart.
    int s = ((phw + 63 - 16) / 64) * 64 + 16;
    if (s < phw) s += 64;
    return s;
}

struct Tiling {
    int tile_h, tile_w, ph, pw, ps;
    long waste;
};

bool choose_tiling(const Desc& d, const CfgInfo& c, int h_eff, int w_eff, int ho_eff, int wo_eff,
                   Tiling* best) {
    const conv2d_params_t& p = d.p;
    bool found = false;
    for (int tw = 8; tw <= c.bn; tw *= 2) {
        const int th = c.bn / tw;
        const int ph = (th - 1) * p.stride_h + (p.k_h - 1) * p.dilation_h + 1;
        const int pw = (tw - 1) * p.stride_w + (p.k_w - 1) * p.dilation_w + 1;
        if (c.ck * ph * pw > kThreads * c.xpt) continue;
        if (ph * pw >= 65536 || c.ck * ph * pw >= 65536) continue;
        const int ps = patch_stride_for(ph * pw);
        const int khw = p.k_h * p.k_w;
        if (c.bm * c.ck * khw > kThreads * c.wpt) continue;
        const int lds = 2 * c.stage_floats(ps, khw);
        if ((lds > c.red_floats ? lds : c.red_floats) * 4 > 64 * 1024) continue;
        const long tiles = (long)((ho_eff + th - 1) / th) * ((wo_eff + tw - 1) / tw);
        const long waste = tiles * c.bn - (long)ho_eff * wo_eff;
        // Prefer less waste; on ties prefer wider rows (longer coalesced runs).
        if (!found || waste < best->waste || (waste == best->waste && tw > best->tile_w)) {
            *best = Tiling{th, tw, ph, pw, ps, waste};
            found = true;
        }
    }
    (void)h_eff; (void)w_eff;
    return found;
}

}  // namespace

bool plan_igemm_f32(Desc& d) {
    const conv2d_params_t& p = d.p;
    const bool is3 = p.k_h == 3 && p.k_w == 3;
    const bool is1 = p.k_h == 1 && p.k_w == 1;
    d.flatten_1x1 = is1 && p.stride_h == 1 && p.stride_w == 1 && p.pad_top == 0 &&
                    p.pad_left == 0 && p.pad_bottom == 0 && p.pad_right == 0;
    const int h_eff = d.flatten_1x1 ? 1 : p.h;
    const int w_eff = d.flatten_1x1 ? p.h * p.w : p.w;
    const int ho_eff = d.flatten_1x1 ? 1 : d.ho;
    const int wo_eff = d.flatten_1x1 ? d.ho * d.wo : d.wo;
    if (d.flatten_1x1 && (int64_t)p.h * p.w > INT32_MAX / 2) return false;

    // Candidate configs in order of preference.
    int cands[4];
    int nc = 0;
    const int m = d.cout_g;
    if (is3) {
        if (m <= 16) cands[nc++] = 3;
        else if (m <= 32) cands[nc++] = 0;
        else if (m <= 64) cands[nc++] = 1;
        else cands[nc++] = 2;
        cands[nc++] = m <= 16 ? 8 : 7;
    } else if (is1) {
        if (m <= 32) cands[nc++] = 4;
        else if (m <= 64) cands[nc++] = 5;
        else cands[nc++] = 6;
        cands[nc++] = m <= 16 ? 8 : 7;
    } else {
        cands[nc++] = m <= 16 ? 8 : 7;
    }
    for (int k = 0; k < nc; ++k) {
        const CfgInfo& c = cfg(cands[k]);
        if (c.kh && (c.kh != p.k_h || c.kw != p.k_w)) continue;
        Tiling t;
        if (d.flatten_1x1) {
            // One row of h*w pixels: the patch is the tile itself.
            t.tile_h = 1; t.tile_w = c.bn; t.ph = 1; t.pw = c.bn;
            t.ps = patch_stride_for(c.bn);
            if (c.ck * c.bn > kThreads * c.xpt || c.bm * c.ck > kThreads * c.wpt) continue;
        } else if (!choose_tiling(d, c, h_eff, w_eff, ho_eff, wo_eff, &t)) {
            continue;
        }
        const int khw = p.k_h * p.k_w;
        const int lds = 2 * c.stage_floats(t.ps, khw);
        d.cfg = cands[k];
        d.tile_h = t.tile_h;
        d.tile_w = t.tile_w;
        d.lds_bytes = 4 * (lds > c.red_floats ? lds : c.red_floats);
        (void)h_eff; (void)w_eff;
        return true;
    }
    return false;
}

void fill_tiling(const Desc& d, ConvArgs& a) {
    // Shared by the implicit-GEMM planners: derive the per-tile geometry.
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

hipError_t launch_igemm_f32(const Desc& d, ConvArgs a, hipStream_t s) {
    const CfgInfo& c = cfg(d.cfg);
    fill_tiling(d, a);
    a.co_tiles = (d.cout_g + c.bm - 1) / c.bm;
    a.chunks = (d.cin_g + c.ck - 1) / c.ck;
    const uint64_t blocks = (uint64_t)a.co_tiles * a.groups * a.tiles_h * a.tiles_w * a.n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0xFFFFFFFFull) return hipErrorInvalidConfiguration;
    a.num_blocks = (uint32_t)blocks;
    void* args[] = {&a};
    return hipLaunchKernel(c.fn, dim3((uint32_t)blocks), dim3(kThreads), args, d.lds_bytes, s);
}

}  // namespace conv2d
