// Fused pointwise 1x1 -> depthwise kxk (the FusedPwDw step of the yscv
// "ONNX CPU Kernels" page, section "Hot kernel paths": an inverted-bottleneck
// expansion followed by its depthwise conv, with the expanded tensor never
// written to main memory).
//
// Workgroup tile: one image, TH output rows, CE = 32 expanded channels, the
// full image width.
//   1. The pointwise input rows the tile needs (TH + (kh-1)*dh rows, halo
//      included) are loaded for a chunk of KC input channels, every thread
//      issuing all of its 16-byte loads before writing any of them to LDS,
//      together with the CE x KC pointwise weights.  E = W_pw * X runs on the
//      fp32 matrix cores (v_mfma_f32_16x16x4f32; M = the CE channels, N = the
//      rows' pixels): each of the eight waves owns every 16-pixel fragment
//      j == wave (mod 8) for both 16-channel halves, so its MFMAs accumulate
//      into independent registers.
//   2. Bias + activation of the pointwise conv go into an LDS tile of
//      W + pad_left + pad_right columns per row.  Rows and columns outside
//      the image hold the depthwise pad_value: the depthwise padding applies
//      to the pointwise output, not to pw(pad).
//   3. The depthwise conv reads R x VO output blocks out of that tile through
//      a register window, adds its bias, applies its activation and writes
//      each output row with a 16-byte store.
// The halo rows are recomputed by the tiles above and below
// (((TH-1)*stride + kh) / TH pointwise work) instead of being exchanged.
// The depthwise may have any stride (the pages' depthwise steps are 3x3 and
// 5x5 at stride 1 or 2); the fixed 3x3 register-window path is stride 1.
#include "device_common.h"

namespace conv2d {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int CE = 32;       // expanded channels per workgroup
constexpr int KC = 32;       // input channels per pointwise chunk
constexpr int CEP = 48;      // LDS row stride of the weight tile (4 k-rows land 16 banks apart)
constexpr int NJMAX = 8;     // max 16-pixel fragments per wave (the NJ template parameter)
constexpr int NVX = 8;       // max 16-byte input loads per thread and chunk
constexpr int VO = 4;        // depthwise outputs per thread and row
constexpr int RR = 4;        // depthwise output rows per thread

struct FusedArgs {
    ConvArgs pw, dw;
    int32_t tile_h, tiles_h, ce_tiles;
    int32_t rows;          // pointwise rows per tile: TH + (kh-1)*dh
    int32_t xs_stride;     // LDS floats per input-channel plane (rows * w, = 16 mod 64)
    int32_t ew;            // LDS row length of the expanded tile
    int32_t es_stride;     // LDS floats per expanded channel
    int32_t vec;           // input rows move as 16-byte vectors
    uint32_t num_blocks;
    DivU32 dv_ce_tiles, dv_tiles_h;
    FastDiv div_w;         // division by the image width (pixel -> row)
    FastDiv div_w4;        // division by w/4 (load unit -> row)
    FastDiv div_rw4;       // division by rows*w/4 (load unit -> channel)
    DivU32 dv_rows;        // expanded row index -> channel
    DivU32 dv_uw;          // depthwise thread -> channel (by the VO-column groups per row)
};

// NJ: 16-pixel pointwise fragments per wave (register budget: 4 keeps two
// workgroups per compute unit).
// 4 bytes per lane from global memory straight into LDS (global_load_lds_dword):
// lane l reads src (its own address) and writes lds_base + 4*l, lds_base
// wave-uniform; completion is counted by vmcnt like any load.  Inline
// assembly, so the compiler does not hold later LDS accesses behind it; the
// kernel orders it (every wave waits for all of its loads before its first
// LDS write of the chunk, and a barrier follows).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy4_to_lds(const float* src, const float* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(m) : "memory", "m0");
#endif
}
#pragma clang diagnostic pop

template <int KH, int KW, int NJ>
__global__ __launch_bounds__(kThreads) void fused_pw_dw_kernel(FusedArgs f) {
    extern __shared__ __align__(16) float lds[];
    const ConvArgs& P = f.pw;
    const ConvArgs& D = f.dw;
    constexpr bool FIXED = KH > 0;
    const int kh = FIXED ? KH : D.k_h, kw = FIXED ? KW : D.k_w;
    const int dh = FIXED ? 1 : D.dilation_h, dwl = FIXED ? 1 : D.dilation_w;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    uint32_t L = xcd_remap(blockIdx.x, f.num_blocks);
    uint32_t Q = divu(L, f.dv_ce_tiles);
    const int cet = L - Q * f.ce_tiles;
    L = Q; Q = divu(L, f.dv_tiles_h);
    const int tht = L - Q * f.tiles_h;
    const int n = Q;
    const int ce0 = cet * CE;
    const int ho0 = tht * f.tile_h;
    const int sh = FIXED ? 1 : D.stride_h, sw = FIXED ? 1 : D.stride_w;
    const int ih_lo = ho0 * sh - D.pad_top;     // image row of pointwise row 0
    const int W = P.w, H = P.h;
    const int npix = f.rows * W;                 // pointwise pixels of the tile
    const int nfn = (npix + 15) / 16;
    const int ce_valid = min(CE, P.c_out - ce0);
    const int64_t HW = (int64_t)H * W;
    const int XS = f.xs_stride;

    const float* __restrict__ xg = (const float*)P.xptr + ((int64_t)n * P.in_total + P.in_off) * HW;
    const float* __restrict__ wpw = (const float*)P.wptr;

    float* xs = lds;                       // [KC][XS]
    float* ws = lds + KC * XS;             // [KC][CEP]

    f32x4 acc[2][NJ];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[m][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // ---- 1. pointwise on the matrix cores ----
    for (int k0 = 0; k0 < P.c_in; k0 += KC) {
        // The chunk's CE x KC weights go straight to LDS first, so their round
        // trip overlaps the input rows': slot s of ws is (k = s / CEP,
        // ce = s % CEP).  Columns past CE, channels past the layer's and
        // inputs past its channels read a valid weight: those columns are
        // never read, those channels' results are discarded, and those
        // inputs are zero in xs.
#pragma unroll
        for (int k = 0; k < (KC * CEP / 64 + kWaves - 1) / kWaves; ++k) {
            const int r = wave + kWaves * k;
            if (r < KC * CEP / 64) {
                const int sl = 64 * r + lane;
                const int kc = sl / CEP, ce = sl - (sl / CEP) * CEP;
                const int cew = min(ce, ce_valid - 1);
                copy4_to_lds(wpw + (int64_t)(ce0 + cew) * P.c_in + min(k0 + kc, P.c_in - 1), ws + 64 * r);
            }
        }
        if (f.vec) {
            // Units of four pixels: (channel, row, column group); all loads first.
            const int w4 = W >> 2;
            const int units = KC * f.rows * w4;
            float4 buf[NVX];
#pragma unroll
            for (int i = 0; i < NVX; ++i) {
                const int u = tid + i * kThreads;
                const int kc = (int)fdiv(u, f.div_rw4);
                const int rem = u - kc * (f.rows * w4);
                const int r = (int)fdiv(rem, f.div_w4);
                const int c4 = rem - r * w4;
                const int ih = ih_lo + r;
                buf[i] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (u < units && k0 + kc < P.c_in && (unsigned)ih < (unsigned)H)
                    buf[i] = *(const float4*)(xg + (int64_t)(k0 + kc) * HW + (int64_t)ih * W + 4 * c4);
            }
#pragma unroll
            for (int i = 0; i < NVX; ++i) {
                const int u = tid + i * kThreads;
                if (u < units) {
                    const int kc = (int)fdiv(u, f.div_rw4);
                    const int rem = u - kc * (f.rows * w4);
                    *(float4*)(xs + kc * XS + 4 * rem) = buf[i];
                }
            }
        } else {
            for (int e = tid; e < KC * npix; e += kThreads) {
                const int kc = e / npix;
                const int p = e - kc * npix;
                const int r = (int)fdiv(p, f.div_w);
                const int c = p - r * W;
                const int ih = ih_lo + r;
                float v = 0.0f;
                if (k0 + kc < P.c_in && (unsigned)ih < (unsigned)H) v = xg[(int64_t)(k0 + kc) * HW + (int64_t)ih * W + c];
                xs[kc * XS + p] = v;
            }
        }
        __builtin_amdgcn_s_waitcnt(0x3f70);           // vmcnt(0): this wave's weight copies have landed
        __syncthreads();
        // A lane reads weight row ce = lane%16 (+16) at k = lane/16; B lane reads
        // input plane k = lane/16 at pixel 16*frag + lane%16.
#pragma unroll
        for (int kq = 0; kq < KC; kq += 4) {
            const int kr = kq + (lane >> 4);
            const float a0 = ws[kr * CEP + (lane & 15)];
            const float a1 = ws[kr * CEP + 16 + (lane & 15)];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int fj = wave + kWaves * j;
                if (fj < nfn) {
                    const float b = xs[kr * XS + fj * 16 + (lane & 15)];
                    acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b, acc[0][j], 0, 0, 0);
                    acc[1][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b, acc[1][j], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }

    // ---- 2. pointwise epilogue into the expanded tile (aliases xs/ws) ----
    float* es = lds;   // [CE][es_stride], pointwise row r at r*ew, image column c at c + pad_left
    const float dpad = D.pad_value;
    {
        // This lane's pixel in each fragment: LDS offset within a channel
        // (-1 = no pixel) and whether its row is inside the image.
        int eoff[NJ];
        bool ein[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int fj = wave + kWaves * j;
            const int p = fj * 16 + (lane & 15);
            eoff[j] = -1;
            ein[j] = false;
            if (fj < nfn && p < npix) {
                const int r = (int)fdiv(p, f.div_w);
                eoff[j] = r * f.ew + (p - r * W) + D.pad_left;
                ein[j] = (unsigned)(ih_lo + r) < (unsigned)H;
            }
        }
        const ActP pa = act_params(P);
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int ce = m * 16 + (lane >> 4) * 4 + v;
                const bool cv = ce < ce_valid;
                const int cg = ce0 + (cv ? ce : 0);
                const float bb = P.bias ? P.bias[cg] : 0.0f;
                const float sl = act_slope(P, pa, cg);
                float* ech = es + ce * f.es_stride;
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    if (eoff[j] >= 0)
                        ech[eoff[j]] = (ein[j] && cv) ? act_apply(acc[m][j][v] + bb, sl, pa.lo, pa.hi) : dpad;
            }
    }
    // pad columns of every row (one row per thread)
    for (int rr = tid; rr < CE * f.rows; rr += kThreads) {
        const int ce = (int)divu((uint32_t)rr, f.dv_rows);
        float* row = es + ce * f.es_stride + (rr - ce * f.rows) * f.ew;
        for (int c = 0; c < D.pad_left; ++c) row[c] = dpad;
        for (int c = D.pad_left + W; c < f.ew; ++c) row[c] = dpad;
    }
    __syncthreads();

    // ---- 3. depthwise from LDS ----
    const int th_n = min(f.tile_h, D.ho - ho0);
    const int uw = (D.wo + VO - 1) / VO;
    const int64_t oplane = (int64_t)D.ho * D.wo;
    float* __restrict__ yg = (float*)D.yptr;
    const float* __restrict__ wdw = (const float*)D.wptr;
    const bool vec_ok = (D.wo % VO) == 0 && (((uintptr_t)D.yptr) % 16) == 0;
    const ActP da = act_params(D);
    auto store_row = [&](float* dst, const float (&accd)[VO], float dbb, float dsl, int q0)
        __attribute__((always_inline)) {
        float outv[VO];
#pragma unroll
        for (int q = 0; q < VO; ++q) outv[q] = act_apply(accd[q] + dbb, dsl, da.lo, da.hi);
        if (vec_ok && q0 + VO <= D.wo) {
            *(float4*)dst = make_float4(outv[0], outv[1], outv[2], outv[3]);
        } else {
#pragma unroll
            for (int q = 0; q < VO; ++q)
                if (q0 + q < D.wo) dst[q] = outv[q];
        }
    };
    if constexpr (FIXED) {
        // 3x3, stride 1: a thread owns one channel and VO output columns and
        // walks down the tile's output rows with a window of three expanded
        // rows in registers (each row's VO + 2 floats read once, as a float4
        // and a float2: rows are 16-byte aligned), so an output costs its 9
        // FMAs and little else.  Output column q0 + q, tap s reads LDS column
        // q0 + q + s (LDS column = image column + pad_left).
        const int pairs = ce_valid * uw;
        for (int pr = tid; pr < pairs; pr += kThreads) {
            const int ce = (int)divu((uint32_t)pr, f.dv_uw);
            const int q0 = (pr - ce * uw) * VO;
            const int cg = ce0 + ce;
            const float* wch = wdw + (int64_t)cg * 9;
            float wt[9];
#pragma unroll
            for (int i = 0; i < 9; ++i) wt[i] = wch[i];
            const float dbb = D.bias ? D.bias[cg] : 0.0f;
            const float dsl = act_slope(D, da, cg);
            const float* ech = es + ce * f.es_stride + q0;
            auto load = [&](float (&v)[VO + 2], int row) __attribute__((always_inline)) {
                const float4 a4 = *(const float4*)(ech + row * f.ew);
                const float2 b2 = *(const float2*)(ech + row * f.ew + 4);
                v[0] = a4.x; v[1] = a4.y; v[2] = a4.z; v[3] = a4.w; v[4] = b2.x; v[5] = b2.y;
            };
            float ra[VO + 2], rb[VO + 2];
            load(ra, 0);
            load(rb, 1);
            float* dst = yg + ((int64_t)n * D.out_total + D.out_off + cg) * oplane + (int64_t)ho0 * D.wo + q0;
            for (int o = 0; o < th_n; ++o) {
                float rc[VO + 2];
                load(rc, o + 2);
                float accd[VO];
#pragma unroll
                for (int q = 0; q < VO; ++q) {
                    float v = 0.0f;
#pragma unroll
                    for (int s2 = 0; s2 < 3; ++s2) v = fmaf(ra[q + s2], wt[s2], v);
#pragma unroll
                    for (int s2 = 0; s2 < 3; ++s2) v = fmaf(rb[q + s2], wt[3 + s2], v);
#pragma unroll
                    for (int s2 = 0; s2 < 3; ++s2) v = fmaf(rc[q + s2], wt[6 + s2], v);
                    accd[q] = v;
                }
                store_row(dst + (int64_t)o * D.wo, accd, dbb, dsl, q0);
#pragma unroll
                for (int t = 0; t < VO + 2; ++t) { ra[t] = rb[t]; rb[t] = rc[t]; }
            }
        }
    } else {
        // Any window, stride and dilation: RR x VO outputs per unit.
        const int uh = (th_n + RR - 1) / RR;
        const int units = ce_valid * uh * uw;
        for (int u = tid; u < units; u += kThreads) {
            const int ce = u / (uh * uw);
            const int rem = u - ce * uh * uw;
            const int rr = rem / uw;
            const int q0 = (rem - rr * uw) * VO;
            const int r0 = rr * RR;
            const int cg = ce0 + ce;
            float accd[RR][VO];
#pragma unroll
            for (int i = 0; i < RR; ++i)
#pragma unroll
                for (int q = 0; q < VO; ++q) accd[i][q] = 0.0f;
            const float* ech = es + ce * f.es_stride;
            const float* wch = wdw + (int64_t)cg * kh * kw;
            const float dbb = D.bias ? D.bias[cg] : 0.0f;
            const float dsl = act_slope(D, da, cg);
#pragma unroll
            for (int orow = 0; orow < RR; ++orow) {
                if (r0 + orow >= th_n) break;
                for (int r = 0; r < kh; ++r) {
                    const float* row = ech + ((r0 + orow) * sh + r * dh) * f.ew;
                    for (int s2 = 0; s2 < kw; ++s2) {
                        const float wv = wch[r * kw + s2];
#pragma unroll
                        for (int q = 0; q < VO; ++q) {
                            // Columns past the row end belong to masked outputs; clamp the read.
                            const int col = min(q0 + q, D.wo - 1) * sw + s2 * dwl;
                            accd[orow][q] = fmaf(row[col], wv, accd[orow][q]);
                        }
                    }
                }
            }
#pragma unroll
            for (int orow = 0; orow < RR; ++orow) {
                const int th = r0 + orow;
                if (th >= th_n) break;
                store_row(yg + ((int64_t)n * D.out_total + D.out_off + cg) * oplane + (int64_t)(ho0 + th) * D.wo + q0,
                          accd[orow], dbb, dsl, q0);
            }
        }
    }
}

// Channel stride of the expanded tile: >= rows * ew and = 4 (mod 16), so the
// four lane groups of an MFMA result (four channels apart) write 16 banks apart.
int es_stride_for(int n) {
    return n % 16 <= 4 ? n - n % 16 + 4 : n - n % 16 + 20;
}

int xs_stride_for(int npix) {
    int s = ((npix + 63 - 16) / 64) * 64 + 16;
    if (s < npix) s += 64;
    return s;
}

struct FusedPlan {
    int tile_h, rows, xs_stride, ew, es_stride, lds_floats, vec;
};

bool plan(const Desc& pw, const Desc& dw, FusedPlan* out) {
    const conv2d_params_t& d = dw.p;
    const int W = pw.p.w;
    // Rows of a multiple of 4 floats (16-byte aligned), the columns past the
    // right pad holding pad_value too.
    const int ew = (W + d.pad_left + d.pad_right + 3) / 4 * 4;
    const bool vec = W % 4 == 0;
    const long per_image = (long)((pw.p.c_out + CE - 1) / CE) * pw.p.n;
    bool ok = false;
    long best_cost = 0;
    for (int th = 1; th <= dw.ho; ++th) {
        const int rows = (th - 1) * d.stride_h + (d.k_h - 1) * d.dilation_h + 1;
        const int npix = rows * W;
        if ((npix + 15) / 16 > NJMAX * kWaves) break;               // fragments per wave
        if (vec && KC * rows * (W / 4) > NVX * kThreads) break;     // loads per thread
        if (npix >= 65536) break;
        const int xs = xs_stride_for(npix);
        const int es = es_stride_for(rows * ew);
        const int fl1 = KC * xs + KC * CEP;
        const int fl2 = CE * es + 8;   // 8 floats of slack: the last column group's window may run past the tile
        const int lds = fl1 > fl2 ? fl1 : fl2;
        if (lds * 4 > 96 * 1024) break;
        // Time ~ rounds of resident workgroups x pointwise rows per workgroup
        // (halo recompute included).
        const long blocks = per_image * ((dw.ho + th - 1) / th);
        long per_cu = (160 * 1024) / (lds * 4) > 0 ? (160 * 1024) / (lds * 4) : 1;
        const long per_cu_regs = (npix + 15) / 16 <= 4 * kWaves ? 2 : 1;   // NJ = 4 or 8 register budget
        if (per_cu > per_cu_regs) per_cu = per_cu_regs;
        const long rounds = (blocks + per_cu * device_cu_count() - 1) / (per_cu * device_cu_count());
        const long cost = rounds * rows;
        if (!ok || cost < best_cost) {
            *out = FusedPlan{th, rows, xs, ew, es, lds, vec ? 1 : 0};
            best_cost = cost;
            ok = true;
        }
    }
    return ok;
}

}  // namespace

bool plan_fused_pw_dw(const Desc& pw, const Desc& dw, int32_t* tile_h, int32_t* lds_bytes) {
    if (dw.p.k_h > 5 || dw.p.k_w > 5) return false;
    FusedPlan fp{};
    if (!plan(pw, dw, &fp)) return false;
    *tile_h = fp.tile_h;
    *lds_bytes = fp.lds_floats * 4;
    return true;
}

hipError_t launch_fused_pw_dw(const Desc& pw, const Desc& dw, ConvArgs apw, ConvArgs adw, hipStream_t s) {
    FusedPlan fp{};
    if (!plan(pw, dw, &fp)) return hipErrorInvalidConfiguration;
    FusedArgs f;
    f.pw = apw;
    f.dw = adw;
    f.tile_h = fp.tile_h;
    f.tiles_h = (dw.ho + fp.tile_h - 1) / fp.tile_h;
    f.ce_tiles = (pw.p.c_out + CE - 1) / CE;
    f.rows = fp.rows;
    f.xs_stride = fp.xs_stride;
    f.ew = fp.ew;
    f.es_stride = fp.es_stride;
    f.vec = fp.vec && ((uintptr_t)apw.xptr % 16) == 0;
    f.div_w = make_fastdiv((uint32_t)pw.p.w);
    f.div_w4 = make_fastdiv((uint32_t)(pw.p.w / 4 > 0 ? pw.p.w / 4 : 1));
    f.div_rw4 = make_fastdiv((uint32_t)(fp.rows * (pw.p.w / 4) > 0 ? fp.rows * (pw.p.w / 4) : 1));
    f.dv_rows = make_divu32((uint32_t)fp.rows);
    f.dv_uw = make_divu32((uint32_t)((dw.wo + VO - 1) / VO));
    f.dv_ce_tiles = make_divu32((uint32_t)f.ce_tiles);
    f.dv_tiles_h = make_divu32((uint32_t)f.tiles_h);
    const uint64_t blocks = (uint64_t)f.ce_tiles * f.tiles_h * apw.n;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0xFFFFFFFFull) return hipErrorInvalidConfiguration;
    f.num_blocks = (uint32_t)blocks;
    const bool k3 = dw.p.k_h == 3 && dw.p.k_w == 3 && dw.p.dilation_h == 1 && dw.p.dilation_w == 1 &&
                    dw.p.stride_h == 1 && dw.p.stride_w == 1;
    const bool nj4 = (fp.rows * pw.p.w + 15) / 16 <= 4 * kWaves;
    const void* fn = k3 ? (nj4 ? (const void*)fused_pw_dw_kernel<3, 3, 4> : (const void*)fused_pw_dw_kernel<3, 3, 8>)
                        : (nj4 ? (const void*)fused_pw_dw_kernel<0, 0, 4> : (const void*)fused_pw_dw_kernel<0, 0, 8>);
    if (fp.lds_floats * 4 > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, fp.lds_floats * 4);
        if (e != hipSuccess) return e;
    }
    void* args[] = {&f};
    return hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(kThreads), args, fp.lds_floats * 4, s);
}

}  // namespace conv2d
