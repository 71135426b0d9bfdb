// Internal declarations shared by the C ABI layer and the gfx950 kernels.
// Nothing here is part of the public ABI (include/conv2d.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/conv2d.h"

namespace conv2d {

// Kernel classes chosen by the descriptor.
enum KernelClass : int32_t {
    KC_IGEMM_F32 = 0,    // implicit GEMM, fp32 MFMA (dense, grouped, pointwise)
    KC_IGEMM_BF16 = 1,   // implicit GEMM, bf16 MFMA, fp32 accumulate
    KC_DW = 2,           // depthwise (groups == c_in == c_out), VALU, LDS halo tiles
    KC_QDW = 3,          // int8 depthwise, VALU int32 MACs
    KC_QPW = 4,          // int8 pointwise 1x1, i8 MFMA
    KC_DIRECT = 5,       // direct convolution, one thread per output (any shape)
    KC_GROUPED = 6,      // grouped 3x3 with 4 or 8 channels per group, VALU
    KC_WINOGRAD_F32 = 7, // Winograd F(2x2, 3x3), fp32 MFMA (3x3, stride 1, dilation 1, one group)
    KC_PW_F32 = 8,       // pointwise 1x1 with K <= 256, fp32 MFMA, every output channel per workgroup
    KC_IGEMM_I8 = 9,     // int8 dense / grouped implicit GEMM, i8 MFMA
    KC_SMALL_F32 = 10,   // small fp32 3x3 layers on the vector units, one thread per output pixel
    KC_WINOGRAD4_F32 = 11, // Winograd F(4x4, 3x3), fp32 MFMA, bound weights only
    KC_PWG_F32 = 12,     // pointwise 1x1 with a deep reduction, 128 x 128 GEMM tiles shared in LDS
    KC_PWN_F32 = 13,     // pointwise 1x1 with 64 < K <= 256 and <= 32 output channels, 32-pixel tiles
};

// Fast unsigned division by a runtime constant d (1 <= d < 2^16) for
// numerators below 2^16: q = umulhi(x, m) with m = ceil(2^32 / d).
struct FastDiv {
    uint32_t d;
    uint32_t m;
};

inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    f.m = (uint32_t)((((uint64_t)1 << 32) + d - 1) / d);
    return f;
}

// Division of any 32-bit unsigned numerator by a runtime constant d >= 1
// (Granlund and Montgomery, "Division by Invariant Integers using
// Multiplication", 1994, round-up method): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, the quotient is
// (t + ((x - t) >> 1)) >> (l - 1), t = umulhi(x, m).
struct DivU32 {
    uint32_t d;
    uint32_t m;
    uint32_t s;   // l - 1 (unused for d == 1)
};

inline DivU32 make_divu32(uint32_t d) {
    DivU32 r;
    r.d = d;
    r.m = 0;
    r.s = 0;
    if (d > 1) {
        uint32_t l = 0;
        while (((uint64_t)1 << l) < d) ++l;
        r.m = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1);
        r.s = l - 1;
    }
    return r;
}

// Everything a forward kernel needs, passed by value.  Sizes are element
// counts; offsets into x and y are computed in 64-bit inside the kernels.
struct ConvArgs {
    const void* xptr;      // input (n, in_total, h, w)
    const void* wptr;      // weights OIHW
    const float* bias;     // null when absent
    const float* slope;    // null unless PReLU
    void* yptr;            // output (n, out_total, ho, wo)

    int32_t n, c_in, h, w, c_out, k_h, k_w;
    int32_t pad_top, pad_left;
    int32_t stride_h, stride_w, dilation_h, dilation_w;
    int32_t groups, cin_g, cout_g;
    int32_t ho, wo;
    int32_t in_total, in_off, out_total, out_off;
    float pad_value;
    int32_t act;
    float act_a, act_b;    // leaky alpha / clip lo, clip hi
    int32_t slope_count;

    // Tiling decided on the host.
    int32_t tile_h, tile_w;          // output pixels per tile (rows, cols)
    int32_t tiles_h, tiles_w;        // tiles per image
    int32_t co_tiles;                // output-channel tiles per group
    int32_t patch_h, patch_w;        // input window of one tile (rows, cols)
    int32_t patch_stride;            // LDS stride between channel planes
    int32_t chunks;                  // number of input-channel chunks
    int32_t stages;                  // LDS pipeline stages (1 or 2)
    uint32_t num_blocks;             // grid size (for the XCD remap)
    FastDiv div_patch_hw, div_patch_w, div_tile_w;
    int32_t patch_shift;             // fp32 igemm: input column of LDS column 0 is iw_lo - patch_shift
    int32_t pt_vertical;             // fp32 igemm: a block's pixel sub-tiles stack along rows (1) or columns (0)
    int32_t vec_store;               // outputs may be written as 16-byte vectors
    int32_t dma;                     // fp32 igemm: copy chunks with direct global->LDS loads
    DivU32 dv_co_tiles, dv_groups, dv_tiles_w, dv_tiles_h;   // block index decomposition
    int32_t lds_rs, lds_plane, col_half;  // bf16 igemm: patch row / plane strides in LDS cells, stride-2 split

    // int8 requant
    float composite;
    int32_t y_zp;
    int32_t rounding;
    const int32_t* qbias;
};

// Host-side descriptor (opaque to callers).
struct Desc {
    conv2d_params_t p;
    int32_t ho, wo;
    int32_t cin_g, cout_g, in_total, out_total;
    KernelClass kclass;
    // tiling choice for the implicit GEMM / depthwise kernels
    int32_t cfg;                 // kernel variant index within the class
    int32_t cfg_ap = -1;         // fp32 implicit GEMM: variant that reads packed weights (-1 = none)
    int32_t tile_h, tile_w;
    int32_t lds_bytes;
    int32_t stages;
    int32_t pt_vertical;
    bool flatten_1x1;            // 1x1/s1/p0: treat [h][w] as one row of h*w pixels
    // bf16 and int8 3x3 implicit GEMM, forward calls given OIHW weights: the
    // weights re-laid into the kernel's per-chunk LDS images before every
    // such call.
    // The buffer is allocated by the first such call, on the device current
    // then; wpack_ev is recorded after each call's kernels, and the next call
    // waits for it on its own stream before it refills the buffer, so calls
    // on any streams see their own weights; mu serialises the host side.
    void* wpack = nullptr;
    int64_t wpack_bytes = 0;
    int wpack_device = -1;
    hipEvent_t wpack_ev = nullptr;
    std::mutex mu;
    // bf16 implicit GEMM: patch geometry fixed at planning (rows, columns,
    // column shift, 8-pixel vectors per row, LDS row / plane stride in cells,
    // stride-2 half width)
    int32_t g_ph = 0, g_span = 0, g_shift = 0, g_nvr = 0, g_rs = 0, g_plane = 0, g_half = 0;
    // fp32 implicit GEMM: bytes of the fragment-order weight image its
    // packed-weight kernel reads (0 = the configuration has none).
    int64_t apack_bytes = 0;
    // AUTO fp32 3x3 descriptor whose bound weights run the Winograd kernel:
    // set at bind when winograd_bound_preferred holds; the packed image is
    // then U = G g G^T (pack_winograd_f32_weights), and calls that pass
    // their own weights keep the implicit GEMM.
    bool wino_bound = false;
    bool wino4_bound = false;   // AUTO fp32 3x3 with bound weights: Winograd F(4x4)
    // Weights bound with conv2d_desc_bind_weights: an OIHW copy at wbound,
    // followed for the bf16 implicit GEMM, the Winograd kernel, the int8 3x3
    // implicit GEMM (and the fp32 implicit GEMM when apack_bytes > 0) by the
    // packed image at wbound + wbound_pack_off (0 = no packed image).
    void* wbound = nullptr;
    int64_t wbound_bytes = 0;
    int64_t wbound_pack_off = 0;
    int wbound_device = -1;
    bool bound = false;
};

// Launchers (implemented next to their kernels).  Each returns the
// hipError_t of the launch.
// wpacked: the bound weights in fragment order (pack_igemm_f32_weights), or
// null; the packed-weight kernel runs when the configuration has one and the
// input is 16-byte aligned, else the kernel reading a.wptr (OIHW).
hipError_t launch_igemm_f32(const Desc& d, ConvArgs a, hipStream_t s, const void* wpacked = nullptr);
// OIHW fp32 weights -> the fragment-order image at dst (d.apack_bytes bytes).
hipError_t pack_igemm_f32_weights(const Desc& d, const void* w, void* dst, hipStream_t s);
// packed: the weights already in the kernel's layout (bound weights), or
// null to pack a.wptr (OIHW) into pack_buf (d.wpack_bytes bytes) first.
hipError_t launch_igemm_bf16(const Desc& d, ConvArgs a, hipStream_t s, const void* packed, void* pack_buf);
// OIHW bf16 weights -> the bf16 implicit GEMM's per-chunk LDS images at dst
// (d.wpack_bytes bytes).
hipError_t pack_igemm_bf16_weights(const Desc& d, const void* w, void* dst, hipStream_t s);
hipError_t launch_dw(const Desc& d, ConvArgs a, hipStream_t s);
hipError_t launch_qdw(const Desc& d, ConvArgs a, hipStream_t s);
// wpacked: the weights re-laid into the 3x3 kernel's per-chunk LDS images
// (pack_igemm_i8_weights), or null for the kernel that reads a.wptr (OIHW).
// The 3x3 kernel runs when wpacked is given and igemm_i8_fast holds.
hipError_t launch_igemm_i8(const Desc& d, ConvArgs a, hipStream_t s, const void* wpacked = nullptr);
// Bytes of the int8 3x3 kernel's weight images (0: the shape has no such kernel).
int64_t igemm_i8_pack_bytes(const Desc& d);
// The shape has the 3x3 kernel and x is word-aligned.
bool igemm_i8_fast(const Desc& d, const void* x);
// OIHW int8 weights -> the 3x3 kernel's per-chunk LDS images at dst
// (igemm_i8_pack_bytes bytes).
hipError_t pack_igemm_i8_weights(const Desc& d, const void* w, void* dst, hipStream_t s);
hipError_t launch_qpw(const Desc& d, ConvArgs a, hipStream_t s);
hipError_t launch_direct(const Desc& d, ConvArgs a, hipStream_t s);
hipError_t launch_grouped(const Desc& d, ConvArgs a, hipStream_t s);
// upacked: the bound weights transformed and packed (pack_winograd_f32_weights),
// or null to transform a.wptr (OIHW) in the kernel.
hipError_t launch_winograd_f32(const Desc& d, ConvArgs a, hipStream_t s, const void* upacked = nullptr);
// Bytes of the packed Winograd U image, and the pack (OIHW fp32 -> U in the
// kernel's per-lane register order).
int64_t winograd_u_bytes(const Desc& d);
hipError_t pack_winograd_f32_weights(const Desc& d, const void* w, void* dst, hipStream_t s);
// Needs 16-byte aligned rows (pointers, plane sizes and channel offsets);
// pointwise_f32_fits says whether a call's tensors allow it.
hipError_t launch_pointwise_f32(const Desc& d, ConvArgs a, hipStream_t s);
bool pointwise_f32_fits(const Desc& d, const ConvArgs& a);
hipError_t launch_qdw3(const Desc& d, ConvArgs a, hipStream_t s);
hipError_t launch_fused_pw_dw(const Desc& pw, const Desc& dw, ConvArgs apw, ConvArgs adw,
                              hipStream_t s);
hipError_t launch_fused_dw_pw(const Desc& dw, const Desc& pw, ConvArgs adw, ConvArgs apw,
                              hipStream_t s);
hipError_t launch_qfused_dw_pw(const Desc& dw, const Desc& pw, ConvArgs adw, ConvArgs apw, float comp_dw,
                               float comp_pw, int y_zp, hipStream_t s);
hipError_t launch_qfused_pw_dw(const Desc& pw, const Desc& dw, ConvArgs apw, ConvArgs adw, float comp_pw,
                               float comp_dw, int y_zp, hipStream_t s);

// Tile planners (host): fill the tiling fields of d; return false if the
// shape cannot use the class (the caller then falls back to KC_DIRECT).
bool plan_igemm_f32(Desc& d);
bool plan_igemm_bf16(Desc& d);
bool plan_dw(Desc& d);
bool plan_qdw(Desc& d);
bool plan_qpw(Desc& d);
bool plan_igemm_i8(const Desc& d);
bool plan_grouped(const Desc& d);
bool plan_winograd_f32(const Desc& d);
// Winograd F(4x4, 3x3): U packed once at bind (winograd4_u_bytes of it) and
// read by the kernel (upacked must be that image).
bool plan_winograd4_f32(const Desc& d);
// AUTO with bound weights: shapes where F(4x4) has been measured faster
// than F(2x2) and the implicit GEMM with packed weights.
bool winograd4_bound_preferred(const Desc& d);
int64_t winograd4_u_bytes(const Desc& d);
hipError_t pack_winograd4_f32_weights(const Desc& d, const void* w, void* dst, hipStream_t s);
hipError_t launch_winograd4_f32(const Desc& d, ConvArgs a, hipStream_t s, const void* upacked);
// Small fp32 3x3 layers (AUTO only): see small_f32.hip.
bool plan_small_f32(const Desc& d);
hipError_t launch_small_f32(const Desc& d, ConvArgs a, hipStream_t s);
// AUTO with bound weights: shapes where the packed-U Winograd kernel has
// been measured faster than the fp32 implicit GEMM with packed weights.
bool winograd_bound_preferred(const Desc& d);
bool plan_pointwise_f32(const Desc& d);
// fp32 pointwise 1x1 as shared 128-pixel x 128-channel GEMM tiles (pw_gemm_f32.hip);
// launch_pw_gemm_f32 needs the 16-byte alignment pointwise_f32_fits checks.
bool plan_pw_gemm_f32(const Desc& d);
hipError_t launch_pw_gemm_f32(const Desc& d, ConvArgs a, hipStream_t s);
// fp32 pointwise 1x1 narrowing a deep input to <= 32 channels (pw_narrow_f32.hip);
// same alignment needs.
bool plan_pw_narrow_f32(const Desc& d);
hipError_t launch_pw_narrow_f32(const Desc& d, ConvArgs a, hipStream_t s);
bool plan_qdw3(const Desc& d);
bool plan_fused_pw_dw(const Desc& pw, const Desc& dw, int32_t* tile_h, int32_t* lds_bytes);
// x: the input pointer (its alignment decides between vector and scalar row loads).
bool plan_fused_dw_pw(const Desc& dw, const Desc& pw, const void* x);
bool plan_qfused_dw_pw(const Desc& dw, const Desc& pw);
bool plan_qfused_pw_dw(const Desc& pw, const Desc& dw);

// Compute units of the current device (256 on MI355X; also the answer when
// no device is visible, e.g. when a descriptor is planned on a host without
// one).  Read once per process.
int device_cu_count();

// Fill the tile-dependent ConvArgs fields from a planned descriptor.


}  // namespace conv2d
