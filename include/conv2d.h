/*
 * conv2d.h -- C ABI of libconv2d.so: NCHW 2-D convolution forward on one
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes (sources: the ncnn developer guide
 * "operators.md", sections "convolution" and "convolutiondepthwise"; the Go
 * package docs "ops" of github.com/0verkilll/onnx, sections ConvOp,
 * ConvLeakyReluOp, ConvPReluOp, ConcatFusedTailOp, ReluOp, LeakyReluOp,
 * PReluOp, ClipOp; the yscv page "ONNX CPU Kernels (Conv/MatMul) -- Runtime
 * Map", section "Hot kernel paths"): every output element is the sum, over
 * the input channels of its group and the k_h x k_w window taps placed by
 * stride and dilation, of input times weight, where a tap that falls outside
 * the input image reads pad_value; the channel's bias is added to that sum
 * and the activation (none, ReLU, LeakyReLU, PReLU or Clip) is applied last.
 *
 * Layouts (all tensors dense, row-major):
 *   x       [n][in_total_channels][h][w]; the convolution reads channels
 *           [in_channel_offset, in_channel_offset + c_in).
 *   weight  OIHW: [c_out][c_in/groups][k_h][k_w].
 *   y       [n][out_total_channels][Ho][Wo]; the convolution writes channels
 *           [out_channel_offset, out_channel_offset + c_out) and no others
 *           (ConcatFusedTail: the producer writes the tail slice of a concat
 *           buffer directly, for any n).
 *   Ho = floor((h + pad_top + pad_bottom - dilation_h*(k_h-1) - 1)/stride_h) + 1,
 *   and likewise Wo.
 *   Output channel co belongs to group g = co / (c_out/groups) and reads input
 *   channels [g*c_in/groups, (g+1)*c_in/groups).
 *
 * Ownership: the caller allocates and owns every input and output buffer;
 * forward calls launch kernels asynchronously on the caller's HIP stream and
 * return, and allocate nothing (one exception, below).  Descriptors are owned by the library from
 * conv2d_desc_create until conv2d_desc_destroy; their attributes are fixed at
 * creation, and the only later change is weights bound with
 * conv2d_desc_bind_weights (a device copy the descriptor owns; see there).
 * conv2d_desc_create allocates no device memory.  Apart from the bound copy,
 * one exception to "no library device memory": a BF16 descriptor whose kernel
 * is the implicit GEMM (any BF16 dense or grouped convolution that is not
 * depthwise; conv2d_desc_kernel_name starts with "igemm_bf16") re-lays OIHW
 * weights passed to conv2d_forward into the kernel's layout in a buffer the
 * descriptor owns.  The first such call allocates it (once, on the current
 * device; freed by conv2d_desc_destroy); every such call refills it.  The
 * descriptor orders these calls itself (each one waits, on its own stream,
 * for the previous one's kernels, through an event the descriptor records),
 * so calls sharing one descriptor may come from any streams or host threads
 * and each convolves with its own weights; they then run one after another
 * on the GPU.  Calls with bound weights (w null) use no such buffer.  The
 * buffer stays on its device: a later call from another device returns
 * INVALID_ARG.
 *
 * Errors: every call returns a conv_status_t and never aborts; no C++
 * exception crosses the ABI.  conv2d_last_error() returns a thread-local
 * message for the last failing call on the calling thread.  Validation is
 * done once at descriptor creation; forward calls only check pointers and
 * aliasing, then launch.
 */
#ifndef CONV2D_MI355X_H
#define CONV2D_MI355X_H

#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define CONV2D_API __attribute__((visibility("default")))
#else
#define CONV2D_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CONV_OK = 0,
    CONV_ERR_INVALID_ARG = 1,          /* bad attribute value or null pointer */
    CONV_ERR_INCOMPATIBLE_SHAPES = 2,  /* channel/group/slope/offset shapes disagree */
    CONV_ERR_UNSUPPORTED = 3,          /* valid request outside this library's scope */
    CONV_ERR_ALIAS = 4,                /* output overlaps an input */
    CONV_ERR_HIP = 5                   /* a HIP runtime call or kernel launch failed */
} conv_status_t;

/* Activation codes of this library (ncnn does not print its numeric codes). */
typedef enum {
    CONV_ACT_NONE = 0,
    CONV_ACT_RELU = 1,        /* max(0, v) */
    CONV_ACT_LEAKY_RELU = 2,  /* v >= 0 ? v : act_params[0] * v        (alpha, default 0.01) */
    CONV_ACT_PRELU = 3,       /* v >= 0 ? v : slope[co or 0] * v       (slope passed at forward) */
    CONV_ACT_CLIP = 4         /* min(max(v, act_params[0]), act_params[1]) (defaults -FLT_MAX, FLT_MAX) */
} conv_act_t;

typedef enum {
    CONV_DTYPE_F32 = 0,   /* x, weight, y float32; fp32 accumulate */
    CONV_DTYPE_BF16 = 1,  /* x, weight, y bfloat16; fp32 accumulate and epilogue; y rounded to nearest even */
    CONV_DTYPE_I8 = 2     /* x, weight, y int8; int32 accumulate; requant (qconv2d_forward only) */
} conv_dtype_t;

typedef enum {
    CONV_ROUND_HALF_EVEN = 0,  /* default requant rounding */
    CONV_ROUND_HALF_AWAY = 1   /* ties away from zero, as the yscv requant epilogue does */
} conv_rounding_t;

/* Convolution attributes.  Fill with conv2d_params_init() and then set what
 * differs from the defaults.  Pads are ONNX order (top, left, bottom, right);
 * ncnn's chained defaults (pad_top = pad_left, ...) are the caller's job. */
/* Algorithm of a float convolution.  AUTO lets the library choose: the
 * direct tiled classes; for an F32 3x3 single-group layer with at most 64
 * input channels and at most 64K output elements, a vector-unit kernel with
 * one short chain per output pixel (conv2d_desc_kernel_name "small_f32");
 * and, binding weights to an F32 3x3 stride-1 dilation-1 single-group
 * descriptor with >= 32 input channels switches its calls with bound weights
 * to Winograd where it was measured faster (calls passing their own weights
 * keep the implicit GEMM): F(4x4, 3x3) when that grid has >= one workgroup
 * per compute unit (2 x 8 output tiles of 4 x 4 pixels x 32 output channels
 * each; conv2d_desc_kernel_name "winograd4_f32"), else F(2x2, 3x3) for <= 64
 * output channels and a grid of >= 256 workgroups (2 x 8 tiles of 2 x 2
 * pixels x 32 output channels; "winograd_f32"); DIRECT uses only the tiled classes (no
 * Winograd, no small-layer kernel); WINOGRAD
 * requests the F(2x2, 3x3) minimal
 * filtering algorithm (Lavin and Gray, CVPR 2016) for the "Winograd cells"
 * the Go package doc "ops" names among its conv fan-out sites (section
 * WorkerPool): F32 only, 3x3 window, stride 1, dilation 1, one group, any
 * pads, bias, activation and channel offsets; conv2d_desc_create returns
 * CONV_ERR_UNSUPPORTED for any other shape.  Its results differ from the
 * direct sum by fp32 rounding only.  WINOGRAD4 requests the larger tile of
 * the same paper, F(4x4, 3x3) (36 multiplies per 4x4 output tile and input
 * channel instead of 144), for the same shapes; its filter transform is
 * computed once, when the weights are bound, so conv2d_forward and
 * conv2d_forward_noalloc take only w = NULL on such a descriptor (a call
 * with weights returns CONV_ERR_UNSUPPORTED).  Its rounding differs from the
 * direct sum more than F(2x2)'s: the tests bound it by 1e-4 * (1 + |y|). */
typedef enum {
    CONV_ALGO_AUTO = 0,
    CONV_ALGO_DIRECT = 1,
    CONV_ALGO_WINOGRAD = 2,
    CONV_ALGO_WINOGRAD4 = 3
} conv_algo_t;

typedef struct {
    int32_t n, c_in, h, w;        /* input batch, channels, height, width */
    int32_t c_out, k_h, k_w;      /* output channels, kernel size */
    int32_t pad_top, pad_left, pad_bottom, pad_right;   /* >= 0, default 0 */
    int32_t stride_h, stride_w;   /* >= 1, default 1 */
    int32_t dilation_h, dilation_w; /* >= 1, default 1 */
    int32_t groups;               /* divides c_in and c_out, default 1 */
    int32_t has_bias;             /* 0/1, default 0 */
    float pad_value;              /* value of padded taps, default 0 (float paths only) */
    int32_t act_type;             /* conv_act_t, default CONV_ACT_NONE */
    float act_params[2];          /* leaky alpha; clip lo/hi.  NaN (the init value) selects
                                     the default: alpha 0.01; clip -FLT_MAX / FLT_MAX */
    int32_t prelu_slope_count;    /* 1 or c_out, default 1 */
    int32_t in_channel_offset;    /* default 0 */
    int32_t in_total_channels;    /* 0 means c_in */
    int32_t out_channel_offset;   /* default 0 */
    int32_t out_total_channels;   /* 0 means c_out */
    int32_t dtype;                /* conv_dtype_t, default CONV_DTYPE_F32 */
    int32_t int8_rounding;        /* conv_rounding_t, default CONV_ROUND_HALF_EVEN */
    int32_t algo;                 /* conv_algo_t, default CONV_ALGO_AUTO */
} conv2d_params_t;

typedef struct conv2d_desc* conv2d_desc_t;

/* Fill *p with the defaults listed above (all sizes 0).  p must not be null. */
CONV2D_API void conv2d_params_init(conv2d_params_t* p);

/* Validate *p, infer Ho/Wo and choose the kernel.  On success *out receives a
 * new descriptor owned by the library.  Errors:
 *   INVALID_ARG           null pointer; size <= 0; negative pad; stride,
 *                         dilation or kernel < 1; unknown act/dtype/rounding;
 *                         clip lo > hi; non-finite pad_value or leaky alpha;
 *                         Ho or Wo < 1 (empty output)
 *   INCOMPATIBLE_SHAPES   groups not dividing c_in and c_out; slope count not
 *                         1 or c_out; channel offset + count beyond the total
 *   UNSUPPORTED           I8 with pad_value != 0 or an activation other than
 *                         NONE/RELU; tensors beyond 2^40 elements, planes
 *                         beyond 2^31 elements */
CONV2D_API conv_status_t conv2d_desc_create(const conv2d_params_t* p, conv2d_desc_t* out);

/* Release a descriptor (null is allowed). */
CONV2D_API void conv2d_desc_destroy(conv2d_desc_t d);

/* out[0..3] = n, out_total_channels, Ho, Wo of the output buffer. */
CONV2D_API conv_status_t conv2d_desc_get_output_shape(conv2d_desc_t d, int32_t out[4]);

/* Name of the kernel class chosen at creation (static string; for logs). */
CONV2D_API const char* conv2d_desc_kernel_name(conv2d_desc_t d);

/* Bind weights to the descriptor once, as ncnn transforms and packs weights
 * once when a layer's pipeline is created instead of on every forward (the
 * yscv page, section "Hot kernel paths", likewise packs int8 weights once at
 * load).  The library copies w (OIHW, the descriptor's dtype; device
 * pointer) into a device buffer it allocates on the first bind, on the
 * current device, and owns until conv2d_desc_destroy; for the BF16 implicit
 * GEMM it also re-lays the copy into the kernel's per-chunk layout, so
 * forward calls that use the bound weights skip that step, and for the F32
 * implicit GEMM of 3x3 windows (conv2d_desc_kernel_name "igemm_f32") it packs
 * a second copy in the matrix-core operand order, which forward calls with
 * bound weights read straight into registers (calls whose input is not
 * 16-byte aligned read the OIHW copy).  The results are those of the OIHW
 * kernel bit for bit for up to 32 output channels per group; with more, the
 * packed kernel sums the input channels in another order (same tolerance).
 * For a WINOGRAD descriptor, and for an AUTO one in the Winograd regime
 * (conv_algo_t), it computes the filter transform U = G g G^T once and packs
 * it in the Winograd kernel's operand order instead; bound-weight calls then
 * run that kernel (bitwise equal to the WINOGRAD descriptor's per-call
 * weights) and conv2d_desc_kernel_name reports "winograd_f32".  Forward calls
 * (conv2d_forward, fused_pw_dw_forward, qconv2d_forward) use the bound copy
 * when their weight pointer is null.  The copy and the re-layout are queued
 * on `stream` (hipStream_t, null = default stream): forward calls on the same
 * stream see them; calls on other streams must be ordered by the caller.
 * Binding again replaces the bound weights in place (ordered the same way
 * against forward calls still reading the old ones).  Errors: INVALID_ARG for
 * a null descriptor or w, or a device other than the descriptor's; ALIAS if w
 * is the descriptor's own bound copy; HIP if the buffer cannot be allocated or
 * a copy/launch fails (no weights are then bound). */
CONV2D_API conv_status_t conv2d_desc_bind_weights(conv2d_desc_t d, const void* w, void* stream);

/* Float convolution (dtype F32 or BF16).
 *   x, w, y   device pointers of the dtype's element type, layouts above;
 *             w null = the weights bound to the descriptor (INVALID_ARG if
 *             none are bound, or they were bound on another device)
 *   bias      device float32[c_out]; required iff has_bias, else ignored
 *   slope     device float32[prelu_slope_count]; required iff act is PRELU
 *   stream    hipStream_t (null = default stream)
 * y may be the same buffer as x only when their channel ranges are disjoint
 * (ConcatFusedTail with in/out offsets); any other overlap of y with x, w,
 * bias or slope returns CONV_ERR_ALIAS.  A dtype of I8 returns INVALID_ARG. */
CONV2D_API conv_status_t conv2d_forward(conv2d_desc_t d, const void* x, const void* w, const float* bias,
                             const float* slope, void* y, void* stream);

/* Size of the device scratch array that conv2d_forward_noalloc uses on each
 * GPU (8 MiB). */
#define CONV2D_NOALLOC_SCRATCH_BYTES (8 << 20)

/* conv2d_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, checks, kernels and results as conv2d_forward, and it
 * allocates nothing.  The one buffer conv2d_forward may allocate -- the
 * re-laid weights of a BF16 implicit-GEMM descriptor given OIHW weights --
 * is replaced by a fixed device array of CONV2D_NOALLOC_SCRATCH_BYTES per
 * GPU, which the library holds from its first use on that GPU until the
 * process ends.  A descriptor whose re-laid weights do not fit returns
 * UNSUPPORTED (bind its weights instead: bound weights need no scratch).
 * Every such call on one GPU shares that array, and it keeps the last call's
 * contents (each call refills what it reads): calls that may overlap on one
 * GPU -- unordered streams, or several host threads -- race and must be
 * ordered by the caller.  Calls with bound weights (w null) and descriptors of
 * every other kernel class use no scratch and behave as conv2d_forward. */
CONV2D_API conv_status_t conv2d_forward_noalloc(conv2d_desc_t d, const void* x, const void* w,
                                                const float* bias, const float* slope, void* y, void* stream);

/* Fused pointwise 1x1 -> depthwise kxk (the yscv FusedPwDw step).  desc_pw:
 * 1x1, stride 1, pads 0, groups 1; desc_dw: groups == c_in == c_out ==
 * desc_pw.c_out, same n/h/w, same dtype (F32).  The expanded tensor stays in
 * on-chip memory; the depthwise padding applies to the pointwise output, so
 * taps outside the image read desc_dw.pad_value.  y layout is desc_dw's.
 * Pointers as in conv2d_forward (b_* / slope_* nullable per descriptor; a
 * null w_pw or w_dw selects that descriptor's bound weights).
 * The depthwise window is up to 5x5, with any stride, dilation and pads.
 * Errors: INCOMPATIBLE_SHAPES for a pair that does not chain; UNSUPPORTED for
 * a dtype other than F32, a window beyond 5x5 or rows too wide for the
 * on-chip tile; ALIAS as above. */
CONV2D_API conv_status_t fused_pw_dw_forward(conv2d_desc_t desc_pw, conv2d_desc_t desc_dw, const void* x,
                                  const void* w_pw, const float* b_pw, const float* slope_pw,
                                  const void* w_dw, const float* b_dw, const float* slope_dw,
                                  void* y, void* stream);

/* Fused depthwise kxk -> pointwise 1x1 (the yscv FusedDwPw step).  desc_dw:
 * groups == c_in == c_out, window up to 5x5, any stride, dilation and pads;
 * its input may be a channel slice of a larger buffer (in_channel_offset /
 * in_total_channels).  desc_pw: 1x1, stride 1, pads 0, groups 1, c_in ==
 * desc_dw.c_out, h/w == desc_dw's output size, same n and dtype (F32); its
 * output may be a channel slice (ConcatFusedTail).  The depthwise output stays
 * in on-chip memory; y layout is desc_pw's.  Pointers as in
 * fused_pw_dw_forward (a null w_dw or w_pw selects that descriptor's bound
 * weights).  Errors: INCOMPATIBLE_SHAPES for a pair that does not chain (or a
 * depthwise output / pointwise input with channel offsets, which have no
 * buffer here); UNSUPPORTED for a dtype other than F32, a window beyond 5x5
 * or rows too wide for the on-chip tile; ALIAS as above. */
CONV2D_API conv_status_t fused_dw_pw_forward(conv2d_desc_t desc_dw, conv2d_desc_t desc_pw, const void* x,
                                  const void* w_dw, const float* b_dw, const float* slope_dw,
                                  const void* w_pw, const float* b_pw, const float* slope_pw,
                                  void* y, void* stream);

/* Symmetric int8 QLinearConv (dtype I8): int32 accumulation, + int32 bias,
 * then q = saturate_int8(round(f32(acc + bias) * composite) + y_zp), with
 * composite = f32(f32(x_scale * w_scale) / y_scale) computed on the host and
 * round = the descriptor's int8_rounding; ReLU (if set) is max(q, y_zp).
 *   x, w, y   device int8 pointers (layouts above); w null = bound weights
 *   bias      device int32[c_out] or null
 * The sum acc + bias is formed in int32: a bias with |bias[co]| above
 * 2^31 - 1 - 128*128*(c_in/groups)*k_h*k_w may overflow it, and the output
 * is then unspecified (no such bias is rejected: the library does not read
 * device data on the host).  Any positive finite composite is allowed; the
 * saturation holds for every product, infinite ones included.
 * Errors: UNSUPPORTED if x_zp != 0 or w_zp != 0 (symmetric scheme only);
 * INVALID_ARG if a scale is not finite and positive or dtype is not I8. */
CONV2D_API conv_status_t qconv2d_forward(conv2d_desc_t d, const int8_t* x, float x_scale, int8_t x_zp,
                              const int8_t* w, float w_scale, int8_t w_zp, const int32_t* bias,
                              float y_scale, int8_t y_zp, int8_t* y, void* stream);

/* Fused int8 depthwise kxk -> pointwise 1x1 (the yscv QuantizedDwPw step):
 * two symmetric QLinearConvs as in qconv2d_forward, each with its own scale
 * triple, the int8 intermediate kept in on-chip memory.  desc_dw: I8,
 * groups == c_in == c_out, window up to 5x5, any stride, dilation and pads;
 * desc_pw: I8, 1x1, stride 1, pads 0, groups 1, c_in == desc_dw.c_out, h/w ==
 * desc_dw's output size; the depthwise output and pointwise input are plain
 * (no channel offsets), the depthwise input and pointwise output may be
 * channel slices.  The depthwise stage requantises with the composite of
 * (dw_x_scale, dw_w_scale, dw_y_scale), zero point 0 and its descriptor's
 * rounding and ReLU; the pointwise stage reads that int8 tensor and
 * requantises with the composite of (pw_x_scale, pw_w_scale, pw_y_scale),
 * y_zp and its descriptor's rounding and ReLU.  The output is bitwise that
 * of qconv2d_forward(desc_dw, x, dw_x_scale, 0, w_dw, dw_w_scale, 0, b_dw,
 * dw_y_scale, 0, tmp) followed by qconv2d_forward(desc_pw, tmp, pw_x_scale,
 * 0, w_pw, pw_w_scale, 0, b_pw, pw_y_scale, y_zp, y) (pw_x_scale is normally
 * dw_y_scale; both are taken so that any pair of stages fuses).  Null w_dw /
 * w_pw select bound weights; biases are device int32 or null.  Errors:
 * INVALID_ARG for a non-I8 descriptor, a scale or composite that is not
 * finite and positive, or null pointers; INCOMPATIBLE_SHAPES / UNSUPPORTED /
 * ALIAS as for fused_dw_pw_forward. */
CONV2D_API conv_status_t qfused_dw_pw_forward(conv2d_desc_t desc_dw, conv2d_desc_t desc_pw, const int8_t* x,
                                   const int8_t* w_dw, const int32_t* b_dw, float dw_x_scale,
                                   float dw_w_scale, float dw_y_scale, const int8_t* w_pw,
                                   const int32_t* b_pw, float pw_x_scale, float pw_w_scale,
                                   float pw_y_scale, int8_t y_zp, int8_t* y, void* stream);

/* Fused int8 pointwise 1x1 -> depthwise kxk (the yscv QuantizedPwDw step):
 * two symmetric QLinearConvs as in qconv2d_forward, each with its own scale
 * triple, the int8 expansion kept in on-chip memory.  desc_pw: I8, 1x1,
 * stride 1, pads 0, groups 1; desc_dw: I8, groups == c_in == c_out ==
 * desc_pw.c_out, same n/h/w, window up to 5x5, any stride, dilation and
 * pads.  The pointwise input may be a channel slice (in_channel_offset /
 * in_total_channels) and the depthwise output may be one (ConcatFusedTail);
 * the expansion has no buffer, so the pointwise output and depthwise input
 * carry no channel offsets.  The pointwise stage requantises with the
 * composite of (pw_x_scale, pw_w_scale, pw_y_scale), zero point 0 and its
 * descriptor's rounding and ReLU; the depthwise stage reads that int8 tensor,
 * its taps outside the image reading the intermediate's zero point (0: the
 * depthwise padding applies to the pointwise output), and requantises with
 * the composite of (dw_x_scale, dw_w_scale, dw_y_scale), y_zp and its
 * descriptor's rounding and ReLU.  The output is bitwise that of
 * qconv2d_forward(desc_pw, x, pw_x_scale, 0, w_pw, pw_w_scale, 0, b_pw,
 * pw_y_scale, 0, tmp) followed by qconv2d_forward(desc_dw, tmp, dw_x_scale,
 * 0, w_dw, dw_w_scale, 0, b_dw, dw_y_scale, y_zp, y).  Null w_pw / w_dw
 * select bound weights; biases are device int32 or null.  Errors as for
 * qfused_dw_pw_forward (UNSUPPORTED also for image rows too wide for the
 * on-chip tile). */
CONV2D_API conv_status_t qfused_pw_dw_forward(conv2d_desc_t desc_pw, conv2d_desc_t desc_dw, const int8_t* x,
                                   const int8_t* w_pw, const int32_t* b_pw, float pw_x_scale,
                                   float pw_w_scale, float pw_y_scale, const int8_t* w_dw,
                                   const int32_t* b_dw, float dw_x_scale, float dw_w_scale,
                                   float dw_y_scale, int8_t y_zp, int8_t* y, void* stream);

/* Human-readable name of a status code (static string). */
CONV2D_API const char* conv2d_status_string(conv_status_t s);

/* Detail of the last error on this thread ("" if none). */
CONV2D_API const char* conv2d_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CONV2D_MI355X_H */
