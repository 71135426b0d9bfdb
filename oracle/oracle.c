/*
 * oracle.c -- plain, slow, obviously correct CPU reference for NCHW conv2d.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only tests/, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant with the
 * HIP library.
 *
 * What it computes (the sources it follows):
 *
 *  - ncnn developer guide "operators.md", sections "convolution" and
 *    "convolutiondepthwise": pad the input with pad_value, correlate it with
 *    the kernel (kernel_h x kernel_w, stride, dilation, group), add the bias,
 *    then apply the activation.  Param ids 1..18 of those tables give the
 *    attributes and their defaults (pads top/left/bottom/right, pad_value
 *    0 by default).
 *  - Go package "ops" (github.com/0verkilll/onnx/ops), sections ConvOp,
 *    ConvLeakyReluOp, ConvPReluOp: ONNX Conv in NCHW with strides, pads
 *    (top, left, bottom, right) and dilations; bias optional; the fused
 *    activation is applied per output channel after the bias.
 *  - Same page, sections ReluOp, LeakyReluOp (x >= 0 ? x : alpha*x, alpha
 *    default 0.01), PReluOp (x >= 0 ? x : slope*x, slope scalar or one per
 *    channel), ClipOp; ncnn "clip" section (defaults -FLT_MAX / FLT_MAX).
 *  - yscv "ONNX CPU Kernels (Conv/MatMul) -- Runtime Map", section "Hot
 *    kernel paths", fused INT8 chains: int32 accumulation, requant of
 *    (acc + bias) as f32 times a composite scale, plus the output zero point,
 *    clamp to [-128, 127], optional Relu; symmetric (zero zero-points) and
 *    per-tensor scales only.
 *
 * Floating point: every product and sum is done in double.  The output size
 * is floor((H + pad_top + pad_bottom - dilation*(k-1) - 1) / stride) + 1.
 * Weights are OIHW: [c_out][c_in/groups][k_h][k_w].  Output channel co
 * belongs to group g = co / (c_out/groups) and reads input channels
 * [g*c_in/groups, (g+1)*c_in/groups).
 *
 * Integer path: the same loops with int64 accumulation (exact); padded taps
 * read the input zero point, which the symmetric scheme fixes at 0.  The
 * requant step is done in float32 scalar arithmetic: yf = f32(acc + bias) *
 * composite, then an explicit round-to-nearest (ties to even by default, ties
 * away from zero as an option), then + y_zp, then saturation.  composite is
 * f32(f32(x_scale * w_scale) / y_scale).
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (see build.py).
 */
#include <stdint.h>
#include <stddef.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_ACT_NONE = 0, ORACLE_ACT_RELU = 1, ORACLE_ACT_LEAKY_RELU = 2,
       ORACLE_ACT_PRELU = 3, ORACLE_ACT_CLIP = 4 };
enum { ORACLE_ROUND_HALF_EVEN = 0, ORACLE_ROUND_HALF_AWAY = 1 };

/* The attributes of one convolution.  Mirrored by a ctypes Structure in
 * oracle/__init__.py; all sizes are plain element counts. */
typedef struct {
    int64_t n, c_in, h, w, c_out, k_h, k_w;
    int64_t pad_top, pad_left, pad_bottom, pad_right;
    int64_t stride_h, stride_w, dilation_h, dilation_w, groups;
    double pad_value;
    int64_t act_type;
    double act_p0, act_p1;     /* leaky: alpha; clip: lo, hi */
    int64_t slope_count;       /* prelu: 1 or c_out */
} oracle_conv_t;

int64_t oracle_out_h(const oracle_conv_t* p) {
    int64_t num = p->h + p->pad_top + p->pad_bottom - p->dilation_h * (p->k_h - 1) - 1;
    return num < 0 ? 0 : num / p->stride_h + 1;
}

int64_t oracle_out_w(const oracle_conv_t* p) {
    int64_t num = p->w + p->pad_left + p->pad_right - p->dilation_w * (p->k_w - 1) - 1;
    return num < 0 ? 0 : num / p->stride_w + 1;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Activation applied after the bias (ncnn "convolution": y = activation(x3)). */
static double activate(const oracle_conv_t* p, const double* slope, int64_t co, double v) {
    switch (p->act_type) {
    case ORACLE_ACT_RELU:
        return v > 0.0 ? v : 0.0;
    case ORACLE_ACT_LEAKY_RELU:
        return v >= 0.0 ? v : p->act_p0 * v;
    case ORACLE_ACT_PRELU: {
        double a = slope[p->slope_count == 1 ? 0 : co];
        return v >= 0.0 ? v : a * v;
    }
    case ORACLE_ACT_CLIP: {
        double t = v < p->act_p0 ? p->act_p0 : v;
        return t > p->act_p1 ? p->act_p1 : t;
    }
    default:
        return v;
    }
}

/* Pre-activation value of output element (n, co, ho, wo): the correlation of
 * the pad_value-padded input with the kernel, plus the bias. */
static double conv_point(const oracle_conv_t* p, const double* x, const double* w,
                         const double* bias, int64_t n, int64_t co, int64_t ho, int64_t wo) {
    const int64_t cin_g = p->c_in / p->groups;
    const int64_t cout_g = p->c_out / p->groups;
    const int64_t g = co / cout_g;
    double acc = 0.0;
    for (int64_t ci = 0; ci < cin_g; ++ci) {
        const int64_t c = g * cin_g + ci;
        for (int64_t r = 0; r < p->k_h; ++r) {
            const int64_t ih = ho * p->stride_h - p->pad_top + r * p->dilation_h;
            for (int64_t s = 0; s < p->k_w; ++s) {
                const int64_t iw = wo * p->stride_w - p->pad_left + s * p->dilation_w;
                double xv;
                if (ih >= 0 && ih < p->h && iw >= 0 && iw < p->w)
                    xv = x[((n * p->c_in + c) * p->h + ih) * p->w + iw];
                else
                    xv = p->pad_value;
                const double wv = w[((co * cin_g + ci) * p->k_h + r) * p->k_w + s];
                acc += xv * wv;
            }
        }
    }
    return acc + (bias ? bias[co] : 0.0);
}

/* Full output y[n][c_out][Ho][Wo] (dense, its own buffer). */
void oracle_conv2d_f64(const oracle_conv_t* p, const double* x, const double* w,
                       const double* bias, const double* slope, double* y) {
    const int64_t ho_n = oracle_out_h(p), wo_n = oracle_out_w(p);
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t n = 0; n < p->n; ++n)
        for (int64_t co = 0; co < p->c_out; ++co)
            for (int64_t ho = 0; ho < ho_n; ++ho)
                for (int64_t wo = 0; wo < wo_n; ++wo) {
                    double v = conv_point(p, x, w, bias, n, co, ho, wo);
                    y[((n * p->c_out + co) * ho_n + ho) * wo_n + wo] = activate(p, slope, co, v);
                }
}

/* Selected outputs only: idx[i] is a flat index into [n][c_out][Ho][Wo]. */
void oracle_conv2d_points_f64(const oracle_conv_t* p, const double* x, const double* w,
                              const double* bias, const double* slope,
                              const int64_t* idx, int64_t count, double* out) {
    const int64_t ho_n = oracle_out_h(p), wo_n = oracle_out_w(p);
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i) {
        int64_t t = idx[i];
        const int64_t wo = t % wo_n; t /= wo_n;
        const int64_t ho = t % ho_n; t /= ho_n;
        const int64_t co = t % p->c_out; t /= p->c_out;
        const int64_t n = t;
        out[i] = activate(p, slope, co, conv_point(p, x, w, bias, n, co, ho, wo));
    }
}

/* ---------------------------------------------------------------- int8 --- */

/* Exact int64 accumulation of output (n, co, ho, wo); padded taps read x_zp. */
static int64_t qconv_point(const oracle_conv_t* p, const int8_t* x, const int8_t* w,
                           int64_t x_zp, int64_t n, int64_t co, int64_t ho, int64_t wo) {
    const int64_t cin_g = p->c_in / p->groups;
    const int64_t cout_g = p->c_out / p->groups;
    const int64_t g = co / cout_g;
    int64_t acc = 0;
    for (int64_t ci = 0; ci < cin_g; ++ci) {
        const int64_t c = g * cin_g + ci;
        for (int64_t r = 0; r < p->k_h; ++r) {
            const int64_t ih = ho * p->stride_h - p->pad_top + r * p->dilation_h;
            for (int64_t s = 0; s < p->k_w; ++s) {
                const int64_t iw = wo * p->stride_w - p->pad_left + s * p->dilation_w;
                int64_t xv;
                if (ih >= 0 && ih < p->h && iw >= 0 && iw < p->w)
                    xv = x[((n * p->c_in + c) * p->h + ih) * p->w + iw];
                else
                    xv = x_zp;
                acc += xv * (int64_t)w[((co * cin_g + ci) * p->k_h + r) * p->k_w + s];
            }
        }
    }
    return acc;
}

/* composite = f32(f32(x_scale * w_scale) / y_scale), each step rounded to f32. */
float oracle_composite_scale(float x_scale, float w_scale, float y_scale) {
    volatile float prod = x_scale * w_scale;
    volatile float comp = prod / y_scale;
    return comp;
}

/* Round a float to the nearest integer; exact halves go to the even integer
 * (mode 0) or away from zero (mode 1).  Written out from the definition, so it
 * does not depend on the floating-point environment. */
static float round_to_integer(float v, int mode) {
    const float a = fabsf(v);
    const float f = floorf(a);
    const float d = a - f;           /* exact: f and a share the exponent range */
    float r;
    if (d > 0.5f)
        r = f + 1.0f;
    else if (d < 0.5f)
        r = f;
    else if (mode == ORACLE_ROUND_HALF_AWAY)
        r = f + 1.0f;
    else
        r = (fmodf(f, 2.0f) == 0.0f) ? f : f + 1.0f;
    return v < 0.0f ? -r : r;
}

/* Requantise one int32 value (accumulator plus bias) to int8. */
int8_t oracle_requant(int64_t v, float composite, int rounding, int64_t y_zp, int relu) {
    const float vf = (float)v;       /* exact for |v| < 2^24 */
    volatile float yf = vf * composite;
    float r = round_to_integer(yf, rounding);
    /* Saturation to int8 makes every |r| beyond 256 equivalent; bounding r
       first keeps the integer conversion defined for any product, an
       infinite one (a large composite) included. */
    if (r > 512.0f) r = 512.0f;
    if (r < -512.0f) r = -512.0f;
    int64_t q = (int64_t)r + y_zp;
    if (q < -128) q = -128;
    if (q > 127) q = 127;
    if (relu && q < y_zp) q = y_zp;
    return (int8_t)q;
}

/* Exact accumulators (no bias), dense [n][c_out][Ho][Wo] int64. */
void oracle_qconv2d_acc(const oracle_conv_t* p, const int8_t* x, const int8_t* w,
                        int64_t x_zp, int64_t* acc) {
    const int64_t ho_n = oracle_out_h(p), wo_n = oracle_out_w(p);
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t n = 0; n < p->n; ++n)
        for (int64_t co = 0; co < p->c_out; ++co)
            for (int64_t ho = 0; ho < ho_n; ++ho)
                for (int64_t wo = 0; wo < wo_n; ++wo)
                    acc[((n * p->c_out + co) * ho_n + ho) * wo_n + wo] =
                        qconv_point(p, x, w, x_zp, n, co, ho, wo);
}

/* Full int8 QLinearConv output: accumulate, + bias, requantise. */
void oracle_qconv2d(const oracle_conv_t* p, const int8_t* x, const int8_t* w,
                    const int32_t* bias, int64_t x_zp, float composite, int rounding,
                    int64_t y_zp, int relu, int8_t* y) {
    const int64_t ho_n = oracle_out_h(p), wo_n = oracle_out_w(p);
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t n = 0; n < p->n; ++n)
        for (int64_t co = 0; co < p->c_out; ++co)
            for (int64_t ho = 0; ho < ho_n; ++ho)
                for (int64_t wo = 0; wo < wo_n; ++wo) {
                    int64_t v = qconv_point(p, x, w, x_zp, n, co, ho, wo) + (bias ? bias[co] : 0);
                    y[((n * p->c_out + co) * ho_n + ho) * wo_n + wo] =
                        oracle_requant(v, composite, rounding, y_zp, relu);
                }
}

/* Selected int8 outputs, flat indices into [n][c_out][Ho][Wo]. */
void oracle_qconv2d_points(const oracle_conv_t* p, const int8_t* x, const int8_t* w,
                           const int32_t* bias, int64_t x_zp, float composite, int rounding,
                           int64_t y_zp, int relu, const int64_t* idx, int64_t count,
                           int8_t* out) {
    const int64_t ho_n = oracle_out_h(p), wo_n = oracle_out_w(p);
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i) {
        int64_t t = idx[i];
        const int64_t wo = t % wo_n; t /= wo_n;
        const int64_t ho = t % ho_n; t /= ho_n;
        const int64_t co = t % p->c_out; t /= p->c_out;
        const int64_t n = t;
        int64_t v = qconv_point(p, x, w, x_zp, n, co, ho, wo) + (bias ? bias[co] : 0);
        out[i] = oracle_requant(v, composite, rounding, y_zp, relu);
    }
}

/* Elementwise requant of a list of int64 values (for tests of that step). */
void oracle_requant_array(const int64_t* v, int64_t count, float composite, int rounding,
                          int64_t y_zp, int relu, int8_t* out) {
    for (int64_t i = 0; i < count; ++i)
        out[i] = oracle_requant(v[i], composite, rounding, y_zp, relu);
}
