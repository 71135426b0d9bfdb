// C ABI of libconv2d.so: descriptor creation and validation, kernel choice,
// pointer and alias checks, dispatch.  Host code only.
//
// Attributes are checked once, when the descriptor is made, and the forward
// calls then only check their pointers: the prepared-execution design of the
// onnx-light-cpu "Binary Kernel Design" page (sections "Prepared execution"
// and "Compute, scheduling, and safety").  The output may share a buffer
// with the input only where the two channel ranges are disjoint, so no input
// element is overwritten before a kernel has read it; any other overlap is
// refused.  Status codes follow the error returns of the Go "ops" page
// (section PReluOp: a slope count that is neither 1 nor the channel count is
// ErrIncompatibleShapes).
#include <cfloat>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>

#include "conv2d_internal.h"

using namespace conv2d;

int conv2d::device_cu_count() {
    static const int n = [] {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            return v;
        return 256;
    }();
    return n;
}

namespace {

thread_local char g_last_error[512] = "";

conv_status_t fail(conv_status_t s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

conv_status_t ok() {
    g_last_error[0] = '\0';
    return CONV_OK;
}

const char* kernel_name(const Desc& d) {
    switch (d.kclass) {
    case KC_IGEMM_F32:
        return d.wino4_bound ? "winograd4_f32"
               : d.wino_bound ? "winograd_f32"
               : d.flatten_1x1 ? "igemm_f32_pointwise"
                               : "igemm_f32";
    case KC_IGEMM_BF16: return d.flatten_1x1 ? "igemm_bf16_pointwise" : "igemm_bf16";
    case KC_DW: return d.p.dtype == CONV_DTYPE_BF16 ? "depthwise_bf16" : "depthwise_f32";
    case KC_QDW: return d.cfg == 1 ? "depthwise_i8_dot4" : "depthwise_i8";
    case KC_QPW: return "pointwise_i8_mfma";
    case KC_DIRECT: return "direct";
    case KC_GROUPED: return d.p.dtype == CONV_DTYPE_BF16 ? "grouped_bf16" : "grouped_f32";
    case KC_WINOGRAD_F32: return "winograd_f32";
    case KC_WINOGRAD4_F32: return "winograd4_f32";
    case KC_PW_F32: return "pointwise_f32";
    case KC_PWG_F32: return "pw_gemm_f32";
    case KC_PWN_F32: return "pw_narrow_f32";
    case KC_IGEMM_I8: return "igemm_i8";
    case KC_SMALL_F32: return "small_f32";
    }
    return "?";
}

size_t elem_size(int32_t dtype) {
    return dtype == CONV_DTYPE_F32 ? 4 : dtype == CONV_DTYPE_BF16 ? 2 : 1;
}

// Byte ranges of a tensor view: n blocks of `len` bytes, `stride` apart.
struct View {
    uintptr_t base;
    int64_t n;
    int64_t stride;
    int64_t len;
    int64_t first() const { return 0; }
};

// Do two strided views overlap?  Both are lists of n equal-length blocks at a
// constant stride; walk them in address order (two pointers, O(n1 + n2)).
bool views_overlap(const View& a, const View& b) {
    if (a.len == 0 || b.len == 0 || a.n == 0 || b.n == 0) return false;
    const uintptr_t a_end = a.base + (uintptr_t)((a.n - 1) * a.stride + a.len);
    const uintptr_t b_end = b.base + (uintptr_t)((b.n - 1) * b.stride + b.len);
    if (a_end <= b.base || b_end <= a.base) return false;
    int64_t i = 0, j = 0;
    while (i < a.n && j < b.n) {
        const uintptr_t as = a.base + (uintptr_t)(i * a.stride), ae = as + (uintptr_t)a.len;
        const uintptr_t bs = b.base + (uintptr_t)(j * b.stride), be = bs + (uintptr_t)b.len;
        if (as < be && bs < ae) return true;
        if (ae <= be) ++i; else ++j;
    }
    return false;
}

View flat(const void* p, int64_t bytes) { return View{(uintptr_t)p, 1, 0, bytes}; }

View x_view(const Desc& d, const void* x) {
    const int64_t plane = (int64_t)d.p.h * d.p.w * (int64_t)elem_size(d.p.dtype);
    return View{(uintptr_t)x + (uintptr_t)(d.p.in_channel_offset * plane), d.p.n,
                (int64_t)d.in_total * plane, (int64_t)d.p.c_in * plane};
}

View y_view(const Desc& d, const void* y) {
    const int64_t plane = (int64_t)d.ho * d.wo * (int64_t)elem_size(d.p.dtype);
    return View{(uintptr_t)y + (uintptr_t)(d.p.out_channel_offset * plane), d.p.n,
                (int64_t)d.out_total * plane, (int64_t)d.p.c_out * plane};
}

int64_t w_bytes(const Desc& d) {
    return (int64_t)d.p.c_out * d.cin_g * d.p.k_h * d.p.k_w * (int64_t)elem_size(d.p.dtype);
}

ConvArgs make_args(const Desc& d, const void* x, const void* w, const float* bias, const float* slope,
                   void* y) {
    ConvArgs a;
    memset(&a, 0, sizeof(a));
    const conv2d_params_t& p = d.p;
    a.xptr = x; a.wptr = w; a.bias = p.has_bias ? bias : nullptr;
    a.slope = p.act_type == CONV_ACT_PRELU ? slope : nullptr;
    a.yptr = y;
    a.n = p.n; a.c_in = p.c_in; a.h = p.h; a.w = p.w; a.c_out = p.c_out; a.k_h = p.k_h; a.k_w = p.k_w;
    a.pad_top = p.pad_top; a.pad_left = p.pad_left;
    a.stride_h = p.stride_h; a.stride_w = p.stride_w; a.dilation_h = p.dilation_h; a.dilation_w = p.dilation_w;
    a.groups = p.groups; a.cin_g = d.cin_g; a.cout_g = d.cout_g;
    a.ho = d.ho; a.wo = d.wo;
    a.in_total = d.in_total; a.in_off = p.in_channel_offset;
    a.out_total = d.out_total; a.out_off = p.out_channel_offset;
    a.pad_value = p.pad_value;
    a.act = p.act_type; a.act_a = p.act_params[0]; a.act_b = p.act_params[1];
    a.slope_count = p.prelu_slope_count;
    return a;
}

conv_status_t hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(CONV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

conv_status_t check_desc(conv2d_desc_t d) {
    if (!d) return fail(CONV_ERR_INVALID_ARG, "null descriptor");
    return CONV_OK;
}

// Weights a forward call uses: w itself, or (w null) the descriptor's bound
// copy, which must live on the current device.  what names the operand.
conv_status_t resolve_weights(const Desc& d, const void*& w, const char* what) {
    if (w) return CONV_OK;
    if (!d.bound) return fail(CONV_ERR_INVALID_ARG, "null %s and no weights bound to the descriptor", what);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != d.wbound_device)
        return fail(CONV_ERR_INVALID_ARG, "%s were bound on device %d, current device is %d", what, d.wbound_device, dev);
    w = d.wbound;
    return CONV_OK;
}

void free_on(void* ptr, int device) {
    if (!ptr) return;
    int cur = -1;
    const bool switched = hipGetDevice(&cur) == hipSuccess && cur != device && hipSetDevice(device) == hipSuccess;
    (void)hipFree(ptr);
    if (switched) (void)hipSetDevice(cur);
}

// AUTO picks Winograd only where it has been measured faster than the
// implicit GEMM (none yet).
bool winograd_preferred(const Desc& d) {
    (void)d;
    return false;
}

conv_status_t forward_float(conv2d_desc_t dd, const void* x, const void* w, const float* bias, const float* slope,
                            void* y, void* stream, bool noalloc);

// Scratch of conv2d_forward_noalloc: the bf16 implicit GEMM's per-call weight
// re-layout goes here instead of into a buffer the descriptor allocates.  A
// file-scope device array: every GPU the library runs on holds its own copy,
// at its own address, until the process ends.  Host code never passes the
// array's name to a kernel or a copy (on the host it is only a stand-in for
// the symbol); it uses the device address hipGetSymbolAddress returns, looked
// up once per device with that device current and kept in g_scratch_ptr.
constexpr int64_t kScratchBytes = CONV2D_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

conv_status_t scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(CONV_ERR_HIP, "no current HIP device");
    if (dev < 0 || dev >= kMaxDevices) return fail(CONV_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return fail(CONV_ERR_HIP, "address of the scratch array on device %d: %s", dev,
                                               hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CONV_OK;
}

// A bf16 (or int8 3x3) implicit-GEMM forward call given OIHW weights:
// re-lay them into the descriptor's pack buffer, then convolve.  The buffer
// is allocated by the first such call, on the current device.  Each call
// waits, on its own stream, for the event recorded after the previous call's
// kernels (which read the buffer), refills the buffer, convolves and records
// the event, all under the descriptor's mutex: calls sharing the descriptor
// may come from any streams and host threads and each one convolves with its
// own weights.
conv_status_t forward_repack(Desc& d, const ConvArgs& a, hipStream_t s) {
    std::lock_guard<std::mutex> lock(d.mu);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(CONV_ERR_HIP, "no current HIP device");
    if (!d.wpack) {
        hipError_t e = hipMalloc(&d.wpack, (size_t)d.wpack_bytes);
        if (e != hipSuccess) {
            d.wpack = nullptr;
            return fail(CONV_ERR_HIP, "allocating %lld bytes for the packed weights: %s",
                        (long long)d.wpack_bytes, hipGetErrorString(e));
        }
        e = hipEventCreateWithFlags(&d.wpack_ev, hipEventDisableTiming);
        if (e != hipSuccess) {
            (void)hipFree(d.wpack);
            d.wpack = nullptr;
            d.wpack_ev = nullptr;
            return hip_status(e, "creating the pack buffer's event");
        }
        d.wpack_device = dev;
    } else if (dev != d.wpack_device) {
        return fail(CONV_ERR_INVALID_ARG, "the weight pack buffer lives on device %d, current device is %d",
                    d.wpack_device, dev);
    }
    hipError_t e = hipStreamWaitEvent(s, d.wpack_ev, 0);
    if (d.kclass == KC_IGEMM_I8) {
        if (e == hipSuccess) e = pack_igemm_i8_weights(d, a.wptr, d.wpack, s);
        if (e == hipSuccess) e = launch_igemm_i8(d, a, s, d.wpack);
    } else {
        if (e == hipSuccess) e = launch_igemm_bf16(d, a, s, nullptr, d.wpack);
    }
    if (e == hipSuccess) e = hipEventRecord(d.wpack_ev, s);
    return hip_status(e, kernel_name(d));
}

}  // namespace

extern "C" {

void conv2d_params_init(conv2d_params_t* p) {
    if (!p) return;
    memset(p, 0, sizeof(*p));
    p->stride_h = p->stride_w = 1;
    p->dilation_h = p->dilation_w = 1;
    p->groups = 1;
    p->pad_value = 0.0f;
    p->act_type = CONV_ACT_NONE;
    // NaN selects the activation's default at descriptor creation.
    p->act_params[0] = NAN;
    p->act_params[1] = NAN;
    p->prelu_slope_count = 1;
    p->dtype = CONV_DTYPE_F32;
    p->int8_rounding = CONV_ROUND_HALF_EVEN;
    p->algo = CONV_ALGO_AUTO;
}

conv_status_t conv2d_desc_create(const conv2d_params_t* pin, conv2d_desc_t* out) {
    if (!pin || !out) return fail(CONV_ERR_INVALID_ARG, "null params or output pointer");
    *out = nullptr;
    conv2d_params_t p = *pin;
    // Activation defaults: LeakyReLU alpha 0.01 (Go ops LeakyReluOp); Clip
    // -FLT_MAX / FLT_MAX (ncnn clip).  Unused slots are zeroed.
    if (p.act_type == CONV_ACT_LEAKY_RELU) {
        if (std::isnan(p.act_params[0])) p.act_params[0] = 0.01f;
        p.act_params[1] = 0.0f;
    } else if (p.act_type == CONV_ACT_CLIP) {
        if (std::isnan(p.act_params[0])) p.act_params[0] = -FLT_MAX;
        if (std::isnan(p.act_params[1])) p.act_params[1] = FLT_MAX;
    } else {
        p.act_params[0] = p.act_params[1] = 0.0f;
    }
    if (p.n <= 0 || p.c_in <= 0 || p.h <= 0 || p.w <= 0 || p.c_out <= 0)
        return fail(CONV_ERR_INVALID_ARG, "n, c_in, h, w, c_out must be positive");
    if (p.k_h <= 0 || p.k_w <= 0) return fail(CONV_ERR_INVALID_ARG, "kernel size must be positive");
    if (p.stride_h <= 0 || p.stride_w <= 0) return fail(CONV_ERR_INVALID_ARG, "stride must be >= 1");
    if (p.dilation_h <= 0 || p.dilation_w <= 0) return fail(CONV_ERR_INVALID_ARG, "dilation must be >= 1");
    if (p.pad_top < 0 || p.pad_left < 0 || p.pad_bottom < 0 || p.pad_right < 0)
        return fail(CONV_ERR_INVALID_ARG, "pads must be >= 0");
    if (p.dtype < CONV_DTYPE_F32 || p.dtype > CONV_DTYPE_I8) return fail(CONV_ERR_INVALID_ARG, "unknown dtype %d", p.dtype);
    if (p.act_type < CONV_ACT_NONE || p.act_type > CONV_ACT_CLIP)
        return fail(CONV_ERR_INVALID_ARG, "unknown activation %d", p.act_type);
    if (p.int8_rounding != CONV_ROUND_HALF_EVEN && p.int8_rounding != CONV_ROUND_HALF_AWAY)
        return fail(CONV_ERR_INVALID_ARG, "unknown rounding %d", p.int8_rounding);
    if (p.has_bias != 0 && p.has_bias != 1) return fail(CONV_ERR_INVALID_ARG, "has_bias must be 0 or 1");
    if (p.algo < CONV_ALGO_AUTO || p.algo > CONV_ALGO_WINOGRAD4) return fail(CONV_ERR_INVALID_ARG, "unknown algo %d", p.algo);
    if (!std::isfinite(p.pad_value)) return fail(CONV_ERR_INVALID_ARG, "pad_value must be finite");
    if (p.groups <= 0) return fail(CONV_ERR_INVALID_ARG, "groups must be >= 1");
    if (p.c_in % p.groups || p.c_out % p.groups)
        return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "groups (%d) must divide c_in (%d) and c_out (%d)", p.groups,
                    p.c_in, p.c_out);
    if (p.act_type == CONV_ACT_LEAKY_RELU && !std::isfinite(p.act_params[0]))
        return fail(CONV_ERR_INVALID_ARG, "leaky alpha must be finite");
    if (p.act_type == CONV_ACT_CLIP) {
        if (p.act_params[0] > p.act_params[1]) return fail(CONV_ERR_INVALID_ARG, "clip lo > hi");
    }
    if (p.act_type == CONV_ACT_PRELU && p.prelu_slope_count != 1 && p.prelu_slope_count != p.c_out)
        return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "PReLU slope count %d is neither 1 nor c_out (%d)",
                    p.prelu_slope_count, p.c_out);
    const int32_t in_total = p.in_total_channels ? p.in_total_channels : p.c_in;
    const int32_t out_total = p.out_total_channels ? p.out_total_channels : p.c_out;
    if (p.in_total_channels < 0 || p.out_total_channels < 0 || p.in_channel_offset < 0 || p.out_channel_offset < 0)
        return fail(CONV_ERR_INVALID_ARG, "channel offsets and totals must be >= 0");
    if ((int64_t)p.in_channel_offset + p.c_in > in_total)
        return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "input channels [%d, %d) exceed in_total_channels %d",
                    p.in_channel_offset, p.in_channel_offset + p.c_in, in_total);
    if ((int64_t)p.out_channel_offset + p.c_out > out_total)
        return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "output channels [%d, %d) exceed out_total_channels %d",
                    p.out_channel_offset, p.out_channel_offset + p.c_out, out_total);
    const int64_t hnum = (int64_t)p.h + p.pad_top + p.pad_bottom - (int64_t)p.dilation_h * (p.k_h - 1) - 1;
    const int64_t wnum = (int64_t)p.w + p.pad_left + p.pad_right - (int64_t)p.dilation_w * (p.k_w - 1) - 1;
    if (hnum < 0 || wnum < 0) return fail(CONV_ERR_INVALID_ARG, "empty output: kernel extent exceeds padded input");
    const int64_t ho = hnum / p.stride_h + 1, wo = wnum / p.stride_w + 1;
    if (ho > INT32_MAX || wo > INT32_MAX) return fail(CONV_ERR_UNSUPPORTED, "output too large");
    if ((int64_t)p.n * in_total * p.h * p.w >= (int64_t)1 << 40 ||
        (int64_t)p.n * out_total * ho * wo >= (int64_t)1 << 40)
        return fail(CONV_ERR_UNSUPPORTED, "tensor too large");
    if ((int64_t)p.h * p.w > INT32_MAX || ho * wo > INT32_MAX || (int64_t)p.c_in * p.k_h * p.k_w > INT32_MAX)
        return fail(CONV_ERR_UNSUPPORTED, "plane or filter too large");
    if (p.dtype == CONV_DTYPE_I8) {
        if (p.pad_value != 0.0f)
            return fail(CONV_ERR_UNSUPPORTED, "int8: padded taps read the zero point (0); pad_value must be 0");
        if (p.act_type != CONV_ACT_NONE && p.act_type != CONV_ACT_RELU)
            return fail(CONV_ERR_UNSUPPORTED, "int8: only NONE or RELU may follow the requant");
    }

    Desc* d = new (std::nothrow) Desc();
    if (!d) return fail(CONV_ERR_INVALID_ARG, "out of host memory");
    d->p = p;
    d->ho = (int32_t)ho;
    d->wo = (int32_t)wo;
    d->cin_g = p.c_in / p.groups;
    d->cout_g = p.c_out / p.groups;
    d->in_total = in_total;
    d->out_total = out_total;
    d->flatten_1x1 = false;
    const bool depthwise = p.groups == p.c_in && p.groups == p.c_out;

    bool planned = false;
    if (p.algo == CONV_ALGO_WINOGRAD) {
        if (!plan_winograd_f32(*d)) {
            delete d;
            return fail(CONV_ERR_UNSUPPORTED, "Winograd F(2x2,3x3) needs F32, a 3x3 window, stride 1, dilation 1 "
                                              "and one group");
        }
        d->kclass = KC_WINOGRAD_F32;
        planned = true;
    } else if (p.algo == CONV_ALGO_WINOGRAD4) {
        if (!plan_winograd4_f32(*d)) {
            delete d;
            return fail(CONV_ERR_UNSUPPORTED, "Winograd F(4x4,3x3) needs F32, a 3x3 window, stride 1, dilation 1 "
                                              "and one group");
        }
        d->kclass = KC_WINOGRAD4_F32;
        planned = true;
    } else if (p.algo == CONV_ALGO_AUTO && winograd_preferred(*d)) {
        d->kclass = KC_WINOGRAD_F32;
        planned = true;
    } else if (p.dtype == CONV_DTYPE_I8) {
        if (depthwise) {
            d->kclass = KC_QDW;
            planned = plan_qdw(*d);
        } else if (plan_qpw(*d)) {
            d->kclass = KC_QPW;
            planned = true;
        } else {
            d->kclass = KC_IGEMM_I8;
            planned = plan_igemm_i8(*d);
            d->wpack_bytes = planned ? igemm_i8_pack_bytes(*d) : 0;
        }
    } else if (depthwise) {
        d->kclass = KC_DW;
        planned = plan_dw(*d);
    } else if (p.algo == CONV_ALGO_AUTO && plan_small_f32(*d)) {
        d->kclass = KC_SMALL_F32;
        planned = true;
    } else if (plan_grouped(*d)) {
        d->kclass = KC_GROUPED;
        planned = true;
    } else if (p.dtype == CONV_DTYPE_F32) {
        // The implicit GEMM is planned in every case: it also serves the
        // pointwise class when a call's tensors are not 16-byte aligned.
        d->kclass = KC_IGEMM_F32;
        planned = plan_igemm_f32(*d);
        if (planned && plan_pointwise_f32(*d)) d->kclass = KC_PW_F32;
        else if (planned && plan_pw_gemm_f32(*d)) d->kclass = KC_PWG_F32;
        else if (planned && plan_pw_narrow_f32(*d)) d->kclass = KC_PWN_F32;
    } else {
        d->kclass = KC_IGEMM_BF16;
        planned = plan_igemm_bf16(*d);
    }
    if (!planned) {
        d->kclass = KC_DIRECT;
        d->flatten_1x1 = false;
        d->wpack_bytes = 0;
    }
    *out = (conv2d_desc_t)d;
    return ok();
}

void conv2d_desc_destroy(conv2d_desc_t dd) {
    Desc* d = (Desc*)dd;
    if (!d) return;
    if (d->wpack_ev) {
        // The last call that read the pack buffer may still be running.
        (void)hipEventSynchronize(d->wpack_ev);
        (void)hipEventDestroy(d->wpack_ev);
    }
    free_on(d->wpack, d->wpack_device);
    free_on(d->wbound, d->wbound_device);
    delete d;
}

conv_status_t conv2d_desc_bind_weights(conv2d_desc_t dd, const void* w, void* stream) {
    if (check_desc(dd) != CONV_OK) return CONV_ERR_INVALID_ARG;
    Desc& d = *(Desc*)dd;
    if (!w) return fail(CONV_ERR_INVALID_ARG, "null weights");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(CONV_ERR_HIP, "no current HIP device");
    if (d.wbound && dev != d.wbound_device)
        return fail(CONV_ERR_INVALID_ARG, "weights were first bound on device %d, current device is %d",
                    d.wbound_device, dev);
    const int64_t wb = w_bytes(d);
    // AUTO fp32 3x3 layers switch to Winograd with bound weights where it was
    // measured faster: F(4x4) on grids that fill the GPU, else F(2x2).
    const bool auto_f32 = d.kclass == KC_IGEMM_F32 && d.p.algo == CONV_ALGO_AUTO;
    const bool wino4 = d.kclass == KC_WINOGRAD4_F32 || (auto_f32 && winograd4_bound_preferred(d));
    const bool wino = !wino4 && (d.kclass == KC_WINOGRAD_F32 || (auto_f32 && winograd_bound_preferred(d)));
    const bool i8pack = d.kclass == KC_IGEMM_I8 && d.wpack_bytes > 0;
    const bool packs =
        d.kclass == KC_IGEMM_BF16 || (d.kclass == KC_IGEMM_F32 && d.apack_bytes > 0) || wino || i8pack || wino4;
    const int64_t pack_bytes = d.kclass == KC_IGEMM_BF16 || i8pack ? d.wpack_bytes
                               : wino                     ? winograd_u_bytes(d)
                               : wino4                    ? winograd4_u_bytes(d)
                                                          : d.apack_bytes;
    const int64_t off = packs ? (wb + 255) / 256 * 256 : 0;
    const int64_t total = packs ? off + pack_bytes : wb;
    if (views_overlap(flat(w, wb), flat(d.wbound, d.wbound_bytes)))
        return fail(CONV_ERR_ALIAS, "w is the descriptor's own bound copy");
    if (!d.wbound) {
        const hipError_t e = hipMalloc(&d.wbound, (size_t)total);
        if (e != hipSuccess) {
            d.wbound = nullptr;
            return fail(CONV_ERR_HIP, "allocating %lld bytes for the bound weights: %s", (long long)total,
                        hipGetErrorString(e));
        }
        d.wbound_bytes = total;
        d.wbound_device = dev;
    }
    d.wbound_pack_off = packs ? off : 0;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(d.wbound, w, (size_t)wb, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess && packs)
        e = d.kclass == KC_IGEMM_BF16 ? pack_igemm_bf16_weights(d, d.wbound, (char*)d.wbound + off, s)
            : i8pack                   ? pack_igemm_i8_weights(d, d.wbound, (char*)d.wbound + off, s)
            : wino                     ? pack_winograd_f32_weights(d, d.wbound, (char*)d.wbound + off, s)
            : wino4                    ? pack_winograd4_f32_weights(d, d.wbound, (char*)d.wbound + off, s)
                                       : pack_igemm_f32_weights(d, d.wbound, (char*)d.wbound + off, s);
    if (e != hipSuccess) {
        d.bound = false;
        d.wino_bound = false;
        d.wino4_bound = false;
        return hip_status(e, "binding weights");
    }
    d.bound = true;
    d.wino_bound = wino && d.kclass == KC_IGEMM_F32;
    d.wino4_bound = wino4 && d.kclass == KC_IGEMM_F32;
    return ok();
}

conv_status_t conv2d_desc_get_output_shape(conv2d_desc_t dd, int32_t out[4]) {
    if (check_desc(dd) != CONV_OK) return CONV_ERR_INVALID_ARG;
    if (!out) return fail(CONV_ERR_INVALID_ARG, "null output array");
    const Desc& d = *(const Desc*)dd;
    out[0] = d.p.n;
    out[1] = d.out_total;
    out[2] = d.ho;
    out[3] = d.wo;
    return ok();
}

const char* conv2d_desc_kernel_name(conv2d_desc_t dd) {
    if (!dd) return "";
    return kernel_name(*(const Desc*)dd);
}

conv_status_t conv2d_forward(conv2d_desc_t dd, const void* x, const void* w, const float* bias,
                             const float* slope, void* y, void* stream) {
    return forward_float(dd, x, w, bias, slope, y, stream, false);
}

conv_status_t conv2d_forward_noalloc(conv2d_desc_t dd, const void* x, const void* w, const float* bias,
                                     const float* slope, void* y, void* stream) {
    return forward_float(dd, x, w, bias, slope, y, stream, true);
}

}  // extern "C"

namespace {

conv_status_t forward_float(conv2d_desc_t dd, const void* x, const void* w, const float* bias, const float* slope,
                            void* y, void* stream, bool noalloc) {
    if (check_desc(dd) != CONV_OK) return CONV_ERR_INVALID_ARG;
    Desc& d = *(Desc*)dd;
    if (d.p.dtype == CONV_DTYPE_I8) return fail(CONV_ERR_INVALID_ARG, "int8 descriptor: use qconv2d_forward");
    if (!x || !y) return fail(CONV_ERR_INVALID_ARG, "null x or y");
    const bool use_bound = !w;
    if (resolve_weights(d, w, "weights") != CONV_OK) return CONV_ERR_INVALID_ARG;
    if (d.p.has_bias && !bias) return fail(CONV_ERR_INVALID_ARG, "has_bias set but bias is null");
    if (d.p.act_type == CONV_ACT_PRELU && !slope) return fail(CONV_ERR_INVALID_ARG, "PReLU needs a slope pointer");
    const View yv = y_view(d, y);
    if (views_overlap(yv, x_view(d, x))) return fail(CONV_ERR_ALIAS, "y overlaps the input channels read");
    if (views_overlap(yv, flat(w, w_bytes(d)))) return fail(CONV_ERR_ALIAS, "y overlaps the weights");
    if (d.p.has_bias && views_overlap(yv, flat(bias, 4 * (int64_t)d.p.c_out)))
        return fail(CONV_ERR_ALIAS, "y overlaps the bias");
    if (d.p.act_type == CONV_ACT_PRELU && views_overlap(yv, flat(slope, 4 * (int64_t)d.p.prelu_slope_count)))
        return fail(CONV_ERR_ALIAS, "y overlaps the PReLU slopes");
    ConvArgs a = make_args(d, x, w, bias, slope, y);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    switch (d.kclass) {
    case KC_IGEMM_F32:
        if (use_bound && d.wino4_bound)
            e = launch_winograd4_f32(d, a, s, (const char*)d.wbound + d.wbound_pack_off);
        else if (use_bound && d.wino_bound)
            e = launch_winograd_f32(d, a, s, (const char*)d.wbound + d.wbound_pack_off);
        else
            e = launch_igemm_f32(d, a, s, use_bound && d.apack_bytes > 0 ? (const char*)d.wbound + d.wbound_pack_off
                                                                         : nullptr);
        break;
    case KC_IGEMM_BF16:
        if (use_bound) {
            e = launch_igemm_bf16(d, a, s, (const char*)d.wbound + d.wbound_pack_off, nullptr);
        } else if (noalloc) {
            // The re-layout goes to this GPU's scratch array instead of a
            // buffer of the descriptor's (nothing allocated, no event).
            if (d.wpack_bytes > kScratchBytes)
                return fail(CONV_ERR_UNSUPPORTED,
                            "the re-laid bf16 weights need %lld bytes, more than the %lld-byte scratch of "
                            "conv2d_forward_noalloc (bind the weights, or use conv2d_forward)",
                            (long long)d.wpack_bytes, (long long)kScratchBytes);
            void* sp = nullptr;
            const conv_status_t st = scratch_on_current_device(&sp);
            if (st != CONV_OK) return st;
            e = launch_igemm_bf16(d, a, s, nullptr, sp);
        } else {
            const conv_status_t st = forward_repack(d, a, s);
            if (st != CONV_OK) return st;
            e = hipSuccess;
        }
        break;
    case KC_DW: e = launch_dw(d, a, s); break;
    case KC_GROUPED: e = launch_grouped(d, a, s); break;
    case KC_WINOGRAD_F32:
        e = launch_winograd_f32(d, a, s, use_bound ? (const char*)d.wbound + d.wbound_pack_off : nullptr);
        break;
    case KC_WINOGRAD4_F32:
        // U exists only as the image packed when the weights were bound.
        if (!use_bound)
            return fail(CONV_ERR_UNSUPPORTED, "Winograd F(4x4,3x3) runs on bound weights: bind them with "
                                              "conv2d_desc_bind_weights and pass w = NULL");
        e = launch_winograd4_f32(d, a, s, (const char*)d.wbound + d.wbound_pack_off);
        break;
    case KC_PW_F32:
        e = pointwise_f32_fits(d, a) ? launch_pointwise_f32(d, a, s) : launch_igemm_f32(d, a, s);
        break;
    case KC_PWG_F32:
        e = pointwise_f32_fits(d, a) ? launch_pw_gemm_f32(d, a, s) : launch_igemm_f32(d, a, s);
        break;
    case KC_PWN_F32:
        e = pointwise_f32_fits(d, a) ? launch_pw_narrow_f32(d, a, s) : launch_igemm_f32(d, a, s);
        break;
    case KC_SMALL_F32: e = launch_small_f32(d, a, s); break;
    default: e = launch_direct(d, a, s); break;
    }
    return hip_status(e, kernel_name(d));
}

}  // namespace

extern "C" {

conv_status_t fused_pw_dw_forward(conv2d_desc_t dpw, conv2d_desc_t ddw, const void* x, const void* w_pw,
                                  const float* b_pw, const float* slope_pw, const void* w_dw, const float* b_dw,
                                  const float* slope_dw, void* y, void* stream) {
    if (!dpw || !ddw) return fail(CONV_ERR_INVALID_ARG, "null descriptor");
    const Desc& pw = *(const Desc*)dpw;
    const Desc& dw = *(const Desc*)ddw;
    const conv2d_params_t& P = pw.p;
    const conv2d_params_t& D = dw.p;
    if (P.dtype != D.dtype) return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "pw and dw dtypes differ");
    if (P.dtype != CONV_DTYPE_F32) return fail(CONV_ERR_UNSUPPORTED, "fused pw->dw supports F32 only");
    if (P.k_h != 1 || P.k_w != 1 || P.stride_h != 1 || P.stride_w != 1 || P.groups != 1 || P.pad_top ||
        P.pad_left || P.pad_bottom || P.pad_right)
        return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "first descriptor must be a 1x1, stride 1, unpadded, ungrouped conv");
    if (!(D.groups == D.c_in && D.groups == D.c_out))
        return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "second descriptor must be depthwise (groups == c_in == c_out)");
    if (D.c_in != P.c_out || D.n != P.n || D.h != P.h || D.w != P.w)
        return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "pw output [%d,%d,%d,%d] does not match dw input [%d,%d,%d,%d]",
                    P.n, P.c_out, P.h, P.w, D.n, D.c_in, D.h, D.w);
    if (pw.out_total != P.c_out || P.out_channel_offset != 0 || D.in_channel_offset != 0 || dw.in_total != D.c_in)
        return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "the expanded tensor has no buffer: pw output and dw input must be "
                                                  "plain (no channel offsets)");
    int32_t th = 0, lds = 0;
    if (!plan_fused_pw_dw(pw, dw, &th, &lds))
        return fail(CONV_ERR_UNSUPPORTED, "image rows too wide for the fused tile");
    if (!x || !y) return fail(CONV_ERR_INVALID_ARG, "null x or y");
    if (resolve_weights(pw, w_pw, "pointwise weights") != CONV_OK ||
        resolve_weights(dw, w_dw, "depthwise weights") != CONV_OK)
        return CONV_ERR_INVALID_ARG;
    if (P.has_bias && !b_pw) return fail(CONV_ERR_INVALID_ARG, "pw has_bias set but bias is null");
    if (D.has_bias && !b_dw) return fail(CONV_ERR_INVALID_ARG, "dw has_bias set but bias is null");
    if (P.act_type == CONV_ACT_PRELU && !slope_pw) return fail(CONV_ERR_INVALID_ARG, "pw PReLU needs slopes");
    if (D.act_type == CONV_ACT_PRELU && !slope_dw) return fail(CONV_ERR_INVALID_ARG, "dw PReLU needs slopes");
    const View yv = y_view(dw, y);
    if (views_overlap(yv, x_view(pw, x))) return fail(CONV_ERR_ALIAS, "y overlaps x");
    if (views_overlap(yv, flat(w_pw, w_bytes(pw))) || views_overlap(yv, flat(w_dw, w_bytes(dw))))
        return fail(CONV_ERR_ALIAS, "y overlaps the weights");
    if ((P.has_bias && views_overlap(yv, flat(b_pw, 4 * (int64_t)P.c_out))) ||
        (D.has_bias && views_overlap(yv, flat(b_dw, 4 * (int64_t)D.c_out))))
        return fail(CONV_ERR_ALIAS, "y overlaps a bias");
    if ((P.act_type == CONV_ACT_PRELU && views_overlap(yv, flat(slope_pw, 4 * (int64_t)P.prelu_slope_count))) ||
        (D.act_type == CONV_ACT_PRELU && views_overlap(yv, flat(slope_dw, 4 * (int64_t)D.prelu_slope_count))))
        return fail(CONV_ERR_ALIAS, "y overlaps PReLU slopes");
    ConvArgs apw = make_args(pw, x, w_pw, b_pw, slope_pw, nullptr);
    ConvArgs adw = make_args(dw, nullptr, w_dw, b_dw, slope_dw, y);
    return hip_status(launch_fused_pw_dw(pw, dw, apw, adw, (hipStream_t)stream), "fused_pw_dw");
}

conv_status_t fused_dw_pw_forward(conv2d_desc_t ddw, conv2d_desc_t dpw, const void* x, const void* w_dw,
                                  const float* b_dw, const float* slope_dw, const void* w_pw, const float* b_pw,
                                  const float* slope_pw, void* y, void* stream) {
    if (!ddw || !dpw) return fail(CONV_ERR_INVALID_ARG, "null descriptor");
    const Desc& dw = *(const Desc*)ddw;
    const Desc& pw = *(const Desc*)dpw;
    const conv2d_params_t& D = dw.p;
    const conv2d_params_t& P = pw.p;
    if (P.dtype != D.dtype) return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "dw and pw dtypes differ");
    if (D.dtype != CONV_DTYPE_F32) return fail(CONV_ERR_UNSUPPORTED, "fused dw->pw supports F32 only");
    if (!(D.groups == D.c_in && D.groups == D.c_out))
        return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "first descriptor must be depthwise (groups == c_in == c_out)");
    if (P.k_h != 1 || P.k_w != 1 || P.stride_h != 1 || P.stride_w != 1 || P.groups != 1 || P.pad_top ||
        P.pad_left || P.pad_bottom || P.pad_right)
        return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "second descriptor must be a 1x1, stride 1, unpadded, ungrouped conv");
    if (P.c_in != D.c_out || P.n != D.n || P.h != dw.ho || P.w != dw.wo)
        return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "dw output [%d,%d,%d,%d] does not match pw input [%d,%d,%d,%d]",
                    D.n, D.c_out, dw.ho, dw.wo, P.n, P.c_in, P.h, P.w);
    if (dw.out_total != D.c_out || D.out_channel_offset != 0 || P.in_channel_offset != 0 || pw.in_total != P.c_in)
        return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "the depthwise output has no buffer: dw output and pw input must be "
                                                  "plain (no channel offsets)");
    if (D.k_h > 5 || D.k_w > 5) return fail(CONV_ERR_UNSUPPORTED, "fused dw->pw supports depthwise windows up to 5x5");
    if (!x || !y) return fail(CONV_ERR_INVALID_ARG, "null x or y");
    if (!plan_fused_dw_pw(dw, pw, x)) return fail(CONV_ERR_UNSUPPORTED, "image rows too wide for the fused tile");
    if (resolve_weights(dw, w_dw, "depthwise weights") != CONV_OK ||
        resolve_weights(pw, w_pw, "pointwise weights") != CONV_OK)
        return CONV_ERR_INVALID_ARG;
    if (D.has_bias && !b_dw) return fail(CONV_ERR_INVALID_ARG, "dw has_bias set but bias is null");
    if (P.has_bias && !b_pw) return fail(CONV_ERR_INVALID_ARG, "pw has_bias set but bias is null");
    if (D.act_type == CONV_ACT_PRELU && !slope_dw) return fail(CONV_ERR_INVALID_ARG, "dw PReLU needs slopes");
    if (P.act_type == CONV_ACT_PRELU && !slope_pw) return fail(CONV_ERR_INVALID_ARG, "pw PReLU needs slopes");
    const View yv = y_view(pw, y);
    if (views_overlap(yv, x_view(dw, x))) return fail(CONV_ERR_ALIAS, "y overlaps x");
    if (views_overlap(yv, flat(w_dw, w_bytes(dw))) || views_overlap(yv, flat(w_pw, w_bytes(pw))))
        return fail(CONV_ERR_ALIAS, "y overlaps the weights");
    if ((D.has_bias && views_overlap(yv, flat(b_dw, 4 * (int64_t)D.c_out))) ||
        (P.has_bias && views_overlap(yv, flat(b_pw, 4 * (int64_t)P.c_out))))
        return fail(CONV_ERR_ALIAS, "y overlaps a bias");
    if ((D.act_type == CONV_ACT_PRELU && views_overlap(yv, flat(slope_dw, 4 * (int64_t)D.prelu_slope_count))) ||
        (P.act_type == CONV_ACT_PRELU && views_overlap(yv, flat(slope_pw, 4 * (int64_t)P.prelu_slope_count))))
        return fail(CONV_ERR_ALIAS, "y overlaps PReLU slopes");
    ConvArgs adw = make_args(dw, x, w_dw, b_dw, slope_dw, nullptr);
    ConvArgs apw = make_args(pw, nullptr, w_pw, b_pw, slope_pw, y);
    return hip_status(launch_fused_dw_pw(dw, pw, adw, apw, (hipStream_t)stream), "fused_dw_pw");
}

namespace {
// composite = f32(f32(in_scale * w_scale) / out_scale), each step rounded to
// f32 (the requant scale of an int8 stage); false if not positive and finite.
bool composite_scale(float in_scale, float w_scale, float out_scale, float* out) {
    if (!(std::isfinite(in_scale) && in_scale > 0) || !(std::isfinite(w_scale) && w_scale > 0) ||
        !(std::isfinite(out_scale) && out_scale > 0))
        return false;
    volatile float prod = in_scale * w_scale;
    volatile float comp = prod / out_scale;
    *out = comp;
    return std::isfinite(*out) && *out > 0;
}
}  // namespace

conv_status_t qfused_dw_pw_forward(conv2d_desc_t ddw, conv2d_desc_t dpw, const int8_t* x, const int8_t* w_dw,
                                   const int32_t* b_dw, float dw_x_scale, float dw_w_scale, float dw_y_scale,
                                   const int8_t* w_pw, const int32_t* b_pw, float pw_x_scale, float pw_w_scale,
                                   float pw_y_scale, int8_t y_zp, int8_t* y, void* stream) {
    if (!ddw || !dpw) return fail(CONV_ERR_INVALID_ARG, "null descriptor");
    const Desc& dw = *(const Desc*)ddw;
    const Desc& pw = *(const Desc*)dpw;
    const conv2d_params_t& D = dw.p;
    const conv2d_params_t& P = pw.p;
    if (D.dtype != CONV_DTYPE_I8 || P.dtype != CONV_DTYPE_I8)
        return fail(CONV_ERR_INVALID_ARG, "qfused_dw_pw_forward needs two I8 descriptors");
    if (!(D.groups == D.c_in && D.groups == D.c_out))
        return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "first descriptor must be depthwise (groups == c_in == c_out)");
    if (P.k_h != 1 || P.k_w != 1 || P.stride_h != 1 || P.stride_w != 1 || P.groups != 1 || P.pad_top ||
        P.pad_left || P.pad_bottom || P.pad_right)
        return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "second descriptor must be a 1x1, stride 1, unpadded, ungrouped conv");
    if (P.c_in != D.c_out || P.n != D.n || P.h != dw.ho || P.w != dw.wo)
        return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "dw output [%d,%d,%d,%d] does not match pw input [%d,%d,%d,%d]",
                    D.n, D.c_out, dw.ho, dw.wo, P.n, P.c_in, P.h, P.w);
    if (dw.out_total != D.c_out || D.out_channel_offset != 0 || P.in_channel_offset != 0 || pw.in_total != P.c_in)
        return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "the depthwise output has no buffer: dw output and pw input must be "
                                                  "plain (no channel offsets)");
    if (D.k_h > 5 || D.k_w > 5) return fail(CONV_ERR_UNSUPPORTED, "fused int8 dw->pw supports windows up to 5x5");
    if (!plan_qfused_dw_pw(dw, pw)) return fail(CONV_ERR_UNSUPPORTED, "image rows too wide for the fused tile");
    float comp_dw = 0.0f, comp_pw = 0.0f;
    if (!composite_scale(dw_x_scale, dw_w_scale, dw_y_scale, &comp_dw) ||
        !composite_scale(pw_x_scale, pw_w_scale, pw_y_scale, &comp_pw))
        return fail(CONV_ERR_INVALID_ARG, "scales (and their composites) must be finite and positive");
    if (!x || !y) return fail(CONV_ERR_INVALID_ARG, "null x or y");
    const void* wdv = w_dw;
    const void* wpv = w_pw;
    if (resolve_weights(dw, wdv, "depthwise weights") != CONV_OK || resolve_weights(pw, wpv, "pointwise weights") != CONV_OK)
        return CONV_ERR_INVALID_ARG;
    if (D.has_bias && !b_dw) return fail(CONV_ERR_INVALID_ARG, "dw has_bias set but bias is null");
    if (P.has_bias && !b_pw) return fail(CONV_ERR_INVALID_ARG, "pw has_bias set but bias is null");
    const View yv = y_view(pw, y);
    if (views_overlap(yv, x_view(dw, x))) return fail(CONV_ERR_ALIAS, "y overlaps x");
    if (views_overlap(yv, flat(wdv, w_bytes(dw))) || views_overlap(yv, flat(wpv, w_bytes(pw))))
        return fail(CONV_ERR_ALIAS, "y overlaps the weights");
    if ((D.has_bias && views_overlap(yv, flat(b_dw, 4 * (int64_t)D.c_out))) ||
        (P.has_bias && views_overlap(yv, flat(b_pw, 4 * (int64_t)P.c_out))))
        return fail(CONV_ERR_ALIAS, "y overlaps a bias");
    ConvArgs adw = make_args(dw, x, wdv, nullptr, nullptr, nullptr);
    adw.qbias = D.has_bias ? b_dw : nullptr;
    ConvArgs apw = make_args(pw, nullptr, wpv, nullptr, nullptr, y);
    apw.qbias = P.has_bias ? b_pw : nullptr;
    return hip_status(launch_qfused_dw_pw(dw, pw, adw, apw, comp_dw, comp_pw, y_zp, (hipStream_t)stream),
                      "qfused_dw_pw");
}

conv_status_t qfused_pw_dw_forward(conv2d_desc_t dpw, conv2d_desc_t ddw, const int8_t* x, const int8_t* w_pw,
                                   const int32_t* b_pw, float pw_x_scale, float pw_w_scale, float pw_y_scale,
                                   const int8_t* w_dw, const int32_t* b_dw, float dw_x_scale, float dw_w_scale,
                                   float dw_y_scale, int8_t y_zp, int8_t* y, void* stream) {
    if (!dpw || !ddw) return fail(CONV_ERR_INVALID_ARG, "null descriptor");
    const Desc& pw = *(const Desc*)dpw;
    const Desc& dw = *(const Desc*)ddw;
    const conv2d_params_t& P = pw.p;
    const conv2d_params_t& D = dw.p;
    if (P.dtype != CONV_DTYPE_I8 || D.dtype != CONV_DTYPE_I8)
        return fail(CONV_ERR_INVALID_ARG, "qfused_pw_dw_forward needs two I8 descriptors");
    if (P.k_h != 1 || P.k_w != 1 || P.stride_h != 1 || P.stride_w != 1 || P.groups != 1 || P.pad_top ||
        P.pad_left || P.pad_bottom || P.pad_right)
        return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "first descriptor must be a 1x1, stride 1, unpadded, ungrouped conv");
    if (!(D.groups == D.c_in && D.groups == D.c_out))
        return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "second descriptor must be depthwise (groups == c_in == c_out)");
    if (D.c_in != P.c_out || D.n != P.n || D.h != P.h || D.w != P.w)
        return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "pw output [%d,%d,%d,%d] does not match dw input [%d,%d,%d,%d]",
                    P.n, P.c_out, P.h, P.w, D.n, D.c_in, D.h, D.w);
    if (pw.out_total != P.c_out || P.out_channel_offset != 0 || D.in_channel_offset != 0 || dw.in_total != D.c_in)
        return fail(CONV_ERR_INCOMPATIBLE_SHAPES, "the expanded tensor has no buffer: pw output and dw input must be "
                                                  "plain (no channel offsets)");
    if (D.k_h > 5 || D.k_w > 5) return fail(CONV_ERR_UNSUPPORTED, "fused int8 pw->dw supports windows up to 5x5");
    if (!plan_qfused_pw_dw(pw, dw)) return fail(CONV_ERR_UNSUPPORTED, "image rows too wide for the fused tile");
    float comp_pw = 0.0f, comp_dw = 0.0f;
    if (!composite_scale(pw_x_scale, pw_w_scale, pw_y_scale, &comp_pw) ||
        !composite_scale(dw_x_scale, dw_w_scale, dw_y_scale, &comp_dw))
        return fail(CONV_ERR_INVALID_ARG, "scales (and their composites) must be finite and positive");
    if (!x || !y) return fail(CONV_ERR_INVALID_ARG, "null x or y");
    const void* wpv = w_pw;
    const void* wdv = w_dw;
    if (resolve_weights(pw, wpv, "pointwise weights") != CONV_OK || resolve_weights(dw, wdv, "depthwise weights") != CONV_OK)
        return CONV_ERR_INVALID_ARG;
    if (P.has_bias && !b_pw) return fail(CONV_ERR_INVALID_ARG, "pw has_bias set but bias is null");
    if (D.has_bias && !b_dw) return fail(CONV_ERR_INVALID_ARG, "dw has_bias set but bias is null");
    const View yv = y_view(dw, y);
    if (views_overlap(yv, x_view(pw, x))) return fail(CONV_ERR_ALIAS, "y overlaps x");
    if (views_overlap(yv, flat(wpv, w_bytes(pw))) || views_overlap(yv, flat(wdv, w_bytes(dw))))
        return fail(CONV_ERR_ALIAS, "y overlaps the weights");
    if ((P.has_bias && views_overlap(yv, flat(b_pw, 4 * (int64_t)P.c_out))) ||
        (D.has_bias && views_overlap(yv, flat(b_dw, 4 * (int64_t)D.c_out))))
        return fail(CONV_ERR_ALIAS, "y overlaps a bias");
    ConvArgs apw = make_args(pw, x, wpv, nullptr, nullptr, nullptr);
    apw.qbias = P.has_bias ? b_pw : nullptr;
    ConvArgs adw = make_args(dw, nullptr, wdv, nullptr, nullptr, y);
    adw.qbias = D.has_bias ? b_dw : nullptr;
    return hip_status(launch_qfused_pw_dw(pw, dw, apw, adw, comp_pw, comp_dw, y_zp, (hipStream_t)stream),
                      "qfused_pw_dw");
}

conv_status_t qconv2d_forward(conv2d_desc_t dd, const int8_t* x, float x_scale, int8_t x_zp, const int8_t* w,
                              float w_scale, int8_t w_zp, const int32_t* bias, float y_scale, int8_t y_zp,
                              int8_t* y, void* stream) {
    if (check_desc(dd) != CONV_OK) return CONV_ERR_INVALID_ARG;
    const Desc& d = *(const Desc*)dd;
    if (d.p.dtype != CONV_DTYPE_I8) return fail(CONV_ERR_INVALID_ARG, "qconv2d_forward needs an I8 descriptor");
    if (x_zp != 0 || w_zp != 0)
        return fail(CONV_ERR_UNSUPPORTED, "symmetric int8 only: x and w zero points must be 0 (got %d, %d)", x_zp, w_zp);
    if (!(std::isfinite(x_scale) && x_scale > 0) || !(std::isfinite(w_scale) && w_scale > 0) ||
        !(std::isfinite(y_scale) && y_scale > 0))
        return fail(CONV_ERR_INVALID_ARG, "scales must be finite and positive");
    // composite = f32(f32(x_scale * w_scale) / y_scale), each step rounded to f32.
    volatile float prod = x_scale * w_scale;
    volatile float comp = prod / y_scale;
    const float composite = comp;
    if (!(std::isfinite(composite) && composite > 0))
        return fail(CONV_ERR_INVALID_ARG, "composite scale x_scale*w_scale/y_scale is not a positive finite float");
    if (!x || !y) return fail(CONV_ERR_INVALID_ARG, "null x or y");
    const void* wv = w;
    if (resolve_weights(d, wv, "weights") != CONV_OK) return CONV_ERR_INVALID_ARG;
    if (d.p.has_bias && !bias) return fail(CONV_ERR_INVALID_ARG, "has_bias set but bias is null");
    const View yv = y_view(d, y);
    if (views_overlap(yv, x_view(d, x))) return fail(CONV_ERR_ALIAS, "y overlaps the input channels read");
    if (views_overlap(yv, flat(wv, w_bytes(d)))) return fail(CONV_ERR_ALIAS, "y overlaps the weights");
    if (d.p.has_bias && views_overlap(yv, flat(bias, 4 * (int64_t)d.p.c_out)))
        return fail(CONV_ERR_ALIAS, "y overlaps the bias");
    ConvArgs a = make_args(d, x, wv, nullptr, nullptr, y);
    a.qbias = d.p.has_bias ? bias : nullptr;
    a.composite = composite;
    a.y_zp = y_zp;
    a.rounding = d.p.int8_rounding;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    switch (d.kclass) {
    case KC_QDW: e = launch_qdw(d, a, s); break;
    case KC_QPW: e = launch_qpw(d, a, s); break;
    case KC_IGEMM_I8:
        if (!igemm_i8_fast(d, x)) {
            e = launch_igemm_i8(d, a, s);
        } else if (!w) {
            e = launch_igemm_i8(d, a, s, (const char*)d.wbound + d.wbound_pack_off);
        } else {
            return forward_repack(*(Desc*)dd, a, s);
        }
        break;
    default: e = launch_direct(d, a, s); break;
    }
    return hip_status(e, kernel_name(d));
}

const char* conv2d_status_string(conv_status_t s) {
    switch (s) {
    case CONV_OK: return "CONV_OK";
    case CONV_ERR_INVALID_ARG: return "CONV_ERR_INVALID_ARG";
    case CONV_ERR_INCOMPATIBLE_SHAPES: return "CONV_ERR_INCOMPATIBLE_SHAPES";
    case CONV_ERR_UNSUPPORTED: return "CONV_ERR_UNSUPPORTED";
    case CONV_ERR_ALIAS: return "CONV_ERR_ALIAS";
    case CONV_ERR_HIP: return "CONV_ERR_HIP";
    }
    return "CONV_ERR_UNKNOWN";
}

const char* conv2d_last_error(void) { return g_last_error; }

}  // extern "C"
