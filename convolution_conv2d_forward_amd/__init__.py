"""Python binding of libconv2d.so (NCHW conv2d forward for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  Tensors are torch tensors (device memory and the
current HIP stream come from torch); the binding checks that each tensor is
contiguous, on the GPU, of the descriptor's dtype and large enough for the
view the descriptor describes, then passes raw pointers through the C ABI
declared in include/conv2d.h.  There is no fallback: if the library is not
built, importing this package raises.

Names and argument order follow the C ABI:
    conv2d_params_init, conv2d_desc_create, conv2d_desc_destroy,
    conv2d_desc_get_output_shape, conv2d_desc_kernel_name,
    conv2d_desc_bind_weights, conv2d_forward, conv2d_forward_noalloc,
    fused_pw_dw_forward, fused_dw_pw_forward, qconv2d_forward, qfused_dw_pw_forward,
    qfused_pw_dw_forward,
    conv2d_status_string,
    conv2d_last_error
plus ``make_params`` (keyword construction of a params struct).
"""
import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libconv2d.so")

CONV_OK, CONV_ERR_INVALID_ARG, CONV_ERR_INCOMPATIBLE_SHAPES, CONV_ERR_UNSUPPORTED, CONV_ERR_ALIAS, \
    CONV_ERR_HIP = range(6)
ACT_NONE, ACT_RELU, ACT_LEAKY_RELU, ACT_PRELU, ACT_CLIP = range(5)
DTYPE_F32, DTYPE_BF16, DTYPE_I8 = range(3)
ROUND_HALF_EVEN, ROUND_HALF_AWAY = range(2)
ALGO_AUTO, ALGO_DIRECT, ALGO_WINOGRAD, ALGO_WINOGRAD4 = range(4)
ALGOS = {"auto": ALGO_AUTO, "direct": ALGO_DIRECT, "winograd": ALGO_WINOGRAD, "winograd4": ALGO_WINOGRAD4}

_ACT_NAMES = {"none": ACT_NONE, "relu": ACT_RELU, "leaky_relu": ACT_LEAKY_RELU, "prelu": ACT_PRELU,
              "clip": ACT_CLIP}
_DTYPE_NAMES = {"f32": DTYPE_F32, "float32": DTYPE_F32, "bf16": DTYPE_BF16, "bfloat16": DTYPE_BF16,
                "i8": DTYPE_I8, "int8": DTYPE_I8}


class conv2d_params_t(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in (
        "n", "c_in", "h", "w", "c_out", "k_h", "k_w",
        "pad_top", "pad_left", "pad_bottom", "pad_right",
        "stride_h", "stride_w", "dilation_h", "dilation_w", "groups", "has_bias")] + [
        ("pad_value", ctypes.c_float),
        ("act_type", ctypes.c_int32),
        ("act_params", ctypes.c_float * 2),
        ("prelu_slope_count", ctypes.c_int32),
        ("in_channel_offset", ctypes.c_int32),
        ("in_total_channels", ctypes.c_int32),
        ("out_channel_offset", ctypes.c_int32),
        ("out_total_channels", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("int8_rounding", ctypes.c_int32),
        ("algo", ctypes.c_int32),
    ]


class ConvError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{conv2d_status_string(status)}: {message}")
        self.status = status


def _load():
    # Load torch first: libconv2d.so then binds the HIP runtime torch already
    # loaded (same soname), so torch's device memory and stream handles are
    # valid inside the library.  Loading the library first would bring in a
    # second runtime copy that cannot use torch's streams.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m convolution_conv2d_forward_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, i8 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_int8
    P = ctypes.POINTER
    lib.conv2d_params_init.argtypes = [P(conv2d_params_t)]
    lib.conv2d_params_init.restype = None
    lib.conv2d_desc_create.argtypes = [P(conv2d_params_t), P(vp)]
    lib.conv2d_desc_create.restype = i32
    lib.conv2d_desc_destroy.argtypes = [vp]
    lib.conv2d_desc_destroy.restype = None
    lib.conv2d_desc_get_output_shape.argtypes = [vp, P(i32)]
    lib.conv2d_desc_get_output_shape.restype = i32
    lib.conv2d_desc_kernel_name.argtypes = [vp]
    lib.conv2d_desc_kernel_name.restype = ctypes.c_char_p
    lib.conv2d_desc_bind_weights.argtypes = [vp, vp, vp]
    lib.conv2d_desc_bind_weights.restype = i32
    lib.conv2d_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.conv2d_forward.restype = i32
    lib.conv2d_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.conv2d_forward_noalloc.restype = i32
    lib.fused_pw_dw_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.fused_pw_dw_forward.restype = i32
    lib.fused_dw_pw_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.fused_dw_pw_forward.restype = i32
    lib.qconv2d_forward.argtypes = [vp, vp, f32, i8, vp, f32, i8, vp, f32, i8, vp, vp]
    lib.qconv2d_forward.restype = i32
    lib.qfused_dw_pw_forward.argtypes = [vp, vp, vp, vp, vp, f32, f32, f32, vp, vp, f32, f32, f32, i8, vp, vp]
    lib.qfused_dw_pw_forward.restype = i32
    lib.qfused_pw_dw_forward.argtypes = [vp, vp, vp, vp, vp, f32, f32, f32, vp, vp, f32, f32, f32, i8, vp, vp]
    lib.qfused_pw_dw_forward.restype = i32
    lib.conv2d_probe_copy.argtypes = [vp, vp, ctypes.c_int64, vp]
    lib.conv2d_probe_copy.restype = i32
    lib.conv2d_status_string.argtypes = [i32]
    lib.conv2d_status_string.restype = ctypes.c_char_p
    lib.conv2d_last_error.argtypes = []
    lib.conv2d_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load()

# C ABI symbols this binding relies on (the header declares exactly these).
EXPORTED = ("conv2d_params_init", "conv2d_desc_create", "conv2d_desc_destroy", "conv2d_desc_get_output_shape",
            "conv2d_desc_kernel_name", "conv2d_desc_bind_weights", "conv2d_forward", "conv2d_forward_noalloc",
            "fused_pw_dw_forward",
            "fused_dw_pw_forward", "qconv2d_forward", "qfused_dw_pw_forward", "qfused_pw_dw_forward", "conv2d_status_string",
            "conv2d_last_error")


def conv2d_status_string(status: int) -> str:
    return _lib.conv2d_status_string(int(status)).decode()


def conv2d_last_error() -> str:
    return _lib.conv2d_last_error().decode()


def _check(status):
    if status != CONV_OK:
        raise ConvError(status, conv2d_last_error())


def conv2d_params_init() -> conv2d_params_t:
    p = conv2d_params_t()
    _lib.conv2d_params_init(ctypes.byref(p))
    return p


def _pair(v):
    if isinstance(v, (tuple, list)):
        return int(v[0]), int(v[1])
    return int(v), int(v)


def make_params(n, c_in, h, w, c_out, k, *, stride=1, pads=0, dilation=1, groups=1, has_bias=False,
                pad_value=0.0, act="none", alpha=None, clip=None, prelu_slope_count=1, in_channel_offset=0,
                in_total_channels=0, out_channel_offset=0, out_total_channels=0, dtype="f32",
                int8_rounding=ROUND_HALF_EVEN, algo=0) -> conv2d_params_t:
    """Build a conv2d_params_t.  pads: int, or (top, left, bottom, right)."""
    p = conv2d_params_init()
    p.n, p.c_in, p.h, p.w, p.c_out = int(n), int(c_in), int(h), int(w), int(c_out)
    p.k_h, p.k_w = _pair(k)
    if isinstance(pads, (tuple, list)):
        p.pad_top, p.pad_left, p.pad_bottom, p.pad_right = (int(v) for v in pads)
    else:
        p.pad_top = p.pad_left = p.pad_bottom = p.pad_right = int(pads)
    p.stride_h, p.stride_w = _pair(stride)
    p.dilation_h, p.dilation_w = _pair(dilation)
    p.groups = int(groups)
    p.has_bias = int(bool(has_bias))
    p.pad_value = float(pad_value)
    p.act_type = _ACT_NAMES[act] if isinstance(act, str) else int(act)
    if alpha is not None:
        p.act_params[0] = float(alpha)
    if clip is not None:
        p.act_params[0], p.act_params[1] = float(clip[0]), float(clip[1])
    p.prelu_slope_count = int(prelu_slope_count)
    p.in_channel_offset, p.in_total_channels = int(in_channel_offset), int(in_total_channels)
    p.out_channel_offset, p.out_total_channels = int(out_channel_offset), int(out_total_channels)
    p.dtype = _DTYPE_NAMES[dtype] if isinstance(dtype, str) else int(dtype)
    p.int8_rounding = int(int8_rounding)
    p.algo = int(ALGOS.get(algo, algo) if isinstance(algo, str) else algo)
    return p


class Desc:
    """Owns a conv2d_desc_t; destroyed with the object or by conv2d_desc_destroy."""

    def __init__(self, handle, params):
        self.handle = handle
        self.params = params
        # Kept on the instance: module globals may already be gone when the
        # last descriptors are collected at interpreter exit.
        self._destroy = _lib.conv2d_desc_destroy

    def __del__(self):
        if getattr(self, "handle", None) and getattr(self, "_destroy", None) is not None:
            self._destroy(self.handle)
            self.handle = None


def conv2d_desc_create(params: conv2d_params_t) -> Desc:
    h = ctypes.c_void_p()
    _check(_lib.conv2d_desc_create(ctypes.byref(params), ctypes.byref(h)))
    p = conv2d_params_t()
    ctypes.memmove(ctypes.byref(p), ctypes.byref(params), ctypes.sizeof(params))
    return Desc(h, p)


def conv2d_desc_destroy(desc: Desc) -> None:
    if desc.handle:
        _lib.conv2d_desc_destroy(desc.handle)
        desc.handle = None


def conv2d_desc_get_output_shape(desc: Desc):
    out = (ctypes.c_int32 * 4)()
    _check(_lib.conv2d_desc_get_output_shape(desc.handle, out))
    return tuple(int(v) for v in out)


def conv2d_desc_kernel_name(desc: Desc) -> str:
    return _lib.conv2d_desc_kernel_name(desc.handle).decode()


# ------------------------------------------------------------ marshalling --

def _torch():
    import torch
    return torch


_ELEM = {DTYPE_F32: "float32", DTYPE_BF16: "bfloat16", DTYPE_I8: "int8"}


_DTYPES = {}


def _dtype(name):
    dt = _DTYPES.get(name)
    if dt is None:
        dt = _DTYPES[name] = getattr(_torch(), name)
    return dt


def _ptr(t, what, dtype_name, min_numel):
    """Raw device pointer of a contiguous GPU tensor holding >= min_numel elements."""
    if t is None:
        return None
    # Fast path: one pass over the conditions; the checked path below names
    # the first one that fails.
    try:
        if t.is_cuda and t.dtype is _dtype(dtype_name) and t.numel() >= min_numel and t.is_contiguous():
            return t.data_ptr()
    except AttributeError:
        pass
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: torch.Tensor expected")
    if not t.is_cuda:
        raise ValueError(f"{what}: tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{what}: tensor must be contiguous")
    if str(t.dtype) != "torch." + dtype_name:
        raise TypeError(f"{what}: dtype {t.dtype}, expected torch.{dtype_name}")
    if t.numel() < min_numel:
        raise ValueError(f"{what}: {t.numel()} elements, the descriptor needs {min_numel}")
    return t.data_ptr()


_RAW_STREAM = None


def _stream(stream):
    """hipStream_t of `stream` (a torch stream or a raw handle); None = the
    current torch stream of the current device."""
    global _RAW_STREAM
    if stream is None:
        if _RAW_STREAM is None:
            C = _torch()._C
            get_raw, get_dev = getattr(C, "_cuda_getCurrentRawStream", None), getattr(C, "_cuda_getDevice", None)
            if get_raw is not None and get_dev is not None:
                _RAW_STREAM = lambda: get_raw(get_dev())
            else:
                _RAW_STREAM = lambda: _torch().cuda.current_stream().cuda_stream
        return _RAW_STREAM()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _sizes(desc):
    """(x, w, y) element counts a call on desc reads and writes (cached: a
    descriptor's shapes never change)."""
    sz = desc.__dict__.get("_sz")
    if sz is None:
        p = desc.params
        n, ot, ho, wo = conv2d_desc_get_output_shape(desc)
        in_total = p.in_total_channels or p.c_in
        sz = desc._sz = (p.n * in_total * p.h * p.w, p.c_out * (p.c_in // p.groups) * p.k_h * p.k_w, n * ot * ho * wo)
    return sz


def conv2d_desc_bind_weights(desc: Desc, w, stream=None) -> None:
    """Copy (and, where the kernel wants it, re-lay) w into the descriptor;
    forward calls given w=None then use that copy."""
    p = desc.params
    _, wn, _ = _sizes(desc)
    _check(_lib.conv2d_desc_bind_weights(desc.handle, _ptr(w, "w", _ELEM[p.dtype], wn), _stream(stream)))


def conv2d_forward(desc: Desc, x, w, bias, slope, y, stream=None) -> None:
    """Float convolution (F32 or BF16 descriptor), launched on `stream`.
    w=None uses the weights bound with conv2d_desc_bind_weights."""
    p = desc.params
    et = _ELEM[p.dtype]
    xn, wn, yn = _sizes(desc)
    _check(_lib.conv2d_forward(
        desc.handle, _ptr(x, "x", et, xn), _ptr(w, "w", et, wn),
        _ptr(bias, "bias", "float32", p.c_out) if p.has_bias else None,
        _ptr(slope, "slope", "float32", p.prelu_slope_count) if p.act_type == ACT_PRELU else None,
        _ptr(y, "y", et, yn), _stream(stream)))


def conv2d_forward_noalloc(desc: Desc, x, w, bias, slope, y, stream=None) -> None:
    """conv2d_forward that allocates no device memory (a fixed per-GPU scratch
    array holds the bf16 weight re-layout); overlapping calls on one GPU race."""
    p = desc.params
    et = _ELEM[p.dtype]
    xn, wn, yn = _sizes(desc)
    _check(_lib.conv2d_forward_noalloc(
        desc.handle, _ptr(x, "x", et, xn), _ptr(w, "w", et, wn),
        _ptr(bias, "bias", "float32", p.c_out) if p.has_bias else None,
        _ptr(slope, "slope", "float32", p.prelu_slope_count) if p.act_type == ACT_PRELU else None,
        _ptr(y, "y", et, yn), _stream(stream)))


def fused_pw_dw_forward(desc_pw: Desc, desc_dw: Desc, x, w_pw, b_pw, slope_pw, w_dw, b_dw, slope_dw, y,
                        stream=None) -> None:
    """Fused pointwise 1x1 -> depthwise (F32)."""
    pp, pd = desc_pw.params, desc_dw.params
    et = _ELEM[pp.dtype]
    xn, wpn, _ = _sizes(desc_pw)
    _, wdn, yn = _sizes(desc_dw)
    _check(_lib.fused_pw_dw_forward(
        desc_pw.handle, desc_dw.handle, _ptr(x, "x", et, xn), _ptr(w_pw, "w_pw", et, wpn),
        _ptr(b_pw, "b_pw", "float32", pp.c_out) if pp.has_bias else None,
        _ptr(slope_pw, "slope_pw", "float32", pp.prelu_slope_count) if pp.act_type == ACT_PRELU else None,
        _ptr(w_dw, "w_dw", et, wdn),
        _ptr(b_dw, "b_dw", "float32", pd.c_out) if pd.has_bias else None,
        _ptr(slope_dw, "slope_dw", "float32", pd.prelu_slope_count) if pd.act_type == ACT_PRELU else None,
        _ptr(y, "y", et, yn), _stream(stream)))


def fused_dw_pw_forward(desc_dw: Desc, desc_pw: Desc, x, w_dw, b_dw, slope_dw, w_pw, b_pw, slope_pw, y,
                        stream=None) -> None:
    """Fused depthwise kxk -> pointwise 1x1 (F32)."""
    pd, pp = desc_dw.params, desc_pw.params
    et = _ELEM[pd.dtype]
    xn, wdn, _ = _sizes(desc_dw)
    _, wpn, yn = _sizes(desc_pw)
    _check(_lib.fused_dw_pw_forward(
        desc_dw.handle, desc_pw.handle, _ptr(x, "x", et, xn), _ptr(w_dw, "w_dw", et, wdn),
        _ptr(b_dw, "b_dw", "float32", pd.c_out) if pd.has_bias else None,
        _ptr(slope_dw, "slope_dw", "float32", pd.prelu_slope_count) if pd.act_type == ACT_PRELU else None,
        _ptr(w_pw, "w_pw", et, wpn),
        _ptr(b_pw, "b_pw", "float32", pp.c_out) if pp.has_bias else None,
        _ptr(slope_pw, "slope_pw", "float32", pp.prelu_slope_count) if pp.act_type == ACT_PRELU else None,
        _ptr(y, "y", et, yn), _stream(stream)))


def qconv2d_forward(desc: Desc, x, x_scale, x_zp, w, w_scale, w_zp, bias, y_scale, y_zp, y, stream=None) -> None:
    """Symmetric int8 QLinearConv (I8 descriptor)."""
    p = desc.params
    xn, wn, yn = _sizes(desc)
    _check(_lib.qconv2d_forward(
        desc.handle, _ptr(x, "x", "int8", xn), ctypes.c_float(x_scale), ctypes.c_int8(int(x_zp)),
        _ptr(w, "w", "int8", wn), ctypes.c_float(w_scale), ctypes.c_int8(int(w_zp)),
        _ptr(bias, "bias", "int32", p.c_out) if p.has_bias else None,
        ctypes.c_float(y_scale), ctypes.c_int8(int(y_zp)), _ptr(y, "y", "int8", yn), _stream(stream)))


def qfused_dw_pw_forward(desc_dw: Desc, desc_pw: Desc, x, w_dw, b_dw, dw_scales, w_pw, b_pw, pw_scales, y_zp, y,
                         stream=None) -> None:
    """Fused int8 depthwise -> pointwise: two symmetric QLinearConvs, each with
    its (x_scale, w_scale, y_scale) triple."""
    pd, pp = desc_dw.params, desc_pw.params
    xn, wdn, _ = _sizes(desc_dw)
    _, wpn, yn = _sizes(desc_pw)
    f = ctypes.c_float
    _check(_lib.qfused_dw_pw_forward(
        desc_dw.handle, desc_pw.handle, _ptr(x, "x", "int8", xn), _ptr(w_dw, "w_dw", "int8", wdn),
        _ptr(b_dw, "b_dw", "int32", pd.c_out) if pd.has_bias else None, *(f(v) for v in dw_scales),
        _ptr(w_pw, "w_pw", "int8", wpn), _ptr(b_pw, "b_pw", "int32", pp.c_out) if pp.has_bias else None,
        *(f(v) for v in pw_scales), ctypes.c_int8(int(y_zp)), _ptr(y, "y", "int8", yn), _stream(stream)))


def qfused_pw_dw_forward(desc_pw: Desc, desc_dw: Desc, x, w_pw, b_pw, pw_scales, w_dw, b_dw, dw_scales, y_zp, y,
                         stream=None) -> None:
    """Fused int8 pointwise -> depthwise: two symmetric QLinearConvs, each with
    its (x_scale, w_scale, y_scale) triple."""
    pp, pd = desc_pw.params, desc_dw.params
    xn, wpn, _ = _sizes(desc_pw)
    _, wdn, yn = _sizes(desc_dw)
    f = ctypes.c_float
    _check(_lib.qfused_pw_dw_forward(
        desc_pw.handle, desc_dw.handle, _ptr(x, "x", "int8", xn), _ptr(w_pw, "w_pw", "int8", wpn),
        _ptr(b_pw, "b_pw", "int32", pp.c_out) if pp.has_bias else None, *(f(v) for v in pw_scales),
        _ptr(w_dw, "w_dw", "int8", wdn), _ptr(b_dw, "b_dw", "int32", pd.c_out) if pd.has_bias else None,
        *(f(v) for v in dw_scales), ctypes.c_int8(int(y_zp)), _ptr(y, "y", "int8", yn), _stream(stream)))


def conv2d_probe_copy(dst, src, stream=None) -> None:
    """Streaming 16-byte device copy of src into dst (the attainable-bandwidth
    reference of the benchmark; include/conv2d_probe.h)."""
    torch = _torch()
    for t, what in ((dst, "dst"), (src, "src")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{what}: contiguous GPU tensor expected")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst smaller than src")
    _check(_lib.conv2d_probe_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                                  ctypes.c_int64(nbytes), _stream(stream)))


def output_shape(desc: Desc):
    """(n, out_total_channels, Ho, Wo) -- alias of conv2d_desc_get_output_shape."""
    return conv2d_desc_get_output_shape(desc)


def flops(params: conv2d_params_t) -> int:
    """2 * multiply-accumulates of one forward, padded taps included."""
    hnum = params.h + params.pad_top + params.pad_bottom - params.dilation_h * (params.k_h - 1) - 1
    wnum = params.w + params.pad_left + params.pad_right - params.dilation_w * (params.k_w - 1) - 1
    ho, wo = hnum // params.stride_h + 1, wnum // params.stride_w + 1
    return 2 * params.n * params.c_out * ho * wo * (params.c_in // params.groups) * params.k_h * params.k_w


__all__ = [n for n in dir() if not n.startswith("_") and n not in ("ctypes", "math", "os")]
