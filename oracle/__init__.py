"""CPU oracle for NCHW conv2d forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The product library never
calls it; it shares no code with the HIP path.

The arithmetic lives in ``oracle.c`` (float64 direct 7-loop convolution,
int64 accumulation plus float32 requant for int8).  This module only
marshals numpy arrays into it.  Function by function:

* ``conv2d`` / ``conv2d_points`` -- ncnn operators.md "convolution" and
  "convolutiondepthwise": pad with pad_value, correlate with kernel, stride,
  dilation and group, add bias, apply the activation; activations as the Go
  "ops" page defines ReluOp, LeakyReluOp, PReluOp and ClipOp.
* ``qconv2d`` / ``qconv2d_acc`` / ``requant`` / ``composite_scale`` -- the
  symmetric int8 QLinearConv of the yscv "ONNX CPU Kernels" page (fused INT8
  chains, requant epilogue): int32 accumulate, + int32 bias, f32 multiply by
  the composite scale, round, + y_zp, saturate to int8, optional Relu.  Ties
  go to even by default (the plainest reading of a "round-half-to-even"
  requant); ties away from zero reproduce the yscv page's own rounding.

Every function here is pinned by ``tests/test_oracle.py`` against hand cases,
closed forms, invariants and independent library formulations.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

ACT_NONE, ACT_RELU, ACT_LEAKY_RELU, ACT_PRELU, ACT_CLIP = 0, 1, 2, 3, 4
ROUND_HALF_EVEN, ROUND_HALF_AWAY = 0, 1
FLT_MAX = float(np.finfo(np.float32).max)


class _Conv(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in (
        "n", "c_in", "h", "w", "c_out", "k_h", "k_w",
        "pad_top", "pad_left", "pad_bottom", "pad_right",
        "stride_h", "stride_w", "dilation_h", "dilation_w", "groups")] + [
        ("pad_value", ctypes.c_double),
        ("act_type", ctypes.c_int64),
        ("act_p0", ctypes.c_double),
        ("act_p1", ctypes.c_double),
        ("slope_count", ctypes.c_int64),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp = ctypes.c_void_p
        lib.oracle_out_h.restype = ctypes.c_int64
        lib.oracle_out_h.argtypes = [P(_Conv)]
        lib.oracle_out_w.restype = ctypes.c_int64
        lib.oracle_out_w.argtypes = [P(_Conv)]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_conv2d_f64.argtypes = [P(_Conv), vp, vp, vp, vp, vp]
        lib.oracle_conv2d_points_f64.argtypes = [P(_Conv), vp, vp, vp, vp, vp, ctypes.c_int64, vp]
        lib.oracle_composite_scale.restype = ctypes.c_float
        lib.oracle_composite_scale.argtypes = [ctypes.c_float] * 3
        lib.oracle_requant.restype = ctypes.c_int8
        lib.oracle_requant.argtypes = [ctypes.c_int64, ctypes.c_float, ctypes.c_int,
                                       ctypes.c_int64, ctypes.c_int]
        lib.oracle_qconv2d_acc.argtypes = [P(_Conv), vp, vp, ctypes.c_int64, vp]
        lib.oracle_qconv2d.argtypes = [P(_Conv), vp, vp, vp, ctypes.c_int64, ctypes.c_float,
                                       ctypes.c_int, ctypes.c_int64, ctypes.c_int, vp]
        lib.oracle_qconv2d_points.argtypes = [P(_Conv), vp, vp, vp, ctypes.c_int64, ctypes.c_float,
                                              ctypes.c_int, ctypes.c_int64, ctypes.c_int, vp,
                                              ctypes.c_int64, vp]
        lib.oracle_requant_array.argtypes = [vp, ctypes.c_int64, ctypes.c_float, ctypes.c_int,
                                             ctypes.c_int64, ctypes.c_int, vp]
        _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle runs on."""
    return int(_load().oracle_num_threads())


def _pair(v):
    if isinstance(v, (tuple, list)):
        return int(v[0]), int(v[1])
    return int(v), int(v)


def _params(x_shape, w_shape, stride=1, pads=(0, 0, 0, 0), dilation=1, groups=1,
            pad_value=0.0, act=ACT_NONE, alpha=0.01, clip=(-FLT_MAX, FLT_MAX), slope_count=1):
    n, c_in, h, w = (int(s) for s in x_shape)
    c_out, cin_g, k_h, k_w = (int(s) for s in w_shape)
    if groups < 1 or c_in % groups or c_out % groups or cin_g != c_in // groups:
        raise ValueError("inconsistent group / channel counts")
    sh, sw = _pair(stride)
    dh, dw = _pair(dilation)
    pt, pl, pb, pr = (int(p) for p in pads)
    if min(sh, sw, dh, dw, k_h, k_w) < 1 or min(pt, pl, pb, pr) < 0:
        raise ValueError("bad conv attributes")
    p = _Conv(n=n, c_in=c_in, h=h, w=w, c_out=c_out, k_h=k_h, k_w=k_w,
              pad_top=pt, pad_left=pl, pad_bottom=pb, pad_right=pr,
              stride_h=sh, stride_w=sw, dilation_h=dh, dilation_w=dw, groups=int(groups),
              pad_value=float(pad_value), act_type=int(act),
              act_p0=float(alpha if act == ACT_LEAKY_RELU else clip[0]),
              act_p1=float(clip[1]), slope_count=int(slope_count))
    return p


def output_shape(x_shape, w_shape, stride=1, pads=(0, 0, 0, 0), dilation=1, groups=1):
    lib = _load()
    p = _params(x_shape, w_shape, stride, pads, dilation, groups)
    return (p.n, p.c_out, int(lib.oracle_out_h(ctypes.byref(p))), int(lib.oracle_out_w(ctypes.byref(p))))


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data


def conv2d(x, w, bias=None, *, stride=1, pads=(0, 0, 0, 0), dilation=1, groups=1,
           pad_value=0.0, act=ACT_NONE, alpha=0.01, clip=(-FLT_MAX, FLT_MAX), slope=None):
    """Float64 direct convolution; returns y[n, c_out, Ho, Wo] as float64.

    Inputs are taken at the exact values given (e.g. fp32 or bf16-representable
    numbers), widened to float64 without change."""
    lib = _load()
    x = _f64(x)
    w = _f64(w)
    b = None if bias is None else _f64(bias)
    s = None if slope is None else _f64(slope).reshape(-1)
    p = _params(x.shape, w.shape, stride, pads, dilation, groups, pad_value, act, alpha, clip,
                1 if s is None else s.size)
    if act == ACT_PRELU and (s is None or s.size not in (1, p.c_out)):
        raise ValueError("prelu slope must hold 1 or c_out values")
    ho, wo = int(lib.oracle_out_h(ctypes.byref(p))), int(lib.oracle_out_w(ctypes.byref(p)))
    y = np.empty((p.n, p.c_out, ho, wo), dtype=np.float64)
    if y.size:
        lib.oracle_conv2d_f64(ctypes.byref(p), _ptr(x), _ptr(w), _ptr(b), _ptr(s), _ptr(y))
    return y


def conv2d_points(x, w, bias, flat_idx, *, stride=1, pads=(0, 0, 0, 0), dilation=1, groups=1,
                  pad_value=0.0, act=ACT_NONE, alpha=0.01, clip=(-FLT_MAX, FLT_MAX), slope=None):
    """The same definition evaluated only at flat indices of [n, c_out, Ho, Wo]."""
    lib = _load()
    x = _f64(x)
    w = _f64(w)
    b = None if bias is None else _f64(bias)
    s = None if slope is None else _f64(slope).reshape(-1)
    p = _params(x.shape, w.shape, stride, pads, dilation, groups, pad_value, act, alpha, clip,
                1 if s is None else s.size)
    idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64).reshape(-1))
    out = np.empty(idx.size, dtype=np.float64)
    if idx.size:
        lib.oracle_conv2d_points_f64(ctypes.byref(p), _ptr(x), _ptr(w), _ptr(b), _ptr(s),
                                     _ptr(idx), idx.size, _ptr(out))
    return out


def composite_scale(x_scale, w_scale, y_scale) -> np.float32:
    """f32(f32(x_scale*w_scale)/y_scale) from float32 scale values."""
    return np.float32(_load().oracle_composite_scale(float(np.float32(x_scale)),
                                                      float(np.float32(w_scale)),
                                                      float(np.float32(y_scale))))


def requant(values, composite, *, rounding=ROUND_HALF_EVEN, y_zp=0, relu=False):
    """Requantise int64 values (accumulator + bias) to int8, elementwise."""
    v = np.ascontiguousarray(np.asarray(values, dtype=np.int64).reshape(-1))
    out = np.empty(v.size, dtype=np.int8)
    if v.size:
        _load().oracle_requant_array(_ptr(v), v.size, float(np.float32(composite)), int(rounding),
                                     int(y_zp), int(bool(relu)), _ptr(out))
    return out.reshape(np.shape(values))


def _i8(a):
    a = np.asarray(a)
    if a.dtype != np.int8:
        raise TypeError("int8 operand expected")
    return np.ascontiguousarray(a)


def qconv2d_acc(x, w, *, stride=1, pads=(0, 0, 0, 0), dilation=1, groups=1, x_zp=0):
    """Exact int64 accumulators of the int8 convolution (no bias)."""
    lib = _load()
    x = _i8(x)
    w = _i8(w)
    p = _params(x.shape, w.shape, stride, pads, dilation, groups)
    ho, wo = int(lib.oracle_out_h(ctypes.byref(p))), int(lib.oracle_out_w(ctypes.byref(p)))
    acc = np.empty((p.n, p.c_out, ho, wo), dtype=np.int64)
    if acc.size:
        lib.oracle_qconv2d_acc(ctypes.byref(p), _ptr(x), _ptr(w), int(x_zp), _ptr(acc))
    return acc


def qconv2d(x, w, bias, x_scale, w_scale, y_scale, *, stride=1, pads=(0, 0, 0, 0), dilation=1,
            groups=1, x_zp=0, y_zp=0, rounding=ROUND_HALF_EVEN, relu=False):
    """Symmetric int8 QLinearConv: returns y[n, c_out, Ho, Wo] as int8."""
    lib = _load()
    x = _i8(x)
    w = _i8(w)
    b = None if bias is None else np.ascontiguousarray(np.asarray(bias, dtype=np.int32))
    p = _params(x.shape, w.shape, stride, pads, dilation, groups)
    ho, wo = int(lib.oracle_out_h(ctypes.byref(p))), int(lib.oracle_out_w(ctypes.byref(p)))
    comp = composite_scale(x_scale, w_scale, y_scale)
    y = np.empty((p.n, p.c_out, ho, wo), dtype=np.int8)
    if y.size:
        lib.oracle_qconv2d(ctypes.byref(p), _ptr(x), _ptr(w), _ptr(b), int(x_zp), float(comp),
                           int(rounding), int(y_zp), int(bool(relu)), _ptr(y))
    return y


def qconv2d_points(x, w, bias, x_scale, w_scale, y_scale, flat_idx, *, stride=1,
                   pads=(0, 0, 0, 0), dilation=1, groups=1, x_zp=0, y_zp=0,
                   rounding=ROUND_HALF_EVEN, relu=False):
    """int8 outputs at flat indices of [n, c_out, Ho, Wo]."""
    lib = _load()
    x = _i8(x)
    w = _i8(w)
    b = None if bias is None else np.ascontiguousarray(np.asarray(bias, dtype=np.int32))
    p = _params(x.shape, w.shape, stride, pads, dilation, groups)
    comp = composite_scale(x_scale, w_scale, y_scale)
    idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64).reshape(-1))
    out = np.empty(idx.size, dtype=np.int8)
    if idx.size:
        lib.oracle_qconv2d_points(ctypes.byref(p), _ptr(x), _ptr(w), _ptr(b), int(x_zp),
                                  float(comp), int(rounding), int(y_zp), int(bool(relu)),
                                  _ptr(idx), idx.size, _ptr(out))
    return out
