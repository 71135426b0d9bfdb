"""Host-only tests of the C ABI (no GPU): the library loads, exports every
symbol include/conv2d.h declares, fills defaults, validates descriptors with
the documented status codes, infers output shapes, and rejects aliasing and
non-symmetric int8 before any launch."""
import ctypes
import math
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "conv2d.h")


def cc():
    import convolution_conv2d_forward_amd as m
    return m


PROBE_HEADER = os.path.join(ROOT, "include", "conv2d_probe.h")


def declared_symbols(path=HEADER):
    text = open(path).read()
    return sorted(set(re.findall(r"CONV2D_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


def test_header_symbols_exported():
    syms = declared_symbols()
    assert len(syms) == 15, syms
    lib = ctypes.CDLL(cc().LIB_PATH)
    for s in syms:
        assert hasattr(lib, s), f"{s} declared in conv2d.h but not exported"
    assert sorted(cc().EXPORTED) == syms
    # every header under include/ (the measurement probe too)
    probe = declared_symbols(PROBE_HEADER)
    assert probe == ["conv2d_probe_copy"], probe
    for s in probe:
        assert hasattr(lib, s), f"{s} declared in conv2d_probe.h but not exported"


def test_probe_copy_rejects_before_launch():
    """Misaligned or overlapping ranges are refused without a HIP call."""
    lib = ctypes.CDLL(cc().LIB_PATH)
    f = lib.conv2d_probe_copy
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    f.restype = ctypes.c_int32
    assert f(None, ctypes.c_void_p(4096), 64, None) == cc().CONV_ERR_INVALID_ARG
    assert f(ctypes.c_void_p(4096 + 4), ctypes.c_void_p(1 << 20), 64, None) == cc().CONV_ERR_INVALID_ARG
    assert f(ctypes.c_void_p(4096), ctypes.c_void_p(1 << 20), 60, None) == cc().CONV_ERR_INVALID_ARG
    assert f(ctypes.c_void_p(4096), ctypes.c_void_p(4096 + 32), 64, None) == cc().CONV_ERR_ALIAS
    assert f(ctypes.c_void_p(4096), ctypes.c_void_p(1 << 20), 0, None) == cc().CONV_OK


def test_params_layout_matches_header(tmp_path):
    """The ctypes mirror of conv2d_params_t has the header's size and field
    offsets (the header compiled with gcc)."""
    P = cc().conv2d_params_t
    names = [f[0] for f in P._fields_]
    src = tmp_path / "layout.c"
    hdr = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "conv2d.h")
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "%s"\nint main(void) {\n'
                   '  printf("%%zu\\n", sizeof(conv2d_params_t));\n%s  return 0;\n}\n'
                   % (hdr, "".join('  printf("%%zu\\n", offsetof(conv2d_params_t, %s));\n' % n for n in names)))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", str(src), "-o", str(exe)], check=True)
    out = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    assert out[0] == ctypes.sizeof(P)
    assert out[1:] == [getattr(P, n).offset for n in names]


def test_params_defaults():
    p = cc().conv2d_params_init()
    assert (p.stride_h, p.stride_w, p.dilation_h, p.dilation_w, p.groups) == (1, 1, 1, 1, 1)
    assert (p.pad_top, p.pad_left, p.pad_bottom, p.pad_right) == (0, 0, 0, 0)
    assert p.pad_value == 0.0 and p.has_bias == 0 and p.act_type == cc().ACT_NONE
    assert math.isnan(p.act_params[0]) and math.isnan(p.act_params[1])
    assert p.prelu_slope_count == 1 and p.dtype == cc().DTYPE_F32 and p.int8_rounding == cc().ROUND_HALF_EVEN


def _status(**kw):
    base = dict(n=1, c_in=4, h=8, w=8, c_out=4, k=3, pads=1)
    base.update(kw)
    args = [base.pop(k) for k in ("n", "c_in", "h", "w", "c_out", "k")]
    p = cc().make_params(*args, **base)
    try:
        cc().conv2d_desc_create(p)
        return cc().CONV_OK
    except cc().ConvError as e:
        return e.status


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(n=0), 1), (dict(c_in=-1), 1), (dict(h=0), 1), (dict(c_out=0), 1), (dict(k=0), 1),
    (dict(stride=0), 1), (dict(dilation=0), 1), (dict(pads=(-1, 0, 0, 0)), 1),
    (dict(k=9, pads=0), 1),                                     # empty output
    (dict(act=7), 1), (dict(dtype=5), 1), (dict(int8_rounding=3), 1),
    (dict(pad_value=float("nan")), 1), (dict(pad_value=float("inf")), 1),
    (dict(act="clip", clip=(1.0, -1.0)), 1),
    (dict(act="leaky_relu", alpha=float("inf")), 1),
    (dict(groups=0), 1),
    (dict(groups=3), 2),                                        # does not divide 4
    (dict(c_in=6, groups=3), 2),                                # c_out 4 % 3
    (dict(act="prelu", prelu_slope_count=3), 2),
    (dict(act="prelu", prelu_slope_count=4), 0),
    (dict(out_channel_offset=2, out_total_channels=5), 2),
    (dict(out_channel_offset=1, out_total_channels=5), 0),
    (dict(in_channel_offset=3, in_total_channels=6), 2),
    (dict(dtype="i8", pad_value=1.0), 3),
    (dict(dtype="i8", act="leaky_relu"), 3),
    (dict(dtype="i8", act="relu"), 0),
])
def test_descriptor_status_codes(kw, status):
    assert _status(**kw) == status


def test_status_strings_and_last_error():
    assert cc().conv2d_status_string(0) == "CONV_OK"
    assert cc().conv2d_status_string(4) == "CONV_ERR_ALIAS"
    assert _status(groups=3) == 2
    assert "groups" in cc().conv2d_last_error()


def test_output_shape_matches_oracle():
    rng = np.random.default_rng(42)
    for _ in range(200):
        L = workloads.random_layer(rng)
        p = cc().make_params(L.n, L.c_in, L.h, L.w, L.c_out, L.k, stride=L.stride, pads=L.pads,
                             dilation=L.dilation, groups=L.groups, out_total_channels=L.c_out + 3,
                             out_channel_offset=2)
        d = cc().conv2d_desc_create(p)
        n, ot, ho, wo = cc().conv2d_desc_get_output_shape(d)
        on, oc, oh, ow = oracle.output_shape(L.x_shape, L.w_shape, L.stride, L.pads, L.dilation, L.groups)
        assert (n, ot, ho, wo) == (on, L.c_out + 3, oh, ow)


def test_kernel_choice_for_the_workloads():
    names = {}
    for L in workloads.dense_block_layers() + workloads.bottleneck().layers + workloads.mixed_sweep_layers():
        d = cc().conv2d_desc_create(cc().make_params(L.n, L.c_in, L.h, L.w, L.c_out, L.k, stride=L.stride,
                                                     pads=L.pads, dilation=L.dilation, groups=L.groups))
        names[L.name] = cc().conv2d_desc_kernel_name(d)
    assert names["conv0"] == "igemm_f32" and names["conv4"] == "igemm_f32"
    assert names["pw1"] == "pointwise_f32" and names["pw2"] == "pw_narrow_f32"
    assert names["dw"] == "depthwise_f32"
    assert names["g32"] == "grouped_f32" and names["pw"] == "pw_gemm_f32"
    for L in workloads.int8_chain_layers():
        d = cc().conv2d_desc_create(cc().make_params(L.n, L.c_in, L.h, L.w, L.c_out, L.k, stride=L.stride,
                                                     pads=L.pads, groups=L.groups, dtype="i8"))
        names[L.name] = cc().conv2d_desc_kernel_name(d)
    assert names["dw_s1"] == names["dw_s2"] == "depthwise_i8_dot4" and names["pw"] == "pointwise_i8_mfma"
    # the int8 bottleneck's depthwise (56-byte rows: 8-byte copy chunks)
    d = cc().conv2d_desc_create(cc().make_params(8, 192, 56, 56, 192, (3, 3), pads=1, groups=192, dtype="i8"))
    assert cc().conv2d_desc_kernel_name(d) == "depthwise_i8_dot4"
    # int8 dense, strided and grouped convolutions: the i8 implicit GEMM
    for L in workloads.mixed_sweep_layers():
        if L.name == "pw":
            continue
        d = cc().conv2d_desc_create(cc().make_params(L.n, L.c_in, L.h, L.w, L.c_out, L.k, stride=L.stride,
                                                     pads=L.pads, dilation=L.dilation, groups=L.groups, dtype="i8"))
        assert cc().conv2d_desc_kernel_name(d) == "igemm_i8", L.name
    # the single conv: the small-layer kernel under AUTO, the implicit GEMM under DIRECT
    L = workloads.single_conv().layers[0]
    for algo, want in (("auto", "small_f32"), ("direct", "igemm_f32")):
        d = cc().conv2d_desc_create(cc().make_params(L.n, L.c_in, L.h, L.w, L.c_out, L.k, pads=L.pads, has_bias=True,
                                                     algo=algo))
        assert cc().conv2d_desc_kernel_name(d) == want, algo
    # just past the small-layer limits: 65 input channels, or more than 64K outputs
    for ci, hw in ((65, 32), (16, 46)):
        d = cc().conv2d_desc_create(cc().make_params(1, ci, hw, hw, 32, (3, 3), pads=1))
        assert cc().conv2d_desc_kernel_name(d) == "igemm_f32", (ci, hw)


def _raw(fn, *args):
    return fn(*[ctypes.c_void_p(a) if isinstance(a, int) else a for a in args])


def test_alias_rejected_before_launch():
    """Fake device addresses: every call below must return before any HIP call."""
    lib = cc()._lib
    L = dict(n=2, c_in=4, h=8, w=8, c_out=4, k=3, pads=1)
    d = cc().conv2d_desc_create(cc().make_params(2, 4, 8, 8, 4, 3, pads=1))
    X = 0x10000000
    xb = 2 * 4 * 64 * 4
    assert _raw(lib.conv2d_forward, d.handle, X, X + 10 * xb, None, None, X + xb - 4, None) == cc().CONV_ERR_ALIAS
    assert _raw(lib.conv2d_forward, d.handle, X, X + 10 * xb, None, None, X + 10 * xb + 8, None) == cc().CONV_ERR_ALIAS
    assert _raw(lib.conv2d_forward, d.handle, 0, X, None, None, X + xb, None) == cc().CONV_ERR_INVALID_ARG
    # concat buffer: input channels [0, 4) and output channels [4, 8) of the same
    # 8-channel buffer are disjoint for every image -> only the overlap case fails.
    pin = cc().make_params(2, 4, 8, 8, 4, 3, pads=1, in_total_channels=8, out_total_channels=8,
                           out_channel_offset=3)
    din = cc().conv2d_desc_create(pin)
    assert _raw(lib.conv2d_forward, din.handle, X, X + 100 * xb, None, None, X, None) == cc().CONV_ERR_ALIAS
    # has_bias without bias pointer
    db = cc().conv2d_desc_create(cc().make_params(2, 4, 8, 8, 4, 3, pads=1, has_bias=True))
    assert _raw(lib.conv2d_forward, db.handle, X, X + 10 * xb, None, None, X + 20 * xb, None) == cc().CONV_ERR_INVALID_ARG
    # int8 descriptor through the float entry point, and non-symmetric int8
    dq = cc().conv2d_desc_create(cc().make_params(2, 4, 8, 8, 4, 3, pads=1, dtype="i8"))
    assert _raw(lib.conv2d_forward, dq.handle, X, X + 10 * xb, None, None, X + 20 * xb, None) == cc().CONV_ERR_INVALID_ARG
    q = lib.qconv2d_forward
    f = ctypes.c_float
    assert q(dq.handle, ctypes.c_void_p(X), f(0.1), ctypes.c_int8(2), ctypes.c_void_p(X + xb), f(0.1),
             ctypes.c_int8(0), None, f(0.1), ctypes.c_int8(0), ctypes.c_void_p(X + 9 * xb), None) == cc().CONV_ERR_UNSUPPORTED
    assert q(dq.handle, ctypes.c_void_p(X), f(-0.1), ctypes.c_int8(0), ctypes.c_void_p(X + xb), f(0.1),
             ctypes.c_int8(0), None, f(0.1), ctypes.c_int8(0), ctypes.c_void_p(X + 9 * xb), None) == cc().CONV_ERR_INVALID_ARG
    assert q(dq.handle, ctypes.c_void_p(X), f(1e30), ctypes.c_int8(0), ctypes.c_void_p(X + xb), f(1e30),
             ctypes.c_int8(0), None, f(1e-30), ctypes.c_int8(0), ctypes.c_void_p(X + 9 * xb), None) == cc().CONV_ERR_INVALID_ARG
    assert q(dq.handle, ctypes.c_void_p(X), f(0.1), ctypes.c_int8(0), ctypes.c_void_p(X), f(0.1),
             ctypes.c_int8(0), None, f(0.1), ctypes.c_int8(0), ctypes.c_void_p(X + 10), None) == cc().CONV_ERR_ALIAS


def test_fused_pair_validation():
    lib = cc()._lib
    X = 0x20000000
    pw = cc().conv2d_desc_create(cc().make_params(2, 8, 10, 10, 16, 1))
    dw = cc().conv2d_desc_create(cc().make_params(2, 16, 10, 10, 16, 3, pads=1, groups=16))
    bad_dw = cc().conv2d_desc_create(cc().make_params(2, 12, 10, 10, 12, 3, pads=1, groups=12))
    dense = cc().conv2d_desc_create(cc().make_params(2, 16, 10, 10, 16, 3, pads=1))
    dw7 = cc().conv2d_desc_create(cc().make_params(2, 16, 10, 10, 16, 7, pads=3, groups=16))
    args = [ctypes.c_void_p(X + i * 0x100000) for i in range(3)]
    call = lambda a, b, y: lib.fused_pw_dw_forward(a.handle, b.handle, args[0], args[1], None, None, args[2],
                                                   None, None, ctypes.c_void_p(y), None)
    assert call(pw, bad_dw, X + 0x400000) == cc().CONV_ERR_INCOMPATIBLE_SHAPES
    assert call(pw, dense, X + 0x400000) == cc().CONV_ERR_INCOMPATIBLE_SHAPES
    assert call(dw, dw, X + 0x400000) == cc().CONV_ERR_INCOMPATIBLE_SHAPES
    assert call(pw, dw7, X + 0x400000) == cc().CONV_ERR_UNSUPPORTED
    assert call(pw, dw, X) == cc().CONV_ERR_ALIAS


def test_bound_weights_validation():
    """Null weights need bound ones; a null bind is refused.  Every call
    below returns before any HIP call (nothing is bound, so none reaches the
    device)."""
    lib = cc()._lib
    X = 0x30000000
    xb = 2 * 4 * 64 * 4
    d = cc().conv2d_desc_create(cc().make_params(2, 4, 8, 8, 4, 3, pads=1))
    assert _raw(lib.conv2d_desc_bind_weights, d.handle, 0, None) == cc().CONV_ERR_INVALID_ARG
    assert _raw(lib.conv2d_forward, d.handle, X, 0, None, None, X + 10 * xb, None) == cc().CONV_ERR_INVALID_ARG
    assert "no weights bound" in cc().conv2d_last_error()
    assert _raw(lib.conv2d_desc_bind_weights, 0, X, None) == cc().CONV_ERR_INVALID_ARG
    dq = cc().conv2d_desc_create(cc().make_params(2, 4, 8, 8, 4, 3, pads=1, dtype="i8"))
    f = ctypes.c_float
    assert lib.qconv2d_forward(dq.handle, ctypes.c_void_p(X), f(0.1), ctypes.c_int8(0), None, f(0.1),
                               ctypes.c_int8(0), None, f(0.1), ctypes.c_int8(0), ctypes.c_void_p(X + 9 * xb),
                               None) == cc().CONV_ERR_INVALID_ARG
    pw = cc().conv2d_desc_create(cc().make_params(2, 8, 10, 10, 16, 1))
    dw = cc().conv2d_desc_create(cc().make_params(2, 16, 10, 10, 16, 3, pads=1, groups=16))
    assert lib.fused_pw_dw_forward(pw.handle, dw.handle, ctypes.c_void_p(X), None, None, None,
                                   ctypes.c_void_p(X + 0x100000), None, None, ctypes.c_void_p(X + 0x400000),
                                   None) == cc().CONV_ERR_INVALID_ARG


def test_fused_dw_pw_rejects():
    lib = cc()._lib
    X = 0x40000000
    dw = cc().conv2d_desc_create(cc().make_params(2, 16, 10, 10, 16, 3, pads=1, groups=16))
    pw = cc().conv2d_desc_create(cc().make_params(2, 16, 10, 10, 8, 1))
    pw_bad = cc().conv2d_desc_create(cc().make_params(2, 12, 10, 10, 8, 1))
    dense = cc().conv2d_desc_create(cc().make_params(2, 16, 10, 10, 16, 3, pads=1))
    dw7 = cc().conv2d_desc_create(cc().make_params(2, 16, 16, 16, 16, 7, pads=3, groups=16))
    pw16 = cc().conv2d_desc_create(cc().make_params(2, 16, 16, 16, 8, 1))
    args = [ctypes.c_void_p(X + i * 0x100000) for i in range(3)]
    call = lambda a, b, y: lib.fused_dw_pw_forward(a.handle, b.handle, args[0], args[1], None, None, args[2],
                                                   None, None, ctypes.c_void_p(y), None)
    assert call(dw, pw_bad, X + 0x400000) == cc().CONV_ERR_INCOMPATIBLE_SHAPES
    assert call(dense, pw, X + 0x400000) == cc().CONV_ERR_INCOMPATIBLE_SHAPES
    assert call(pw, dw, X + 0x400000) == cc().CONV_ERR_INCOMPATIBLE_SHAPES
    assert call(dw7, pw16, X + 0x400000) == cc().CONV_ERR_UNSUPPORTED
    assert call(dw, pw, X) == cc().CONV_ERR_ALIAS


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    d = cc().conv2d_desc_create(cc().make_params(1, 4, 8, 8, 4, 3, pads=1))
    x = torch.zeros(4 * 64)
    with pytest.raises(ValueError):
        cc().conv2d_forward(d, x, torch.zeros(144), None, None, torch.zeros(256))


@pytest.mark.parametrize("bad", ["stride", "dilation", "groups", "kernel", "bf16"])
def test_winograd_rejects(bad):
    """algo = WINOGRAD on a shape F(2x2, 3x3) does not cover is refused at
    descriptor creation (no GPU call is made)."""
    kw = dict(stride=1, dilation=1, groups=1, dtype="f32")
    k = (3, 3)
    if bad == "stride":
        kw["stride"] = 2
    elif bad == "dilation":
        kw["dilation"] = 2
    elif bad == "groups":
        kw["groups"] = 2
    elif bad == "kernel":
        k = (5, 5)
    else:
        kw["dtype"] = "bf16"
    p = cc().make_params(1, 8, 16, 16, 8, k, pads=1, algo="winograd", **kw)
    with pytest.raises(cc().ConvError, match="Winograd") as e:
        cc().conv2d_desc_create(p)
    assert e.value.status == cc().CONV_ERR_UNSUPPORTED


def test_algo_field():
    """algo defaults to AUTO; an unknown value is refused; WINOGRAD on a 3x3 s1
    fp32 layer selects the Winograd kernel."""
    p = cc().conv2d_params_init()
    assert p.algo == cc().ALGO_AUTO
    p = cc().make_params(1, 8, 16, 16, 8, (3, 3), pads=1, algo=7)
    with pytest.raises(cc().ConvError):
        cc().conv2d_desc_create(p)
    d = cc().conv2d_desc_create(cc().make_params(1, 8, 16, 16, 8, (3, 3), pads=1, algo="winograd"))
    assert cc().conv2d_desc_kernel_name(d) == "winograd_f32"
    d = cc().conv2d_desc_create(cc().make_params(1, 8, 16, 16, 8, (3, 3), pads=1, algo="direct"))
    assert cc().conv2d_desc_kernel_name(d) != "winograd_f32"
