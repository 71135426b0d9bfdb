"""GPU: weights bound to the descriptor once (conv2d_desc_bind_weights) and
used by forward calls given a null weight pointer.

For every kernel class the bound path must give bitwise the same output as
the same descriptor given the weights explicitly (same kernels, same
arithmetic; only where the weights are read from differs), and match the
oracle at the float tolerances.  Rebinding replaces the weights; an explicit
call in between does not disturb the bound copy."""
import numpy as np
import pytest

import workloads
from helpers import (BF16_TOL, FP32_TOL, Guarded, assert_bitexact, assert_close, bf16_round, layer_params,
                     oracle_layer, to_dev, torch)
from test_gpu_parity import CLASS_CASES

pytestmark = pytest.mark.gpu


def cc():
    import convolution_conv2d_forward_amd as m
    return m


def _layer(i, pad_value=0.0):
    n, ci, h, w, co, k, s, p, d, g, act = CLASS_CASES[i]
    k2 = k if isinstance(k, tuple) else (k, k)
    s2 = s if isinstance(s, tuple) else (s, s)
    d2 = d if isinstance(d, tuple) else (d, d)
    p4 = p if isinstance(p, tuple) else (p, p, p, p)
    return workloads.Layer("case", n, ci, h, w, co, k2, stride=s2, pads=p4, dilation=d2, groups=g,
                           has_bias=True, act=act, alpha=0.1, clip=(-0.5, 0.75), pad_value=pad_value)


def _run(d, L, xd, wd, bd, sd, tdt):
    t = torch()
    n, ot, ho, wo = cc().conv2d_desc_get_output_shape(d)
    y = Guarded(n * ot * ho * wo, tdt, float("nan"))
    cc().conv2d_forward(d, xd, wd, bd, sd, y.view)
    t.cuda.synchronize()
    y.check_guards()
    return y.host().float().numpy().astype(np.float64).reshape(n, ot, ho, wo)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("i", range(len(CLASS_CASES)))
def test_bound_equals_explicit(i, dtype):
    t = torch()
    tdt = t.float32 if dtype == "f32" else t.bfloat16
    tol = FP32_TOL if dtype == "f32" else BF16_TOL
    L = _layer(i, pad_value=-0.25)
    rng = np.random.default_rng(900 + i)
    x, w, b, s = workloads.layer_arrays(rng, L)
    _, w2, _, _ = workloads.layer_arrays(rng, L)
    if dtype == "bf16":
        x, w, w2 = bf16_round(x), bf16_round(w), bf16_round(w2)
    d = cc().conv2d_desc_create(layer_params(L, dtype, prelu_slope_count=s.size))
    kname = cc().conv2d_desc_kernel_name(d)
    print(f"case {i} {dtype} {kname}", flush=True)
    xd, wd, w2d = to_dev(x, tdt), to_dev(w, tdt), to_dev(w2, tdt)
    bd, sd = to_dev(b), to_dev(s) if L.act == workloads.ACT_PRELU else None
    explicit = _run(d, L, xd, wd, bd, sd, tdt)
    cc().conv2d_desc_bind_weights(d, wd)
    wd.fill_(float("nan"))                      # the bound copy must not read the caller's buffer again
    bound = _run(d, L, xd, None, bd, sd, tdt)
    assert_bitexact(bound, explicit, f"case {i} {dtype} ({kname}): bound vs explicit")
    assert_close(bound, oracle_layer(L, x, w, b, s), tol, f"case {i} {dtype} ({kname})")
    # An explicit call with other weights leaves the bound copy alone ...
    other = _run(d, L, xd, w2d, bd, sd, tdt)
    assert_close(other, oracle_layer(L, x, w2, b, s), tol, f"case {i} {dtype}: explicit w2")
    assert_bitexact(_run(d, L, xd, None, bd, sd, tdt), explicit, f"case {i} {dtype}: bound after explicit")
    # ... and binding again replaces it.
    cc().conv2d_desc_bind_weights(d, w2d)
    assert_bitexact(_run(d, L, xd, None, bd, sd, tdt), other, f"case {i} {dtype}: rebound")


def test_bound_bf16_unaligned_input_uses_the_oihw_copy():
    """A bf16 implicit-GEMM descriptor whose input is not 16-byte aligned runs
    the direct kernel, which reads the OIHW copy kept next to the packed one."""
    t = torch()
    L = _layer(1)
    rng = np.random.default_rng(950)
    x, w, b, s = workloads.layer_arrays(rng, L)
    x, w = bf16_round(x), bf16_round(w)
    d = cc().conv2d_desc_create(layer_params(L, "bf16", prelu_slope_count=s.size))
    assert cc().conv2d_desc_kernel_name(d).startswith("igemm_bf16")
    flat = to_dev(np.concatenate([np.zeros(1, np.float32), x.reshape(-1)]), t.bfloat16)
    xd = flat[1:]                                   # 2-byte offset: not 16-byte aligned
    assert xd.data_ptr() % 16 != 0
    cc().conv2d_desc_bind_weights(d, to_dev(w, t.bfloat16))
    y = _run(d, L, xd, None, to_dev(b), None, t.bfloat16)
    assert_close(y, oracle_layer(L, x, w, b, s), BF16_TOL, "unaligned bf16, bound weights")


def test_bound_fused_pw_dw():
    t = torch()
    wl = workloads.bottleneck(n=2, h=20, w=24)
    a = wl.arrays
    L1, L2, _ = wl.layers
    d1, d2 = cc().conv2d_desc_create(layer_params(L1)), cc().conv2d_desc_create(layer_params(L2))
    x, w1, w2 = to_dev(a["x"]), to_dev(a["w_pw1"]), to_dev(a["w_dw"])
    ho, wo = L2.out_hw
    outs = []
    for bound in (False, True):
        if bound:
            cc().conv2d_desc_bind_weights(d1, w1)
            cc().conv2d_desc_bind_weights(d2, w2)
        y = Guarded(L2.n * L2.c_out * ho * wo, t.float32, float("nan"))
        cc().fused_pw_dw_forward(d1, d2, x, None if bound else w1, None, None, None if bound else w2, None, None,
                                 y.view)
        t.cuda.synchronize()
        y.check_guards()
        outs.append(y.host().numpy().reshape(L2.n, L2.c_out, ho, wo))
    assert_bitexact(outs[1], outs[0], "fused: bound vs explicit")
    e = oracle_layer(L1, a["x"], a["w_pw1"], None, None).astype(np.float32)
    assert_close(outs[1], oracle_layer(L2, e, a["w_dw"], None, None), FP32_TOL, "fused bound")


@pytest.mark.parametrize("which", ["dw_s1", "dw_s2", "pw"])
def test_bound_int8(which):
    t = torch()
    layers = {L.name: L for L in workloads.int8_chain_layers(n=2, h=24, w=32)}
    L = layers[which]
    rng = np.random.default_rng(960)
    x = rng.integers(-128, 128, size=(L.n, L.c_in, L.h, L.w), dtype=np.int8)
    w = rng.integers(-127, 128, size=(L.c_out, L.c_in // L.groups) + tuple(L.k), dtype=np.int8)
    b = rng.integers(-500, 501, size=L.c_out, dtype=np.int32)
    sx, sw, sy = workloads.INT8_SCALES
    d = cc().conv2d_desc_create(layer_params(L, "i8"))
    n, ot, ho, wo = cc().conv2d_desc_get_output_shape(d)
    xd, wd, bd = to_dev(x), to_dev(w), to_dev(b)
    outs = []
    for bound in (False, True):
        if bound:
            cc().conv2d_desc_bind_weights(d, wd)
            wd.fill_(0)
        y = Guarded(n * ot * ho * wo, t.int8, 0x5A)
        cc().qconv2d_forward(d, xd, sx, 0, None if bound else wd, sw, 0, bd, sy, 0, y.view)
        t.cuda.synchronize()
        y.check_guards()
        outs.append(y.host().numpy())
    assert_bitexact(outs[1], outs[0], f"int8 {which}: bound vs explicit")
