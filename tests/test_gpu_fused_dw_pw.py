"""GPU parity of the fused depthwise kxk -> pointwise 1x1 path
(fused_dw_pw_forward) against the oracle run as two separate convolutions,
the depthwise output rounded to float32 between them (as the unfused path
stores it).  fp32 tolerance 1e-4 * (1 + |ref|)."""
import numpy as np
import pytest

import workloads
from helpers import FP32_TOL, Guarded, assert_bitexact, assert_close, layer_params, oracle_layer, to_dev, torch

pytestmark = pytest.mark.gpu


def cc():
    import convolution_conv2d_forward_amd as m
    return m


A = workloads
CASES = [
    # n, c, h, w, k, stride, pads, dilation, c_out, dw act, pw act, bias, pad_value
    (2, 40, 9, 24, 3, 1, 1, 1, 24, A.ACT_CLIP, A.ACT_NONE, True, 0.0),          # 3x3 s1, channel tail chunk
    (1, 64, 13, 20, 3, 2, (0, 1, 2, 1), 1, 72, A.ACT_RELU, A.ACT_PRELU, True, -0.5),  # 3x3 s2, 2 co tiles
    (2, 17, 11, 13, 5, 1, 4, 2, 16, A.ACT_LEAKY_RELU, A.ACT_CLIP, False, 0.25),  # 5x5 d2, odd width (scalar rows)
    (1, 96, 7, 56, 3, 1, 1, 1, 130, A.ACT_PRELU, A.ACT_LEAKY_RELU, True, 1.0),  # 3 co tiles, cout % 64 != 0
    (3, 8, 30, 8, (1, 3), (1, 2), (0, 1, 0, 1), 1, 40, A.ACT_NONE, A.ACT_RELU, True, 0.0),  # 1x3 generic window
    (1, 33, 5, 100, 3, 1, 1, 1, 33, A.ACT_CLIP, A.ACT_CLIP, True, 0.0),        # wide rows
    (1, 1, 1, 1, 1, 1, 0, 1, 1, A.ACT_NONE, A.ACT_NONE, False, 0.0),            # smallest
]


def _layers(case):
    n, c, h, w, k, s, p, d, co, a1, a2, bias, pv = case
    k2 = k if isinstance(k, tuple) else (k, k)
    s2 = s if isinstance(s, tuple) else (s, s)
    p4 = p if isinstance(p, tuple) else (p,) * 4
    L1 = A.Layer("dw", n, c, h, w, c, k2, stride=s2, pads=p4, dilation=(d, d), groups=c, has_bias=bias, act=a1,
                 alpha=0.2, clip=(-0.4, 0.6), pad_value=pv)
    ho, wo = L1.out_hw
    L2 = A.Layer("pw", n, c, ho, wo, co, (1, 1), has_bias=bias, act=a2, alpha=0.1, clip=(-0.3, 0.8))
    return L1, L2


def _run(L1, L2, x, w1, b1, s1, w2, b2, s2, *, in_total=0, in_off=0, out_total=0, out_off=0, bind=False):
    t = torch()
    d1 = cc().conv2d_desc_create(layer_params(L1, prelu_slope_count=s1.size, in_total_channels=in_total,
                                              in_channel_offset=in_off))
    d2 = cc().conv2d_desc_create(layer_params(L2, prelu_slope_count=s2.size, out_total_channels=out_total,
                                              out_channel_offset=out_off))
    n, ot, ho, wo = cc().conv2d_desc_get_output_shape(d2)
    y = Guarded(n * ot * ho * wo, t.float32, float("nan"))
    dv = lambda v, on: to_dev(v) if on else None
    wd1, wd2 = to_dev(w1), to_dev(w2)
    if bind:
        cc().conv2d_desc_bind_weights(d1, wd1)
        cc().conv2d_desc_bind_weights(d2, wd2)
        wd1 = wd2 = None
    cc().fused_dw_pw_forward(d1, d2, to_dev(x), wd1, dv(b1, L1.has_bias), dv(s1, L1.act == A.ACT_PRELU), wd2,
                             dv(b2, L2.has_bias), dv(s2, L2.act == A.ACT_PRELU), y.view)
    t.cuda.synchronize()
    y.check_guards()
    return y.host().numpy().reshape(n, ot, ho, wo)


def _oracle(L1, L2, x, w1, b1, s1, w2, b2, s2):
    mid = oracle_layer(L1, x, w1, b1, s1).astype(np.float32)
    return oracle_layer(L2, mid, w2, b2, s2)


@pytest.mark.parametrize("i", range(len(CASES)))
def test_fused_dw_pw_cases(i):
    L1, L2 = _layers(CASES[i])
    rng = np.random.default_rng(500 + i)
    x, w1, b1, s1 = A.layer_arrays(rng, L1)
    _, w2, b2, s2 = A.layer_arrays(rng, L2)
    print(f"case {i} {L1} -> {L2}", flush=True)
    ref = _oracle(L1, L2, x, w1, b1, s1, w2, b2, s2)
    y1 = _run(L1, L2, x, w1, b1, s1, w2, b2, s2)
    assert_close(y1, ref, FP32_TOL, f"fused dw->pw case {i}")
    y2 = _run(L1, L2, x, w1, b1, s1, w2, b2, s2, bind=True)
    assert_bitexact(y2, y1, f"case {i}: bound weights vs explicit")


def test_fused_dw_pw_concat_slices():
    """Depthwise input read from channels [3, 3+c) of a wider buffer; pointwise
    output written to channels [5, 5+co) of a wider buffer (ConcatFusedTail);
    the channels around the slice stay untouched (NaN guard)."""
    L1, L2 = _layers(CASES[0])
    rng = np.random.default_rng(540)
    x, w1, b1, s1 = A.layer_arrays(rng, L1)
    _, w2, b2, s2 = A.layer_arrays(rng, L2)
    big = rng.standard_normal((L1.n, L1.c_in + 7, L1.h, L1.w)).astype(np.float32)
    big[:, 3:3 + L1.c_in] = x
    y = _run(L1, L2, big, w1, b1, s1, w2, b2, s2, in_total=L1.c_in + 7, in_off=3, out_total=L2.c_out + 9,
             out_off=5)
    assert np.isnan(y[:, :5]).all() and np.isnan(y[:, 5 + L2.c_out:]).all()
    assert_close(y[:, 5:5 + L2.c_out], _oracle(L1, L2, x, w1, b1, s1, w2, b2, s2), FP32_TOL, "slices")


def test_fused_dw_pw_bottleneck_full_size():
    """The inverted bottleneck's depthwise 3x3 + Clip(0,6) -> pointwise 192->32
    at full size (N=8, 56x56), fed with the oracle's own pointwise-1 output."""
    wl = A.bottleneck()
    a = wl.arrays
    L1, L2, L3 = wl.layers
    e = oracle_layer(L1, a["x"], a["w_pw1"], None, None).astype(np.float32)
    ref = _oracle(L2, L3, e, a["w_dw"], None, np.zeros(1, np.float32), a["w_pw2"], None, np.zeros(1, np.float32))
    y = _run(L2, L3, e, a["w_dw"], None, np.zeros(1, np.float32), a["w_pw2"], None, np.zeros(1, np.float32))
    assert_close(y, ref, FP32_TOL, "bottleneck dw->pw2")

