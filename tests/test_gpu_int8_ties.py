"""GPU: int8 requant on exact f32 ties, every int8 kernel.

The requant multiplies the int32 sum by the composite scale in f32 and rounds
that f32 product (QLinearConv of the ONNX operator page; the yscv requant
epilogue).  With the composite f32(f32(0.03 * 0.02) / 0.04) = f32(0.015),
sums of 100 * odd give products that are not exactly representable but round
to an exact x.5 in f32 (1700 * f32(0.015) = 25.4999994 -> 25.5).  The tie has
to be decided on that rounded product: a kernel that fuses the multiply into
the rounding step (one fma) sees 25.4999994 and rounds toward zero.

Small value ranges keep the sums away from saturation so that ties are
common; each case first checks that the oracle's two rounding modes disagree
somewhere (the case does contain ties), then that every GPU path is
bit-exact with the oracle in both modes."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import Guarded, assert_bitexact, layer_params, to_dev, torch

pytestmark = pytest.mark.gpu

SC = (0.03, 0.02, 0.04)          # x, w, y: composite f32(0.015)
HALF_EVEN, HALF_AWAY = 0, 1


def cc():
    import convolution_conv2d_forward_amd as m
    return m


LAYERS = [
    # name, n, c_in, h, w, c_out, k, stride, pads, groups
    ("dw3 s1", 2, 32, 12, 32, 32, 3, 1, (1, 1, 1, 1), 32),
    ("dw3 s2 pad 0", 2, 48, 15, 32, 48, 3, 2, (0, 0, 1, 1), 48),
    ("dw5 generic", 1, 24, 9, 13, 24, 5, 1, (2, 2, 2, 2), 24),
    ("pw", 2, 64, 10, 24, 40, 1, 1, (0, 0, 0, 0), 1),
    ("dense 3x3", 1, 16, 9, 11, 24, 3, 1, (1, 1, 1, 1), 1),
]


def _inputs(rng, L):
    x = rng.integers(-20, 20, size=L.x_shape, endpoint=True).astype(np.int8)
    w = rng.integers(-20, 20, size=L.w_shape, endpoint=True).astype(np.int8)
    b = (100 * rng.integers(-5, 5, size=L.c_out, endpoint=True)).astype(np.int32)
    return x, w, b


def _ties(a, b):
    return int(np.count_nonzero(a != b))


@pytest.mark.parametrize("i", range(len(LAYERS)))
def test_qconv2d_ties(i):
    t = torch()
    name, n, ci, h, w, co, k, s, pads, g = LAYERS[i]
    L = workloads.Layer(name, n, ci, h, w, co, (k, k), stride=(s, s), pads=pads, groups=g, has_bias=True)
    rng = np.random.default_rng(900 + i)
    x, wt, b = _inputs(rng, L)
    refs = {r: oracle.qconv2d(x, wt, b, *SC, stride=L.stride, pads=L.pads, groups=L.groups, rounding=r)
            for r in (HALF_EVEN, HALF_AWAY)}
    assert _ties(refs[HALF_EVEN], refs[HALF_AWAY]) > 0, "no ties in this case"
    for r, ref in refs.items():
        d = cc().conv2d_desc_create(layer_params(L, "i8", int8_rounding=r))
        nn, ot, ho, wo = cc().conv2d_desc_get_output_shape(d)
        y = Guarded(nn * ot * ho * wo, t.int8, 0x5A)
        cc().qconv2d_forward(d, to_dev(x), SC[0], 0, to_dev(wt), SC[1], 0, to_dev(b), SC[2], 0, y.view)
        t.cuda.synchronize()
        y.check_guards()
        print(f"{name} rounding {r}: {cc().conv2d_desc_kernel_name(d)}, "
              f"ties {_ties(refs[HALF_EVEN], refs[HALF_AWAY])}", flush=True)
        assert_bitexact(y.host().numpy().reshape(ref.shape), ref, f"{name} rounding {r}")


FUSED = [
    # n, c, h, w, k, stride, pads, c_out  (the first two take the 16-byte row path)
    (2, 48, 15, 32, 3, 2, (0, 0, 1, 1), 24),
    (1, 64, 10, 32, 3, 1, (1, 1, 1, 1), 40),
    (1, 20, 9, 13, 3, 1, (1, 1, 1, 1), 24),
]


@pytest.mark.parametrize("i", range(len(FUSED)))
def test_qfused_ties(i):
    t = torch()
    n, c, h, w, k, s, pads, co = FUSED[i]
    L1 = workloads.Layer("dw", n, c, h, w, c, (k, k), stride=(s, s), pads=pads, groups=c, has_bias=True)
    ho, wo = L1.out_hw
    L2 = workloads.Layer("pw", n, c, ho, wo, co, (1, 1), has_bias=True)
    rng = np.random.default_rng(950 + i)
    x, w1, b1 = _inputs(rng, L1)
    _, w2, b2 = _inputs(rng, L2)
    # the pointwise input scale is the depthwise output scale
    sp = (SC[2], SC[1], SC[2])
    mids, refs = {}, {}
    for r in (HALF_EVEN, HALF_AWAY):
        mids[r] = oracle.qconv2d(x, w1, b1, *SC, stride=L1.stride, pads=L1.pads, groups=L1.groups, rounding=r)
        refs[r] = oracle.qconv2d(mids[r], w2, b2, *sp, rounding=r)
    assert _ties(mids[HALF_EVEN], mids[HALF_AWAY]) > 0, "no depthwise ties in this case"
    for r, ref in refs.items():
        d1 = cc().conv2d_desc_create(layer_params(L1, "i8", int8_rounding=r))
        d2 = cc().conv2d_desc_create(layer_params(L2, "i8", int8_rounding=r))
        nn, ot, h2, w2o = cc().conv2d_desc_get_output_shape(d2)
        y = Guarded(nn * ot * h2 * w2o, t.int8, 0x5A)
        cc().qfused_dw_pw_forward(d1, d2, to_dev(x), to_dev(w1), to_dev(b1), SC, to_dev(w2), to_dev(b2), sp, 0,
                                  y.view)
        t.cuda.synchronize()
        y.check_guards()
        assert_bitexact(y.host().numpy().reshape(ref.shape), ref, f"fused case {i} rounding {r}")


FUSED_PW_DW = [
    # n, c_in, h, w, c_exp, k, stride, pads  (the first two take the 4-byte row path)
    (2, 32, 12, 16, 48, 3, 1, (1, 1, 1, 1)),
    (1, 64, 10, 32, 40, 3, 2, (0, 0, 1, 1)),
    (1, 20, 9, 13, 24, 5, 1, (2, 2, 2, 2)),
]


@pytest.mark.parametrize("i", range(len(FUSED_PW_DW)))
def test_qfused_pw_dw_ties(i):
    t = torch()
    n, c, h, w, ce, k, s, pads = FUSED_PW_DW[i]
    L1 = workloads.Layer("pw", n, c, h, w, ce, (1, 1), has_bias=True)
    L2 = workloads.Layer("dw", n, ce, h, w, ce, (k, k), stride=(s, s), pads=pads, groups=ce, has_bias=True)
    rng = np.random.default_rng(970 + i)
    x, w1, b1 = _inputs(rng, L1)
    _, w2, b2 = _inputs(rng, L2)
    sd = (SC[2], SC[1], SC[2])
    mids, refs = {}, {}
    for r in (HALF_EVEN, HALF_AWAY):
        mids[r] = oracle.qconv2d(x, w1, b1, *SC, rounding=r)
        refs[r] = oracle.qconv2d(mids[r], w2, b2, *sd, stride=L2.stride, pads=L2.pads, groups=L2.groups,
                                 rounding=r)
    assert _ties(mids[HALF_EVEN], mids[HALF_AWAY]) > 0, "no pointwise ties in this case"
    for r, ref in refs.items():
        d1 = cc().conv2d_desc_create(layer_params(L1, "i8", int8_rounding=r))
        d2 = cc().conv2d_desc_create(layer_params(L2, "i8", int8_rounding=r))
        nn, ot, h2, w2o = cc().conv2d_desc_get_output_shape(d2)
        y = Guarded(nn * ot * h2 * w2o, t.int8, 0x5A)
        cc().qfused_pw_dw_forward(d1, d2, to_dev(x), to_dev(w1), to_dev(b1), SC, to_dev(w2), to_dev(b2), sd, 0,
                                  y.view)
        t.cuda.synchronize()
        y.check_guards()
        assert_bitexact(y.host().numpy().reshape(ref.shape), ref, f"fused pw->dw case {i} rounding {r}")
