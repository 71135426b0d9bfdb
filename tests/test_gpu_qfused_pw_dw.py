"""GPU: the fused int8 pointwise -> depthwise path (qfused_pw_dw_forward).

Bit-exact twice over: against the oracle's two QLinearConvs chained through
the int8 expansion (the depthwise padding reads the expansion's zero point),
and against the library's own unfused calls (qconv2d_forward twice)."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import Guarded, assert_bitexact, layer_params, to_dev, torch

pytestmark = pytest.mark.gpu


def cc():
    import convolution_conv2d_forward_amd as m
    return m


TIES = (1.0, 1.0, 2.0, 1.0, 36.0)   # pw composite 0.5 (every odd sum a tie); dw composite 1/36
SYM = (0.02, 0.01, 0.05, 0.01, 0.05)
CASES = [
    # n, c_in, h, w, c_exp, k, stride, pads, dilation, scales (x, w_pw, mid, w_dw, y), pw relu, dw relu, y_zp,
    # rounding
    (2, 32, 14, 16, 64, 3, 1, 1, 1, SYM, False, False, 0, 0),            # bottleneck shape, 2 channel tiles
    (1, 32, 9, 13, 40, 3, 1, 1, 1, SYM, True, False, 0, 0),              # odd width (byte rows), partial tile
    (2, 20, 11, 24, 70, 5, 1, (2, 1, 2, 3), 2, (0.03, 0.02, 0.04, 0.01, 0.09), False, True, 3, 1),  # 5x5 d2
    (1, 130, 6, 8, 16, 3, 2, (0, 1, 1, 0), 1, TIES, True, True, -2, 1),  # ties, 3 K chunks, s2
    (1, 200, 7, 12, 36, 3, 2, 1, 1, TIES, False, False, 0, 0),           # ties ties-to-even, K not a multiple of 16
    (3, 7, 5, 5, 9, 1, 1, 0, 1, SYM, False, False, 5, 0),                # 1x1 depthwise window
    (1, 48, 24, 80, 32, 3, 1, 1, 1, SYM, False, True, 0, 0),             # several row tiles
    (2, 16, 15, 32, 24, 3, 2, (0, 0, 1, 1), 1, (0.03, 0.02, 0.04, 0.01, 0.09), False, True, -3, 1),
    (1, 64, 9, 48, 40, 5, 1, 2, 1, SYM, True, True, 2, 0),               # 5x5 s1
    (1, 16, 10, 32, 16, 5, 2, (2, 1, 2, 1), 1, SYM, False, False, 0, 1), # 5x5 s2, wo 15
    (2, 24, 6, 16, 72, 3, 2, (1, 3, 1, 3), 1, TIES, True, True, -2, 1),  # pad 3
    (4, 8, 3, 4, 8, 3, 1, 1, 1, SYM, False, False, 0, 0),                # tiny images
]


def _layers(case):
    n, c, h, w, ce, k, s, p, d = case[:9]
    p4 = p if isinstance(p, tuple) else (p,) * 4
    L1 = workloads.Layer("pw", n, c, h, w, ce, (1, 1), has_bias=True)
    L2 = workloads.Layer("dw", n, ce, h, w, ce, (k, k), stride=(s, s), pads=p4, dilation=(d, d), groups=ce,
                         has_bias=True)
    return L1, L2


def _desc(L, rounding, relu, **kw):
    p = layer_params(L, "i8", int8_rounding=rounding, **kw)
    if relu:
        p.act_type = 1
    return cc().conv2d_desc_create(p)


def _arrays(rng, L1, L2):
    x = rng.integers(-128, 127, size=L1.x_shape, endpoint=True).astype(np.int8)
    w1 = rng.integers(-127, 127, size=L1.w_shape, endpoint=True).astype(np.int8)
    w2 = rng.integers(-127, 127, size=L2.w_shape, endpoint=True).astype(np.int8)
    b1 = rng.integers(-500, 500, size=L1.c_out, endpoint=True).astype(np.int32)
    b2 = rng.integers(-500, 500, size=L2.c_out, endpoint=True).astype(np.int32)
    return x, w1, w2, b1, b2


def _oracle_chain(L1, L2, x, w1, w2, b1, b2, scales, relu1, relu2, y_zp, rnd):
    sx, swp, smid, swd, sy = scales
    mid = oracle.qconv2d(x, w1, b1, sx, swp, smid, rounding=rnd, relu=relu1)
    ref = oracle.qconv2d(mid, w2, b2, smid, swd, sy, stride=L2.stride, pads=L2.pads, dilation=L2.dilation,
                         groups=L2.groups, y_zp=y_zp, rounding=rnd, relu=relu2)
    return mid, ref


def _fused(d1, d2, xd, w1d, b1d, w2d, b2d, scales, y_zp):
    t = torch()
    sx, swp, smid, swd, sy = scales
    n, ot, ho, wo = cc().conv2d_desc_get_output_shape(d2)
    y = Guarded(n * ot * ho * wo, t.int8, 0x5A)
    cc().qfused_pw_dw_forward(d1, d2, xd, w1d, b1d, (sx, swp, smid), w2d, b2d, (smid, swd, sy), y_zp, y.view)
    t.cuda.synchronize()
    y.check_guards()
    return y.host().numpy().reshape(n, ot, ho, wo)


@pytest.mark.parametrize("i", range(len(CASES)))
def test_qfused_pw_dw_cases(i):
    t = torch()
    case = CASES[i]
    L1, L2 = _layers(case)
    scales = case[9]
    relu1, relu2, y_zp, rnd = case[10:]
    rng = np.random.default_rng(1700 + i)
    x, w1, w2, b1, b2 = _arrays(rng, L1, L2)
    mid, ref = _oracle_chain(L1, L2, x, w1, w2, b1, b2, scales, relu1, relu2, y_zp, rnd)
    if scales is TIES:
        acc = oracle.qconv2d_acc(x, w1) + b1.reshape(1, -1, 1, 1)
        assert np.any(acc % 2 != 0), "tie case without ties"
    print(f"case {i}: {L1} -> {L2}; expansion saturated {np.mean(np.abs(mid.astype(int)) >= 127):.3f}", flush=True)
    d1, d2 = _desc(L1, rnd, relu1), _desc(L2, rnd, relu2)
    xd, w1d, w2d, b1d, b2d = to_dev(x), to_dev(w1), to_dev(w2), to_dev(b1), to_dev(b2)
    got = _fused(d1, d2, xd, w1d, b1d, w2d, b2d, scales, y_zp)
    assert_bitexact(got, ref, f"case {i}: fused vs oracle chain")
    # the library's unfused path
    sx, swp, smid, swd, sy = scales
    n, ot, ho, wo = got.shape
    tmp = t.empty(L1.n * L1.c_out * L1.h * L1.w, dtype=t.int8, device="cuda")
    y2 = t.empty(n * ot * ho * wo, dtype=t.int8, device="cuda")
    cc().qconv2d_forward(d1, xd, sx, 0, w1d, swp, 0, b1d, smid, 0, tmp)
    cc().qconv2d_forward(d2, tmp, smid, 0, w2d, swd, 0, b2d, sy, y_zp, y2)
    t.cuda.synchronize()
    assert_bitexact(got, y2.cpu().numpy().reshape(n, ot, ho, wo), f"case {i}: fused vs unfused")
    # bound weights
    cc().conv2d_desc_bind_weights(d1, w1d)
    cc().conv2d_desc_bind_weights(d2, w2d)
    got3 = _fused(d1, d2, xd, None, b1d, None, b2d, scales, y_zp)
    assert_bitexact(got3, got, f"case {i}: bound weights")


def test_qfused_pw_dw_bottleneck_full_size():
    """The inverted bottleneck's expansion and depthwise in int8 at full size
    (8 x 32 x 56 x 56 -> 192 -> depthwise 3x3), the symmetric scales at both
    stages, against the oracle chain and the unfused pair."""
    t = torch()
    L1 = workloads.Layer("pw", 8, 32, 56, 56, 192, (1, 1), has_bias=True)
    L2 = workloads.Layer("dw", 8, 192, 56, 56, 192, (3, 3), pads=(1, 1, 1, 1), groups=192, has_bias=True)
    rng = np.random.default_rng(1799)
    x, w1, w2, b1, b2 = _arrays(rng, L1, L2)
    _, ref = _oracle_chain(L1, L2, x, w1, w2, b1, b2, SYM, False, False, 0, 0)
    d1, d2 = _desc(L1, 0, False), _desc(L2, 0, False)
    got = _fused(d1, d2, to_dev(x), to_dev(w1), to_dev(b1), to_dev(w2), to_dev(b2), SYM, 0)
    assert_bitexact(got, ref, "bottleneck pw -> dw fused vs oracle")


def test_qfused_pw_dw_slices():
    """Pointwise input from channels [3, 3 + c_in) of a wider buffer; depthwise
    output into channels [4, 4 + c_exp) of a wider one (ConcatFusedTail)."""
    t = torch()
    L1, L2 = _layers(CASES[0])
    rng = np.random.default_rng(1760)
    x, w1, w2, b1, b2 = _arrays(rng, L1, L2)
    _, ref = _oracle_chain(L1, L2, x, w1, w2, b1, b2, SYM, False, False, 0, 0)
    big = rng.integers(-128, 127, size=(L1.n, L1.c_in + 5, L1.h, L1.w), endpoint=True).astype(np.int8)
    big[:, 3:3 + L1.c_in] = x
    d1 = _desc(L1, 0, False, in_total_channels=L1.c_in + 5, in_channel_offset=3)
    d2 = _desc(L2, 0, False, out_total_channels=L2.c_out + 7, out_channel_offset=4)
    got = _fused(d1, d2, to_dev(big), to_dev(w1), to_dev(b1), to_dev(w2), to_dev(b2), SYM, 0)
    assert (got[:, :4] == 0x5A).all() and (got[:, 4 + L2.c_out:] == 0x5A).all()
    assert_bitexact(got[:, 4:4 + L2.c_out], ref, "slices")
