"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself: values worked out
by hand from the ncnn "convolution" definition (tests/golden), closed forms,
invariants of correlation (linearity, stride = subsampling, dilation = a
zero-stuffed kernel, groups = independent convolutions), and special cases
that reduce to library routines (numpy.matmul, scipy.signal.correlate2d,
torch.nn.functional.conv2d in float64, numpy.rint).  A dropped term, a wrong
sign or index, or a transposed operand in oracle.c fails at least one of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ----------------------------------------------------------- hand cases ---

@pytest.mark.parametrize("case", _golden()["conv_cases"], ids=lambda c: c["name"])
def test_hand_cases(case):
    x = np.array(case["x"], dtype=np.float64)[None, None]
    kh, kw = case["k"]
    w = np.ones((1, 1, kh, kw))
    y = oracle.conv2d(x, w, stride=case["stride"], pads=case["pads"], dilation=case["dilation"],
                      pad_value=case["pad_value"])
    np.testing.assert_array_equal(y[0, 0], np.array(case["y"], dtype=np.float64))


def test_hand_group_case():
    c = _golden()["group_case"]
    x = np.array(c["x"], dtype=np.float64).reshape(1, 2, 1, 1)
    w = np.array(c["w"], dtype=np.float64).reshape(2, 1, 1, 1)
    y = oracle.conv2d(x, w, groups=c["groups"])
    np.testing.assert_array_equal(y.reshape(-1), np.array(c["y"], dtype=np.float64))


def test_hand_requant_ties():
    c = _golden()["requant_case"]
    comp = oracle.composite_scale(c["x_scale"], c["w_scale"], c["y_scale"])
    assert comp == np.float32(0.5)
    acc = np.array(c["acc"], dtype=np.int64)
    np.testing.assert_array_equal(oracle.requant(acc, comp, rounding=oracle.ROUND_HALF_EVEN),
                                  np.array(c["half_even"], dtype=np.int8))
    np.testing.assert_array_equal(oracle.requant(acc, comp, rounding=oracle.ROUND_HALF_AWAY),
                                  np.array(c["half_away"], dtype=np.int8))


def test_hand_activation_points():
    c = _golden()["activation_case"]
    v = np.array(c["v"], dtype=np.float64)
    x = v.reshape(1, 1, 1, -1)
    w = np.ones((1, 1, 1, 1))
    relu = oracle.conv2d(x, w, act=oracle.ACT_RELU).reshape(-1)
    leaky = oracle.conv2d(x, w, act=oracle.ACT_LEAKY_RELU, alpha=0.2).reshape(-1)
    prelu = oracle.conv2d(x, w, act=oracle.ACT_PRELU, slope=np.array([0.1])).reshape(-1)
    clip = oracle.conv2d(x, w, act=oracle.ACT_CLIP, clip=(0.0, 6.0)).reshape(-1)
    np.testing.assert_allclose(relu, c["relu"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(leaky, c["leaky_0.2"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(prelu, c["prelu_0.1"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(clip, c["clip_0_6"], rtol=0, atol=1e-15)


def test_activation_defaults_and_per_channel_prelu():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, 3, 4, 5))
    w = np.eye(3).reshape(3, 3, 1, 1)
    b = np.array([0.5, -0.25, 0.0])
    slope = np.array([0.1, 0.2, 0.3])
    y = oracle.conv2d(x, w, b, act=oracle.ACT_PRELU, slope=slope)
    v = x + b.reshape(1, 3, 1, 1)
    np.testing.assert_allclose(y, np.where(v >= 0, v, slope.reshape(1, 3, 1, 1) * v), rtol=0, atol=1e-15)
    # Leaky default alpha is 0.01; clip defaults are -FLT_MAX / FLT_MAX (identity on finite data).
    y = oracle.conv2d(x, w, act=oracle.ACT_LEAKY_RELU)
    np.testing.assert_allclose(y, np.where(x >= 0, x, 0.01 * x), rtol=0, atol=1e-15)
    y = oracle.conv2d(x * 1e30, w, act=oracle.ACT_CLIP)
    np.testing.assert_array_equal(y, x * 1e30)


# ------------------------------------------ independent formulations ------

def _shift_and_add(x, w, b, stride, pads, dilation, groups, pad_value):
    """Correlation as a sum of shifted, strided views of the explicitly padded
    input (numpy.pad + slicing + einsum over the group): no per-element index
    arithmetic shared with the oracle's loops."""
    n, c, _, _ = x.shape
    co, cig, kh, kw = w.shape
    sh, sw = stride
    dh, dw = dilation
    pt, pl, pb, pr = pads
    xp = np.pad(x, ((0, 0), (0, 0), (pt, pb), (pl, pr)), mode="constant", constant_values=pad_value)
    ho = (xp.shape[2] - dh * (kh - 1) - 1) // sh + 1
    wo = (xp.shape[3] - dw * (kw - 1) - 1) // sw + 1
    y = np.zeros((n, groups, co // groups, ho, wo))
    wg = w.reshape(groups, co // groups, cig, kh, kw)
    for r in range(kh):
        for s in range(kw):
            view = xp[:, :, r * dh: r * dh + (ho - 1) * sh + 1: sh, s * dw: s * dw + (wo - 1) * sw + 1: sw]
            view = view.reshape(n, groups, cig, ho, wo)
            y += np.einsum("gok,ngkhw->ngohw", wg[:, :, :, r, s], view)
    y = y.reshape(n, co, ho, wo)
    if b is not None:
        y = y + b.reshape(1, -1, 1, 1)
    return y


def _random_case(rng):
    groups = int(rng.choice([1, 1, 2, 3]))
    cig = int(rng.integers(1, 4))
    cog = int(rng.integers(1, 4))
    c_in, c_out = cig * groups, cog * groups
    kh, kw = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    sh, sw = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    dh, dw = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    pads = tuple(int(v) for v in rng.integers(0, 3, size=4))
    h = int(rng.integers(max(1, dh * (kh - 1) + 1 - pads[0] - pads[2]), 10))
    wd = int(rng.integers(max(1, dw * (kw - 1) + 1 - pads[1] - pads[3]), 10))
    n = int(rng.integers(1, 3))
    x = rng.standard_normal((n, c_in, h, wd))
    w = rng.standard_normal((c_out, cig, kh, kw))
    b = rng.standard_normal(c_out) if rng.random() < 0.5 else None
    pad_value = float(rng.choice([0.0, 0.0, -1.5, 2.25]))
    return x, w, b, (sh, sw), pads, (dh, dw), groups, pad_value


def test_brute_force_tiny_shapes_vs_shift_and_add():
    rng = np.random.default_rng(2024)
    for _ in range(400):
        x, w, b, stride, pads, dil, groups, pv = _random_case(rng)
        ref = _shift_and_add(x, w, b, stride, pads, dil, groups, pv)
        y = oracle.conv2d(x, w, b, stride=stride, pads=pads, dilation=dil, groups=groups, pad_value=pv)
        assert y.shape == ref.shape
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_matches_torch_conv2d_float64():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    rng = np.random.default_rng(99)
    for _ in range(100):
        x, w, b, stride, pads, dil, groups, pv = _random_case(rng)
        pt, pl, pb, pr = pads
        xt = F.pad(torch.from_numpy(x), (pl, pr, pt, pb), value=pv)
        ref = F.conv2d(xt, torch.from_numpy(w), None if b is None else torch.from_numpy(b),
                       stride=stride, dilation=dil, groups=groups).numpy()
        y = oracle.conv2d(x, w, b, stride=stride, pads=pads, dilation=dil, groups=groups, pad_value=pv)
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_pointwise_equals_matmul():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 7, 5, 6))
    w = rng.standard_normal((4, 7, 1, 1))
    b = rng.standard_normal(4)
    y = oracle.conv2d(x, w, b)
    ref = np.matmul(w.reshape(4, 7), x.reshape(2, 7, 30)).reshape(2, 4, 5, 6) + b.reshape(1, 4, 1, 1)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_depthwise_equals_per_channel_correlate2d():
    from scipy.signal import correlate2d
    rng = np.random.default_rng(4)
    c = 5
    x = rng.standard_normal((2, c, 7, 9))
    w = rng.standard_normal((c, 1, 3, 3))
    y = oracle.conv2d(x, w, pads=(1, 1, 1, 1), groups=c)
    for n in range(2):
        for ch in range(c):
            ref = correlate2d(np.pad(x[n, ch], 1), w[ch, 0], mode="valid")
            np.testing.assert_allclose(y[n, ch], ref, rtol=1e-13, atol=1e-13)


def test_grouped_equals_independent_convs():
    rng = np.random.default_rng(5)
    g, cig, cog = 3, 2, 4
    x = rng.standard_normal((2, g * cig, 6, 6))
    w = rng.standard_normal((g * cog, cig, 3, 3))
    y = oracle.conv2d(x, w, pads=(1, 0, 2, 1), groups=g, stride=(2, 1))
    for k in range(g):
        part = oracle.conv2d(x[:, k * cig:(k + 1) * cig], w[k * cog:(k + 1) * cog],
                             pads=(1, 0, 2, 1), stride=(2, 1))
        np.testing.assert_array_equal(y[:, k * cog:(k + 1) * cog], part)


def test_identity_and_corner_delta():
    rng = np.random.default_rng(6)
    c = 3
    x = rng.standard_normal((1, c, 5, 4))
    w = np.zeros((c, c, 3, 3))
    for i in range(c):
        w[i, i, 1, 1] = 1.0
    y = oracle.conv2d(x, w, pads=(1, 1, 1, 1), pad_value=7.0)
    np.testing.assert_array_equal(y, x)
    # A delta at kernel tap (0, 0) with pad 1 shifts the image down-right by
    # one and brings pad_value in at the top row and left column.
    w = np.zeros((c, c, 3, 3))
    for i in range(c):
        w[i, i, 0, 0] = 1.0
    y = oracle.conv2d(x, w, pads=(1, 1, 1, 1), pad_value=-3.0)
    np.testing.assert_array_equal(y[:, :, 1:, 1:], x[:, :, :-1, :-1])
    assert np.all(y[:, :, 0, :] == -3.0) and np.all(y[:, :, :, 0] == -3.0)


def test_linearity():
    rng = np.random.default_rng(8)
    x1 = rng.standard_normal((2, 4, 6, 7))
    x2 = rng.standard_normal((2, 4, 6, 7))
    w = rng.standard_normal((6, 2, 3, 2))
    kw = dict(stride=(1, 2), pads=(1, 2, 0, 1), dilation=(2, 1), groups=2)
    lhs = oracle.conv2d(1.5 * x1 - 0.75 * x2, w, **kw)
    rhs = 1.5 * oracle.conv2d(x1, w, **kw) - 0.75 * oracle.conv2d(x2, w, **kw)
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-12)


def test_stride_is_subsampling():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((1, 3, 11, 10))
    w = rng.standard_normal((2, 3, 3, 3))
    base = oracle.conv2d(x, w, pads=(1, 1, 2, 0), pad_value=0.5)
    for s in (2, 3):
        ys = oracle.conv2d(x, w, pads=(1, 1, 2, 0), stride=s, pad_value=0.5)
        np.testing.assert_array_equal(ys, base[:, :, ::s, ::s])


def test_dilation_is_zero_stuffed_kernel():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((1, 2, 12, 11))
    w = rng.standard_normal((3, 2, 3, 2))
    for d in (2, 3):
        big = np.zeros((3, 2, (3 - 1) * d + 1, (2 - 1) * d + 1))
        big[:, :, ::d, ::d] = w
        yd = oracle.conv2d(x, w, dilation=d, pads=(2, 1, 2, 1), pad_value=0.0)
        yb = oracle.conv2d(x, big, pads=(2, 1, 2, 1), pad_value=0.0)
        np.testing.assert_allclose(yd, yb, rtol=0, atol=1e-13)


def test_pad_value_equals_explicit_padding():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2, 2, 5, 6))
    w = rng.standard_normal((3, 2, 3, 3))
    pads = (2, 1, 0, 3)
    y = oracle.conv2d(x, w, pads=pads, pad_value=-0.625)
    xp = np.pad(x, ((0, 0), (0, 0), (2, 0), (1, 3)), constant_values=-0.625)
    np.testing.assert_allclose(y, oracle.conv2d(xp, w), rtol=0, atol=1e-13)


def test_output_size_floor():
    # (H + pt + pb - d*(k-1) - 1) / s, rounded down, plus one.
    assert oracle.output_shape((1, 1, 7, 8), (1, 1, 3, 3), stride=2, pads=(1, 1, 1, 1)) == (1, 1, 4, 4)
    assert oracle.output_shape((1, 1, 64, 64), (1, 1, 3, 3), stride=2, pads=(1, 1, 1, 1)) == (1, 1, 32, 32)
    assert oracle.output_shape((1, 1, 64, 64), (1, 1, 3, 3), dilation=2, pads=(2, 2, 2, 2)) == (1, 1, 64, 64)
    assert oracle.output_shape((1, 1, 80, 80), (1, 1, 3, 3), stride=2, pads=(1, 1, 1, 1)) == (1, 1, 40, 40)


def test_points_agree_with_full():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((2, 4, 9, 8))
    w = rng.standard_normal((6, 2, 3, 3))
    b = rng.standard_normal(6)
    sl = rng.random(6)
    kw = dict(stride=(2, 1), pads=(1, 1, 1, 1), groups=2, pad_value=0.25, act=oracle.ACT_PRELU, slope=sl)
    full = oracle.conv2d(x, w, b, **kw)
    idx = rng.choice(full.size, size=100, replace=False)
    np.testing.assert_array_equal(oracle.conv2d_points(x, w, b, idx, **kw), full.reshape(-1)[idx])


def test_invalid_arguments_rejected():
    with pytest.raises(ValueError):
        oracle.conv2d(np.zeros((1, 3, 4, 4)), np.zeros((2, 1, 3, 3)), groups=2)
    with pytest.raises(ValueError):
        oracle.conv2d(np.zeros((1, 2, 4, 4)), np.zeros((2, 2, 3, 3)), act=oracle.ACT_PRELU,
                      slope=np.zeros(3))


# --------------------------------------------------------------- int8 -----

def test_composite_bits_for_symmetric_scales():
    comp = oracle.composite_scale(0.02, 0.01, 0.05)
    assert comp.view(np.uint32) == 0x3B83126E


def test_requant_matches_numpy_rint_and_saturates():
    rng = np.random.default_rng(13)
    v = rng.integers(-3_000_000, 3_000_000, size=20000)
    comp = oracle.composite_scale(0.02, 0.01, 0.05)
    ref = np.clip(np.rint(v.astype(np.float32) * comp), -128, 127).astype(np.int8)
    np.testing.assert_array_equal(oracle.requant(v, comp), ref)
    relu = oracle.requant(v, comp, relu=True)
    np.testing.assert_array_equal(relu, np.maximum(ref, 0))
    shifted = oracle.requant(v, comp, y_zp=5)
    np.testing.assert_array_equal(shifted, np.clip(np.rint(v.astype(np.float32) * comp) + 5, -128, 127))


@pytest.mark.parametrize("y_zp", [-100, 0, 100])
@pytest.mark.parametrize("relu", [False, True])
def test_requant_saturates_at_extreme_composites(y_zp, relu):
    """A composite of 1e30 sends every nonzero sum past the int8 range (the
    largest ones to an infinite f32 product): the result is 127 above zero,
    -128 below it and the zero point at zero, raised to the zero point under
    ReLU, whatever y_zp is."""
    comp = np.float32(1e30)
    v = np.array([-2**31, -10**9, -5, -1, 0, 1, 7, 10**9, 2**31 - 1], dtype=np.int64)
    expect = np.where(v > 0, 127, np.where(v < 0, -128, y_zp))
    if relu:
        expect = np.maximum(expect, y_zp)
    for rounding in (oracle.ROUND_HALF_EVEN, oracle.ROUND_HALF_AWAY):
        got = oracle.requant(v, comp, rounding=rounding, y_zp=y_zp, relu=relu)
        np.testing.assert_array_equal(got.astype(np.int64), expect)


def test_requant_equals_exact_rational_rounding_on_unsaturated_range():
    """Over |acc| <= 32000 the f32 formula with composite 0x3B83126E gives the
    exactly rounded (ties to even) value of acc*sx*sw/sy, sx,sw,sy taken as the
    float32 scales."""
    comp = oracle.composite_scale(0.02, 0.01, 0.05)
    v = np.arange(-32000, 32001, dtype=np.int64)
    got = oracle.requant(v, comp).astype(np.int64)
    k = Fraction(float(np.float32(0.02))) * Fraction(float(np.float32(0.01))) / Fraction(float(np.float32(0.05)))
    exact = np.array([round(int(a) * k) for a in v], dtype=np.int64)   # Python round: ties to even
    np.testing.assert_array_equal(got, np.clip(exact, -128, 127))


def _int_shift_and_add(x, w, stride, pads, groups):
    return _shift_and_add(x.astype(np.int64), w.astype(np.int64), None, stride, pads, (1, 1), groups, 0)


def test_int8_accumulators_exact():
    rng = np.random.default_rng(14)
    x = rng.integers(-128, 128, size=(2, 6, 9, 10), dtype=np.int8)
    w = rng.integers(-127, 128, size=(6, 1, 3, 3), dtype=np.int8)
    for s in (1, 2):
        acc = oracle.qconv2d_acc(x, w, stride=s, pads=(1, 1, 1, 1), groups=6)
        ref = _int_shift_and_add(x.astype(np.float64), w.astype(np.float64), (s, s), (1, 1, 1, 1), 6)
        np.testing.assert_array_equal(acc, ref.astype(np.int64))


def test_int8_pointwise_is_integer_matmul_then_requant():
    rng = np.random.default_rng(15)
    x = rng.integers(-128, 128, size=(2, 16, 5, 4), dtype=np.int8)
    w = rng.integers(-127, 128, size=(8, 16, 1, 1), dtype=np.int8)
    b = rng.integers(-500, 501, size=8).astype(np.int32)
    y = oracle.qconv2d(x, w, b, 0.02, 0.01, 0.05)
    acc = np.matmul(w.reshape(8, 16).astype(np.int64), x.reshape(2, 16, 20).astype(np.int64))
    acc = acc + b.astype(np.int64).reshape(1, 8, 1)
    comp = oracle.composite_scale(0.02, 0.01, 0.05)
    ref = np.clip(np.rint(acc.astype(np.float32) * comp), -128, 127).astype(np.int8)
    np.testing.assert_array_equal(y, ref.reshape(2, 8, 5, 4))


def test_int8_saturation_and_identity():
    x = np.full((1, 2, 4, 4), 127, dtype=np.int8)
    w = np.full((2, 1, 3, 3), 127, dtype=np.int8)
    y = oracle.qconv2d(x, w, None, 0.02, 0.01, 0.05, pads=(1, 1, 1, 1), groups=2)
    assert np.all(y == 127)
    y = oracle.qconv2d(x, -w, None, 0.02, 0.01, 0.05, pads=(1, 1, 1, 1), groups=2)
    assert np.all(y == -128)
    # composite 1 and a centre delta: q = clamp(x + bias).
    rng = np.random.default_rng(16)
    x = rng.integers(-128, 128, size=(1, 3, 5, 5), dtype=np.int8)
    w = np.zeros((3, 1, 3, 3), dtype=np.int8)
    w[:, 0, 1, 1] = 1
    b = np.array([0, 100, -100], dtype=np.int32)
    y = oracle.qconv2d(x, w, b, 1.0, 1.0, 1.0, pads=(1, 1, 1, 1), groups=3)
    ref = np.clip(x.astype(np.int64) + b.reshape(1, 3, 1, 1), -128, 127)
    np.testing.assert_array_equal(y, ref)


def test_int8_points_agree_with_full():
    rng = np.random.default_rng(17)
    x = rng.integers(-128, 128, size=(2, 4, 9, 9), dtype=np.int8)
    w = rng.integers(-127, 128, size=(4, 1, 3, 3), dtype=np.int8)
    b = rng.integers(-500, 501, size=4).astype(np.int32)
    full = oracle.qconv2d(x, w, b, 0.02, 0.01, 0.05, stride=2, pads=(1, 1, 1, 1), groups=4)
    idx = rng.choice(full.size, 50, replace=False)
    pts = oracle.qconv2d_points(x, w, b, 0.02, 0.01, 0.05, idx, stride=2, pads=(1, 1, 1, 1), groups=4)
    np.testing.assert_array_equal(pts, full.reshape(-1)[idx])
