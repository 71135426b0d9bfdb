"""GPU: int8 dense and grouped convolution on the i8 matrix cores (igemm_i8),
bit-exact against the oracle's int64 QLinearConv.

Cases reach every path of the kernel: one and several 64-channel chunks with
partial ones, 3x3 chunks held in registers (one and two fragments per wave,
1, 2 and 4 sixteen-channel groups per item list), output-channel tiles of 64 (windows up to 9 taps) and 32
(larger windows), one and two output-row fragments per wave, stride,
dilation, asymmetric pads, non-square windows, grouped convolutions with 4,
8, 16 and 72 channels per group and a channel multiplier, rows that are not
whole 4-byte words, channel counts that are not multiples of 4 (byte weight
loads), an input that is not 4-byte aligned, channel slices in and out, bound
weights, and both rounding modes with zero points and ReLU."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import Guarded, assert_bitexact, layer_params, to_dev, torch

pytestmark = pytest.mark.gpu


def cc():
    import convolution_conv2d_forward_amd as m
    return m


SYM = (0.02, 0.01, 0.05)
CASES = [
    # n, c_in, h, w, c_out, k, stride, pads, dilation, groups
    (2, 16, 9, 11, 24, 3, 1, 1, 1, 1),           # odd width: byte rows
    (1, 64, 16, 32, 64, 3, 1, 1, 1, 1),          # one full chunk, one channel tile
    (2, 72, 12, 20, 100, 3, 1, 1, 1, 1),         # partial second chunk, two channel tiles, ragged
    (1, 130, 8, 16, 16, 3, 1, 1, 1, 1),          # three chunks, cin_g % 4 = 2 (byte weights)
    (2, 32, 17, 33, 48, 3, 2, (0, 1, 2, 1), 1, 1),   # stride 2, asymmetric pads
    (1, 24, 20, 24, 40, 3, 1, 2, 2, 1),          # dilation 2
    (1, 20, 11, 13, 36, 5, 1, 2, 1, 1),          # 5x5: 32-channel tiles
    (1, 8, 12, 16, 12, 7, 1, 3, 1, 1),           # 7x7: one fragment per wave, large LDS
    (2, 12, 10, 14, 20, (1, 3), 1, (0, 1, 0, 1), 1, 1),  # 1x3
    (1, 12, 9, 16, 20, (3, 1), (2, 1), (1, 0, 1, 0), 1, 1),  # 3x1, stride (2, 1)
    (2, 16, 8, 12, 16, 1, 2, 0, 1, 1),           # 1x1 stride 2 (not the pointwise kernel)
    (1, 16, 9, 9, 16, 2, 1, 0, 1, 1),            # 2x2, even window
    (2, 32, 10, 12, 32, 3, 1, 1, 1, 8),          # grouped, 4 channels per group
    (1, 64, 12, 16, 64, 3, 2, 1, 1, 8),          # grouped, 8 per group, stride 2
    (2, 64, 9, 20, 32, 3, 1, 1, 1, 4),           # grouped, 16 in / 8 out per group
    (1, 144, 8, 8, 144, 3, 1, 1, 1, 2),          # grouped, 72 per group (two chunks per group)
    (1, 6, 9, 11, 12, 3, 1, 1, 1, 6),            # channel multiplier 2 (groups == c_in < c_out)
    (3, 5, 6, 7, 9, 3, 1, 1, 1, 1),              # tiny, odd everything
    # 3x3 over word-aligned rows and filters: the chunk held in registers
    (1, 128, 20, 40, 64, 3, 2, 1, 1, 1),         # stride 2, two chunks, one fragment per wave (patch > 2048 units)
    (2, 8, 16, 24, 16, 3, 1, 1, 1, 1),           # 8 channels: four taps per K step, 16 output channels
    (1, 48, 9, 16, 24, 3, 1, 1, 1, 1),           # 12 of 16 channel quads, 32-channel tile
    (1, 36, 8, 12, 20, 3, 1, 1, 1, 2),           # 18 per group: two 16-channel groups per item list
    (2, 200, 6, 8, 70, 3, 1, (1, 0, 2, 1), 1, 1),  # four chunks (the last 8 channels), ragged channel tile
]


def _layer(case):
    n, ci, h, w, co, k, s, p, d, g = case
    k2 = k if isinstance(k, tuple) else (k, k)
    s2 = s if isinstance(s, tuple) else (s, s)
    p4 = p if isinstance(p, tuple) else (p,) * 4
    return workloads.Layer("q", n, ci, h, w, co, k2, stride=s2, pads=p4, dilation=(d, d), groups=g, has_bias=True)


def _arrays(rng, L):
    x = rng.integers(-128, 127, size=L.x_shape, endpoint=True).astype(np.int8)
    wt = rng.integers(-127, 127, size=L.w_shape, endpoint=True).astype(np.int8)
    b = rng.integers(-500, 500, size=L.c_out, endpoint=True).astype(np.int32)
    return x, wt, b


def _run(L, xd, wd, bd, scales, *, rounding=0, y_zp=0, relu=False, **kw):
    t = torch()
    p = layer_params(L, "i8", int8_rounding=rounding, **kw)
    if relu:
        p.act_type = 1
    d = cc().conv2d_desc_create(p)
    n, ot, ho, wo = cc().conv2d_desc_get_output_shape(d)
    y = Guarded(n * ot * ho * wo, t.int8, 0x5A)
    cc().qconv2d_forward(d, xd, scales[0], 0, wd, scales[1], 0, bd, scales[2], y_zp, y.view)
    t.cuda.synchronize()
    y.check_guards()
    return y.host().numpy().reshape(n, ot, ho, wo), d


@pytest.mark.parametrize("i", range(len(CASES)))
@pytest.mark.parametrize("mode", ["rne", "away_relu_zp"])
def test_igemm_i8_cases(i, mode):
    L = _layer(CASES[i])
    rng = np.random.default_rng(2100 + i)
    x, wt, b = _arrays(rng, L)
    # small-range scales make most sums land inside the int8 range
    scales = SYM if mode == "rne" else (0.01, 0.01, 0.02 * (L.c_in // L.groups) * L.k[0] * L.k[1])
    rounding, y_zp, relu = (0, 0, False) if mode == "rne" else (1, -3, True)
    ref = oracle.qconv2d(x, wt, b, *scales, stride=L.stride, pads=L.pads, dilation=L.dilation, groups=L.groups,
                         y_zp=y_zp, rounding=rounding, relu=relu)
    print(f"case {i} {mode}: {L}; saturated {np.mean((ref == 127) | (ref == -128)):.3f}", flush=True)
    got, d = _run(L, to_dev(x), to_dev(wt), to_dev(b), scales, rounding=rounding, y_zp=y_zp, relu=relu)
    assert cc().conv2d_desc_kernel_name(d) == "igemm_i8"
    assert_bitexact(got, ref, f"igemm_i8 case {i} {mode}")


def test_igemm_i8_unaligned_input_slices_and_bound_weights():
    """Input channels [3, 3 + c_in) of a buffer that starts one byte past a
    word boundary, output into channels [2, 2 + c_out) of a wider buffer;
    then the same layer with its weights bound to the descriptor."""
    t = torch()
    L = _layer((2, 20, 10, 16, 28, 3, 1, 1, 1, 1))
    rng = np.random.default_rng(2199)
    x, wt, b = _arrays(rng, L)
    ref = oracle.qconv2d(x, wt, b, *SYM, stride=L.stride, pads=L.pads, groups=L.groups)
    big = rng.integers(-128, 127, size=(L.n, L.c_in + 5, L.h, L.w), endpoint=True).astype(np.int8)
    big[:, 3:3 + L.c_in] = x
    raw = t.zeros(big.size + 1, dtype=t.int8, device="cuda")
    xv = raw[1:1 + big.size]
    xv.copy_(t.from_numpy(big.reshape(-1)).cuda())
    got, d = _run(L, xv, to_dev(wt), to_dev(b), SYM, in_total_channels=L.c_in + 5, in_channel_offset=3,
                  out_total_channels=L.c_out + 6, out_channel_offset=2)
    assert (got[:, :2] == 0x5A).all() and (got[:, 2 + L.c_out:] == 0x5A).all()
    assert_bitexact(got[:, 2:2 + L.c_out], ref, "unaligned input, slices")
    cc().conv2d_desc_bind_weights(d, to_dev(wt))
    n, ot, ho, wo = cc().conv2d_desc_get_output_shape(d)
    y = Guarded(n * ot * ho * wo, t.int8, 0x5A)
    cc().qconv2d_forward(d, xv, SYM[0], 0, None, SYM[1], 0, to_dev(b), SYM[2], 0, y.view)
    t.cuda.synchronize()
    y.check_guards()
    assert_bitexact(y.host().numpy().reshape(n, ot, ho, wo), got, "bound weights")


@pytest.mark.parametrize("bound", [False, True])
@pytest.mark.parametrize("name", ["s2", "d2", "g32"])
def test_igemm_i8_mixed_sweep_shapes(name, bound):
    """The mixed sweep's strided, dilated and grouped 3x3 layers at full
    size (the bench's batch of 32), every output compared; with the weights
    passed per call and bound to the descriptor (as the bench times them)."""
    L0 = next(L for L in workloads.mixed_sweep_layers() if L.name == name)
    L = workloads.Layer(name, L0.n, L0.c_in, L0.h, L0.w, L0.c_out, L0.k, stride=L0.stride, pads=L0.pads,
                        dilation=L0.dilation, groups=L0.groups, has_bias=True)
    rng = np.random.default_rng(2197)
    x, wt, b = _arrays(rng, L)
    print(f"{name}: {L}", flush=True)
    ref = oracle.qconv2d(x, wt, b, *SYM, stride=L.stride, pads=L.pads, dilation=L.dilation, groups=L.groups)
    if not bound:
        got, d = _run(L, to_dev(x), to_dev(wt), to_dev(b), SYM)
    else:
        t = torch()
        d = cc().conv2d_desc_create(layer_params(L, "i8"))
        cc().conv2d_desc_bind_weights(d, to_dev(wt))
        n, ot, ho, wo = cc().conv2d_desc_get_output_shape(d)
        y = Guarded(n * ot * ho * wo, t.int8, 0x5A)
        cc().qconv2d_forward(d, to_dev(x), SYM[0], 0, None, SYM[1], 0, to_dev(b), SYM[2], 0, y.view)
        t.cuda.synchronize()
        y.check_guards()
        got = y.host().numpy().reshape(n, ot, ho, wo)
    assert cc().conv2d_desc_kernel_name(d) == "igemm_i8"
    assert_bitexact(got, ref, f"mixed sweep {name} ({'bound' if bound else 'per call'})")


def test_igemm_i8_dense_full_size():
    """A dense int8 3x3 layer at the int8 chain's scale (16 x 144 x 40 x 40
    -> 96), every output compared."""
    L = _layer((16, 144, 40, 40, 96, 3, 1, 1, 1, 1))
    rng = np.random.default_rng(2198)
    x, wt, b = _arrays(rng, L)
    ref = oracle.qconv2d(x, wt, b, *SYM, stride=L.stride, pads=L.pads, groups=L.groups)
    got, d = _run(L, to_dev(x), to_dev(wt), to_dev(b), SYM)
    assert cc().conv2d_desc_kernel_name(d) == "igemm_i8"
    assert_bitexact(got, ref, "dense int8 full size")
