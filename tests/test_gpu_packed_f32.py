"""GPU: the fp32 implicit GEMM with bound weights, which reads them in
fragment order (packed once by conv2d_desc_bind_weights) straight into
registers instead of staging OIHW weights through LDS.

For tiles of up to 32 output channels the packed kernel feeds the matrix
cores the same operands in the same order and sums the K slices the same way
as the kernel given OIHW weights, so the bound output must equal the
explicit-weight output bit for bit.  For 64-channel tiles the packed kernel
lets each wave own all 64 channels and splits K eight ways instead of four (a
different summation order), so there the two agree to the fp32 tolerance.
Every output must match the oracle at the fp32 tolerance.  Cases reach the three tile
configurations (<= 16, <= 32, <= 64 output channels per tile), partial
input-channel chunks and output-channel tiles, padding with a pad value,
dilation, groups, batch > 1, concat slices on both sides, the layouts that
fall back to the OIHW kernel (width not a multiple of 4, input not 16-byte
aligned), rebinding, and the dense-block chain at full size.  Descriptors
ask for the tiled classes (algo "direct"): under AUTO the small 3x3 layers
here would run the small-layer kernel and bound dense-block layers Winograd."""
import numpy as np
import pytest

import workloads
from helpers import FP32_TOL, Guarded, assert_bitexact, assert_close, layer_params, oracle_layer, to_dev, torch

pytestmark = pytest.mark.gpu

A = workloads


def cc():
    import convolution_conv2d_forward_amd as m
    return m


CASES = [
    # n, c_in, h, w, c_out, pads (t, l, b, r), dilation, groups, act, bias, pad_value
    (1, 32, 12, 16, 8, (1, 1, 1, 1), 1, 1, A.ACT_RELU, True, 0.0),           # <= 16 outputs, one chunk per wave
    (1, 37, 13, 20, 32, (1, 1, 1, 1), 1, 1, A.ACT_LEAKY_RELU, True, -0.5),   # partial last chunk
    (2, 64, 9, 24, 48, (0, 2, 1, 1), 1, 1, A.ACT_PRELU, True, 0.25),         # partial 64-channel tile, batch 2
    (1, 96, 16, 32, 64, (1, 1, 1, 1), 1, 1, A.ACT_NONE, True, 0.0),          # 64 outputs, two row halves
    (1, 40, 11, 28, 20, (2, 2, 2, 2), 2, 1, A.ACT_CLIP, False, 1.0),         # dilation 2
    (1, 64, 10, 16, 64, (1, 1, 1, 1), 1, 2, A.ACT_RELU, True, 0.0),          # two groups
    (1, 33, 14, 40, 40, (0, 0, 0, 0), 1, 1, A.ACT_NONE, True, 0.0),          # no padding, ragged rows
    (1, 32, 10, 18, 32, (1, 1, 1, 1), 1, 1, A.ACT_RELU, True, 0.0),          # width 18: OIHW kernel
]


def _layer(i):
    n, ci, h, w, co, pads, dil, g, act, bias, pv = CASES[i]
    return A.Layer("packed", n, ci, h, w, co, (3, 3), pads=pads, dilation=(dil, dil), groups=g, has_bias=bias,
                   act=act, alpha=0.2, clip=(-0.3, 0.4), pad_value=pv)


def _same_split(L):
    """Bound and explicit weights take the same K split: tiles of <= 32
    output channels, or the OIHW kernel on both sides (width not a multiple
    of 4)."""
    return L.c_out // L.groups <= 32 or L.w % 4 != 0


def _agree(bound, explicit, L, what):
    if _same_split(L):
        assert_bitexact(bound, explicit, what)
    else:
        assert_close(bound, explicit, FP32_TOL, what)


def _run(d, xd, wd, bd, sd):
    t = torch()
    n, ot, ho, wo = cc().conv2d_desc_get_output_shape(d)
    y = Guarded(n * ot * ho * wo, t.float32, float("nan"))
    cc().conv2d_forward(d, xd, wd, bd, sd, y.view)
    t.cuda.synchronize()
    y.check_guards()
    return y.host().numpy().astype(np.float64).reshape(n, ot, ho, wo)


@pytest.mark.parametrize("i", range(len(CASES)))
def test_packed_equals_explicit(i):
    L = _layer(i)
    rng = np.random.default_rng(3100 + i)
    x, w, b, s = A.layer_arrays(rng, L)
    _, w2, _, _ = A.layer_arrays(rng, L)
    d = cc().conv2d_desc_create(layer_params(L, prelu_slope_count=s.size, algo="direct"))
    kname = cc().conv2d_desc_kernel_name(d)
    print(f"case {i}: {L} ({kname})", flush=True)
    xd, wd, w2d = to_dev(x), to_dev(w), to_dev(w2)
    bd = to_dev(b) if L.has_bias else None
    sd = to_dev(s) if L.act == A.ACT_PRELU else None
    explicit = _run(d, xd, wd, bd, sd)
    assert_close(explicit, oracle_layer(L, x, w, b, s), FP32_TOL, f"case {i} explicit")
    cc().conv2d_desc_bind_weights(d, wd)
    wd.fill_(float("nan"))
    bound = _run(d, xd, None, bd, sd)
    _agree(bound, explicit, L, f"case {i} ({kname}): bound vs explicit")
    assert_close(bound, oracle_layer(L, x, w, b, s), FP32_TOL, f"case {i} bound")
    cc().conv2d_desc_bind_weights(d, w2d)
    rebound = _run(d, xd, None, bd, sd)
    assert_close(rebound, oracle_layer(L, x, w2, b, s), FP32_TOL, f"case {i}: rebound")
    _agree(rebound, _run(d, xd, w2d, bd, sd), L, f"case {i}: rebound vs explicit")


def test_packed_concat_slices_and_unaligned_input():
    """Input channels [5, 5 + c_in) of a wider buffer, output into channels
    [3, 3 + c_out) of another (the channels around stay NaN); then the same
    input one float off 16-byte alignment, which runs the OIHW kernel on the
    bound copy."""
    t = torch()
    L = A.Layer("packed", 2, 36, 10, 24, 32, (3, 3), pads=(1, 1, 1, 1), has_bias=True, act=A.ACT_RELU)
    rng = np.random.default_rng(3150)
    x, w, b, s = A.layer_arrays(rng, L)
    ref = oracle_layer(L, x, w, b, s)
    big = rng.standard_normal((L.n, L.c_in + 9, L.h, L.w)).astype(np.float32)
    big[:, 5:5 + L.c_in] = x
    d = cc().conv2d_desc_create(layer_params(L, algo="direct", in_total_channels=L.c_in + 9, in_channel_offset=5,
                                             out_total_channels=L.c_out + 6, out_channel_offset=3))
    assert cc().conv2d_desc_kernel_name(d) == "igemm_f32"
    cc().conv2d_desc_bind_weights(d, to_dev(w))
    bd = to_dev(b)
    y = _run(d, to_dev(big), None, bd, None)
    assert np.isnan(y[:, :3]).all() and np.isnan(y[:, 3 + L.c_out:]).all()
    assert_close(y[:, 3:3 + L.c_out], ref, FP32_TOL, "packed, concat slices")
    flat = to_dev(np.concatenate([np.zeros(1, np.float32), big.reshape(-1)]))
    xu = flat[1:]
    assert xu.data_ptr() % 16 != 0
    yu = _run(d, xu, None, bd, None)
    assert_close(yu[:, 3:3 + L.c_out], ref, FP32_TOL, "bound weights, unaligned input")


def test_packed_dense_block_full_size():
    """The dense-block chain (1 x 64 x 128 x 128 input in a 256-channel concat
    buffer, five 3x3 layers appending 32, 32, 32, 32 and 64 channels) with
    every layer's weights bound, run in place like the benchmark; each
    layer's output against the oracle fed with the oracle's own previous
    outputs, and against the same chain with explicit weights (bit for bit
    for the 32-channel layers)."""
    t = torch()
    wl = A.dense_block()
    a = wl.arrays
    total = A.DENSE_TOTAL_CHANNELS
    descs = []
    for k, L in enumerate(wl.layers):
        # algo "direct": AUTO would run these bound layers on Winograd
        d = cc().conv2d_desc_create(layer_params(L, in_total_channels=total, out_total_channels=total,
                                                 out_channel_offset=L.c_in, algo="direct"))
        descs.append(d)
    outs = {}
    for bound in (False, True):
        buf = torch().full((1, total, 128, 128), float("nan"), dtype=t.float32, device="cuda")
        buf[:, :64] = to_dev(a["x"])
        for k, (L, d) in enumerate(zip(wl.layers, descs)):
            wd = to_dev(a[f"w{k}"])
            if bound:
                cc().conv2d_desc_bind_weights(d, wd)
                wd = None
            cc().conv2d_forward(d, buf, wd, None, None, buf)
        t.cuda.synchronize()
        outs[bound] = buf.cpu().numpy().astype(np.float64)
    cur = a["x"]
    for k, L in enumerate(wl.layers):
        sl = slice(L.c_in, L.c_in + L.c_out)
        _agree(outs[True][:, sl], outs[False][:, sl], L, f"dense block layer {k}: bound vs explicit")
        ref = oracle_layer(L, cur, a[f"w{k}"], None, None)
        assert_close(outs[True][:, L.c_in:L.c_in + L.c_out], ref, FP32_TOL, f"dense block layer {k}")
        cur = np.concatenate([cur, ref.astype(np.float32)], axis=1)
