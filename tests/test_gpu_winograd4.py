"""GPU parity of the Winograd F(4x4, 3x3) path (algo = WINOGRAD4, weights
bound to the descriptor) against the oracle's direct float64 convolution,
fp32 tolerance 1e-4 * (1 + |ref|).

F(4x4) reaches the convolution's result through larger transforms than
F(2x2) (6x6 input tiles, 36 channel sums per output tile), so its fp32
rounding is the larger one; the oracle stays the plain definition.  The
cases cover partial 4x4 output tiles and partial 8x32 workgroup tiles, every
pad layout with a nonzero pad_value, partial 16-channel chunks and 32-channel
tiles, each activation with bias, batch > 1, concat slices on both sides, the
entry point that allocates nothing, and the five dense-block layers at full
size."""
import numpy as np
import pytest

import workloads
from helpers import FP32_TOL, Guarded, assert_close, layer_params, oracle_layer, to_dev, torch

pytestmark = pytest.mark.gpu

A = workloads


def cc():
    import convolution_conv2d_forward_amd as m
    return m


CASES = [
    # n, c_in, h, w, c_out, pads (t, l, b, r), act, bias, pad_value
    (1, 16, 8, 32, 32, (1, 1, 1, 1), A.ACT_NONE, False, 0.0),          # one workgroup, exact tiles
    (1, 20, 13, 17, 24, (1, 1, 1, 1), A.ACT_RELU, True, 0.0),          # partial tiles, partial chunk
    (2, 35, 9, 30, 40, (0, 2, 1, 0), A.ACT_LEAKY_RELU, True, 0.5),     # asymmetric pads, pad_value, 2 channel tiles
    (1, 64, 24, 40, 33, (2, 2, 2, 2), A.ACT_PRELU, True, -1.0),        # pads of 2, PReLU per channel
    (3, 7, 5, 6, 5, (0, 0, 0, 0), A.ACT_CLIP, True, 0.0),              # no pads, tiny
    (1, 1, 3, 3, 1, (0, 0, 0, 0), A.ACT_NONE, False, 0.0),             # a single output
    (1, 48, 33, 65, 64, (1, 0, 0, 1), A.ACT_NONE, True, 0.25),         # several workgroups per row, ragged edges
    (2, 24, 128, 128, 64, (1, 1, 1, 1), A.ACT_RELU, True, 0.0),        # many workgroups, 64 output channels
    (1, 160, 40, 44, 32, (1, 1, 1, 1), A.ACT_LEAKY_RELU, False, 0.0),  # ten chunks
]


def _desc(L, s, **kw):
    d = cc().conv2d_desc_create(layer_params(L, prelu_slope_count=s.size, algo="winograd4", **kw))
    assert cc().conv2d_desc_kernel_name(d) == "winograd4_f32"
    return d


def _run(L, x, w, b, s, *, in_total=0, in_off=0, out_total=0, out_off=0, noalloc=False):
    t = torch()
    d = _desc(L, s, in_total_channels=in_total, in_channel_offset=in_off, out_total_channels=out_total,
              out_channel_offset=out_off)
    n, ot, ho, wo = cc().conv2d_desc_get_output_shape(d)
    y = Guarded(n * ot * ho * wo, t.float32, float("nan"))
    cc().conv2d_desc_bind_weights(d, to_dev(w))
    fwd = cc().conv2d_forward_noalloc if noalloc else cc().conv2d_forward
    fwd(d, to_dev(x), None, to_dev(b) if L.has_bias else None, to_dev(s) if L.act == A.ACT_PRELU else None, y.view)
    t.cuda.synchronize()
    y.check_guards()
    return y.host().numpy().reshape(n, ot, ho, wo)


def _layer(i):
    n, ci, h, w, co, pads, act, bias, pv = CASES[i]
    return A.Layer("wino4", n, ci, h, w, co, (3, 3), pads=pads, has_bias=bias, act=act, alpha=0.2,
                   clip=(-0.3, 0.4), pad_value=pv)


@pytest.mark.parametrize("i", range(len(CASES)))
def test_winograd4_cases(i):
    L = _layer(i)
    rng = np.random.default_rng(900 + i)
    x, wt, b, s = A.layer_arrays(rng, L)
    print(f"case {i}: {L}", flush=True)
    ref = oracle_layer(L, x, wt, b, s)
    got = _run(L, x, wt, b, s)
    err = np.max(np.abs(got - ref) / (1 + np.abs(ref))) if ref.size else 0.0
    print(f"case {i}: max |y - ref| / (1 + |ref|) = {err:.3g}", flush=True)
    assert_close(got, ref, FP32_TOL, f"winograd4 case {i}")


def test_winograd4_concat_slices():
    """Input channels [5, 5 + c_in) of a wider buffer, output into channels
    [3, 3 + c_out) of another; the channels around the slice stay NaN."""
    L = A.Layer("wino4", 2, 24, 10, 18, 20, (3, 3), pads=(1, 1, 1, 1), has_bias=True, act=A.ACT_RELU)
    rng = np.random.default_rng(980)
    x, wt, b, s = A.layer_arrays(rng, L)
    big = rng.standard_normal((L.n, L.c_in + 9, L.h, L.w)).astype(np.float32)
    big[:, 5:5 + L.c_in] = x
    y = _run(L, big, wt, b, s, in_total=L.c_in + 9, in_off=5, out_total=L.c_out + 6, out_off=3)
    assert np.isnan(y[:, :3]).all() and np.isnan(y[:, 3 + L.c_out:]).all()
    assert_close(y[:, 3:3 + L.c_out], oracle_layer(L, x, wt, b, s), FP32_TOL, "winograd4 slices")


def test_winograd4_noalloc_matches_forward():
    """conv2d_forward_noalloc runs the same kernel on the bound image: bitwise
    the output of conv2d_forward."""
    L = _layer(2)
    rng = np.random.default_rng(990)
    x, wt, b, s = A.layer_arrays(rng, L)
    assert np.array_equal(_run(L, x, wt, b, s, noalloc=True), _run(L, x, wt, b, s))


def test_winograd4_needs_bound_weights():
    """A call that passes OIHW weights is refused (the filter transform exists
    only as the image packed at bind); the output buffer is left untouched."""
    t = torch()
    L = _layer(1)
    rng = np.random.default_rng(995)
    x, wt, b, s = A.layer_arrays(rng, L)
    d = _desc(L, s)
    n, ot, ho, wo = cc().conv2d_desc_get_output_shape(d)
    y = Guarded(n * ot * ho * wo, t.float32, float("nan"))
    with pytest.raises(cc().ConvError) as e:
        cc().conv2d_forward(d, to_dev(x), to_dev(wt), to_dev(b), None, y.view)
    assert e.value.status == cc().CONV_ERR_UNSUPPORTED
    t.cuda.synchronize()
    y.check_guards()
    assert np.isnan(y.host().numpy()).all()


def test_winograd4_dense_block_full_size():
    """The dense-block chain's five layers (1 x Cin x 128 x 128, Cin = 64 + 32k),
    each fed with the oracle's own previous outputs, at full size."""
    wl = A.dense_block()
    a = wl.arrays
    cur = a["x"]
    for k, L in enumerate(wl.layers):
        w = a[f"w{k}"]
        ref = oracle_layer(L, cur, w, None, None)
        b0, s0 = np.zeros(L.c_out, np.float32), np.zeros(1, np.float32)
        got = _run(L, cur, w, b0, s0)
        print(f"layer {k}: max |y - ref| / (1 + |ref|) = {np.max(np.abs(got - ref) / (1 + np.abs(ref))):.3g}",
              flush=True)
        assert_close(got, ref, FP32_TOL, f"dense block layer {k}")
        cur = np.concatenate([cur, ref.astype(np.float32)], axis=1)


def test_auto_bound_weights_pick_winograd4_on_full_grids():
    """An AUTO descriptor whose F(4x4) grid fills the GPU (8 images of 64x64,
    64 -> 64 channels: 256 workgroups) keeps the implicit GEMM for per-call
    weights and runs F(4x4) once its weights are bound: bitwise the output of
    an algo="winograd4" descriptor, and within the fp32 tolerance of the
    oracle."""
    t = torch()
    L = A.Layer("wino4", 8, 64, 64, 64, 64, (3, 3), pads=(1, 1, 1, 1), has_bias=True, act=A.ACT_RELU)
    rng = np.random.default_rng(997)
    x, wt, b, s = A.layer_arrays(rng, L)
    d = cc().conv2d_desc_create(layer_params(L))
    assert cc().conv2d_desc_kernel_name(d) == "igemm_f32"
    cc().conv2d_desc_bind_weights(d, to_dev(wt))
    assert cc().conv2d_desc_kernel_name(d) == "winograd4_f32"
    n, ot, ho, wo = cc().conv2d_desc_get_output_shape(d)
    y = Guarded(n * ot * ho * wo, t.float32, float("nan"))
    cc().conv2d_forward(d, to_dev(x), None, to_dev(b), None, y.view)
    t.cuda.synchronize()
    y.check_guards()
    got = y.host().numpy().reshape(n, ot, ho, wo)
    assert np.array_equal(got, _run(L, x, wt, b, s)), "AUTO bound differs from the winograd4 descriptor"
    assert_close(got, oracle_layer(L, x, wt, b, s), FP32_TOL, "AUTO winograd4")
