"""GPU parity of the fp32 pointwise kernels for deep reductions (the
128 x 128 GEMM-tile kernel pw_gemm_f32, and pw_narrow_f32 for <= 32 output
channels; see the cases further down) against the oracle.

pw_gemm_f32: 1x1
stride 1, no pads, one group, >= 128 input and output channels, grids of at
least two workgroups per compute unit) against the oracle's direct float64
convolution, fp32 tolerance 1e-4 * (1 + |ref|).

The cases cover pixel counts that are not multiples of the 128-pixel tile,
output-channel counts that are not multiples of the 128-channel tile, input
channel counts that end in a partial 16-channel chunk, every activation with
and without bias, concat slices on both sides, bound weights, a call whose
input is not 16-byte aligned (served by the implicit GEMM instead), and the
mixed sweep's 1x1 256 -> 512 layer at full size (batch 32)."""
import numpy as np
import pytest

import workloads as A
from helpers import FP32_TOL, Guarded, assert_close, layer_params, oracle_layer, to_dev, torch

pytestmark = pytest.mark.gpu


def cc():
    import convolution_conv2d_forward_amd as m
    return m


CASES = [
    # n, c_in, h, w, c_out, act, bias (each grid >= 512 workgroups of 128 pixels x 128 channels)
    (128, 128, 16, 32, 128, A.ACT_NONE, False),      # whole tiles, 8 chunks
    (64, 132, 20, 20, 136, A.ACT_RELU, True),        # ragged pixels, channels and chunk
    (256, 260, 9, 12, 200, A.ACT_PRELU, True),       # 108-pixel planes (one partial tile per image)
    (96, 144, 14, 14, 384, A.ACT_LEAKY_RELU, True),  # 3 channel tiles
    (80, 192, 28, 28, 128, A.ACT_CLIP, False),       # 784-pixel planes
]


def _run(L, x, w, b, s, *, in_total=0, in_off=0, out_total=0, out_off=0, bound=False, xdev=None):
    t = torch()
    d = cc().conv2d_desc_create(layer_params(L, prelu_slope_count=s.size, in_total_channels=in_total,
                                             in_channel_offset=in_off, out_total_channels=out_total,
                                             out_channel_offset=out_off))
    assert cc().conv2d_desc_kernel_name(d) == "pw_gemm_f32"
    n, ot, ho, wo = cc().conv2d_desc_get_output_shape(d)
    y = Guarded(n * ot * ho * wo, t.float32, float("nan"))
    wd = to_dev(w)
    if bound:
        cc().conv2d_desc_bind_weights(d, wd)
        wd = None
    cc().conv2d_forward(d, to_dev(x) if xdev is None else xdev, wd, to_dev(b) if L.has_bias else None,
                        to_dev(s) if L.act == A.ACT_PRELU else None, y.view)
    t.cuda.synchronize()
    y.check_guards()
    return y.host().numpy().reshape(n, ot, ho, wo)


def _layer(i):
    n, ci, h, w, co, act, bias = CASES[i]
    return A.Layer("pwg", n, ci, h, w, co, (1, 1), has_bias=bias, act=act, alpha=0.2, clip=(-0.3, 0.4))


@pytest.mark.parametrize("i", range(len(CASES)))
def test_pw_gemm_cases(i):
    L = _layer(i)
    rng = np.random.default_rng(700 + i)
    x, wt, b, s = A.layer_arrays(rng, L)
    print(f"case {i}: {L}", flush=True)
    assert_close(_run(L, x, wt, b, s, bound=i % 2 == 1), oracle_layer(L, x, wt, b, s), FP32_TOL, f"pw_gemm case {i}")


def test_pw_gemm_concat_slices():
    """Input channels [3, 3 + c_in) of a wider buffer, output into channels
    [8, 8 + c_out) of another; the channels around the slice stay NaN."""
    L = _layer(1)
    rng = np.random.default_rng(760)
    x, wt, b, s = A.layer_arrays(rng, L)
    big = rng.standard_normal((L.n, L.c_in + 7, L.h, L.w)).astype(np.float32)
    big[:, 3:3 + L.c_in] = x
    y = _run(L, big, wt, b, s, in_total=L.c_in + 7, in_off=3, out_total=L.c_out + 12, out_off=8)
    assert np.isnan(y[:, :8]).all() and np.isnan(y[:, 8 + L.c_out:]).all()
    assert_close(y[:, 8:8 + L.c_out], oracle_layer(L, x, wt, b, s), FP32_TOL, "pw_gemm slices")


def test_pw_gemm_unaligned_input_falls_back():
    """An input one float past a 16-byte boundary: the descriptor still names
    pw_gemm_f32, the call runs on the implicit GEMM, results within the
    tolerance."""
    t = torch()
    L = _layer(0)
    rng = np.random.default_rng(770)
    x, wt, b, s = A.layer_arrays(rng, L)
    raw = t.zeros(x.size + 4, dtype=t.float32, device="cuda")
    xv = raw[1:1 + x.size]
    xv.copy_(t.from_numpy(x.reshape(-1)).cuda())
    assert_close(_run(L, x, wt, b, s, xdev=xv), oracle_layer(L, x, wt, b, s), FP32_TOL, "pw_gemm unaligned")


def test_pw_gemm_mixed_sweep_pointwise_full_size():
    """The mixed sweep's 1x1 256 -> 512 layer (batch 32, 32 x 32, bias,
    PReLU), compared in full with the oracle."""
    L = [l for l in A.mixed_sweep_layers() if l.name == "pw"][0]
    rng = np.random.default_rng(780)
    x, wt, b, s = A.layer_arrays(rng, L)
    got = _run(L, x, wt, b, s, bound=True)
    ref = oracle_layer(L, x, wt, b, s)
    print(f"max |y - ref| / (1 + |ref|) = {np.max(np.abs(got - ref) / (1 + np.abs(ref))):.3g}", flush=True)
    assert_close(got, ref, FP32_TOL, "mixed sweep pw")


# pw_narrow_f32: 1x1 with 64 < K <= 256 and <= 32 output channels, 32-pixel
# tiles (ragged when the plane is not a multiple of 32), K split over four
# waves in 16-channel chunks (partial last chunk when K % 16 != 0).
NARROW_CASES = [
    # n, c_in, h, w, c_out, act, bias
    (2, 68, 10, 10, 32, A.ACT_RELU, True),          # 5 chunks, the last with 4 channels; 100-pixel planes
    (3, 256, 8, 12, 1, A.ACT_NONE, False),          # K at its maximum, one output channel
    (1, 132, 7, 4, 17, A.ACT_PRELU, True),          # 28 pixels: one partial tile; 17 channels
    (4, 96, 33, 20, 24, A.ACT_LEAKY_RELU, True),    # 6 chunks, several tiles per image
    (2, 200, 16, 16, 32, A.ACT_CLIP, False),        # 13 chunks: waves take 4, 3, 3, 3
]


def _narrow(i):
    n, ci, h, w, co, act, bias = NARROW_CASES[i]
    return A.Layer("pwn", n, ci, h, w, co, (1, 1), has_bias=bias, act=act, alpha=0.2, clip=(-0.3, 0.4))


def _run_narrow(L, x, w, b, s, *, bound=False, xdev=None, **kw):
    t = torch()
    d = cc().conv2d_desc_create(layer_params(L, prelu_slope_count=s.size, **kw))
    assert cc().conv2d_desc_kernel_name(d) == "pw_narrow_f32"
    n, ot, ho, wo = cc().conv2d_desc_get_output_shape(d)
    y = Guarded(n * ot * ho * wo, t.float32, float("nan"))
    wd = to_dev(w)
    if bound:
        cc().conv2d_desc_bind_weights(d, wd)
        wd = None
    cc().conv2d_forward(d, to_dev(x) if xdev is None else xdev, wd, to_dev(b) if L.has_bias else None,
                        to_dev(s) if L.act == A.ACT_PRELU else None, y.view)
    t.cuda.synchronize()
    y.check_guards()
    return y.host().numpy().reshape(n, ot, ho, wo)


@pytest.mark.parametrize("i", range(len(NARROW_CASES)))
def test_pw_narrow_cases(i):
    L = _narrow(i)
    rng = np.random.default_rng(800 + i)
    x, wt, b, s = A.layer_arrays(rng, L)
    print(f"narrow case {i}: {L}", flush=True)
    assert_close(_run_narrow(L, x, wt, b, s, bound=i % 2 == 0), oracle_layer(L, x, wt, b, s), FP32_TOL,
                 f"pw_narrow case {i}")


def test_pw_narrow_slices_and_unaligned_input():
    """Channels [2, 2 + c_in) of a wider input into channels [6, 6 + c_out)
    of a wider output (the rest stays NaN); then an input one float past a
    16-byte boundary, served by the implicit GEMM."""
    t = torch()
    L = _narrow(3)
    rng = np.random.default_rng(850)
    x, wt, b, s = A.layer_arrays(rng, L)
    ref = oracle_layer(L, x, wt, b, s)
    big = rng.standard_normal((L.n, L.c_in + 5, L.h, L.w)).astype(np.float32)
    big[:, 2:2 + L.c_in] = x
    y = _run_narrow(L, big, wt, b, s, in_total_channels=L.c_in + 5, in_channel_offset=2,
                    out_total_channels=L.c_out + 10, out_channel_offset=6)
    assert np.isnan(y[:, :6]).all() and np.isnan(y[:, 6 + L.c_out:]).all()
    assert_close(y[:, 6:6 + L.c_out], ref, FP32_TOL, "pw_narrow slices")
    raw = t.zeros(x.size + 4, dtype=t.float32, device="cuda")
    xv = raw[1:1 + x.size]
    xv.copy_(t.from_numpy(x.reshape(-1)).cuda())
    assert_close(_run_narrow(L, x, wt, b, s, xdev=xv), ref, FP32_TOL, "pw_narrow unaligned")
