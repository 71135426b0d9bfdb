"""GPU parity of the Winograd F(2x2, 3x3) path (algo = WINOGRAD) against the
oracle's direct float64 convolution, fp32 tolerance 1e-4 * (1 + |ref|).

Winograd reaches the convolution's result by a different arithmetic (input,
filter and output transforms around 16 channel sums), so the oracle stays the
plain definition; the cases cover partial output tiles (odd sizes), every pad
layout with a nonzero pad_value, partial channel chunks and channel tiles,
each activation with bias, batch > 1, concat slices on both sides, and the
five dense-block layers at full size."""
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
    (1, 16, 8, 16, 32, (1, 1, 1, 1), A.ACT_NONE, False, 0.0),          # one workgroup, exact tiles
    (1, 20, 13, 17, 24, (1, 1, 1, 1), A.ACT_RELU, True, 0.0),          # odd sizes: partial tiles, partial chunk
    (2, 35, 9, 30, 40, (0, 2, 1, 0), A.ACT_LEAKY_RELU, True, 0.5),     # asymmetric pads, pad_value, 2 channel tiles
    (1, 64, 24, 40, 33, (2, 2, 2, 2), A.ACT_PRELU, True, -1.0),        # pads of 2, PReLU per channel
    (3, 7, 5, 6, 5, (0, 0, 0, 0), A.ACT_CLIP, True, 0.0),              # no pads, tiny
    (1, 1, 3, 3, 1, (0, 0, 0, 0), A.ACT_NONE, False, 0.0),             # a single output
    (1, 48, 33, 65, 64, (1, 0, 0, 1), A.ACT_NONE, True, 0.25),         # several workgroups per row, ragged edges
    (2, 24, 128, 128, 64, (1, 1, 1, 1), A.ACT_RELU, True, 0.0),        # enough workgroups for 64-channel tiles
]


def _run(L, x, w, b, s, *, in_total=0, in_off=0, out_total=0, out_off=0, bound=False):
    t = torch()
    d = cc().conv2d_desc_create(layer_params(L, prelu_slope_count=s.size, in_total_channels=in_total,
                                             in_channel_offset=in_off, out_total_channels=out_total,
                                             out_channel_offset=out_off, algo="winograd"))
    assert cc().conv2d_desc_kernel_name(d) == "winograd_f32"
    n, ot, ho, wo = cc().conv2d_desc_get_output_shape(d)
    y = Guarded(n * ot * ho * wo, t.float32, float("nan"))
    if bound:
        cc().conv2d_desc_bind_weights(d, to_dev(w))
    cc().conv2d_forward(d, to_dev(x), None if bound else to_dev(w), to_dev(b) if L.has_bias else None,
                        to_dev(s) if L.act == A.ACT_PRELU else None, y.view)
    t.cuda.synchronize()
    y.check_guards()
    return y.host().numpy().reshape(n, ot, ho, wo)


@pytest.mark.parametrize("i", range(len(CASES)))
def test_winograd_cases(i):
    n, ci, h, w, co, pads, act, bias, pv = CASES[i]
    L = A.Layer("wino", n, ci, h, w, co, (3, 3), pads=pads, has_bias=bias, act=act, alpha=0.2, clip=(-0.3, 0.4),
                pad_value=pv)
    rng = np.random.default_rng(800 + i)
    x, wt, b, s = A.layer_arrays(rng, L)
    print(f"case {i}: {L}", flush=True)
    ref = oracle_layer(L, x, wt, b, s)
    assert_close(_run(L, x, wt, b, s), ref, FP32_TOL, f"winograd case {i}")


def test_winograd_concat_slices():
    """Input channels [5, 5 + c_in) of a wider buffer, output into channels
    [3, 3 + c_out) of another; the channels around the slice stay NaN."""
    L = A.Layer("wino", 2, 24, 10, 18, 20, (3, 3), pads=(1, 1, 1, 1), has_bias=True, act=A.ACT_RELU)
    rng = np.random.default_rng(880)
    x, wt, b, s = A.layer_arrays(rng, L)
    big = rng.standard_normal((L.n, L.c_in + 9, L.h, L.w)).astype(np.float32)
    big[:, 5:5 + L.c_in] = x
    y = _run(L, big, wt, b, s, in_total=L.c_in + 9, in_off=5, out_total=L.c_out + 6, out_off=3)
    assert np.isnan(y[:, :3]).all() and np.isnan(y[:, 3 + L.c_out:]).all()
    assert_close(y[:, 3:3 + L.c_out], oracle_layer(L, x, wt, b, s), FP32_TOL, "winograd slices")


def test_winograd_dense_block_full_size():
    """The dense-block chain's five layers (1 x Cin x 128 x 128, Cin = 64 + 32k),
    each fed with the oracle's own previous outputs, at full size; with the
    weights passed per call and bound to the descriptor (bitwise equal)."""
    wl = A.dense_block()
    a = wl.arrays
    cur = a["x"]
    for k, L in enumerate(wl.layers):
        w = a[f"w{k}"]
        ref = oracle_layer(L, cur, w, None, None)
        b0, s0 = np.zeros(L.c_out, np.float32), np.zeros(1, np.float32)
        got = _run(L, cur, w, b0, s0)
        assert_close(got, ref, FP32_TOL, f"dense block layer {k}")
        assert np.array_equal(_run(L, cur, w, b0, s0, bound=True), got), f"dense block layer {k}: bound weights"
        cur = np.concatenate([cur, ref.astype(np.float32)], axis=1)


@pytest.mark.parametrize("i", range(len(CASES)))
def test_winograd_bound_weights(i):
    """Weights bound to the descriptor: U = G g G^T is computed once and packed
    in the kernel's register order.  The output is bitwise that of the same
    descriptor given the OIHW weights (the same transform arithmetic), and
    matches the oracle."""
    t = torch()
    n, ci, h, w, co, pads, act, bias, pv = CASES[i]
    L = A.Layer("wino", n, ci, h, w, co, (3, 3), pads=pads, has_bias=bias, act=act, alpha=0.2, clip=(-0.3, 0.4),
                pad_value=pv)
    rng = np.random.default_rng(850 + i)
    x, wt, b, s = A.layer_arrays(rng, L)
    d = cc().conv2d_desc_create(layer_params(L, prelu_slope_count=s.size, algo="winograd"))
    nn, ot, ho, wo = cc().conv2d_desc_get_output_shape(d)
    xd, wd = to_dev(x), to_dev(wt)
    bd = to_dev(b) if L.has_bias else None
    sd = to_dev(s) if L.act == A.ACT_PRELU else None
    outs = []
    for bound in (False, True):
        if bound:
            cc().conv2d_desc_bind_weights(d, wd)
        y = Guarded(nn * ot * ho * wo, t.float32, float("nan"))
        cc().conv2d_forward(d, xd, None if bound else wd, bd, sd, y.view)
        t.cuda.synchronize()
        y.check_guards()
        outs.append(y.host().numpy().reshape(nn, ot, ho, wo))
    assert np.array_equal(outs[0], outs[1]), "bound weights differ from explicit weights"
    assert_close(outs[1], oracle_layer(L, x, wt, b, s), FP32_TOL, f"winograd bound case {i}")


def test_auto_dense_block_bound_weights_use_winograd():
    """AUTO descriptors of the dense-block layers (in a 256-channel concat
    buffer, run in place) keep the implicit GEMM for per-call weights and
    switch to the packed-U Winograd kernel once their weights are bound: the
    bound chain equals the chain of algo="winograd" descriptors with bound
    weights bit for bit, and every layer matches the oracle."""
    t = torch()
    wl = A.dense_block()
    a = wl.arrays
    total = A.DENSE_TOTAL_CHANNELS
    outs = {}
    for algo in ("auto", "winograd"):
        buf = t.full((1, total, 128, 128), float("nan"), dtype=t.float32, device="cuda")
        buf[:, :64] = to_dev(a["x"])
        for k, L in enumerate(wl.layers):
            d = cc().conv2d_desc_create(layer_params(L, in_total_channels=total, out_total_channels=total,
                                                     out_channel_offset=L.c_in, algo=algo))
            if algo == "auto":
                assert cc().conv2d_desc_kernel_name(d) == "igemm_f32"
            cc().conv2d_desc_bind_weights(d, to_dev(a[f"w{k}"]))
            assert cc().conv2d_desc_kernel_name(d) == "winograd_f32", (algo, k)
            cc().conv2d_forward(d, buf, None, None, None, buf)
        t.cuda.synchronize()
        outs[algo] = buf.cpu().numpy().astype(np.float64)
    assert np.array_equal(outs["auto"], outs["winograd"]), "AUTO bound chain differs from the Winograd chain"
    cur = a["x"]
    for k, L in enumerate(wl.layers):
        ref = oracle_layer(L, cur, a[f"w{k}"], None, None)
        assert_close(outs["auto"][:, L.c_in:L.c_in + L.c_out], ref, FP32_TOL, f"dense block layer {k}")
        cur = np.concatenate([cur, ref.astype(np.float32)], axis=1)


@pytest.mark.parametrize("algo,kernel", [("auto", "small_f32"), ("direct", "igemm_f32")])
def test_auto_small_bound_layer_keeps_its_kernel(algo, kernel):
    """A 3x3 layer too small to fill the GPU with Winograd workgroups keeps
    its kernel after binding."""
    L = A.Layer("small", 1, 64, 16, 16, 32, (3, 3), pads=(1, 1, 1, 1))
    d = cc().conv2d_desc_create(layer_params(L, algo=algo))
    assert cc().conv2d_desc_kernel_name(d) == kernel
    cc().conv2d_desc_bind_weights(d, to_dev(np.zeros(L.w_shape, np.float32)))
    assert cc().conv2d_desc_kernel_name(d) == kernel
