"""Shared test helpers: run the HIP path through the binding, compare with the
oracle at the stated tolerances, guard bands around outputs."""
import numpy as np

import oracle
import workloads

FP32_TOL = 1e-4     # max |gpu - ref| <= tol * (1 + |ref|)
BF16_TOL = 2e-2
GUARD = 256         # elements of sentinel before and after every output


def torch():
    import torch as t
    return t


def dev():
    t = torch()
    assert t.cuda.is_available(), "GPU test run without a GPU"
    return t.device("cuda:0")


def to_dev(a, dtype=None):
    t = torch()
    x = t.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        x = x.to(dtype)
    return x.to(dev())


def bf16_round(a):
    """float32 -> bfloat16 (round to nearest even) -> float32, via torch."""
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(t.bfloat16).to(t.float32).numpy()


class Guarded:
    """A device buffer of `numel` elements between two sentinel bands."""

    def __init__(self, numel, dtype, fill):
        t = torch()
        self.numel = numel
        self.buf = t.full((numel + 2 * GUARD,), fill, dtype=dtype, device=dev())
        self.fill = fill
        self.view = self.buf[GUARD:GUARD + numel]

    def check_guards(self):
        t = torch()
        host = self.buf.cpu()
        head, tail = host[:GUARD], host[GUARD + self.numel:]
        if isinstance(self.fill, float) and np.isnan(self.fill):
            assert t.isnan(head.float()).all() and t.isnan(tail.float()).all(), "write outside the output"
        else:
            assert (head == self.fill).all() and (tail == self.fill).all(), "write outside the output"

    def host(self):
        return self.view.cpu()


def assert_close(gpu, ref, tol, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if gpu.size == 0:
        return
    assert np.isfinite(gpu).all(), f"{what}: non-finite output at {np.argwhere(~np.isfinite(gpu))[:5].tolist()}"
    excess = np.abs(gpu - ref) - tol * (1.0 + np.abs(ref))
    worst = int(np.argmax(excess))
    if excess.reshape(-1)[worst] > 0:
        idx = np.unravel_index(worst, gpu.shape)
        raise AssertionError(
            f"{what}: max excess {excess.reshape(-1)[worst]:.3e} at {idx}: gpu={gpu[idx]!r} ref={ref[idx]!r} "
            f"(tol {tol}*(1+|ref|)); {int((excess > 0).sum())} of {gpu.size} out of tolerance")


def assert_bitexact(gpu, ref, what=""):
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    bad = np.argwhere(gpu != ref)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {gpu.size} mismatches; first at {i}: gpu={gpu[i]} ref={ref[i]}")


def layer_params(L: workloads.Layer, dtype="f32", **kw):
    import convolution_conv2d_forward_amd as cc
    return cc.make_params(L.n, L.c_in, L.h, L.w, L.c_out, L.k, stride=L.stride, pads=L.pads,
                          dilation=L.dilation, groups=L.groups, has_bias=L.has_bias, pad_value=L.pad_value,
                          act=L.act, alpha=L.alpha if L.act == workloads.ACT_LEAKY_RELU else None,
                          clip=L.clip if L.act == workloads.ACT_CLIP else None, dtype=dtype, **kw)


def oracle_layer(L: workloads.Layer, x, w, b, s, pad_value=None):
    """Oracle output of one float layer (x, w, b, s already the values the GPU consumes)."""
    return oracle.conv2d(x, w, b if L.has_bias else None, stride=L.stride, pads=L.pads, dilation=L.dilation,
                         groups=L.groups, pad_value=L.pad_value if pad_value is None else pad_value,
                         act=L.act, alpha=np.float32(L.alpha), clip=tuple(np.float32(c) for c in L.clip),
                         slope=s if L.act == workloads.ACT_PRELU else None)


def gpu_layer(L: workloads.Layer, x, w, b, s, *, dtype="f32", out_total=None, out_off=0, repeat=1, bound=False,
              algo="auto"):
    """Run one float layer on the GPU into a NaN-guarded output; returns
    (host output as float64 [n, out_total, ho, wo], kernel name, all runs).
    bound: bind the weights to the descriptor and call with w=None."""
    import convolution_conv2d_forward_amd as cc
    t = torch()
    tdt = t.float32 if dtype == "f32" else t.bfloat16
    p = layer_params(L, dtype, prelu_slope_count=(s.size if L.act == workloads.ACT_PRELU else 1),
                     out_total_channels=out_total or 0, out_channel_offset=out_off, algo=algo)
    d = cc.conv2d_desc_create(p)
    n, ot, ho, wo = cc.conv2d_desc_get_output_shape(d)
    xd = to_dev(x.astype(np.float32), tdt)
    wd = to_dev(w.astype(np.float32), tdt)
    bd = to_dev(b.astype(np.float32)) if L.has_bias else None
    sd = to_dev(s.astype(np.float32)) if L.act == workloads.ACT_PRELU else None
    if bound:
        cc.conv2d_desc_bind_weights(d, wd)
        t.cuda.synchronize()
        wd = None
    runs = []
    for _ in range(repeat):
        y = Guarded(n * ot * ho * wo, tdt, float("nan"))
        cc.conv2d_forward(d, xd, wd, bd, sd, y.view)
        t.cuda.synchronize()
        y.check_guards()
        runs.append(y.host().float().numpy().astype(np.float64).reshape(n, ot, ho, wo))
    return runs[0], cc.conv2d_desc_kernel_name(d), runs
