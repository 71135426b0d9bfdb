"""GPU: calls that share one bf16 (or int8 3x3) implicit-GEMM descriptor from
several streams and host threads, each given its own weights.

Such a descriptor re-lays OIHW weights into a buffer it owns before every
convolution; the descriptor orders those calls itself, so each call must
convolve with the weights it was given, whatever the other calls do.  The
outputs are compared with the oracle at the bf16 tolerance (int8:
bit-exact)."""
import threading

import numpy as np
import pytest

import oracle
import workloads
from helpers import (BF16_TOL, assert_bitexact, assert_close, bf16_round, layer_params, oracle_layer, to_dev,
                     torch)

pytestmark = pytest.mark.gpu


def cc():
    import convolution_conv2d_forward_amd as m
    return m


def _case():
    L = workloads.Layer("b", 2, 128, 32, 32, 256, (3, 3), stride=(2, 2), pads=(1, 1, 1, 1), has_bias=True,
                        act=workloads.ACT_PRELU)
    rng = np.random.default_rng(4242)
    x, w1, b, s = workloads.layer_arrays(rng, L)
    _, w2, _, _ = workloads.layer_arrays(rng, L)
    x, w1, w2 = bf16_round(x), bf16_round(w1), bf16_round(w2)
    refs = [oracle_layer(L, x, w, b, s) for w in (w1, w2)]
    return L, x, (w1, w2), b, s, refs


def _outputs(L, n):
    t = torch()
    ho, wo = L.out_hw
    return [t.full((L.n, L.c_out, ho, wo), float("nan"), dtype=t.bfloat16, device="cuda") for _ in range(n)]


def test_bf16_descriptor_shared_by_two_streams():
    t = torch()
    L, x, ws, b, s, refs = _case()
    d = cc().conv2d_desc_create(layer_params(L, "bf16", prelu_slope_count=s.size))
    assert cc().conv2d_desc_kernel_name(d).startswith("igemm_bf16")
    xd, bd, sd = to_dev(x, t.bfloat16), to_dev(b), to_dev(s)
    wd = [to_dev(w, t.bfloat16) for w in ws]
    streams = [t.cuda.Stream(), t.cuda.Stream()]
    reps = 6
    ys = [_outputs(L, reps), _outputs(L, reps)]
    t.cuda.synchronize()
    for i in range(reps):
        for k in (0, 1):
            cc().conv2d_forward(d, xd, wd[k], bd, sd, ys[k][i], stream=streams[k])
    t.cuda.synchronize()
    for k in (0, 1):
        for i in range(reps):
            got = ys[k][i].float().cpu().numpy().astype(np.float64)
            assert_close(got, refs[k], BF16_TOL, f"stream {k} call {i}")


def test_bf16_descriptor_shared_by_two_threads():
    t = torch()
    L, x, ws, b, s, refs = _case()
    d = cc().conv2d_desc_create(layer_params(L, "bf16", prelu_slope_count=s.size))
    xd, bd, sd = to_dev(x, t.bfloat16), to_dev(b), to_dev(s)
    wd = [to_dev(w, t.bfloat16) for w in ws]
    reps = 8
    ys = [_outputs(L, reps), _outputs(L, reps)]
    t.cuda.synchronize()
    errors = []

    def worker(k):
        try:
            st = t.cuda.Stream()
            for i in range(reps):
                cc().conv2d_forward(d, xd, wd[k], bd, sd, ys[k][i], stream=st)
            st.synchronize()
        except Exception as e:   # reported in the main thread
            errors.append(e)

    th = [threading.Thread(target=worker, args=(k,)) for k in (0, 1)]
    for h in th:
        h.start()
    for h in th:
        h.join()
    t.cuda.synchronize()
    assert not errors, errors
    for k in (0, 1):
        for i in range(reps):
            got = ys[k][i].float().cpu().numpy().astype(np.float64)
            assert_close(got, refs[k], BF16_TOL, f"thread {k} call {i}")


def test_int8_descriptor_shared_by_two_streams():
    """An int8 3x3 layer whose per-call weights are re-laid into the
    descriptor's buffer before each call, on two streams with different
    weights."""
    t = torch()
    L = workloads.Layer("q", 2, 64, 24, 32, 96, (3, 3), stride=(2, 2), pads=(1, 1, 1, 1), has_bias=True)
    rng = np.random.default_rng(4243)
    x = rng.integers(-128, 127, size=L.x_shape, endpoint=True).astype(np.int8)
    ws = [rng.integers(-127, 127, size=L.w_shape, endpoint=True).astype(np.int8) for _ in range(2)]
    b = rng.integers(-500, 500, size=L.c_out, endpoint=True).astype(np.int32)
    sc = (0.02, 0.01, 0.05)
    refs = [oracle.qconv2d(x, w, b, *sc, stride=L.stride, pads=L.pads) for w in ws]
    d = cc().conv2d_desc_create(layer_params(L, "i8"))
    assert cc().conv2d_desc_kernel_name(d) == "igemm_i8"
    xd, bd = to_dev(x), to_dev(b)
    wd = [to_dev(w) for w in ws]
    ho, wo = L.out_hw
    streams = [t.cuda.Stream(), t.cuda.Stream()]
    reps = 6
    ys = [[t.zeros((L.n, L.c_out, ho, wo), dtype=t.int8, device="cuda") for _ in range(reps)] for _ in range(2)]
    t.cuda.synchronize()
    for i in range(reps):
        for k in (0, 1):
            cc().qconv2d_forward(d, xd, sc[0], 0, wd[k], sc[1], 0, bd, sc[2], 0, ys[k][i], stream=streams[k])
    t.cuda.synchronize()
    for k in (0, 1):
        for i in range(reps):
            assert_bitexact(ys[k][i].cpu().numpy(), refs[k], f"stream {k} call {i}")


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 3 << 20])
def test_probe_copy_copies(nbytes):
    """The measurement copy moves exactly the bytes asked for (the tail past
    them in dst is untouched)."""
    t = torch()
    n = nbytes // 4
    src = t.arange(n, dtype=t.float32, device="cuda")
    dst = t.full((n + 64,), -1.0, dtype=t.float32, device="cuda")
    cc().conv2d_probe_copy(dst, src)
    t.cuda.synchronize()
    assert t.equal(dst[:n], src)
    assert (dst[n:] == -1.0).all()
