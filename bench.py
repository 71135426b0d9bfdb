"""Benchmark of the conv2d forward path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME] [--no-cpu-baseline] [--no-extra]

A step is one pass of the dense-block chain: input 1x64x128x128 in a
1x256x128x128 fp32 concat buffer, five 3x3 s1 p1 convolutions with
Cin = 64+32k and Cout = 32 (last 64), LeakyReLU(0.2) on all but the last,
each writing the buffer's next channel slice (ConcatFusedTail), no bias.
`value` is conv GFLOP/s (2 * MACs, padded taps counted) over K timed steps.
Steps rotate over buffer sets (>= 1 GiB in all) so that inputs come from HBM,
not from the 256 MB last-level cache.

The JSON line also carries:
  roofline      the dominant kernel of the step against the fp32 MFMA peak;
                its duration comes from HIP events on the launch stream around
                a run of back-to-back launches of each layer, queued behind a
                GPU delay (so no host launch time inside the run; the mean
                per launch is the kernel plus the dispatch gap between
                kernels)
  cpu_baseline  the float64 CPU oracle timed on this host's cores on a sample
                of the same workload's outputs
  per_config    the other synthetic workloads (single conv, inverted
                bottleneck fused/unfused, mixed sweep fp32/bf16, int8 chain
                unfused/fused, int8 bottleneck fused/unfused, int8 dense
                layers, dense-block layers with Winograd beside the implicit
                GEMM), each layer timed in such a run the same way, with its
                binding roofline; HBM-bound entries also carry the time of the
                library's streaming 16-byte copy moving the same bytes
                (copy_us) and their speed as a fraction of it (copy_frac)
Everything on stdout except the final JSON line goes to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "conv GFLOP/s (2·MACs) and depthwise GB/s, % of MFMA/HBM roofline"
PEAK = {"f32": 157.3e12, "bf16": 2516.6e12, "i8": 5033.2e12, "hbm": 8.0e12}
ROTATE_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", default="all",
                    help="all | dense_block | single_conv | bottleneck | mixed_f32 | mixed_bf16 | int8_chain | "
                         "int8_bottleneck | int8_dense | winograd | copy")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--reps", type=int, default=20, help="timed launches per layer for per_config")
    return ap.parse_args()


# ------------------------------------------------------------------ setup --

def torch_mod():
    import torch
    return torch


def dev():
    return torch_mod().device("cuda:0")


def t_(a, dtype=None):
    t = torch_mod().from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev())


def params_of(L, dtype="f32", **kw):
    import convolution_conv2d_forward_amd as cc
    import workloads
    return cc.make_params(L.n, L.c_in, L.h, L.w, L.c_out, L.k, stride=L.stride, pads=L.pads, dilation=L.dilation,
                          groups=L.groups, has_bias=L.has_bias, pad_value=L.pad_value, act=L.act,
                          alpha=L.alpha if L.act == workloads.ACT_LEAKY_RELU else None,
                          clip=L.clip if L.act == workloads.ACT_CLIP else None, dtype=dtype,
                          prelu_slope_count=L.c_out if L.act == workloads.ACT_PRELU else 1, **kw)


def layer_bytes(L, esize, wsize=None, extra=0):
    """Algorithmic HBM bytes: x once + weights + bias/slope + y once."""
    ho, wo = L.out_hw
    wsize = esize if wsize is None else wsize
    b = L.n * L.c_in * L.h * L.w * esize + L.c_out * (L.c_in // L.groups) * L.k[0] * L.k[1] * wsize
    b += L.n * L.c_out * ho * wo * esize
    if L.has_bias:
        b += 4 * L.c_out
    if L.act == 3:
        b += 4 * L.c_out
    return b + extra


_SLEEP_CYCLES_PER_US = None


def gpu_delay(us):
    """Queue a spin kernel of about `us` microseconds on the current stream.
    Launches enqueued behind it then run back to back, so the HIP events
    around each one time GPU work rather than waits for the host's next
    launch call (a 10 us kernel is comparable to one ctypes call)."""
    global _SLEEP_CYCLES_PER_US
    torch = torch_mod()
    if _SLEEP_CYCLES_PER_US is None:
        n = 2_000_000
        torch.cuda._sleep(n)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        torch.cuda._sleep(n)
        e.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_US = n / (s.elapsed_time(e) * 1e3)
    torch.cuda._sleep(int(us * _SLEEP_CYCLES_PER_US))


class EventTimer:
    """HIP events around each launch, on the current (launch) stream."""

    def __init__(self):
        self.pairs = {}

    def run(self, key, fn):
        torch = torch_mod()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.pairs.setdefault(key, []).append((s, e))

    def mean_us(self, key):
        torch_mod().cuda.synchronize()
        ts = [s.elapsed_time(e) * 1e3 for s, e in self.pairs[key]]
        return float(np.mean(ts)), float(np.median(ts)), len(ts)


def run_time_us(fns, reps, delay_per_launch_us=200.0):
    """Mean HIP-event time of one launch in a run of `reps` back-to-back
    launches (fns[i % len(fns)] for launch i): two events on the launch
    stream around the whole run, queued behind a GPU delay so that the host
    has enqueued every launch before the first one starts.  The mean is the
    kernel's duration plus the dispatch gap between consecutive kernels; an
    event between every pair of launches would add its own GPU-side cost to
    each launch."""
    torch = torch_mod()
    delay = delay_per_launch_us * reps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gpu_delay(delay)
    t0 = time.perf_counter()
    e0.record()
    for i in range(reps):
        fns[i % len(fns)]()
    e1.record()
    t_enq = (time.perf_counter() - t0) * 1e6
    torch.cuda.synchronize()
    if t_enq > delay:
        log(f"host enqueue {t_enq:.0f} us outran the {delay:.0f} us GPU delay")
    return e0.elapsed_time(e1) * 1e3 / reps


def roofline_entry(flops, bytes_, t_us, dtype, bound=None):
    t = t_us * 1e-6
    mf = flops / t / PEAK[dtype]
    hb = bytes_ / t / PEAK["hbm"]
    t_roof = max(flops / PEAK[dtype], bytes_ / PEAK["hbm"])
    if bound is None:
        bound = "mfma" if flops / PEAK[dtype] >= bytes_ / PEAK["hbm"] else "hbm"
    return {"us": round(t_us, 3), "gflops": round(flops / t / 1e9, 1), "gbps": round(bytes_ / t / 1e9, 1),
            "mfma_frac": round(mf, 4), "hbm_frac": round(hb, 4), "bound": bound,
            "roofline_frac": round(t_roof / t, 4), "flops": int(flops), "bytes": int(bytes_)}


# ------------------------------------------------------------ dense block --

class DenseBlock:
    """The chain: 5 convs into one concat buffer, rotated over buffer sets.
    bound: each layer's weights are bound to its descriptor once at set-up
    (conv2d_desc_bind_weights, which packs them for the fp32 implicit GEMM, as
    ncnn packs weights when a layer's pipeline is created) and every step
    passes w=None; else every call passes the OIHW weights."""

    def __init__(self, h=128, w=128, bound=True):
        import convolution_conv2d_forward_amd as cc
        import workloads
        torch = torch_mod()
        self.cc = cc
        wl = workloads.dense_block(h, w)
        self.layers = wl.layers
        total = workloads.DENSE_TOTAL_CHANNELS
        buf_bytes = total * h * w * 4
        self.nsets = max(1, -(-ROTATE_BYTES // buf_bytes))
        x = t_(wl.arrays["x"])
        self.bufs = []
        for _ in range(self.nsets):
            b = torch.zeros((1, total, h, w), device=dev())
            b[:, :64] = x
            self.bufs.append(b)
        self.descs = [cc.conv2d_desc_create(params_of(L, in_total_channels=total, out_total_channels=total,
                                                       out_channel_offset=L.c_in)) for L in self.layers]
        self.w = [t_(wl.arrays[f"w{k}"]) for k in range(len(self.layers))]
        self.bound = bound
        if bound:
            for d, wk in zip(self.descs, self.w):
                cc.conv2d_desc_bind_weights(d, wk)
            torch.cuda.synchronize()
            self.w = [None] * len(self.layers)
        # after binding: AUTO runs bound 3x3 layers of this size on Winograd
        self.kernels = [cc.conv2d_desc_kernel_name(d) for d in self.descs]
        self.flops = [L.flops for L in self.layers]
        # x slice read once + weights + the written slice
        self.bytes = [4 * (L.c_in * h * w + L.c_out * L.c_in * 9 + L.c_out * h * w) for L in self.layers]
        self.i = 0

    def step(self):
        """One pass of the chain."""
        buf = self.bufs[self.i % self.nsets]
        self.i += 1
        for d, w in zip(self.descs, self.w):
            self.cc.conv2d_forward(d, buf, w, None, None, buf)

    def layer_fns(self, k):
        """Launches of layer k alone, one per buffer set."""
        d, w = self.descs[k], self.w[k]
        return [lambda b=b: self.cc.conv2d_forward(d, b, w, None, None, b) for b in self.bufs]


def bench_dense_block(steps, warmup, bound=True):
    torch = torch_mod()
    db = DenseBlock(bound=bound)
    log(f"dense block: {db.nsets} buffer sets, kernels {db.kernels}, weights {'bound' if bound else 'per call'}")
    for _ in range(warmup):
        db.step()
    torch.cuda.synchronize()
    # Wall-clock pass: K steps, no events.
    t0 = time.perf_counter()
    for _ in range(steps):
        db.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # Per-layer times: each layer in a run of back-to-back launches of its
    # own (inputs from the passes above), events around the run.
    reps = max(steps, 20)
    per = []
    for k in range(len(db.layers)):
        t = run_time_us(db.layer_fns(k), reps)
        per.append((t, t, reps))
    return db, wall, per


def dense_roofline(db, per):
    """Roofline of the dominant kernel: the instantiation with the largest
    total event time in the step (layers sharing a kernel are pooled).
    achieved counts the convolution's own 2*MACs; for Winograd F(2x2,3x3),
    which issues 16 products per 2x2 output tile and channel pair instead of
    36, the MFMA flops it executes are given beside it."""
    groups = {}
    for k, name in enumerate(db.kernels):
        if db.bound and name == "igemm_f32":
            name = "igemm_f32_packed"
        L = db.layers[k]
        cfg = f"{name}/M{64 if L.c_out > 32 else 32}"
        g = groups.setdefault(cfg, {"layers": [], "flops": 0, "exec": 0, "bytes": 0, "us": 0.0})
        g["layers"].append(L.name)
        g["flops"] += db.flops[k]
        g["exec"] += (2 * 16 * L.c_out * L.c_in * ((L.h + 1) // 2) * ((L.w + 1) // 2)
                      if name == "winograd_f32" else db.flops[k])
        g["bytes"] += db.bytes[k]
        g["us"] += per[k][0]
    dom = max(groups, key=lambda g: groups[g]["us"])
    g = groups[dom]
    n = len(g["layers"])
    achieved = g["flops"] / (g["us"] * 1e-6) / 1e12
    roof = {
        "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK["f32"] / 1e12, "unit": "TFLOP/s",
        "frac": round(achieved * 1e12 / PEAK["f32"], 4), "traffic": traffic_for(dom, n),
        "kernel": dom, "launches_per_step": n, "avg_launch_us": round(g["us"] / n, 3),
        "flops_per_launch": int(g["flops"] / n), "layers": g["layers"],
    }
    if g["exec"] != g["flops"]:
        ex = g["exec"] / (g["us"] * 1e-6) / 1e12
        roof.update(executed_flops_per_launch=int(g["exec"] / n), executed_tflops=round(ex, 2),
                    executed_frac=round(ex * 1e12 / PEAK["f32"], 4))
    return dom, g, roof


def _source_sha(rel):
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(kernel, launches):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else null."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec or rec.get("source_sha") != _source_sha(rec["source"]):
        return None
    return rec.get("bytes_per_launch")


# -------------------------------------------------------------- per config --

def _rotating(make, footprint, target=ROTATE_BYTES, cap=64):
    n = int(min(cap, max(1, -(-target // max(1, footprint)))))
    return [make() for _ in range(n)]


def time_layer(key, fn_sets, reps, warm=3):
    """Mean HIP-event time of one launch.  fn_sets: list of callables (one per
    rotating buffer set); the timed launches run back to back behind a GPU
    delay with events around the whole run (run_time_us)."""
    torch = torch_mod()
    for i in range(warm):
        fn_sets[i % len(fn_sets)]()
    torch.cuda.synchronize()
    return run_time_us(fn_sets, reps)


def float_layer_fns(L, x, w, b, s, dtype, reps, bound=False):
    """Time one float layer.  bound: the weights are bound to the descriptor
    once (conv2d_desc_bind_weights, re-laid for the kernel at that point) and
    every timed call passes w=None."""
    import convolution_conv2d_forward_amd as cc
    torch = torch_mod()
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    esize = 4 if dtype == "f32" else 2
    d = cc.conv2d_desc_create(params_of(L, dtype))
    ho, wo = L.out_hw
    wd = t_(w, tdt)
    if bound:
        cc.conv2d_desc_bind_weights(d, wd)
        torch.cuda.synchronize()
        wd = None
    bd = t_(b) if L.has_bias else None
    sd = t_(s) if L.act == 3 else None
    xs = t_(x, tdt)
    foot = (x.size + L.n * L.c_out * ho * wo) * esize

    def make():
        xi = xs.clone()
        yi = torch.empty((L.n, L.c_out, ho, wo), dtype=tdt, device=dev())
        return lambda: cc.conv2d_forward(d, xi, wd, bd, sd, yi)

    fns = _rotating(make, foot)
    t = time_layer(L.name, fns, reps)
    return t, cc.conv2d_desc_kernel_name(d)


def per_config(reps, only="all"):
    """Per-configuration table; `only` selects one section (single_conv,
    bottleneck, mixed_f32, mixed_bf16, int8_chain, int8_bottleneck, int8_dense,
    winograd)
    or all of them."""
    import convolution_conv2d_forward_amd as cc
    import workloads
    torch = torch_mod()
    out = {}

    def want(name):
        return only in ("all", name)

    # single conv (latency)
    if want("single_conv"):
        wl = workloads.single_conv()
        L = wl.layers[0]
        t, k = float_layer_fns(L, wl.arrays["x"], wl.arrays["w"], wl.arrays["b"], None, "f32", reps)
        out["single_conv"] = {"conv": dict(roofline_entry(L.flops, layer_bytes(L, 4), t, "f32", bound="latency"),
                                           kernel=k)}
        log("single_conv", out["single_conv"])

    # inverted bottleneck
    if want("bottleneck"):
        wl = workloads.bottleneck()
        L1, L2, L3 = wl.layers
        a = wl.arrays
        res = {}
        for L, wk in ((L1, "w_pw1"), (L2, "w_dw"), (L3, "w_pw2")):
            rng = np.random.default_rng(3)
            x = a["x"] if L is L1 else rng.standard_normal(L.x_shape).astype(np.float32)
            t, k = float_layer_fns(L, x, a[wk], None, None, "f32", reps)
            res[L.name] = dict(roofline_entry(L.flops, layer_bytes(L, 4), t, "f32"), kernel=k)
        d1, d2 = cc.conv2d_desc_create(params_of(L1)), cc.conv2d_desc_create(params_of(L2))
        w1, w2 = t_(a["w_pw1"]), t_(a["w_dw"])
        xs = t_(a["x"])

        def make_fused():
            xi = xs.clone()
            yi = torch.empty((L2.n, L2.c_out, L2.h, L2.w), device=dev())
            return lambda: cc.fused_pw_dw_forward(d1, d2, xi, w1, None, None, w2, None, None, yi)

        fns = _rotating(make_fused, (L1.n * L1.c_in + L2.n * L2.c_out) * L1.h * L1.w * 4)
        t = time_layer("fused", fns, reps)
        fb = 4 * (L1.n * L1.c_in * L1.h * L1.w + L1.c_out * L1.c_in + L2.c_out * 9 + L2.n * L2.c_out * L2.h * L2.w)
        res["fused_pw_dw"] = dict(roofline_entry(L1.flops + L2.flops, fb, t, "f32"), kernel="fused_pw_dw")
        # dw -> pw2 fused: the depthwise output stays on chip
        d3 = cc.conv2d_desc_create(params_of(L3))
        w3 = t_(a["w_pw2"])
        xe = t_(np.random.default_rng(3).standard_normal(L2.x_shape).astype(np.float32))

        def make_dwpw():
            xi = xe.clone()
            yi = torch.empty((L3.n, L3.c_out, L3.h, L3.w), device=dev())
            return lambda: cc.fused_dw_pw_forward(d2, d3, xi, w2, None, None, w3, None, None, yi)

        fns = _rotating(make_dwpw, (L2.n * L2.c_in + L3.n * L3.c_out) * L2.h * L2.w * 4)
        t = time_layer("fused_dw_pw", fns, reps)
        fb = 4 * (L2.n * L2.c_in * L2.h * L2.w + L2.c_out * 9 + L3.c_out * L3.c_in + L3.n * L3.c_out * L3.h * L3.w)
        res["fused_dw_pw"] = dict(roofline_entry(L2.flops + L3.flops, fb, t, "f32"), kernel="fused_dw_pw")
        out["bottleneck"] = res
        log("bottleneck", res)

    # mixed sweep fp32 / bf16
    for dtype in ("f32", "bf16"):
        if not want(f"mixed_{dtype}"):
            continue
        res = {}
        for name in ("s2", "d2", "g32", "pw"):
            wl = workloads.mixed_sweep(which={name})
            L = [l for l in wl.layers if l.name == name][0]
            a = wl.arrays
            args = (L, a[f"x_{name}"], a[f"w_{name}"], a[f"b_{name}"], a[f"s_{name}"], dtype, reps)
            es = 4 if dtype == "f32" else 2
            # Weights bound at set-up (the timed figure), as a layer's weights
            # are transformed once when it is created: the bf16 implicit GEMM
            # re-lays them into its per-chunk LDS image, the fp32 one packs the
            # 3x3 tiles it can read from registers.  Passing them on every call
            # is reported beside it.
            t, k = float_layer_fns(*args, bound=True)
            t_call, _ = float_layer_fns(*args)
            res[name] = dict(roofline_entry(L.flops, layer_bytes(L, es), t, dtype), kernel=k,
                             weights="bound", us_weights_per_call=round(t_call, 3))
            log("mixed", dtype, name, res[name])
        out[f"mixed_sweep_{dtype}"] = res

    # int8 chain
    if want("int8_chain"):
        wl = workloads.int8_chain()
        a = wl.arrays
        res = {}
        for L in wl.layers:
            d = cc.conv2d_desc_create(params_of(L, "i8"))
            ho, wo = L.out_hw
            rng = np.random.default_rng(5)
            x = a["x"] if L.name == "dw_s1" else rng.integers(-128, 128, size=L.x_shape).astype(np.int8)
            xs = t_(x)
            wd, bd = t_(a[f"w_{L.name}"]), t_(a[f"b_{L.name}"])

            def make(d=d, xs=xs, wd=wd, bd=bd, L=L, ho=ho, wo=wo):
                xi = xs.clone()
                yi = torch.empty((L.n, L.c_out, ho, wo), dtype=torch.int8, device=dev())
                return lambda: cc.qconv2d_forward(d, xi, 0.02, 0, wd, 0.01, 0, bd, 0.05, 0, yi)

            fns = _rotating(make, x.size + L.n * L.c_out * ho * wo)
            t = time_layer(L.name, fns, reps)
            res[L.name] = dict(roofline_entry(L.flops, layer_bytes(L, 1, extra=0), t, "i8"),
                               kernel=cc.conv2d_desc_kernel_name(d))
            log("int8", L.name, res[L.name])
        # dw s2 -> pw fused: the int8 depthwise output stays on chip
        L1, L2 = wl.layers[1], wl.layers[2]
        d1 = cc.conv2d_desc_create(params_of(L1, "i8"))
        d2 = cc.conv2d_desc_create(params_of(L2, "i8"))
        w1, b1, w2, b2 = (t_(a[k]) for k in ("w_dw_s2", "b_dw_s2", "w_pw", "b_pw"))
        xq = t_(np.random.default_rng(5).integers(-128, 128, size=L1.x_shape).astype(np.int8))
        sc = workloads.INT8_SCALES

        def make_q():
            xi = xq.clone()
            yi = torch.empty((L2.n, L2.c_out, L2.h, L2.w), dtype=torch.int8, device=dev())
            return lambda: cc.qfused_dw_pw_forward(d1, d2, xi, w1, b1, sc, w2, b2, sc, 0, yi)

        fns = _rotating(make_q, L1.n * L1.c_in * L1.h * L1.w + L2.n * L2.c_out * L2.h * L2.w)
        t = time_layer("qfused_dw_pw", fns, reps)
        fb = (L1.n * L1.c_in * L1.h * L1.w + L1.c_out * 9 + 4 * L1.c_out + L2.c_out * L2.c_in + 4 * L2.c_out
              + L2.n * L2.c_out * L2.h * L2.w)
        res["qfused_dw_pw"] = dict(roofline_entry(L1.flops + L2.flops, fb, t, "i8"), kernel="qfused_dw_pw")
        log("int8", "qfused_dw_pw", res["qfused_dw_pw"])
        out["int8_chain"] = res

    # int8 inverted bottleneck: pw 32->192 and dw 3x3, unfused and fused
    if want("int8_bottleneck"):
        res = {}
        L1 = workloads.Layer("pw", 8, 32, 56, 56, 192, (1, 1), has_bias=True)
        L2 = workloads.Layer("dw", 8, 192, 56, 56, 192, (3, 3), pads=(1, 1, 1, 1), groups=192, has_bias=True)
        rng = np.random.default_rng(6)
        x = rng.integers(-128, 128, size=L1.x_shape).astype(np.int8)
        w1 = rng.integers(-127, 128, size=L1.w_shape).astype(np.int8)
        w2 = rng.integers(-127, 128, size=L2.w_shape).astype(np.int8)
        b1 = rng.integers(-500, 501, size=192).astype(np.int32)
        b2 = rng.integers(-500, 501, size=192).astype(np.int32)
        d1 = cc.conv2d_desc_create(params_of(L1, "i8"))
        d2 = cc.conv2d_desc_create(params_of(L2, "i8"))
        xq, w1d, w2d, b1d, b2d = t_(x), t_(w1), t_(w2), t_(b1), t_(b2)
        sc = workloads.INT8_SCALES
        e_host = rng.integers(-128, 128, size=L2.x_shape).astype(np.int8)
        eq = t_(e_host)
        for L, d, xs_, wd, bd in ((L1, d1, xq, w1d, b1d), (L2, d2, eq, w2d, b2d)):
            def make(d=d, xs_=xs_, wd=wd, bd=bd, L=L):
                xi = xs_.clone()
                yi = torch.empty((L.n, L.c_out, L.h, L.w), dtype=torch.int8, device=dev())
                return lambda: cc.qconv2d_forward(d, xi, 0.02, 0, wd, 0.01, 0, bd, 0.05, 0, yi)
            fns = _rotating(make, L.n * (L.c_in + L.c_out) * L.h * L.w)
            t = time_layer(L.name, fns, reps)
            res[L.name] = dict(roofline_entry(L.flops, layer_bytes(L, 1, extra=4 * L.c_out), t, "i8"),
                               kernel=cc.conv2d_desc_kernel_name(d))

        def make_f():
            xi = xq.clone()
            yi = torch.empty((L2.n, L2.c_out, L2.h, L2.w), dtype=torch.int8, device=dev())
            return lambda: cc.qfused_pw_dw_forward(d1, d2, xi, w1d, b1d, sc, w2d, b2d, sc, 0, yi)

        fns = _rotating(make_f, L1.n * (L1.c_in + L2.c_out) * L1.h * L1.w)
        t = time_layer("qfused_pw_dw", fns, reps)
        fb = (L1.n * L1.c_in * L1.h * L1.w + L1.c_out * L1.c_in + 4 * L1.c_out + L2.c_out * 9 + 4 * L2.c_out
              + L2.n * L2.c_out * L2.h * L2.w)
        res["qfused_pw_dw"] = dict(roofline_entry(L1.flops + L2.flops, fb, t, "i8"), kernel="qfused_pw_dw")
        log("int8_bottleneck", res)
        out["int8_bottleneck"] = res

    # int8 dense / strided / dilated / grouped convolutions on the i8 matrix cores (the mixed sweep's shapes)
    if want("int8_dense"):
        res = {}
        for L in workloads.mixed_sweep_layers():
            if L.name == "pw":
                continue
            Lq = workloads.Layer(L.name, L.n, L.c_in, L.h, L.w, L.c_out, L.k, stride=L.stride, pads=L.pads,
                                 dilation=L.dilation, groups=L.groups, has_bias=True)
            rng = np.random.default_rng(7)
            x = rng.integers(-128, 128, size=Lq.x_shape).astype(np.int8)
            w = rng.integers(-127, 128, size=Lq.w_shape).astype(np.int8)
            b = rng.integers(-500, 501, size=Lq.c_out).astype(np.int32)
            xs_, wd, bd = t_(x), t_(w), t_(b)
            ho, wo = Lq.out_hw
            # Weights bound at set-up (the timed figure): the 3x3 kernel's
            # weights are re-laid into its per-chunk LDS images once; passing
            # them on every call (a re-lay per call) is reported beside it.
            times = {}
            for bound in (True, False):
                d = cc.conv2d_desc_create(params_of(Lq, "i8"))
                if bound:
                    cc.conv2d_desc_bind_weights(d, wd)

                def make(d=d, xs_=xs_, wd=None if bound else wd, bd=bd, Lq=Lq, ho=ho, wo=wo):
                    xi = xs_.clone()
                    yi = torch.empty((Lq.n, Lq.c_out, ho, wo), dtype=torch.int8, device=dev())
                    return lambda: cc.qconv2d_forward(d, xi, 0.02, 0, wd, 0.01, 0, bd, 0.05, 0, yi)

                fns = _rotating(make, x.size + Lq.n * Lq.c_out * ho * wo)
                times[bound] = time_layer(Lq.name, fns, reps)
            t = times[True]
            res[Lq.name] = dict(roofline_entry(Lq.flops, layer_bytes(Lq, 1, extra=4 * Lq.c_out), t, "i8"),
                                kernel=cc.conv2d_desc_kernel_name(d), weights="bound",
                                us_weights_per_call=round(times[False], 3))
            log("int8_dense", Lq.name, res[Lq.name])
        out["int8_dense"] = res

    # dense-block layers, Winograd F(2x2,3x3) beside the implicit GEMM
    if want("winograd"):
        wl = workloads.dense_block()
        total = workloads.DENSE_TOTAL_CHANNELS
        h, w = wl.layers[0].h, wl.layers[0].w
        nb = max(1, min(64, -(-ROTATE_BYTES // (total * h * w * 4))))
        bufs = [torch.zeros((1, total, h, w), device=dev()) for _ in range(nb)]
        for b in bufs:
            b[:, :64] = t_(wl.arrays["x"])
        res = {}
        for k, L in enumerate(wl.layers):
            wd = t_(wl.arrays[f"w{k}"])
            entry = {}
            for algo, bound in (("direct", False), ("direct", True), ("winograd", False), ("winograd", True),
                                ("winograd4", True)):
                p = params_of(L, in_total_channels=total, out_total_channels=total, out_channel_offset=L.c_in)
                p.algo = cc.ALGOS[algo]
                d = cc.conv2d_desc_create(p)
                wuse = wd
                if bound:
                    cc.conv2d_desc_bind_weights(d, wd)
                    torch.cuda.synchronize()
                    wuse = None
                fns = [lambda d=d, b=b, wuse=wuse: cc.conv2d_forward(d, b, wuse, None, None, b) for b in bufs]
                key = algo + ("_bound" if bound else "")
                t = time_layer(f"{key}{k}", fns, reps)
                entry[key] = dict(roofline_entry(L.flops, 4 * (L.c_in * h * w + L.c_out * L.c_in * 9 + L.c_out * h * w),
                                                 t, "f32"), kernel=cc.conv2d_desc_kernel_name(d))
            # the MFMA work Winograd actually issues: 16 products per 2x2 tile and
            # channel pair, 36 per 4x4 tile for F(4x4)
            for key in ("winograd", "winograd_bound"):
                entry[key]["executed_flops"] = 2 * 16 * L.c_out * L.c_in * ((h + 1) // 2) * ((w + 1) // 2)
            entry["winograd4_bound"]["executed_flops"] = 2 * 36 * L.c_out * L.c_in * ((h + 3) // 4) * ((w + 3) // 4)
            res[L.name] = entry
            log("winograd", L.name, {a: e["us"] for a, e in entry.items()})
        out["dense_block_winograd"] = res
        # a batched 3x3 layer (8 x 128 x 64 x 64 -> 128), whose F(4x4) grid
        # fills the GPU: the shape where the larger tile pays
        L = workloads.Layer("batched_3x3", 8, 128, 64, 64, 128, (3, 3), pads=(1, 1, 1, 1))
        rng = np.random.default_rng(5)
        xs = t_(rng.standard_normal((L.n, L.c_in, L.h, L.w), dtype=np.float32))
        wd = t_((0.05 * rng.standard_normal((L.c_out, L.c_in, 3, 3))).astype(np.float32))
        bufs = _rotating(lambda: (xs.clone(), torch.empty((L.n, L.c_out, L.h, L.w), device=dev())),
                         4 * L.n * (L.c_in + L.c_out) * L.h * L.w)
        entry = {}
        for algo in ("direct", "winograd", "winograd4"):
            p = params_of(L)
            p.algo = cc.ALGOS[algo]
            d = cc.conv2d_desc_create(p)
            cc.conv2d_desc_bind_weights(d, wd)
            torch.cuda.synchronize()
            fns = [lambda d=d, x=x, y=y: cc.conv2d_forward(d, x, None, None, None, y) for x, y in bufs]
            t = time_layer(f"batched_{algo}", fns, reps)
            entry[algo + "_bound"] = dict(roofline_entry(L.flops, 4 * (L.n * L.c_in * L.h * L.w + L.c_out * L.c_in * 9
                                                                       + L.n * L.c_out * L.h * L.w), t, "f32"),
                                          kernel=cc.conv2d_desc_kernel_name(d))
        tiles2, tiles4 = L.n * (L.h // 2) * (L.w // 2), L.n * (L.h // 4) * (L.w // 4)
        entry["winograd_bound"]["executed_flops"] = 2 * 16 * L.c_out * L.c_in * tiles2
        entry["winograd4_bound"]["executed_flops"] = 2 * 36 * L.c_out * L.c_in * tiles4
        log("winograd", L.name, {a: e["us"] for a, e in entry.items()})
        out["batched_3x3_winograd"] = {L.name: entry}
    add_copy_context(out, reps)
    return out


def copy_us(nbytes, reps):
    """HIP-event time of the library's streaming 16-byte copy
    (conv2d_probe_copy) moving nbytes in all (half read, half written), cold:
    rotated over buffer sets like the layers, queued back to back the same
    way."""
    import convolution_conv2d_forward_amd as cc
    torch = torch_mod()
    n = max(4, nbytes // 8 // 4 * 4)      # float32 elements per side, whole 16-byte pieces
    sets = int(min(64, max(1, ROTATE_BYTES // max(1, 8 * n))))
    src = [torch.ones(n, device=dev()) for _ in range(sets)]
    dst = [torch.empty(n, device=dev()) for _ in range(sets)]
    fns = [lambda s=s_, d=d_: cc.conv2d_probe_copy(d, s) for s_, d_ in zip(src, dst)]
    t = time_layer("copy", fns, reps)
    del src, dst
    return t


def add_copy_context(out, reps):
    """Beside every HBM-bound entry: the time a plain device copy of the same
    bytes takes here, and the entry's speed as a fraction of it (what a copy
    of that size reaches on this machine, not the 8 TB/s peak)."""
    cache = {}
    for sec in out.values():
        for e in sec.values():
            if isinstance(e, dict) and e.get("bound") == "hbm" and e.get("bytes"):
                nb = e["bytes"]
                if nb not in cache:
                    cache[nb] = copy_us(nb, reps)
                e["copy_us"] = round(cache[nb], 3)
                e["copy_frac"] = round(cache[nb] / e["us"], 4)


def copy_probe(reps):
    """The library's streaming copy: one of known size (1 GiB each way, which
    calibrates the HBM byte counters) and a sweep over the byte counts of the
    HBM-bound layers (read + written, cold, back to back), as the attainable
    bandwidth at each size."""
    import convolution_conv2d_forward_amd as cc
    torch = torch_mod()
    n = 256 << 20   # 1 GiB of float32
    a = torch.ones(n, device=dev())
    b = torch.empty_like(a)
    for _ in range(3):
        cc.conv2d_probe_copy(b, a)
    torch.cuda.synchronize()
    timer = EventTimer()
    for _ in range(reps):
        timer.run("copy", lambda: cc.conv2d_probe_copy(b, a))
    t = timer.mean_us("copy")[0]
    out = {"bytes_read": 4 * n, "bytes_written": 4 * n, "us": t, "gbps": 8 * n / (t * 1e-6) / 1e9}
    del a, b
    sweep = {}
    for mb in (4, 8, 16, 22.5, 38.5, 64, 128, 256, 512):
        nb = int(mb * 1e6)
        tu = copy_us(nb, max(reps, 20))
        sweep[f"{mb}MB"] = {"us": round(tu, 3), "gbps": round(nb / (tu * 1e-6) / 1e9, 1)}
    out["sweep"] = sweep
    return out


# ------------------------------------------------------------ cpu baseline --

def cpu_baseline(target_s=6.0):
    """The oracle (as it stands) on the host cores.

    value: whole passes of the benchmark step (the five dense-block layers,
    each computed in full in float64 from the previous layers' float32
    outputs, the concat buffer assembled by plain concatenation), repeated
    until about target_s seconds have run.  per_config: every layer of the
    other workloads computed once in full (wall seconds and GFLOP/s each; the
    mixed sweep's fp32 inputs, whose float64 arithmetic is the same work as
    its bf16 one; the int8 chain in int64)."""
    import oracle
    import workloads
    layers = workloads.dense_block_layers()
    wl = workloads.dense_block()
    step_flops = sum(L.flops for L in layers)

    def one_pass():
        buf = wl.arrays["x"]
        for k, L in enumerate(layers):
            y = oracle.conv2d(buf, wl.arrays[f"w{k}"], None, pads=L.pads, act=L.act, alpha=L.alpha)
            buf = np.concatenate([buf, y.astype(np.float32)], axis=1)
        return buf

    passes = 0
    t0 = time.perf_counter()
    while True:
        one_pass()
        passes += 1
        s = time.perf_counter() - t0
        if s >= target_s:
            break
    f = passes * step_flops

    per = {}

    def timed(cfg, name, L, fn):
        t1 = time.perf_counter()
        fn()
        dt = time.perf_counter() - t1
        per.setdefault(cfg, {})[name] = {"seconds": round(dt, 4), "gflops": round(L.flops / dt / 1e9, 3),
                                         "gflop": round(L.flops / 1e9, 4)}

    sc = workloads.single_conv()
    L = sc.layers[0]
    timed("single_conv", "conv", L, lambda: oracle.conv2d(sc.arrays["x"], sc.arrays["w"], sc.arrays["b"],
                                                          pads=L.pads, act=L.act))
    bn = workloads.bottleneck()
    a = bn.arrays
    L1, L2, L3 = bn.layers
    e = oracle.conv2d(a["x"], a["w_pw1"], None, act=L1.act, clip=L1.clip)
    timed("bottleneck", "pw1", L1, lambda: oracle.conv2d(a["x"], a["w_pw1"], None, act=L1.act, clip=L1.clip))
    e = e.astype(np.float32)
    dwo = oracle.conv2d(e, a["w_dw"], None, pads=L2.pads, groups=L2.groups, act=L2.act, clip=L2.clip)
    timed("bottleneck", "dw", L2, lambda: oracle.conv2d(e, a["w_dw"], None, pads=L2.pads, groups=L2.groups,
                                                        act=L2.act, clip=L2.clip))
    dwo = dwo.astype(np.float32)
    timed("bottleneck", "pw2", L3, lambda: oracle.conv2d(dwo, a["w_pw2"], None))
    for L in workloads.mixed_sweep_layers():
        m = workloads.mixed_sweep(which={L.name}).arrays
        n_ = L.name
        timed("mixed_sweep", n_, L, lambda: oracle.conv2d(m[f"x_{n_}"], m[f"w_{n_}"], m[f"b_{n_}"], stride=L.stride,
                                                          pads=L.pads, dilation=L.dilation, groups=L.groups,
                                                          act=L.act, slope=m[f"s_{n_}"]))
    q = workloads.int8_chain()
    cur = q.arrays["x"]
    for L in q.layers:
        qa = q.arrays
        res = {}

        def run(L=L, cur=cur):
            res["y"] = oracle.qconv2d(cur, qa[f"w_{L.name}"], qa[f"b_{L.name}"], *workloads.INT8_SCALES,
                                      stride=L.stride, pads=L.pads, groups=L.groups)
        timed("int8_chain", L.name, L, run)
        cur = res["y"]
    total = sum(e["seconds"] for c in per.values() for e in c.values())
    return {"value": round(f / s / 1e9, 3), "unit": "GFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{passes} full pass(es) of the 5-layer dense-block chain "
                      f"({f / 1e9:.2f} GFLOP in {s:.1f} s, float64 direct loops, OpenMP over (n, c_out)); "
                      f"per_config: every layer of the other workloads once in full ({total:.1f} s)",
            "seconds": round(s, 2), "per_config": per}


# ------------------------------------------------------------------- main --

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(there is no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    torch = torch_mod()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import convolution_conv2d_forward_amd as cc   # noqa: F401  (fails loudly if the library is missing)

    if args.only == "copy":
        log(json.dumps(copy_probe(args.steps)))
        return
    if args.only not in ("all", "dense_block"):
        log(json.dumps(per_config(args.reps, args.only)))
        return

    db, wall, per = bench_dense_block(args.steps, args.warmup)
    step_flops = sum(db.flops)
    value = step_flops * args.steps / wall / 1e9
    dom, g, roof = dense_roofline(db, per)
    kname = lambda k: "igemm_f32_packed" if db.bound and db.kernels[k] == "igemm_f32" else db.kernels[k]
    layers = {L.name: dict(roofline_entry(db.flops[k], db.bytes[k], per[k][0], "f32"), kernel=kname(k))
              for k, L in enumerate(db.layers)}
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "dense_block_chain_fp32: 1x64x128x128 input in a 1x256x128x128 concat buffer; "
                               "5 conv3x3 s1 p1, Cin=64+32k, Cout=32 (last 64), LeakyReLU(0.2) except last, "
                               "ConcatFusedTail writes, no bias",
                   "gflop_per_step": round(step_flops / 1e9, 4), "buffer_sets": db.nsets,
                   "kernel_sum_us_per_step": round(sum(p[0] for p in per), 2)},
        "roofline": roof,
        "layers": layers,
    }
    line["config"]["weights"] = ("bound at set-up (AUTO: 3x3 layers of this size then run Winograd F(2x2,3x3) "
                                 "with U = G g G^T packed at bind; otherwise packed for the fp32 implicit GEMM)")
    # The same chain with the OIHW weights passed on every call.
    db2, wall2, per2 = bench_dense_block(args.steps, args.warmup, bound=False)
    line["config"]["weights_per_call"] = {
        "value": round(step_flops * args.steps / wall2 / 1e9, 1), "ms_per_step": round(wall2 / args.steps * 1e3, 4),
        "layers_us": {L.name: round(per2[k][0], 3) for k, L in enumerate(db2.layers)}}
    log("dense block, weights per call", line["config"]["weights_per_call"])
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
        log("cpu_baseline", line["cpu_baseline"])
    if not args.no_extra and args.only == "all":
        line["per_config"] = per_config(args.reps)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
