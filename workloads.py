"""Seeded synthetic workloads for the conv2d forward path.

This module only draws inputs and states layer attributes; it holds none of
the convolution arithmetic.  Both the HIP path (tests, benchmark) and the CPU
oracle consume what it returns.

Generator: numpy.random.Generator(PCG64(seed)), seed = the workload number
(1..5).  Draw order: the input first, then for each layer its weights, bias,
PReLU slopes.  Floating draws are float64, cast to float32 (bf16 copies are
made from those float32 values by the caller, round-to-nearest-even).  Integer
draws use Generator.integers with inclusive bounds as stated.

Workloads (the five synthetic configurations of the conv2d forward task):
  1 single_conv      1x16x32x32 -> 3x3 s1 p1 -> 32, bias, ReLU
  2 dense_block      1x64x128x128 in a 1x256x128x128 concat buffer; 5 convs
                     3x3 s1 p1, Cin = 64+32k, Cout = 32 (last 64), LeakyReLU
                     0.2 except the last, each writing the buffer's next
                     channel slice; no bias
  3 bottleneck       8x32x56x56 -> pw 32->192 Clip(0,6) -> dw 3x3 Clip(0,6)
                     -> pw 192->32 linear; no bias
  4 mixed_sweep      four independent N=32 layers, bias + per-channel PReLU
  5 int8_chain       16x144x80x80 int8 -> dw 3x3 s1 -> dw 3x3 s2 -> pw 144->48
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

ACT_NONE, ACT_RELU, ACT_LEAKY_RELU, ACT_PRELU, ACT_CLIP = 0, 1, 2, 3, 4
FLT_MAX = float(np.finfo(np.float32).max)


@dataclass
class Layer:
    """Attributes of one convolution (input shape [n, c_in, h, w], OIHW weights)."""
    name: str
    n: int
    c_in: int
    h: int
    w: int
    c_out: int
    k: Tuple[int, int]
    stride: Tuple[int, int] = (1, 1)
    pads: Tuple[int, int, int, int] = (0, 0, 0, 0)   # top, left, bottom, right
    dilation: Tuple[int, int] = (1, 1)
    groups: int = 1
    has_bias: bool = False
    act: int = ACT_NONE
    alpha: float = 0.01
    clip: Tuple[float, float] = (-FLT_MAX, FLT_MAX)
    pad_value: float = 0.0

    @property
    def w_shape(self):
        return (self.c_out, self.c_in // self.groups, self.k[0], self.k[1])

    @property
    def x_shape(self):
        return (self.n, self.c_in, self.h, self.w)

    @property
    def out_hw(self):
        kh, kw = self.k
        ho = (self.h + self.pads[0] + self.pads[2] - self.dilation[0] * (kh - 1) - 1) // self.stride[0] + 1
        wo = (self.w + self.pads[1] + self.pads[3] - self.dilation[1] * (kw - 1) - 1) // self.stride[1] + 1
        return ho, wo

    @property
    def flops(self) -> int:
        """2 * multiply-accumulates, padded taps included."""
        ho, wo = self.out_hw
        kh, kw = self.k
        return 2 * self.n * self.c_out * ho * wo * (self.c_in // self.groups) * kh * kw


@dataclass
class Workload:
    name: str
    seed: int
    layers: list
    arrays: dict = field(default_factory=dict)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _normal(rng, shape, var):
    return (rng.standard_normal(shape) * np.sqrt(var)).astype(np.float32)


def _uniform(rng, shape, lo, hi):
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def single_conv() -> Workload:
    L = Layer("conv", 1, 16, 32, 32, 32, (3, 3), pads=(1, 1, 1, 1), has_bias=True, act=ACT_RELU)
    rng = _rng(1)
    a = {"x": _uniform(rng, L.x_shape, -1.0, 1.0),
         "w": _normal(rng, L.w_shape, 1.0 / (16 * 9)),
         "b": _uniform(rng, (32,), -0.1, 0.1)}
    return Workload("single_conv", 1, [L], a)


DENSE_TOTAL_CHANNELS = 256


def dense_block_layers(h=128, w=128):
    layers = []
    for k in range(5):
        c_in = 64 + 32 * k
        c_out = 64 if k == 4 else 32
        act = ACT_NONE if k == 4 else ACT_LEAKY_RELU
        layers.append(Layer(f"conv{k}", 1, c_in, h, w, c_out, (3, 3), pads=(1, 1, 1, 1),
                            act=act, alpha=0.2))
    return layers


def dense_block(h=128, w=128) -> Workload:
    layers = dense_block_layers(h, w)
    rng = _rng(2)
    a = {"x": _uniform(rng, (1, 64, h, w), -1.0, 1.0)}
    for k, L in enumerate(layers):
        a[f"w{k}"] = _normal(rng, L.w_shape, 1.0 / (9 * L.c_in))
    return Workload("dense_block", 2, layers, a)


def bottleneck(n=8, h=56, w=56) -> Workload:
    clip6 = (0.0, 6.0)
    layers = [Layer("pw1", n, 32, h, w, 192, (1, 1), act=ACT_CLIP, clip=clip6),
              Layer("dw", n, 192, h, w, 192, (3, 3), pads=(1, 1, 1, 1), groups=192,
                    act=ACT_CLIP, clip=clip6),
              Layer("pw2", n, 192, h, w, 32, (1, 1))]
    rng = _rng(3)
    a = {"x": _normal(rng, (n, 32, h, w), 1.0),
         "w_pw1": _normal(rng, (192, 32, 1, 1), 1.0 / 32),
         "w_dw": _normal(rng, (192, 1, 3, 3), 1.0 / 9),
         "w_pw2": _normal(rng, (32, 192, 1, 1), 1.0 / 192)}
    return Workload("bottleneck", 3, layers, a)


def mixed_sweep_layers(n=32):
    return [Layer("s2", n, 128, 64, 64, 256, (3, 3), stride=(2, 2), pads=(1, 1, 1, 1),
                  has_bias=True, act=ACT_PRELU),
            Layer("d2", n, 128, 64, 64, 128, (3, 3), pads=(2, 2, 2, 2), dilation=(2, 2),
                  has_bias=True, act=ACT_PRELU),
            Layer("g32", n, 256, 32, 32, 256, (3, 3), pads=(1, 1, 1, 1), groups=32,
                  has_bias=True, act=ACT_PRELU),
            Layer("pw", n, 256, 32, 32, 512, (1, 1), has_bias=True, act=ACT_PRELU)]


def mixed_sweep(n=32, which=None) -> Workload:
    """Four independent layers; each gets its own input, weights, bias, slopes
    in that order.  `which` restricts generation to a subset of layer names
    (draws for the skipped layers are still made, so values do not depend on
    the subset)."""
    layers = mixed_sweep_layers(n)
    rng = _rng(4)
    a = {}
    for L in layers:
        keep = which is None or L.name in which
        fan_in = (L.c_in // L.groups) * L.k[0] * L.k[1]
        x = _normal(rng, L.x_shape, 1.0)
        w = _normal(rng, L.w_shape, 1.0 / fan_in)
        b = _uniform(rng, (L.c_out,), -0.1, 0.1)
        s = _uniform(rng, (L.c_out,), 0.0, 0.3)
        if keep:
            a[f"x_{L.name}"], a[f"w_{L.name}"], a[f"b_{L.name}"], a[f"s_{L.name}"] = x, w, b, s
    return Workload("mixed_sweep", 4, layers, a)


INT8_SCALES = (0.02, 0.01, 0.05)   # x, w, y; zero points 0


def int8_chain_layers(n=16, h=80, w=80):
    return [Layer("dw_s1", n, 144, h, w, 144, (3, 3), pads=(1, 1, 1, 1), groups=144, has_bias=True),
            Layer("dw_s2", n, 144, h, w, 144, (3, 3), stride=(2, 2), pads=(1, 1, 1, 1), groups=144,
                  has_bias=True),
            Layer("pw", n, 144, (h + 1) // 2, (w + 1) // 2, 48, (1, 1), has_bias=True)]


def int8_chain(n=16, h=80, w=80, w_range=127) -> Workload:
    layers = int8_chain_layers(n, h, w)
    rng = _rng(5)
    a = {"x": rng.integers(-128, 127, size=(n, 144, h, w), endpoint=True).astype(np.int8)}
    for L in layers:
        a[f"w_{L.name}"] = rng.integers(-w_range, w_range, size=L.w_shape, endpoint=True).astype(np.int8)
        a[f"b_{L.name}"] = rng.integers(-500, 500, size=(L.c_out,), endpoint=True).astype(np.int32)
    return Workload("int8_chain", 5, layers, a)


def random_layer(rng, *, max_c=12, max_hw=23, dtype="f32") -> Tuple[Layer, Optional[dict]]:
    """A random small layer for parity sweeps (shape and attributes only)."""
    groups = int(rng.choice([1, 1, 1, 2, 4]))
    cig = int(rng.integers(1, max(2, max_c // groups)))
    cog = int(rng.integers(1, max(2, max_c // groups)))
    kh, kw = int(rng.choice([1, 2, 3, 5])), int(rng.choice([1, 3, 4]))
    sh, sw = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    dh, dw = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    pads = tuple(int(v) for v in rng.integers(0, 3, size=4))
    h = int(rng.integers(max(1, dh * (kh - 1) + 1 - pads[0] - pads[2]), max_hw))
    w = int(rng.integers(max(1, dw * (kw - 1) + 1 - pads[1] - pads[3]), max_hw))
    n = int(rng.integers(1, 4))
    act = int(rng.integers(0, 5))
    L = Layer("rand", n, cig * groups, h, w, cog * groups, (kh, kw), stride=(sh, sw), pads=pads,
              dilation=(dh, dw), groups=groups, has_bias=bool(rng.random() < 0.6), act=act,
              alpha=float(np.float32(rng.uniform(0.01, 0.3))),
              clip=(float(np.float32(-rng.uniform(0, 1))), float(np.float32(rng.uniform(0.2, 2)))),
              pad_value=float(rng.choice([0.0, 0.0, -0.5, 1.25])))
    return L


def layer_arrays(rng, L: Layer, *, x_dist="normal"):
    """Seeded x, w, bias, slope for a layer (float32)."""
    fan_in = (L.c_in // L.groups) * L.k[0] * L.k[1]
    x = _normal(rng, L.x_shape, 1.0) if x_dist == "normal" else _uniform(rng, L.x_shape, -1, 1)
    w = _normal(rng, L.w_shape, 1.0 / fan_in)
    b = _uniform(rng, (L.c_out,), -0.1, 0.1) if L.has_bias else None
    s = _uniform(rng, (L.c_out if rng.random() < 0.7 else 1,), 0.0, 0.3)
    return x, w, b, s
