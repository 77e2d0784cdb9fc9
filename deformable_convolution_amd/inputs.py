"""Seeded synthetic inputs for the 1D deformable convolution forward.

This module only draws random tensors of the right shapes; it holds none of
the method's arithmetic (it does not even compute the output length: every
workload states its own ``L_out``).  Tests, the bench and the smoke check
draw here and hand the same tensors to the GPU path and to the oracle.

Recipe (one CPU ``torch.Generator`` seeded per call; draws always in the
order x, offsets, mask, weight, bias; every draw in float32, then cast to
the storage dtype, so both sides read the same stored values):

* ``("uniform", a, b)``  -> a + (b - a) * U[0, 1)
* ``("normal", mu, var)`` -> mu + sqrt(var) * N(0, 1)   (second number is
  the variance)
* mask ``("sigmoid_normal", mu, var)`` -> sigmoid of such a normal draw
* bias ``"zeros"`` -> a zero tensor that is still passed; ``None`` -> no bias

The named workloads are the layer shapes the dc1d page uses (its
DeformConv1d usage example: B16, C512, K16, dilation 3, "valid", L128) and
four further synthetic shapes that cover a tiny case, a long bf16 sequence,
the depthwise offsets the DTCN paper uses, and a strided modulated layer.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import torch

Dist = Tuple  # ("uniform", a, b) | ("normal", mu, var) | ("sigmoid_normal", mu, var)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    C_in: int
    C_out: int
    L_in: int
    K: int
    stride: int
    padding: int
    dilation: int
    groups: int
    G: int  # offset groups
    L_out: int
    dtype: str  # "f32" | "bf16"
    x_dist: Dist
    off_dist: Dist
    mask_dist: Optional[Dist]
    w_var: float
    bias: Optional[str]  # "normal" (N(0, 0.1)), "zeros", or None

    def with_batch(self, B: int) -> "Workload":
        return dataclasses.replace(self, B=B, name="%s[B=%d]" % (self.name, B))


WORKLOADS = {
    "tiny": Workload("tiny", 1, 4, 4, 32, 3, 1, 0, 1, 1, 1, 30, "f32",
                     ("uniform", 0.0, 1.0), ("uniform", -2.0, 2.0), None, 1.0 / 12, "normal"),
    "dc1d_layer": Workload("dc1d_layer", 16, 512, 512, 128, 16, 1, 0, 3, 1, 1, 83, "f32",
                           ("uniform", 0.0, 1.0), ("normal", 0.0, 1.0), None, 1.0 / 8192, "normal"),
    "long_seq_bf16": Workload("long_seq_bf16", 8, 256, 256, 16384, 3, 1, 1, 1, 1, 4, 16384, "bf16",
                              ("normal", 0.0, 1.0), ("normal", 0.0, 2.0), None, 1.0 / 768, "zeros"),
    "depthwise": Workload("depthwise", 16, 512, 512, 4096, 5, 1, 2, 2, 512, 512, 4092, "f32",
                          ("normal", 0.0, 1.0), ("uniform", -4.0, 4.0), None, 1.0 / 5, "normal"),
    "dcnv2_bf16": Workload("dcnv2_bf16", 32, 1024, 1024, 2048, 3, 2, 1, 1, 1, 8, 1024, "bf16",
                           ("normal", 0.0, 1.0), ("normal", 0.0, 1.5), ("sigmoid_normal", 0.0, 1.0),
                           1.0 / 3072, "normal"),
}
# The order the five workloads are listed in everywhere (1..5).
WORKLOAD_ORDER = ["tiny", "dc1d_layer", "long_seq_bf16", "depthwise", "dcnv2_bf16"]


def _draw(gen, shape, dist):
    kind = dist[0]
    if kind == "uniform":
        a, b = dist[1], dist[2]
        return torch.rand(shape, generator=gen, dtype=torch.float32) * (b - a) + a
    if kind == "normal":
        mu, var = dist[1], dist[2]
        return torch.randn(shape, generator=gen, dtype=torch.float32) * math.sqrt(var) + mu
    if kind == "sigmoid_normal":
        mu, var = dist[1], dist[2]
        return torch.sigmoid(torch.randn(shape, generator=gen, dtype=torch.float32) * math.sqrt(var) + mu)
    raise ValueError("unknown distribution %r" % (dist,))


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_inputs(w: Workload, seed: int = 0) -> dict:
    """CPU tensors x, offsets, mask (or None), weight, bias (or None)."""
    gen = torch.Generator().manual_seed(seed)
    dt = torch_dtype(w.dtype)
    x = _draw(gen, (w.B, w.C_in, w.L_in), w.x_dist)
    offsets = _draw(gen, (w.B, w.G, w.L_out, w.K), w.off_dist)
    mask = _draw(gen, (w.B, w.G, w.L_out, w.K), w.mask_dist) if w.mask_dist is not None else None
    weight = torch.randn((w.C_out, w.C_in // w.groups, w.K), generator=gen, dtype=torch.float32) * math.sqrt(w.w_var)
    if w.bias == "normal":
        bias = torch.randn((w.C_out,), generator=gen, dtype=torch.float32) * math.sqrt(0.1)
    elif w.bias == "zeros":
        bias = torch.zeros((w.C_out,), dtype=torch.float32)
    else:
        bias = None
    cast = lambda t: None if t is None else t.to(dt).contiguous()
    return {"x": cast(x), "offsets": cast(offsets), "mask": cast(mask),
            "weight": cast(weight), "bias": cast(bias)}


def custom(name="custom", *, B, C_in, C_out, L_in, K, stride=1, padding=0, dilation=1, groups=1, G=1,
           L_out, dtype="f32", x_dist=("normal", 0.0, 1.0), off_dist=("normal", 0.0, 1.0),
           mask_dist=None, w_var=None, bias="normal") -> Workload:
    """A workload of arbitrary shape (L_out must be supplied by the caller)."""
    if w_var is None:
        w_var = 1.0 / max(1, (C_in // groups) * K)
    return Workload(name, B, C_in, C_out, L_in, K, stride, padding, dilation, groups, G, L_out, dtype,
                    x_dist, off_dist, mask_dist, w_var, bias)


@dataclasses.dataclass(frozen=True)
class PackedWorkload:
    """The packed layer (offsets, and optionally the mask, generated from x by
    a depthwise trunk and pointwise heads); fp32 storage."""
    name: str
    B: int
    C_in: int
    C_out: int
    L_in: int
    K: int
    stride: int
    padding: int
    dilation: int
    groups: int
    G: int
    L_out: int
    modulated: bool
    off_var: float = 4.0  # offset head weight variance times C_in: offsets of a few positions

    def with_batch(self, B: int) -> "PackedWorkload":
        return dataclasses.replace(self, B=B, name="%s[B=%d]" % (self.name, B))


# The dc1d page's PackedDeformConv1d usage example (C 64, K 3, dilation 4,
# groups 64, offset groups 64, "same"; input [4, 64, 256]), its modulated
# variant, and the same layer on a longer, larger batch for measurement.
PACKED_WORKLOADS = {
    "packed_page": PackedWorkload("packed_page", 4, 64, 64, 256, 3, 1, 4, 4, 64, 64, 256, False),
    "packed_page_modulated": PackedWorkload("packed_page_modulated", 4, 64, 64, 256, 3, 1, 4, 4, 64, 64, 256, True),
    "packed": PackedWorkload("packed", 32, 64, 64, 8192, 3, 1, 4, 4, 64, 64, 8192, True),
}


def make_packed_inputs(w: PackedWorkload, seed: int = 0) -> dict:
    """CPU float32 tensors for the packed layer, drawn in the order x,
    trunk_weight, trunk_bias, off_weight, off_bias, mask_weight, mask_bias
    (both None unless modulated), weight, bias:
    x ~ N(0, 1); trunk_weight ~ N(0, 1/K); off_weight ~ N(0, off_var/C_in);
    mask_weight ~ N(0, 1/C_in); weight ~ N(0, 1/((C_in/groups)*K)); every
    bias ~ N(0, 0.1)."""
    gen = torch.Generator().manual_seed(seed)
    n = lambda shape, var: torch.randn(shape, generator=gen, dtype=torch.float32) * math.sqrt(var)
    GK = w.G * w.K
    t = {"x": n((w.B, w.C_in, w.L_in), 1.0),
         "trunk_weight": n((w.C_in, 1, w.K), 1.0 / w.K),
         "trunk_bias": n((w.C_in,), 0.1),
         "off_weight": n((GK, w.C_in, 1), w.off_var / w.C_in),
         "off_bias": n((GK,), 0.1)}
    t["mask_weight"] = n((GK, w.C_in, 1), 1.0 / w.C_in) if w.modulated else None
    t["mask_bias"] = n((GK,), 0.1) if w.modulated else None
    t["weight"] = n((w.C_out, w.C_in // w.groups, w.K), 1.0 / ((w.C_in // w.groups) * w.K))
    t["bias"] = n((w.C_out,), 0.1)
    return t


def packed_custom(name="packed_custom", *, B, C_in, C_out, L_in, K, stride=1, padding=0, dilation=1, groups=1,
                  G=1, L_out, modulated=False, off_var=4.0) -> PackedWorkload:
    """A packed-layer workload of arbitrary shape (L_out supplied by the caller)."""
    return PackedWorkload(name, B, C_in, C_out, L_in, K, stride, padding, dilation, groups, G, L_out, modulated,
                          off_var)


@dataclasses.dataclass(frozen=True)
class Workload2D:
    """2D modulated deformable convolution (offsets in torchvision's layout)."""
    name: str
    B: int
    C_in: int
    C_out: int
    H: int
    W: int
    kh: int
    kw: int
    stride: Tuple[int, int]
    padding: Tuple[int, int]
    dilation: Tuple[int, int]
    groups: int
    G: int
    Ho: int
    Wo: int
    dtype: str
    modulated: bool
    off_var: float = 1.0

    def with_batch(self, B: int) -> "Workload2D":
        return dataclasses.replace(self, B=B, name="%s[B=%d]" % (self.name, B))


# The deformable convolution article's torchvision example (input
# [1, 64, 28, 28], a 3x3 deformable conv 64 -> 128 with padding 1, offsets
# from a plain conv), modulated here, and a DCNv2 layer of a detection
# backbone's size for measurement, in fp32 and bf16.
WORKLOADS_2D = {
    "dcn2d_article": Workload2D("dcn2d_article", 1, 64, 128, 28, 28, 3, 3, (1, 1), (1, 1), (1, 1), 1, 1, 28, 28,
                                "f32", True),
    "dcn2d": Workload2D("dcn2d", 8, 256, 256, 64, 64, 3, 3, (1, 1), (1, 1), (1, 1), 1, 1, 64, 64, "f32", True),
    "dcn2d_bf16": Workload2D("dcn2d_bf16", 8, 256, 256, 64, 64, 3, 3, (1, 1), (1, 1), (1, 1), 1, 1, 64, 64, "bf16",
                             True),
}


def make_inputs2d(w: Workload2D, seed: int = 0) -> dict:
    """CPU tensors x, offsets, mask (or None), weight, bias, drawn in that
    order in float32 and cast to the storage dtype: x ~ N(0, 1); offsets ~
    N(0, off_var) (row and column alike); mask ~ sigmoid(N(0, 1)); weight ~
    N(0, 1/((C_in/groups)*kh*kw)); bias ~ N(0, 0.1)."""
    gen = torch.Generator().manual_seed(seed)
    dt = torch_dtype(w.dtype)
    T = w.kh * w.kw
    n = lambda shape, var: torch.randn(shape, generator=gen, dtype=torch.float32) * math.sqrt(var)
    x = n((w.B, w.C_in, w.H, w.W), 1.0)
    off = n((w.B, 2 * w.G * T, w.Ho, w.Wo), w.off_var)
    mask = torch.sigmoid(n((w.B, w.G * T, w.Ho, w.Wo), 1.0)) if w.modulated else None
    weight = n((w.C_out, w.C_in // w.groups, w.kh, w.kw), 1.0 / ((w.C_in // w.groups) * T))
    bias = n((w.C_out,), 0.1)
    cast = lambda t: None if t is None else t.to(dt).contiguous()
    return {"x": cast(x), "offsets": cast(off), "mask": cast(mask), "weight": cast(weight), "bias": cast(bias)}


def custom2d(name="custom2d", *, B, C_in, C_out, H, W, kh, kw, stride=(1, 1), padding=(0, 0), dilation=(1, 1),
             groups=1, G=1, Ho, Wo, dtype="f32", modulated=False, off_var=1.0) -> Workload2D:
    """A 2D workload of arbitrary shape (Ho, Wo supplied by the caller)."""
    return Workload2D(name, B, C_in, C_out, H, W, kh, kw, tuple(stride), tuple(padding), tuple(dilation), groups, G,
                      Ho, Wo, dtype, modulated, off_var)
