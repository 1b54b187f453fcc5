"""Seeded synthetic inputs for the modulated deformable convolution forward.

This module holds no arithmetic of the operator itself: it only draws random
tensors of the shapes and value distributions of the workloads below, so that
the GPU path and the CPU oracle can be fed the very same bytes.

Every tensor is drawn in float32 from one CPU ``torch.Generator`` seeded with
``seed``, in the fixed order x, offset, mask, [mask zero draw], weight,
[bias], then rounded to the requested dtype (round-to-nearest-even).

Distributions (standard deviation for "normal"):
  x       N(0, 1)
  offset  N(0, sigma) pixels, or U(-a, a) pixels
  mask    sigmoid(N(0, 1)), or U(0, 1) with a fraction set to exactly 0
  weight  Kaiming normal: N(0, sqrt(2 / ((C/group) * kh * kw)))
  bias    N(0, 0.1)

Tensor layouts are NCHW, as the plugin guide's input table gives them
(page "TensorRT 插件解析：modulatedDeformConvPlugin 可变形卷积插件的原理、参数与使用指南", §二):
  x [N, C, H, W], offset [N, 2*dg*kh*kw, Ho, Wo], mask [N, dg*kh*kw, Ho, Wo],
  weight [Co, C/group, kh, kw], bias [Co].
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Problem:
    """Shapes, attributes and input distributions of one forward call."""
    N: int
    C: int
    Co: int
    H: int
    W: int
    kh: int = 3
    kw: int = 3
    stride: Tuple[int, int] = (1, 1)
    padding: Tuple[int, int] = (1, 1)
    dilation: Tuple[int, int] = (1, 1)
    groups: int = 1
    deformable_groups: int = 1
    bias: bool = True
    offset_dist: Tuple = ("normal", 1.0)      # ("normal", sigma) or ("uniform", a)
    mask_dist: Tuple = ("sigmoid_normal",)    # or ("uniform_zeros", p_zero)
    Ho: Optional[int] = None                  # default: the usual conv formula
    Wo: Optional[int] = None

    def out_hw(self) -> Tuple[int, int]:
        def conv_len(n, k, s, p, d):
            return (n + 2 * p - d * (k - 1) - 1) // s + 1
        ho = self.Ho if self.Ho is not None else conv_len(
            self.H, self.kh, self.stride[0], self.padding[0], self.dilation[0])
        wo = self.Wo if self.Wo is not None else conv_len(
            self.W, self.kw, self.stride[1], self.padding[1], self.dilation[1])
        return ho, wo

    def shapes(self):
        ho, wo = self.out_hw()
        kk = self.kh * self.kw
        return {
            "x": (self.N, self.C, self.H, self.W),
            "offset": (self.N, 2 * self.deformable_groups * kk, ho, wo),
            "mask": (self.N, self.deformable_groups * kk, ho, wo),
            "weight": (self.Co, self.C // self.groups, self.kh, self.kw),
            "bias": (self.Co,) if self.bias else None,
            "out": (self.N, self.Co, ho, wo),
        }

    def flops(self) -> int:
        """Effective flops of one call: 2*N*Co*(C/group)*kh*kw*Ho*Wo."""
        ho, wo = self.out_hw()
        return 2 * self.N * self.Co * (self.C // self.groups) * self.kh * self.kw * ho * wo

    def attrs(self):
        return dict(stride=self.stride, padding=self.padding, dilation=self.dilation,
                    groups=self.groups, deformable_groups=self.deformable_groups)


def generate(problem: Problem, dtype: str = "f32", seed: int = 0):
    """Draw the inputs of ``problem`` on the CPU; returns a dict of tensors."""
    g = torch.Generator().manual_seed(seed)
    s = problem.shapes()
    x = torch.randn(s["x"], generator=g)
    kind = problem.offset_dist[0]
    if kind == "normal":
        offset = torch.randn(s["offset"], generator=g) * problem.offset_dist[1]
    elif kind == "uniform":
        a = problem.offset_dist[1]
        offset = (torch.rand(s["offset"], generator=g) * 2.0 - 1.0) * a
    else:
        raise ValueError(kind)
    kind = problem.mask_dist[0]
    if kind == "sigmoid_normal":
        mask = torch.sigmoid(torch.randn(s["mask"], generator=g))
    elif kind == "uniform_zeros":
        mask = torch.rand(s["mask"], generator=g)
        zero = torch.rand(s["mask"], generator=g) < problem.mask_dist[1]
        mask = torch.where(zero, torch.zeros_like(mask), mask)
    elif kind == "ones":
        mask = torch.ones(s["mask"])
    else:
        raise ValueError(kind)
    fan_in = (problem.C // problem.groups) * problem.kh * problem.kw
    weight = torch.randn(s["weight"], generator=g) * math.sqrt(2.0 / fan_in)
    bias = torch.randn(s["bias"], generator=g) * 0.1 if problem.bias else None
    t = DTYPES[dtype]
    out = {"x": x, "offset": offset, "mask": mask, "weight": weight, "bias": bias}
    return {k: (v.to(t).contiguous() if v is not None else None) for k, v in out.items()}


GRID = (0.0, 0.25, 0.5, 1.0, 1.5, 2.0, 3.0, -0.25, -0.5, -1.0, -1.5, -2.0, -3.0)


def generate_grid(problem: Problem, dtype: str = "f32", seed: int = 0):
    """Inputs on coarse dyadic grids, for checks that need every rounding of
    the reduced-precision path to be an exact operation: x and the weight
    (times 2^-5) and bias (times 2^-3) drawn uniformly from GRID, integer
    offsets in [-2, 2], masks from {0, 0.5, 1}.  Every such value is exact in
    fp32, fp16, bf16 and the 8-bit E4M3 format."""
    g = torch.Generator().manual_seed(seed)
    s = problem.shapes()
    grid = torch.tensor(GRID)

    def pick(shape, values):
        return values[torch.randint(0, len(values), shape, generator=g)]

    x = pick(s["x"], grid)
    offset = torch.randint(-2, 3, s["offset"], generator=g).to(torch.float32)
    mask = pick(s["mask"], torch.tensor([0.0, 0.5, 1.0]))
    weight = pick(s["weight"], grid) * 2.0 ** -5
    bias = pick(s["bias"], grid) * 2.0 ** -3 if problem.bias else None
    t = DTYPES[dtype]
    out = {"x": x, "offset": offset, "mask": mask, "weight": weight, "bias": bias}
    return {k: (v.to(t).contiguous() if v is not None else None) for k, v in out.items()}


# The five benchmark workloads (synthetic stand-ins for OCDNet-style stages).
TINY = Problem(N=1, C=4, Co=4, H=8, W=8, bias=True, offset_dist=("normal", 1.0))
OCDNET_STAGE = Problem(N=4, C=256, Co=256, H=160, W=160, bias=False,
                       offset_dist=("normal", 2.0))
STRIDED_GROUPED = Problem(N=2, C=128, Co=256, H=128, W=128, stride=(2, 2), padding=(2, 2),
                          dilation=(2, 2), groups=2, deformable_groups=4, bias=True,
                          offset_dist=("normal", 3.0))
DEEP_STAGE = Problem(N=16, C=512, Co=512, H=40, W=40, bias=True,
                     offset_dist=("normal", 1.5))
DEPTHWISE = Problem(N=8, C=256, Co=256, H=96, W=96, groups=256, bias=True,
                    offset_dist=("uniform", 48.0), mask_dist=("uniform_zeros", 0.1))

WORKLOADS = {
    "tiny_n1_c4_8x8": (TINY, ("f32",)),
    "ocdnet_n4_c256_160x160": (OCDNET_STAGE, ("f32", "f16")),
    "strided_grouped_n2_c128_co256_128x128": (STRIDED_GROUPED, ("bf16",)),
    "deep_n16_c512_40x40": (DEEP_STAGE, ("f16",)),
    "depthwise_n8_c256_96x96": (DEPTHWISE, ("f32",)),
}
