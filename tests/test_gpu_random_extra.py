"""GPU parity on seeded random problems for the backward pass and the FP8
path (the forward's paths have their own random-problem test).

Problems are drawn from a fixed seed like test_gpu_random_shapes.py (groups
and offset groups that divide the channels, kernel sizes 1..5 with 3x3
weighted up, strides, paddings and dilations, output grids from the formula
or smaller, small or large offsets, masks with exact zeros), smaller here
because the backward oracle is sequential.  Tolerances: the backward's
(test_gpu_backward.py) and the FP8 path's random-input rule
(test_gpu_fp8.py).
"""
import numpy as np
import pytest
import torch

from helpers import ensure_built, within_tolerance

ensure_built()
from modulated_deformable_convolution_amd import mdcn, workloads  # noqa: E402
from modulated_deformable_convolution_amd.workloads import Problem  # noqa: E402
from oracle import oracle  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
ROUNDING = {"f32": 0.0, "f16": 2.0 ** -10, "bf16": 2.0 ** -7}


def _divisors(n):
    return [d for d in range(1, n + 1) if n % d == 0]


def random_problem(rng, max_macs):
    for _ in range(1000):
        groups = int(rng.choice([1, 1, 2, 3]))
        cg = int(rng.choice([1, 4, 8, 16, 24, 32]))
        C = groups * cg
        Co = groups * int(rng.choice([1, 5, 16, 32, 40]))
        dg = int(rng.choice(_divisors(C)[:5]))
        if rng.random() < 0.7:
            kh = kw = 3
        else:
            kh, kw = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        pr = Problem(N=int(rng.integers(1, 3)), C=C, Co=Co, H=int(rng.integers(5, 20)),
                     W=int(rng.integers(5, 20)), kh=kh, kw=kw,
                     stride=(int(rng.choice([1, 1, 2])), int(rng.choice([1, 2]))),
                     padding=(int(rng.integers(0, 3)), int(rng.integers(0, 3))),
                     dilation=(int(rng.choice([1, 1, 2])), int(rng.choice([1, 2]))),
                     groups=groups, deformable_groups=dg, bias=bool(rng.random() < 0.7),
                     offset_dist=(("normal", float(rng.choice([0.5, 1.5, 3.0])))
                                  if rng.random() < 0.8 else ("uniform", 15.0)),
                     mask_dist=(("uniform_zeros", 0.1) if rng.random() < 0.3
                                else ("sigmoid_normal",)))
        ho, wo = pr.out_hw()
        if ho < 1 or wo < 1:
            continue
        if rng.random() < 0.2:
            pr = Problem(**{**pr.__dict__, "Ho": max(1, ho - 2), "Wo": max(1, wo - 1)})
        macs = pr.N * pr.Co * np.prod(pr.out_hw()) * cg * kh * kw
        if macs <= max_macs:
            return pr
    raise RuntimeError("no problem drawn")


def _cases(seed, count, max_macs):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        pr = random_problem(rng, max_macs)
        dtype = str(rng.choice(["f32", "f16", "bf16"]))
        out.append(pytest.param(pr, dtype, id=f"p{i}-{dtype}"))
    return out


@pytest.mark.parametrize("pr,dtype", _cases(4242, 40, 3e6))
def test_random_backward(pr, dtype):
    inp = workloads.generate(pr, dtype, seed=5)
    ho, wo = pr.out_hw()
    go = torch.randn((pr.N, pr.Co, ho, wo), generator=torch.Generator().manual_seed(6))
    go = go.to(workloads.DTYPES[dtype])
    print("random backward", pr, dtype, flush=True)
    ref = oracle.backward(inp["x"], inp["offset"], inp["mask"], inp["weight"], go,
                          with_bias=pr.bias, **pr.attrs())
    g = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    op = mdcn.mdcn_create(pr.stride, pr.padding, pr.dilation, pr.groups, pr.deformable_groups)
    out = mdcn.backward(op, g["x"], g["offset"], g["mask"], g["weight"], go.to(DEV),
                        with_bias=pr.bias)
    torch.cuda.synchronize()
    for k in ("x", "offset", "mask", "weight") + (("bias",) if pr.bias else ()):
        got = out[k].cpu().double().numpy()
        r = ref[k]
        rms = float(np.sqrt(np.mean(r ** 2))) if r.size else 0.0
        bound = 1e-4 * np.maximum(np.abs(r), rms) + ROUNDING[dtype] * np.abs(r)
        if dtype == "f16":
            bound = bound + 2.0 ** -24
        err = np.abs(got - r)
        assert (err <= bound).all(), (k, dtype, float(err.max()))


@pytest.mark.parametrize("pr,dtype", _cases(4343, 40, 2e7))
def test_random_fp8(pr, dtype):
    inp = workloads.generate(pr, dtype, seed=7)
    print("random fp8", pr, dtype, flush=True)
    ref, asum = oracle.forward_fp8(inp["x"], inp["offset"], inp["mask"], inp["weight"],
                                   inp["bias"], **pr.attrs())
    g = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    op = mdcn.mdcn_create(pr.stride, pr.padding, pr.dilation, pr.groups, pr.deformable_groups,
                          path=mdcn.MDCN_PATH_GATHER_GEMM_FP8)
    got = mdcn.forward(op, g["x"], g["offset"], g["mask"], g["weight"], g["bias"])
    torch.cuda.synchronize()
    got = got.cpu().double().numpy()
    _, err, bound = within_tolerance(got, ref, dtype)
    assert (err <= bound + 2.0 ** -11 * asum).all(), (dtype, float((err / (bound + 2.0 ** -11 * asum)).max()))
