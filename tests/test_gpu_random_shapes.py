"""GPU parity on seeded random problems: every path a problem is eligible
for, against the oracle, over the whole output.

The problems are drawn from a fixed seed (so every run checks the same
cases): channel counts that hit and miss the vector widths and the fused /
windowed eligibility rules, groups and deformable groups that divide them,
kernel sizes 1..5 (3x3 weighted up, so the specialised 3x3 kernels are hit
often), strides, paddings and dilations 1..3, output grids from the conv
formula or smaller, offsets small (mostly inside the window margin) or large
(through the fallbacks and off the image), masks with exact zeros.
Tolerances are those of helpers.within_tolerance.
"""
import numpy as np
import pytest
import torch

from helpers import ensure_built, error_report, within_tolerance

ensure_built()
from modulated_deformable_convolution_amd import mdcn, workloads  # noqa: E402
from modulated_deformable_convolution_amd.workloads import Problem  # noqa: E402
from oracle import oracle  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
PATHS = {mdcn.MDCN_PATH_GATHER_GEMM: "gather_gemm", mdcn.MDCN_PATH_DEPTHWISE: "depthwise",
         mdcn.MDCN_PATH_FUSED: "fused", mdcn.MDCN_PATH_WINDOW: "window",
         mdcn.MDCN_PATH_DIRECT: "direct"}


def _divisors(n):
    return [d for d in range(1, n + 1) if n % d == 0]


def random_problem(rng):
    """One problem; sizes small enough that the oracle takes well under a
    second."""
    for _ in range(1000):
        groups = int(rng.choice([1, 1, 1, 2, 3, 4]))
        cg = int(rng.choice([1, 4, 6, 8, 16, 16, 32, 32, 64]))
        C = groups * cg
        mg = int(rng.choice([1, 5, 16, 32, 48, 96, 160]))
        Co = groups * mg
        dg = int(rng.choice(_divisors(C)[:6]))
        if rng.random() < 0.7:
            kh = kw = 3
        else:
            kh, kw = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        sh, sw = int(rng.choice([1, 1, 2, 3])), int(rng.choice([1, 1, 2]))
        dh, dw = int(rng.choice([1, 1, 2, 3])), int(rng.choice([1, 1, 2]))
        ph, pw = int(rng.integers(0, 3)), int(rng.integers(0, 3))
        H, W = int(rng.integers(5, 30)), int(rng.integers(5, 30))
        N = int(rng.integers(1, 4))
        pr = Problem(N=N, C=C, Co=Co, H=H, W=W, kh=kh, kw=kw, stride=(sh, sw),
                     padding=(ph, pw), dilation=(dh, dw), groups=groups,
                     deformable_groups=dg, bias=bool(rng.random() < 0.7),
                     offset_dist=(("normal", float(rng.choice([0.5, 1.5, 3.0])))
                                  if rng.random() < 0.8 else ("uniform", 20.0)),
                     mask_dist=(("uniform_zeros", 0.1) if rng.random() < 0.3
                                else ("sigmoid_normal",)))
        ho, wo = pr.out_hw()
        if ho < 1 or wo < 1:
            continue
        if rng.random() < 0.2:       # an output grid smaller than the formula
            pr = Problem(**{**pr.__dict__, "Ho": max(1, ho - 2), "Wo": max(1, wo - 1)})
        macs = pr.N * pr.Co * np.prod(pr.out_hw()) * cg * kh * kw
        if macs <= 6e7:
            return pr
    raise RuntimeError("no problem drawn")


def _cases():
    rng = np.random.default_rng(20260)
    cases = []
    for i in range(120):
        pr = random_problem(rng)
        dtype = str(rng.choice(["f32", "f16", "bf16"]))
        cases.append(pytest.param(pr, dtype, id=f"p{i}-{dtype}"))
    return cases


def _eligible_paths(pr, dtype):
    op_dims = [int(v) for k in ("x", "offset", "mask", "weight") for v in pr.shapes()[k]]
    code = mdcn.dtype_code(workloads.DTYPES[dtype])
    out = []
    for path in PATHS:
        op = mdcn.mdcn_create(pr.stride, pr.padding, pr.dilation, pr.groups,
                              pr.deformable_groups, path=path)
        try:
            mdcn.mdcn_workspace_bytes(op, code, op_dims)
        except mdcn.MdcnError as e:
            assert e.status == mdcn.MDCN_E_PATH, (path, e)
            continue
        out.append(path)
    return out


@pytest.mark.parametrize("pr,dtype", _cases())
def test_random_problem_every_path(pr, dtype):
    inp = workloads.generate(pr, dtype, seed=3)
    ref = oracle.forward(inp["x"], inp["offset"], inp["mask"], inp["weight"], inp["bias"],
                         **pr.attrs())
    g = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    paths = _eligible_paths(pr, dtype)
    assert mdcn.MDCN_PATH_GATHER_GEMM in paths and mdcn.MDCN_PATH_DIRECT in paths
    for path in [mdcn.MDCN_PATH_AUTO] + paths:
        print("random", pr, dtype, PATHS.get(path, "auto"), flush=True)
        op = mdcn.mdcn_create(pr.stride, pr.padding, pr.dilation, pr.groups,
                              pr.deformable_groups, path=path)
        got = mdcn.forward(op, g["x"], g["offset"], g["mask"], g["weight"], g["bias"])
        torch.cuda.synchronize()
        got = got.cpu().double().numpy()
        ok, err, bound = within_tolerance(got, ref, dtype)
        assert ok, (PATHS.get(path, "auto"), dtype, error_report(got, ref))
