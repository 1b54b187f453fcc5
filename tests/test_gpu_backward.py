"""GPU parity of the backward pass (mdcn_backward, fp32) against the oracle's
backward (oracle.backward, float64, pinned by adjoint identities and finite
differences in test_oracle_backward_pins.py).

Tolerance, per gradient tensor: |g - r| <= 1e-4 * max(|r|, RMS(r)), the
forward's fp32 rule, plus for fp16/bf16 one rounding of the result to the
dtype (2^-10 or 2^-7 of |r|; the oracle gets the same rounded inputs and
grad_out).  Every gradient element is a sum of at most a few thousand fp32
products (grad_weight: N*Ho*Wo of them, accumulated by atomic adds in any
order), so fp32 rounding stays orders of magnitude below it.
The GPU splits each sample coordinate into cell and fraction from the fp32
offset exactly as the oracle does from the same value, so both
differentiate on the same cell.
"""
import numpy as np
import pytest
import torch

from helpers import ensure_built

ensure_built()
from modulated_deformable_convolution_amd import mdcn, workloads  # noqa: E402
from modulated_deformable_convolution_amd.workloads import Problem  # noqa: E402
from oracle import oracle  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

CASES = {
    "basic_3x3": Problem(N=2, C=16, Co=24, H=12, W=14, offset_dist=("normal", 1.5)),
    "grouped_dg": Problem(N=2, C=24, Co=16, H=9, W=11, stride=(2, 1), padding=(1, 2),
                          dilation=(1, 2), groups=2, deformable_groups=3, bias=False),
    "kernel_5x3_far": Problem(N=1, C=8, Co=12, H=10, W=13, kh=5, kw=3, padding=(2, 1),
                              offset_dist=("uniform", 6.0), mask_dist=("uniform_zeros", 0.2)),
    "depthwise": Problem(N=2, C=8, Co=8, H=9, W=9, groups=8),
    "grid_smaller": Problem(N=1, C=12, Co=8, H=11, W=11, Ho=7, Wo=9),
    "wide_channels": Problem(N=1, C=128, Co=64, H=16, W=16, offset_dist=("normal", 2.0)),
    # 128 channels in two offset groups (64-lane teams), an output grid with
    # odd sizes, offsets of sigma 3
    "dg2_ragged": Problem(N=2, C=128, Co=32, H=21, W=19, deformable_groups=2,
                          offset_dist=("normal", 3.0)),
    # ... with groups, stride and dilation 2, far offsets and zero masks
    "grouped_strided_far": Problem(N=1, C=128, Co=64, H=23, W=17, stride=(2, 2),
                                   padding=(2, 2), dilation=(2, 2), groups=2,
                                   deformable_groups=2, offset_dist=("uniform", 6.0),
                                   mask_dist=("uniform_zeros", 0.2)),
    # fp32: both contractions on the MFMA GEMM, the weight gradient in two
    # pixel chunks of 1024 (P = 2048)
    "mfma_split": Problem(N=2, C=32, Co=64, H=32, W=64, offset_dist=("normal", 1.0)),
}


def grads_gpu(pr, inp, go, trace=None):
    g = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    op = mdcn.mdcn_create(pr.stride, pr.padding, pr.dilation, pr.groups, pr.deformable_groups)
    out = mdcn.backward(op, g["x"], g["offset"], g["mask"], g["weight"],
                        go.to(g["x"].dtype).to(DEV), with_bias=pr.bias, trace=trace)
    torch.cuda.synchronize()
    return {k: (v.cpu().double().numpy() if v is not None else None) for k, v in out.items()}


ROUNDING = {"f32": 0.0, "f16": 2.0 ** -10, "bf16": 2.0 ** -7}


def check(got, ref, name, dtype="f32"):
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = np.abs(got - ref)
    bound = 1e-4 * np.maximum(np.abs(ref), rms) + ROUNDING[dtype] * np.abs(ref)
    if dtype == "f16":
        bound = bound + 2.0 ** -24                    # fp16 subnormal spacing
    assert (err <= bound).all(), (name, float(err.max()), float((err / np.maximum(bound, 1e-300)).max()))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_backward_matches_oracle(name, dtype):
    pr = CASES[name]
    inp = workloads.generate(pr, dtype, seed=11)
    ho, wo = pr.out_hw()
    go = torch.randn((pr.N, pr.Co, ho, wo), generator=torch.Generator().manual_seed(12))
    go = go.to(workloads.DTYPES[dtype])                # the values both sides see
    print("backward", name, dtype, flush=True)
    ref = oracle.backward(inp["x"], inp["offset"], inp["mask"], inp["weight"], go,
                          with_bias=pr.bias, **pr.attrs())
    got = grads_gpu(pr, inp, go)
    for k in ("x", "offset", "mask", "weight") + (("bias",) if pr.bias else ()):
        check(got[k], ref[k], (name, k), dtype)
    if not pr.bias:
        assert got["bias"] is None


def test_backward_trace_and_repeat():
    """Kernels in order, and a second call gives the same result (the
    accumulators are cleared by each call)."""
    pr = CASES["basic_3x3"]
    inp = workloads.generate(pr, "f32", seed=13)
    ho, wo = pr.out_hw()
    go = torch.randn((pr.N, pr.Co, ho, wo), generator=torch.Generator().manual_seed(14))
    tr = mdcn.Trace(64)
    a = grads_gpu(pr, inp, go, trace=tr)
    b = grads_gpu(pr, inp, go)
    for k in ("offset", "mask", "bias"):
        assert np.array_equal(a[k], b[k]), k       # no atomics: bit-identical
    for k in ("x", "weight"):
        assert np.allclose(a[k], b[k], rtol=1e-5, atol=1e-6), k
    names = [n for n, _ in tr.read()]
    assert names[:2] == ["bwd_zero", "bwd_bias"] and names[-1] == "bwd_weight_out"
    assert names.count("bwd_sample") == names.count("bwd_col_gemm") == pr.N


def test_backward_zero_mask_and_far_samples():
    """A zero mask: no gradient reaches x or the offsets, grad_weight is 0;
    samples far off the image: all of x, offset, mask and weight get 0."""
    pr = CASES["basic_3x3"]
    inp = workloads.generate(pr, "f32", seed=15)
    ho, wo = pr.out_hw()
    go = torch.randn((pr.N, pr.Co, ho, wo), generator=torch.Generator().manual_seed(16))
    z = dict(inp)
    z["mask"] = torch.zeros_like(inp["mask"])
    g = grads_gpu(pr, z, go)
    assert not g["x"].any() and not g["offset"].any() and not g["weight"].any()
    f = dict(inp)
    f["offset"] = inp["offset"] + 1000.0
    g = grads_gpu(pr, f, go)
    assert not g["x"].any() and not g["offset"].any() and not g["mask"].any()
    assert not g["weight"].any()
    assert np.allclose(g["bias"], go.double().numpy().sum(axis=(0, 2, 3)), rtol=1e-5, atol=1e-4)
