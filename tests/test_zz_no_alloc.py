"""mdcn_forward_noalloc: the forward with its workspace in the library's own
device array (for callers that cannot allocate), against mdcn_forward.

Two calls in a row through the C ABI, the second on a smaller input, each
compared with mdcn_forward on the same inputs and with the oracle (on the
windowed path and, separately, on the windowed FP8 path).  Both calls
split output tiles between workgroups (MDCN_WIN_CTAS), so the first leaves
published partial sums and set flags in the shared array: the second is only
right if the forward clears what must start at zero.  A problem that needs
more workspace than the array holds is rejected before anything is enqueued.
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


def _dev(inp):
    return {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}


def _noalloc(op, g, dtype):
    dims = mdcn.dims_of(g["x"], g["offset"], g["mask"], g["weight"])
    out = torch.full(mdcn.mdcn_output_shape(op, dims), float("nan"), dtype=g["x"].dtype,
                     device=DEV)
    bias = g["bias"]
    st = mdcn.mdcn_forward_noalloc(op, mdcn.dtype_code(workloads.DTYPES[dtype]), dims,
                                   g["x"].data_ptr(), g["offset"].data_ptr(),
                                   g["mask"].data_ptr(), g["weight"].data_ptr(),
                                   bias.data_ptr() if bias is not None else 0,
                                   int(bias.numel()) if bias is not None else 0, out.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
    return st, out


def test_noalloc_matches_forward_twice(monkeypatch):
    # 8 and then 4 output tiles of 8 chunks each over 3 workgroups: tiles are
    # split in both calls (their partial sums go through the array's slots)
    monkeypatch.setenv("MDCN_WIN_CTAS", "3")
    cases = [(Problem(N=2, C=128, Co=64, H=32, W=32, offset_dist=("normal", 2.0)), "f16", 31),
             (Problem(N=1, C=128, Co=64, H=32, W=32, bias=True, offset_dist=("normal", 2.0)),
              "bf16", 32)]
    for pr, dtype, seed in cases:
        print("noalloc", pr, dtype, flush=True)
        op = mdcn.mdcn_create(pr.stride, pr.padding, pr.dilation, pr.groups,
                              pr.deformable_groups, path=mdcn.MDCN_PATH_WINDOW)
        inp = workloads.generate(pr, dtype, seed=seed)
        g = _dev(inp)
        st, got = _noalloc(op, g, dtype)
        assert st == mdcn.MDCN_OK, mdcn.status_string(st)
        ref_fwd = mdcn.forward(op, g["x"], g["offset"], g["mask"], g["weight"], g["bias"],
                               check=True)
        torch.cuda.synchronize()
        a = got.cpu().double().numpy()
        b = ref_fwd.cpu().double().numpy()
        assert np.isfinite(a).all()
        # against the existing entry point on the same inputs, and the oracle
        ok, err, bound = within_tolerance(a, b, dtype)
        assert ok, float((err - bound).max())
        ref = oracle.forward(inp["x"], inp["offset"], inp["mask"], inp["weight"], inp["bias"],
                             **pr.attrs())
        ok, err, bound = within_tolerance(a, ref, dtype)
        assert ok, float((err - bound).max())


def test_noalloc_window_fp8_twice(monkeypatch):
    """The same two calls on the windowed FP8 path (E4M3 weight and row
    scales in the array, split tiles): bit-identical to mdcn_forward, and
    within the FP8 tolerance of the oracle's FP8 mode."""
    monkeypatch.setenv("MDCN_WIN_CTAS", "3")
    cases = [(Problem(N=2, C=128, Co=64, H=32, W=32, offset_dist=("normal", 2.0)), "f16", 33),
             (Problem(N=1, C=128, Co=64, H=32, W=32, bias=True, offset_dist=("normal", 2.0)),
              "bf16", 34)]
    for pr, dtype, seed in cases:
        print("noalloc fp8", pr, dtype, flush=True)
        op = mdcn.mdcn_create(pr.stride, pr.padding, pr.dilation, pr.groups,
                              pr.deformable_groups, path=mdcn.MDCN_PATH_WINDOW_FP8)
        inp = workloads.generate(pr, dtype, seed=seed)
        g = _dev(inp)
        st, got = _noalloc(op, g, dtype)
        assert st == mdcn.MDCN_OK, mdcn.status_string(st)
        ref_fwd = mdcn.forward(op, g["x"], g["offset"], g["mask"], g["weight"], g["bias"],
                               check=True)
        torch.cuda.synchronize()
        assert torch.equal(got, ref_fwd)
        ref, asum = oracle.forward_fp8(inp["x"], inp["offset"], inp["mask"], inp["weight"],
                                       inp["bias"], **pr.attrs())
        _, err, bound = within_tolerance(got.cpu().double().numpy(), ref, dtype)
        assert (err <= bound + 2.0 ** -11 * asum).all()


def test_noalloc_window_fp8_wide_twice(monkeypatch):
    """Two calls on the windowed FP8 path's wide tiles (groups of more than
    256 output channels: 128-pixel x 512-channel tiles, split between
    workgroups), the second smaller: bit-identical to mdcn_forward and within
    the FP8 tolerance of the oracle's FP8 mode."""
    monkeypatch.setenv("MDCN_WIN_CTAS", "5")
    cases = [(Problem(N=2, C=32, Co=288, H=37, W=37, offset_dist=("normal", 3.0)), "f16", 35),
             (Problem(N=1, C=32, Co=320, H=21, W=19, bias=True, offset_dist=("normal", 2.0)),
              "bf16", 36)]
    for pr, dtype, seed in cases:
        print("noalloc fp8 wide", pr, dtype, flush=True)
        op = mdcn.mdcn_create(pr.stride, pr.padding, pr.dilation, pr.groups,
                              pr.deformable_groups, path=mdcn.MDCN_PATH_WINDOW_FP8)
        s = pr.shapes()
        dims = [int(v) for k in ("x", "offset", "mask", "weight") for v in s[k]]
        desc = mdcn.mdcn_describe_plan(op, mdcn.MDCN_F16 if dtype == "f16" else mdcn.MDCN_BF16,
                                       dims)
        assert int(desc.split("tile=")[1].split()[0]) in (4, 5, 6), desc
        inp = workloads.generate(pr, dtype, seed=seed)
        g = _dev(inp)
        st, got = _noalloc(op, g, dtype)
        assert st == mdcn.MDCN_OK, mdcn.status_string(st)
        ref_fwd = mdcn.forward(op, g["x"], g["offset"], g["mask"], g["weight"], g["bias"],
                               check=True)
        torch.cuda.synchronize()
        assert torch.equal(got, ref_fwd)
        ref, asum = oracle.forward_fp8(inp["x"], inp["offset"], inp["mask"], inp["weight"],
                                       inp["bias"], **pr.attrs())
        _, err, bound = within_tolerance(got.cpu().double().numpy(), ref, dtype)
        assert (err <= bound + 2.0 ** -11 * asum).all()


def test_noalloc_rejects_problems_beyond_the_array():
    # the OCDNet-like stage on the gather + GEMM path in fp32: one image's
    # column buffer alone (236 MB) exceeds the array
    pr, _ = workloads.WORKLOADS["ocdnet_n4_c256_160x160"]
    op = mdcn.mdcn_create(pr.stride, pr.padding, pr.dilation, pr.groups, pr.deformable_groups,
                          path=mdcn.MDCN_PATH_GATHER_GEMM)
    s = pr.shapes()
    dims = [int(v) for k in ("x", "offset", "mask", "weight") for v in s[k]]
    _, least = mdcn.mdcn_workspace_bytes(op, mdcn.MDCN_F32, dims)
    assert least > mdcn.MDCN_NOALLOC_SCRATCH_BYTES
    g = {k: torch.zeros(s[k], dtype=torch.float32, device=DEV) for k in
         ("x", "offset", "mask", "weight")}
    g["bias"] = None
    torch.cuda.synchronize()
    st, out = _noalloc(op, g, "f32")
    torch.cuda.synchronize()
    assert st == mdcn.MDCN_E_WORKSPACE
    assert bool(torch.isnan(out).all())          # nothing was enqueued
