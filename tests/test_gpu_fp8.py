"""GPU parity of the FP8 path (MDCN_PATH_GATHER_GEMM_FP8) against the
oracle's FP8 mode (oracle.forward_fp8: columns and scaled weight rows rounded
to E4M3, exact sums).

Two tolerances:
- grid inputs (workloads.generate_grid: x, weights, masks on coarse dyadic
  grids, integer offsets): every column value is an E4M3 number, so the
  quantization decisions cannot differ, and every product and partial sum is
  a small multiple of a power of two, which the FP8 matrix instruction sums
  exactly.  The GPU result is then the oracle's up to the output rounding:
  fp32 |g - r| <= 1e-6 * max(|r|, RMS(r)); fp16/bf16 one unit in the last
  place of the output type.
- random inputs (workloads.generate): the dtype's tolerance
  (helpers.within_tolerance) plus 2^-11 * S, S the oracle's sum of absolute
  scaled products of the output.  The v_mfma_f32_32x32x64_f8f6f4 instruction
  does not sum its 64 products exactly when they span many binades: on
  random operands its error reached 2^-12 of their absolute sum (2^-15.5
  with operands distributed like these workloads), so summing that bound
  over the instructions of one output gives at most 2^-12 * S; 2^-11 leaves
  a factor 2.  The same margin covers a column value whose fp32 sample
  (GPU) and exact sample (oracle) fall on two sides of an E4M3 rounding
  midpoint (an output moves by |w| times one E4M3 spacing of that column).
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
FP8 = mdcn.MDCN_PATH_GATHER_GEMM_FP8

CASES = {
    # several GEMM tiles, ragged pixel count, 2 offset groups
    "multi_tile_dg2": Problem(N=2, C=64, Co=96, H=13, W=17, deformable_groups=2,
                              offset_dist=("normal", 1.5)),
    # groups and offset groups that divide neither way, stride 2
    "grouped_strided": Problem(N=1, C=48, Co=40, H=9, W=11, stride=(2, 1), groups=2,
                               deformable_groups=3, bias=False),
    # 1x1 kernel: Kg = 32 padded to 128, more images
    "pointwise": Problem(N=3, C=32, Co=64, H=20, W=20, kh=1, kw=1, padding=(0, 0)),
    # 6 channels: no 16-byte channel vectors (the scalar gather)
    "narrow_channels": Problem(N=2, C=6, Co=8, H=10, W=12, kh=5, kw=3, padding=(2, 1),
                               dilation=(1, 2)),
    # large offsets: samples off the image and fallbacks
    "far_offsets": Problem(N=1, C=16, Co=16, H=12, W=12, offset_dist=("uniform", 20.0),
                           mask_dist=("uniform_zeros", 0.2)),
}


def make_op(pr):
    return mdcn.mdcn_create(pr.stride, pr.padding, pr.dilation, pr.groups,
                            pr.deformable_groups, path=FP8)


def run(pr, inp, workspace_bytes=None, trace=None):
    g = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    ws = None
    if workspace_bytes is not None:
        ws = torch.empty(max(workspace_bytes, 1), dtype=torch.uint8, device=DEV)
    out = mdcn.forward(make_op(pr), g["x"], g["offset"], g["mask"], g["weight"], g["bias"],
                       workspace=ws, trace=trace)
    torch.cuda.synchronize()
    return out.cpu().double().numpy()


def ulp(r, dtype):
    """One unit in the last place of r in the output type (subnormals included)."""
    if dtype == "f16":
        return np.spacing(np.abs(r).astype(np.float16)).astype(np.float64)
    # bf16: 8 significant bits, normal exponent range of fp32
    a = np.maximum(np.abs(r), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_fp8_grid_inputs_exact(name, dtype):
    pr = CASES[name]
    inp = workloads.generate_grid(pr, dtype, seed=1)
    print("fp8 grid", name, dtype, flush=True)
    ref, _ = oracle.forward_fp8(inp["x"], inp["offset"], inp["mask"], inp["weight"], inp["bias"],
                                **pr.attrs())
    got = run(pr, inp)
    err = np.abs(got - ref)
    if dtype == "f32":
        bound = 1e-6 * np.maximum(np.abs(ref), np.sqrt(np.mean(ref ** 2)))
    else:
        bound = ulp(ref, dtype)
    assert (err <= bound).all(), (name, dtype, float(err.max()), error_report(got, ref))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_fp8_random_inputs(name, dtype):
    pr = CASES[name]
    inp = workloads.generate(pr, dtype, seed=2)
    print("fp8 random", name, dtype, flush=True)
    ref, asum = oracle.forward_fp8(inp["x"], inp["offset"], inp["mask"], inp["weight"],
                                   inp["bias"], **pr.attrs())
    got = run(pr, inp)
    _, err, bound = within_tolerance(got, ref, dtype)
    bound = bound + 2.0 ** -11 * asum
    assert (err <= bound).all(), (name, dtype, float((err / bound).max()),
                                  error_report(got, ref))


@pytest.mark.parametrize("wl,dtype", [("ocdnet_n4_c256_160x160", "f16"),
                                      ("deep_n16_c512_40x40", "f16")])
def test_fp8_benchmark_workload_sampled(wl, dtype):
    """The benchmark shapes at full size, in the launch configuration the
    benchmark times: 4096 random outputs plus the first and last row and
    column of every image's first and last channel, against the oracle."""
    pr = workloads.WORKLOADS[wl][0]
    inp = workloads.generate(pr, dtype, seed=0)
    print("fp8 sampled", wl, dtype, flush=True)
    got = run(pr, inp).reshape(-1)
    N, Co, (Ho, Wo) = pr.N, pr.Co, pr.out_hw()
    rng = np.random.default_rng(3)
    idx = [rng.integers(0, got.size, 4096)]
    for n in (0, N - 1):
        for co in (0, Co - 1):
            base = (n * Co + co) * Ho * Wo
            idx.append(base + np.arange(Wo))                       # first row
            idx.append(base + (Ho - 1) * Wo + np.arange(Wo))       # last row
            idx.append(base + np.arange(Ho) * Wo)                  # first column
            idx.append(base + np.arange(Ho) * Wo + Wo - 1)         # last column
    idx = np.unique(np.concatenate(idx))
    ref, asum = oracle.forward_points_fp8(inp["x"], inp["offset"], inp["mask"], inp["weight"],
                                          inp["bias"], idx, **pr.attrs())
    rms = float(np.sqrt(np.mean(ref ** 2)))
    _, err, bound = within_tolerance(got[idx], ref, dtype, rms=rms)
    bound = bound + 2.0 ** -11 * asum
    assert (err <= bound).all(), (wl, float((err / bound).max()))


def test_fp8_differs_from_exact_by_quantization_only():
    """Against the exact (non-FP8) oracle the FP8 path is off by about the
    E4M3 rounding, visibly more than the fp16 paths and far less than the
    output's scale."""
    pr = CASES["multi_tile_dg2"]
    inp = workloads.generate(pr, "f32", seed=4)
    exact = oracle.forward(inp["x"], inp["offset"], inp["mask"], inp["weight"], inp["bias"],
                           **pr.attrs())
    got = run(pr, inp)
    rel = np.sqrt(np.mean((got - exact) ** 2)) / np.sqrt(np.mean(exact ** 2))
    assert 1e-3 < rel < 0.1, rel


def test_fp8_chunked_workspace_matches_default():
    """With the least workspace (one image per chunk) the weight is quantized
    once, in the first chunk's set-up launch, and the result is bit-identical."""
    pr = CASES["pointwise"]
    inp = workloads.generate(pr, "f16", seed=5)
    op = make_op(pr)
    dims = [pr.N, pr.C, pr.H, pr.W] + list(inp["offset"].shape) + list(inp["mask"].shape) + \
        list(inp["weight"].shape)
    full, least = mdcn.mdcn_workspace_bytes(op, mdcn.MDCN_F16, dims)
    assert least < full
    assert "chunk=1" in mdcn.mdcn_describe_plan(op, mdcn.MDCN_F16, dims, least)
    tr = mdcn.Trace(64)
    a = run(pr, inp)
    b = run(pr, inp, workspace_bytes=least, trace=tr)
    assert np.array_equal(a, b)
    names = [n for n, _ in tr.read()]
    assert names[0] == "prep_nhwc_fp8"
    assert names.count("prep_nhwc_fp8") == 1
    assert names.count("deform_gather_fp8") == names.count("gemm_fp8_bias") == pr.N
    assert names.count("to_nhwc") == pr.N - 1          # the first chunk's is in prep_nhwc_fp8


def test_fp8_zero_mask_gives_bias_exactly():
    pr = CASES["multi_tile_dg2"]
    inp = workloads.generate(pr, "f32", seed=6)
    inp["mask"] = torch.zeros_like(inp["mask"])
    got = run(pr, inp)
    want = np.broadcast_to(inp["bias"].double().numpy()[None, :, None, None], got.shape)
    assert np.array_equal(got, want)


def test_fp8_saturates_large_inputs():
    """Column values beyond 448 saturate to 448 as in the oracle (the convert
    instruction alone would give NaN above 464)."""
    pr = CASES["pointwise"]
    inp = workloads.generate_grid(pr, "f32", seed=7)
    inp["x"] = inp["x"] * 400.0                      # samples up to 1200
    ref, asum = oracle.forward_fp8(inp["x"], inp["offset"], inp["mask"], inp["weight"],
                                   inp["bias"], **pr.attrs())
    got = run(pr, inp)
    assert np.isfinite(got).all()
    _, err, bound = within_tolerance(got, ref, "f32")
    assert (err <= bound + 2.0 ** -11 * asum).all(), float(err.max())
