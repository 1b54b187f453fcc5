"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small problems (several tiles, ragged tails in every GEMM dimension, padded
contraction, scalar and vector gather paths, every dtype and path) are
compared element by element over the whole output.  The five benchmark
workloads are run at full size, in the same launch configuration as the
benchmark, and compared on sampled outputs (seeded random elements plus the
image borders) that the oracle computes one by one.  Tolerances are those of
helpers.within_tolerance.
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

SMALL = {
    # Co = 160: one full and one partial 128-row tile; 3 images x 361 pixels:
    # a ragged column tile; Kg = 288 padded to 320; two offset groups.
    "multi_tile_dg2": Problem(N=3, C=32, Co=160, H=19, W=19, deformable_groups=2,
                              offset_dist=("normal", 2.0)),
    # kh != kw, asymmetric stride/padding/dilation, 3 groups, 6 offset groups.
    "grouped_strided": Problem(N=2, C=48, Co=96, H=17, W=23, kh=3, kw=2, stride=(2, 1),
                               padding=(2, 0), dilation=(1, 2), groups=3, deformable_groups=6,
                               offset_dist=("normal", 1.5)),
    # channel counts that are not a multiple of the 16-byte vector: scalar gather.
    "odd_channels": Problem(N=2, C=6, Co=10, H=11, W=9, deformable_groups=2, bias=False,
                            offset_dist=("normal", 1.0)),
    # depthwise with a channel multiplier of 2 and 3 offset groups.
    "depthwise_mult2": Problem(N=2, C=24, Co=48, H=13, W=13, groups=24, deformable_groups=3,
                               offset_dist=("uniform", 8.0), mask_dist=("uniform_zeros", 0.1)),
    # depthwise: odd offset-group width (one staged plane per workgroup) and a
    # channel multiplier of 6 (two passes of at most 4 outputs per plane)
    "depthwise_mult6_odd": Problem(N=2, C=9, Co=54, H=11, W=7, groups=9, deformable_groups=3,
                                   offset_dist=("uniform", 5.0), mask_dist=("uniform_zeros", 0.1)),
    # depthwise 3x3 with one output per input channel (the persistent
    # kernel): 1517 pixels = two full groups of 512 and a ragged one; an odd
    # plane size (16-bit types stay on the staged kernel)
    "depthwise_3x3_ragged": Problem(N=2, C=12, Co=12, H=37, W=41, groups=12,
                                    deformable_groups=3, offset_dist=("uniform", 16.0),
                                    mask_dist=("uniform_zeros", 0.1)),
    # the same with an even plane size and an odd width (16-bit planes are
    # read two positions at a time, which then straddle rows)
    "depthwise_3x3_even": Problem(N=2, C=16, Co=16, H=30, W=35, groups=16,
                                  deformable_groups=2, offset_dist=("uniform", 12.0),
                                  mask_dist=("uniform_zeros", 0.1)),
    # depthwise with a 5x3 kernel (runtime tap count)
    "depthwise_5x3": Problem(N=2, C=8, Co=8, H=12, W=10, kh=5, kw=3, padding=(2, 1), groups=8,
                             deformable_groups=2, offset_dist=("normal", 2.0)),
    # depthwise plane too large for LDS: the plain kernel
    "depthwise_large_plane": Problem(N=1, C=4, Co=4, H=150, W=150, groups=4,
                                     offset_dist=("uniform", 20.0)),
    "kernel_1x1": Problem(N=2, C=16, Co=24, H=9, W=10, kh=1, kw=1, padding=(0, 0),
                          offset_dist=("normal", 2.0)),
    "kernel_5x5": Problem(N=1, C=16, Co=16, H=12, W=12, kh=5, kw=5, padding=(2, 2)),
    # output grid smaller than the conv formula (taken from the offset dims)
    "smaller_out_grid": Problem(N=2, C=16, Co=32, H=15, W=15, Ho=7, Wo=11),
    "tiny": workloads.TINY,
    # eligible for the fused gather-GEMM (C/group a multiple of 64, C/dg of 32):
    # Co = 160 (a partial weight-row tile), 3 x 169 pixels (ragged columns)
    "fused_multi_tile": Problem(N=3, C=64, Co=160, H=13, W=13, deformable_groups=2,
                                offset_dist=("normal", 2.0)),
    # grouped, strided, dilated, 3x2 kernel, 4 offset groups, Mg = 48
    "fused_grouped": Problem(N=2, C=128, Co=96, H=17, W=15, kh=3, kw=2, stride=(2, 1),
                             padding=(2, 1), dilation=(2, 1), groups=2, deformable_groups=4,
                             offset_dist=("normal", 1.5)),
    # C/dg = 16: the lanes of one output column read different offset groups
    # (f16/bf16: two 16-byte chunks per offset group; f32: four)
    "fused_narrow_dg": Problem(N=2, C=64, Co=64, H=11, W=13, deformable_groups=4,
                               offset_dist=("normal", 2.0)),
    # C/group = 64 and C/dg = 96: group 1 spans offset groups 0 and 1
    "fused_misaligned_groups": Problem(N=2, C=192, Co=96, H=9, W=11, groups=3,
                                       deformable_groups=2, offset_dist=("normal", 2.0)),
    # 5x5 taps: the geometry table only fits beside a 64-column tile
    "fused_5x5": Problem(N=2, C=64, Co=64, H=11, W=10, kh=5, kw=5, padding=(2, 2),
                         offset_dist=("normal", 2.0)),
    # eligible for the windowed kernel (fp16/bf16): Co = 288 (a full and a
    # partial 256-row tile), 37 x 37 (1369 pixels: the planner takes six flat
    # tiles of 256 raster pixels, the last one ragged; MDCN_WIN_TILE forces
    # the ragged rectangular ones in test_every_window_tile), offsets wide
    # enough that some samples leave the window (the fallback)
    "window_multi_tile": Problem(N=2, C=32, Co=288, H=37, W=37,
                                 offset_dist=("normal", 3.0)),
    # stride (2, 1), dilation (1, 2), 2 groups inside 2 offset groups, Mg = 48
    "window_grouped": Problem(N=2, C=64, Co=96, H=23, W=19, stride=(2, 1), padding=(1, 2),
                              dilation=(1, 2), groups=2, deformable_groups=2,
                              offset_dist=("normal", 2.0)),
    # offsets up to 20 px: many samples off the image or outside the window
    "window_far_offsets": Problem(N=1, C=16, Co=32, H=30, W=30,
                                  offset_dist=("uniform", 20.0),
                                  mask_dist=("uniform_zeros", 0.1)),
    # 13 x 21 = 273 output pixels: flat tiles (MDCN_WIN_TILE=3) wrap rows,
    # the last one is ragged, and a plane is not a multiple of 8 pixels
    # (element stores)
    "window_flat_ragged": Problem(N=2, C=32, Co=64, H=13, W=21, offset_dist=("normal", 2.0)),
    # also eligible for the fused kernel (C/group = 64)
    "window_fused_cmp": Problem(N=2, C=64, Co=128, H=21, W=21, offset_dist=("normal", 2.0)),
    # 4 output tiles per image of 8 chunks (16 channels) each: with 3 to 13
    # workgroups the work split cuts tiles (see test_window_split_tiles)
    "window_split_chunks": Problem(N=2, C=128, Co=64, H=32, W=32, offset_dist=("normal", 2.0)),
}


def path_ok(pr, dtype, path):
    """Whether the library accepts `path` for this problem (a host query: an
    op created for that path reports MDCN_E_PATH otherwise)."""
    op = make_op(pr, path)
    shapes = pr.shapes()
    dims = [int(v) for k in ("x", "offset", "mask", "weight") for v in shapes[k]]
    try:
        mdcn.mdcn_workspace_bytes(op, mdcn.dtype_code(workloads.DTYPES[dtype]), dims)
    except mdcn.MdcnError as e:
        assert e.status == mdcn.MDCN_E_PATH
        return False
    return True


def to_dev(inp):
    return {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}


def make_op(pr, path=mdcn.MDCN_PATH_AUTO):
    return mdcn.mdcn_create(pr.stride, pr.padding, pr.dilation, pr.groups,
                            pr.deformable_groups, path=path)


def run_gpu(pr, inp, path=mdcn.MDCN_PATH_AUTO, workspace_bytes=None, trace=None):
    g = to_dev(inp)
    op = make_op(pr, path)
    ws = None
    if workspace_bytes is not None:
        ws = torch.empty(max(workspace_bytes, 1), dtype=torch.uint8, device=DEV)
    # check: every forward also asks mdcn_forward_check whether a bounded wait
    # inside it gave up (only the windowed path waits)
    out = mdcn.forward(op, g["x"], g["offset"], g["mask"], g["weight"], g["bias"],
                       workspace=ws, trace=trace, check=True)
    torch.cuda.synchronize()
    return out.cpu()


def oracle_full(pr, inp):
    return oracle.forward(inp["x"], inp["offset"], inp["mask"], inp["weight"], inp["bias"],
                          **pr.attrs())


def paths_for(pr, dtype):
    paths = [mdcn.MDCN_PATH_GATHER_GEMM, mdcn.MDCN_PATH_DIRECT]
    if pr.C // pr.groups == 1:
        paths.append(mdcn.MDCN_PATH_DEPTHWISE)
    if path_ok(pr, dtype, mdcn.MDCN_PATH_FUSED):
        paths.append(mdcn.MDCN_PATH_FUSED)
    if path_ok(pr, dtype, mdcn.MDCN_PATH_WINDOW):
        paths.append(mdcn.MDCN_PATH_WINDOW)
    return paths


CASES = [(name, dt, path) for name, pr in SMALL.items() for dt in ("f32", "f16", "bf16")
         for path in paths_for(pr, dt)]


@pytest.mark.parametrize("name,dtype,path", CASES)
def test_small_full_tensor(name, dtype, path):
    pr = SMALL[name]
    print("case", name, dtype, "path", path, flush=True)
    inp = workloads.generate(pr, dtype, seed=1)
    got = run_gpu(pr, inp, path).double().numpy()
    ref = oracle_full(pr, inp)
    assert got.shape == ref.shape
    ok, err, bound = within_tolerance(got, ref, dtype)
    assert ok, (name, dtype, error_report(got, ref), float((err / bound).max()))


@pytest.mark.parametrize("pr,path,name", [
    # 146k multiply-adds: the one-launch direct kernel
    (SMALL["depthwise_mult2"], mdcn.MDCN_PATH_DIRECT, "path=direct"),
    # 1.8M multiply-adds, C/group = 1: the depthwise kernel
    (Problem(N=2, C=64, Co=64, H=40, W=40, groups=64, offset_dist=("uniform", 8.0)),
     mdcn.MDCN_PATH_DEPTHWISE, "path=depthwise_direct"),
])
def test_auto_path_matches_forced_paths(pr, path, name):
    inp = workloads.generate(pr, "f32", seed=2)
    shapes = pr.shapes()
    dims = [int(v) for k in ("x", "offset", "mask", "weight") for v in shapes[k]]
    assert mdcn.mdcn_describe_plan(make_op(pr), mdcn.MDCN_F32, dims).startswith(name)
    auto = run_gpu(pr, inp, mdcn.MDCN_PATH_AUTO)
    forced = run_gpu(pr, inp, path)
    assert torch.equal(auto, forced)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_zero_mask_gives_bias_exactly(dtype):
    pr = SMALL["multi_tile_dg2"]
    inp = workloads.generate(pr, dtype, seed=3)
    inp["mask"] = torch.zeros_like(inp["mask"])
    got = run_gpu(pr, inp)
    assert torch.equal(got, inp["bias"][None, :, None, None].expand_as(got))


@pytest.mark.parametrize("path", [mdcn.MDCN_PATH_GATHER_GEMM, mdcn.MDCN_PATH_DEPTHWISE])
def test_off_image_samples_give_bias_exactly(path):
    pr = SMALL["depthwise_mult2"]
    inp = workloads.generate(pr, "f32", seed=4)
    off = inp["offset"]
    # alternate far below/right, far above/left, and the exact edges h = -1 / w = W
    far = torch.full_like(off, 1.0e4)
    far[:, 1::4] = -3.0e7
    far[:, 2::4] = -1.0e9
    inp["offset"] = far
    got = run_gpu(pr, inp, path)
    assert torch.equal(got, inp["bias"][None, :, None, None].expand_as(got))
    # exactly on the line h = -1 for every tap (anchor row + offset == -1)
    Ho, Wo = pr.out_hw()
    off = torch.zeros_like(inp["offset"])
    K = pr.kh * pr.kw
    for q in range(pr.deformable_groups):
        for k in range(K):
            i = k // pr.kw
            anchor = torch.arange(Ho, dtype=torch.float32) * pr.stride[0] - pr.padding[0] \
                + i * pr.dilation[0]
            off[:, q * 2 * K + 2 * k] = (-1.0 - anchor)[:, None]
            off[:, q * 2 * K + 2 * k + 1] = 0.25
    inp["offset"] = off
    got = run_gpu(pr, inp, path)
    assert torch.equal(got, inp["bias"][None, :, None, None].expand_as(got))


@pytest.mark.parametrize("name,path", [("multi_tile_dg2", mdcn.MDCN_PATH_AUTO),
                                       ("fused_multi_tile", mdcn.MDCN_PATH_FUSED),
                                       ("window_multi_tile", mdcn.MDCN_PATH_WINDOW)])
def test_chunked_workspace_matches_default(name, path):
    """The least workspace: one image per chunk; the first chunk's launch
    also repacks the weight (and clears the window path's flags), the later
    chunks only move x."""
    pr = SMALL[name]
    inp = workloads.generate(pr, "f16", seed=5)
    op = make_op(pr, path)
    dims = [pr.N, pr.C, pr.H, pr.W] + list(inp["offset"].shape) + list(inp["mask"].shape) + \
        list(inp["weight"].shape)
    full, least = mdcn.mdcn_workspace_bytes(op, mdcn.MDCN_F16, dims)
    assert least < full
    assert "chunk=1" in mdcn.mdcn_describe_plan(op, mdcn.MDCN_F16, dims, least)
    tr = mdcn.Trace(64)
    a = run_gpu(pr, inp, path)
    b = run_gpu(pr, inp, path, workspace_bytes=least, trace=tr)
    assert torch.equal(a, b)
    names = [n for n, _ in tr.read()]
    assert names[0].startswith("prep_") and not any(n.startswith("prep_") for n in names[1:])
    assert len([n for n in names if n.startswith("to_")]) == pr.N - 1


def test_traced_forward_matches_and_records():
    pr = SMALL["multi_tile_dg2"]
    inp = workloads.generate(pr, "bf16", seed=6)
    tr = mdcn.Trace(64)
    a = run_gpu(pr, inp, trace=tr)
    b = run_gpu(pr, inp)
    assert torch.equal(a, b)
    names = [n for n, _ in tr.read()]
    assert names[0] == "prep_nhwc"
    assert names.count("gemm_bias") == names.count("deform_gather") >= 1
    assert all(ms >= 0 for _, ms in tr.read())


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_unaligned_buffers(dtype):
    """x, out and the workspace at addresses that are not 16-byte aligned."""
    pr = SMALL["multi_tile_dg2"]
    inp = workloads.generate(pr, dtype, seed=13)
    g = to_dev(inp)
    op = make_op(pr)
    shift = 1                                  # one element
    xs = torch.empty(inp["x"].numel() + shift, dtype=g["x"].dtype, device=DEV)
    x = xs[shift:].view(inp["x"].shape)
    x.copy_(g["x"])
    code = mdcn.dtype_code(x.dtype)
    dims = mdcn.dims_of(x, g["offset"], g["mask"], g["weight"])
    shape = mdcn.mdcn_output_shape(op, dims)
    n_out = int(np.prod(shape))
    outs = torch.empty(n_out + shift, dtype=x.dtype, device=DEV)
    out = outs[shift:].view(shape)
    nbytes, _ = mdcn.mdcn_workspace_bytes(op, code, dims)
    ws = torch.empty(nbytes + 8, dtype=torch.uint8, device=DEV)[3:]
    mdcn.forward(op, x, g["offset"], g["mask"], g["weight"], g["bias"], out=out, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle_full(pr, inp)
    ok, err, bound = within_tolerance(out.cpu().double().numpy(), ref, dtype)
    assert ok, error_report(out.cpu().double().numpy(), ref)


def test_repeatable():
    pr = SMALL["grouped_strided"]
    inp = workloads.generate(pr, "f32", seed=7)
    assert torch.equal(run_gpu(pr, inp), run_gpu(pr, inp))


def test_empty_batch():
    pr = SMALL["tiny"]
    inp = workloads.generate(pr, "f32", seed=8)
    for k in ("x", "offset", "mask"):
        inp[k] = inp[k][:0].contiguous()
    got = run_gpu(pr, inp)
    assert tuple(got.shape) == (0, pr.Co, 8, 8)


# ---------------------------------------------------------------- full-size workloads

def sample_indices(shape, n_random, seed):
    """Seeded random flat indices plus every border pixel of two (n, co) planes."""
    N, Co, Ho, Wo = shape
    rng = np.random.default_rng(seed)
    total = N * Co * Ho * Wo
    idx = set(rng.choice(total, size=min(n_random, total), replace=False).tolist())
    for n, co in ((0, 0), (N - 1, Co - 1)):
        base = (n * Co + co) * Ho * Wo
        for h in range(Ho):
            for w in (0, Wo - 1):
                idx.add(base + h * Wo + w)
        for w in range(Wo):
            for h in (0, Ho - 1):
                idx.add(base + h * Wo + w)
    return np.array(sorted(idx), dtype=np.int64)


WORKLOAD_CASES = []
for _name, (_pr, _dts) in workloads.WORKLOADS.items():
    for _dt in sorted(set(_dts) | {"f32"}):
        WORKLOAD_CASES.append((_name, _dt))


@pytest.mark.parametrize("name,dtype", WORKLOAD_CASES)
def test_workload_sampled(name, dtype):
    """Full-size workload, default plan (as benchmarked), sampled outputs.
    fp32 runs of the fp16/bf16 workloads check indexing at a tolerance where
    a single misplaced tap would show."""
    pr, _ = workloads.WORKLOADS[name]
    print("workload", name, dtype, flush=True)
    inp = workloads.generate(pr, dtype, seed=0)
    got = run_gpu(pr, inp)
    shape = tuple(got.shape)
    idx = sample_indices(shape, 4096, seed=11)
    ref = oracle.forward_points(inp["x"], inp["offset"], inp["mask"], inp["weight"],
                                inp["bias"], idx, **pr.attrs())
    g = got.reshape(-1)[torch.from_numpy(idx)].double().numpy()
    # the fp32 rule's scale floor: RMS of the oracle's values at the sampled
    # outputs (an estimate of the whole output's, taken from the reference,
    # never from the result under test)
    rms = float(np.sqrt(np.mean(np.asarray(ref, dtype=np.float64) ** 2)))
    ok, err, bound = within_tolerance(g, ref, dtype, rms=rms)
    assert ok, (name, dtype, error_report(g, ref), float((err / bound).max()))
    assert torch.isfinite(got).all()


def ulp_of(ref, dtype):
    """Spacing of the output dtype at |ref| (normal range; the subnormal
    spacing below it)."""
    mant, emin = {"f32": (23, -126), "f16": (10, -14), "bf16": (7, -126)}[dtype]
    a = np.maximum(np.abs(np.asarray(ref, dtype=np.float64)), 2.0 ** emin)
    return 2.0 ** (np.floor(np.log2(a)) - mant)


GRID_CASES = [
    ("ocdnet_n4_c256_160x160", "f16", mdcn.MDCN_PATH_AUTO, "window"),
    ("deep_n16_c512_40x40", "f16", mdcn.MDCN_PATH_AUTO, "window"),
    ("ocdnet_n4_c256_160x160", "f32", mdcn.MDCN_PATH_AUTO, "fused"),
    ("strided_grouped_n2_c128_co256_128x128", "bf16", mdcn.MDCN_PATH_AUTO, "fused"),
    ("ocdnet_n4_c256_160x160", "f16", mdcn.MDCN_PATH_GATHER_GEMM, "gather_gemm"),
    ("ocdnet_n4_c256_160x160", "f32", mdcn.MDCN_PATH_GATHER_GEMM, "gather_gemm"),
    ("depthwise_n8_c256_96x96", "f32", mdcn.MDCN_PATH_AUTO, "depthwise_direct"),
]


@pytest.mark.parametrize("name,dtype,path,plan", GRID_CASES,
                         ids=["%s-%s-%s" % (c[0].split("_")[0], c[1], c[3]) for c in GRID_CASES])
def test_workload_grid_exact(name, dtype, path, plan):
    """Full-size workloads on grid inputs (workloads.generate_grid: x and the
    weight on coarse dyadic grids, integer offsets, masks in {0, 1/2, 1}).
    Every sample is then a value of the dtype, every product and every fp32
    partial sum is exact, so the result is the exact value rounded once to
    the output dtype: each sampled output must be within one unit in the
    last place of the oracle's value.  A single misplaced tap, channel or
    pixel moves an output by far more than that."""
    pr, _ = workloads.WORKLOADS[name]
    print("grid workload", name, dtype, plan, flush=True)
    inp = workloads.generate_grid(pr, dtype, seed=3)
    op = make_op(pr, path)
    dims = [pr.N, pr.C, pr.H, pr.W] + list(inp["offset"].shape) + list(inp["mask"].shape) + \
        list(inp["weight"].shape)
    code = mdcn.dtype_code(workloads.DTYPES[dtype])
    assert mdcn.mdcn_describe_plan(op, code, dims).startswith("path=%s " % plan)
    got = run_gpu(pr, inp, path)
    idx = sample_indices(tuple(got.shape), 8192, seed=13)
    ref = np.asarray(oracle.forward_points(inp["x"], inp["offset"], inp["mask"], inp["weight"],
                                           inp["bias"], idx, **pr.attrs()), dtype=np.float64)
    g = got.reshape(-1)[torch.from_numpy(idx)].double().numpy()
    err = np.abs(g - ref)
    ulp = ulp_of(ref, dtype)
    assert (err <= ulp).all(), (name, dtype, plan, float((err / ulp).max()),
                                int((err > ulp).sum()))
    # and the reference itself is not trivial: many distinct, mostly nonzero
    # values (a depthwise output sums only 9 grid products: fewer distinct ones)
    distinct = 500 if plan == "depthwise_direct" else 1000
    assert np.count_nonzero(ref) > 0.9 * ref.size and np.unique(ref).size > distinct


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_gather_gemm_workload_sampled(dtype):
    """The OCDNet-like stage on the gather + GEMM path (column buffer, chunks
    of images within the default column budget), random inputs, sampled
    outputs against the oracle."""
    pr, _ = workloads.WORKLOADS["ocdnet_n4_c256_160x160"]
    print("gather_gemm workload", dtype, flush=True)
    inp = workloads.generate(pr, dtype, seed=0)
    got = run_gpu(pr, inp, mdcn.MDCN_PATH_GATHER_GEMM)
    idx = sample_indices(tuple(got.shape), 4096, seed=14)
    ref = oracle.forward_points(inp["x"], inp["offset"], inp["mask"], inp["weight"],
                                inp["bias"], idx, **pr.attrs())
    g = got.reshape(-1)[torch.from_numpy(idx)].double().numpy()
    rms = float(np.sqrt(np.mean(np.asarray(ref, dtype=np.float64) ** 2)))
    ok, err, bound = within_tolerance(g, ref, dtype, rms=rms)
    assert ok, (dtype, error_report(g, ref), float((err / bound).max()))
    assert torch.isfinite(got).all()


# ---------------------------------------------------------------- every GEMM tile shape

GEMM_TILES = range(6)


@pytest.mark.parametrize("tile", GEMM_TILES)
@pytest.mark.parametrize("name,dtype", [("multi_tile_dg2", "f16"), ("multi_tile_dg2", "f32"),
                                        ("grouped_strided", "bf16"), ("odd_channels", "f16")])
def test_every_gemm_tile(tile, name, dtype, monkeypatch):
    """The planner's tile override (MDCN_GEMM_TILE) forces each GEMM tile shape."""
    monkeypatch.setenv("MDCN_GEMM_TILE", str(tile))
    pr = SMALL[name]
    inp = workloads.generate(pr, dtype, seed=12)
    got = run_gpu(pr, inp, mdcn.MDCN_PATH_GATHER_GEMM).double().numpy()
    ref = oracle_full(pr, inp)
    ok, err, bound = within_tolerance(got, ref, dtype)
    assert ok, (tile, name, dtype, error_report(got, ref))


# ---------------------------------------------------------------- depthwise kernel variants

@pytest.mark.parametrize("entry,pixels", [(16, 1), (16, 2), (8, 1), (8, 2), (4, 1), (4, 2),
                                          (2, 1)])
@pytest.mark.parametrize("name,dtype", [("depthwise_mult2", "f32"), ("depthwise_5x3", "f32"),
                                        ("depthwise_mult2", "f16"), ("depthwise_5x3", "bf16"),
                                        ("depthwise_mult6_odd", "f32")])
def test_depthwise_variants(entry, pixels, name, dtype, monkeypatch):
    """The staged depthwise kernel with each LDS entry width (channels staged
    interleaved per plane position) and pixels-per-thread setting
    (MDCN_DW_ENTRY / MDCN_DW_PIXELS; widths a problem cannot use fall back to
    the default)."""
    monkeypatch.setenv("MDCN_DW_ENTRY", str(entry))
    monkeypatch.setenv("MDCN_DW_PIXELS", str(pixels))
    pr = SMALL[name]
    inp = workloads.generate(pr, dtype, seed=14)
    got = run_gpu(pr, inp, mdcn.MDCN_PATH_DEPTHWISE).double().numpy()
    ref = oracle_full(pr, inp)
    ok, err, bound = within_tolerance(got, ref, dtype)
    assert ok, (entry, pixels, name, dtype, error_report(got, ref))


@pytest.mark.parametrize("blocks", [0, 1, 2, 5])
@pytest.mark.parametrize("entry", [16, 8, 4])
@pytest.mark.parametrize("name,dtype", [("depthwise_3x3_ragged", "f32"),
                                        ("depthwise_3x3_even", "f32"),
                                        ("depthwise_3x3_even", "f16"),
                                        ("depthwise_3x3_even", "bf16"),
                                        ("depthwise_3x3_ragged", "bf16")])
def test_depthwise_3x3_persistent(blocks, entry, name, dtype, monkeypatch):
    """3x3 depthwise with one output per input channel: the persistent
    kernel with 1, 2 and up to 5 channel blocks per workgroup (a workgroup's
    run crossing an image boundary; loader waves staging the next block),
    each LDS entry width the problem allows; blocks = 0 is the staged kernel
    (MDCN_DW_PERSISTENT=0)."""
    if blocks == 0:
        monkeypatch.setenv("MDCN_DW_PERSISTENT", "0")
    else:
        monkeypatch.setenv("MDCN_DW_PERSISTENT_BLOCKS", str(blocks))
    monkeypatch.setenv("MDCN_DW_ENTRY", str(entry))
    pr = SMALL[name]
    inp = workloads.generate(pr, dtype, seed=15)
    got = run_gpu(pr, inp, mdcn.MDCN_PATH_DEPTHWISE).double().numpy()
    ref = oracle_full(pr, inp)
    ok, err, bound = within_tolerance(got, ref, dtype)
    assert ok, (blocks, entry, name, dtype, error_report(got, ref))


@pytest.mark.parametrize("name,dtype,path", [
    ("multi_tile_dg2", "f32", mdcn.MDCN_PATH_GATHER_GEMM),
    ("fused_multi_tile", "f16", mdcn.MDCN_PATH_FUSED),
    ("fused_multi_tile", "f32", mdcn.MDCN_PATH_FUSED),
    ("window_multi_tile", "f16", mdcn.MDCN_PATH_WINDOW),
    ("window_grouped", "bf16", mdcn.MDCN_PATH_WINDOW),
    ("depthwise_mult2", "f32", mdcn.MDCN_PATH_DEPTHWISE),
    ("depthwise_5x3", "bf16", mdcn.MDCN_PATH_DEPTHWISE)])
def test_nonfinite_and_huge_offsets(name, dtype, path):
    """A NaN, infinite or far-off-image offset puts its sample off the image:
    it contributes 0, as in the oracle's zero-padded bilinear read (where any
    comparison with NaN fails).  One offset in ten is replaced."""
    pr = SMALL[name]
    inp = workloads.generate(pr, dtype, seed=21)
    flat = inp["offset"].clone().view(-1)
    g = torch.Generator().manual_seed(21)
    idx = torch.randperm(flat.numel(), generator=g)[: flat.numel() // 10]
    big = 1e30 if dtype == "f32" else 6e4
    vals = torch.tensor([float("nan"), float("inf"), float("-inf"), big, -big, 3e3])
    flat[idx] = vals[torch.arange(idx.numel()) % vals.numel()].to(flat.dtype)
    inp["offset"] = flat.view(inp["offset"].shape)
    got = run_gpu(pr, inp, path).double().numpy()
    ref = oracle_full(pr, inp)
    assert np.isfinite(ref).all()
    ok, err, bound = within_tolerance(got, ref, dtype)
    assert ok, (name, dtype, path, error_report(got, ref))


# ---------------------------------------------------------------- fused gather-GEMM tiles

@pytest.mark.parametrize("tile", range(4))
@pytest.mark.parametrize("name,dtype", [("fused_multi_tile", "f16"), ("fused_multi_tile", "f32"),
                                        ("fused_grouped", "bf16"), ("fused_narrow_dg", "f16")])
def test_every_fused_tile(tile, name, dtype, monkeypatch):
    """The planner's fused-tile override (MDCN_FUSED_TILE) forces each tile."""
    monkeypatch.setenv("MDCN_FUSED_TILE", str(tile))
    pr = SMALL[name]
    inp = workloads.generate(pr, dtype, seed=15)
    got = run_gpu(pr, inp, mdcn.MDCN_PATH_FUSED).double().numpy()
    ref = oracle_full(pr, inp)
    ok, err, bound = within_tolerance(got, ref, dtype)
    assert ok, (tile, name, dtype, error_report(got, ref))


def test_fused_matches_gather_gemm_closely():
    """Both paths round the same fp32 sums once; they agree far inside the
    tolerance (the column buffer rounds each sample to the storage dtype, the
    fused path rounds the same samples to the same dtype in LDS)."""
    pr = SMALL["fused_multi_tile"]
    inp = workloads.generate(pr, "f16", seed=16)
    a = run_gpu(pr, inp, mdcn.MDCN_PATH_FUSED).double()
    b = run_gpu(pr, inp, mdcn.MDCN_PATH_GATHER_GEMM).double()
    assert float((a - b).abs().max()) <= 2e-3


# ---------------------------------------------------------------- windowed fused kernel

@pytest.mark.parametrize("tile", range(4))
@pytest.mark.parametrize("margin", [2, 8])
@pytest.mark.parametrize("name,dtype", [("window_multi_tile", "f16"), ("window_grouped", "bf16"),
                                        ("window_far_offsets", "f16"),
                                        ("window_flat_ragged", "f16")])
def test_every_window_tile(tile, margin, name, dtype, monkeypatch):
    """Each tile shape (MDCN_WIN_TILE) with a narrow (many samples through
    the fallback) and the default margin (MDCN_WIN_MARGIN); a tile whose
    window does not fit falls back to the planner's choice."""
    monkeypatch.setenv("MDCN_WIN_TILE", str(tile))
    monkeypatch.setenv("MDCN_WIN_MARGIN", str(margin))
    pr = SMALL[name]
    print("window", name, dtype, tile, margin, flush=True)
    inp = workloads.generate(pr, dtype, seed=17)
    got = run_gpu(pr, inp, mdcn.MDCN_PATH_WINDOW).double().numpy()
    ref = oracle_full(pr, inp)
    ok, err, bound = within_tolerance(got, ref, dtype)
    assert ok, (tile, margin, name, dtype, error_report(got, ref))


def test_window_matches_fused_closely():
    """The windowed and the fused kernel round the same fp32 bilinear sums
    once to fp16 and accumulate in fp32 in different orders: they agree far
    inside the tolerance."""
    pr = SMALL["window_fused_cmp"]
    inp = workloads.generate(pr, "f16", seed=18)
    a = run_gpu(pr, inp, mdcn.MDCN_PATH_WINDOW).double()
    b = run_gpu(pr, inp, mdcn.MDCN_PATH_FUSED).double()
    assert float((a - b).abs().max()) <= 2e-3


@pytest.mark.parametrize("margin", [2, 8])
def test_window_exact_cases(margin, monkeypatch):
    """Exact results on the windowed kernel: a zero mask gives the bias, and
    samples off the image (far away, or exactly on h = -1) give the bias."""
    monkeypatch.setenv("MDCN_WIN_MARGIN", str(margin))
    pr = SMALL["window_multi_tile"]
    inp = workloads.generate(pr, "f16", seed=19)
    bias = inp["bias"][None, :, None, None]
    z = dict(inp, mask=torch.zeros_like(inp["mask"]))
    got = run_gpu(pr, z, mdcn.MDCN_PATH_WINDOW)
    assert torch.equal(got, bias.expand_as(got))
    far = torch.full_like(inp["offset"], 3.0e4)
    far[:, 1::4] = -3.0e4
    got = run_gpu(pr, dict(inp, offset=far), mdcn.MDCN_PATH_WINDOW)
    assert torch.equal(got, bias.expand_as(got))
    Ho, Wo = pr.out_hw()
    off = torch.zeros_like(inp["offset"])
    K = pr.kh * pr.kw
    for k in range(K):
        i = k // pr.kw
        anchor = torch.arange(Ho, dtype=torch.float32) * pr.stride[0] - pr.padding[0] \
            + i * pr.dilation[0]
        off[:, 2 * k] = (-1.0 - anchor)[:, None].to(off.dtype)
        off[:, 2 * k + 1] = 0.25
    got = run_gpu(pr, dict(inp, offset=off), mdcn.MDCN_PATH_WINDOW)
    assert torch.equal(got, bias.expand_as(got))


def assert_tiles_split(pr, inp, monkeypatch, workspace_bytes=None):
    """Some output tile really is split between two workgroups in this
    configuration: with the hand-over wait forced to give up at once
    (MDCN_WIN_SPIN_LIMIT=0) the forward reports MDCN_E_SYNC.  (The work split
    keeps tiles whole when it can, so a workgroup count alone proves nothing.)"""
    monkeypatch.setenv("MDCN_WIN_SPIN_LIMIT", "0")
    with pytest.raises(mdcn.MdcnError) as e:
        run_gpu(pr, inp, mdcn.MDCN_PATH_WINDOW, workspace_bytes=workspace_bytes)
    assert e.value.status == mdcn.MDCN_E_SYNC
    monkeypatch.delenv("MDCN_WIN_SPIN_LIMIT")


@pytest.mark.parametrize("ctas,name,dtype", [
    (3, "window_split_chunks", "f16"), (5, "window_split_chunks", "f16"),
    (7, "window_split_chunks", "bf16"), (7, "window_split_chunks", "f16"),
    (7, "window_multi_tile", "f16"), (11, "window_multi_tile", "bf16"),
    (3, "window_grouped", "bf16")])
def test_window_split_tiles(ctas, name, dtype, monkeypatch):
    """Fewer workgroups than tiles (MDCN_WIN_CTAS): the (tile, chunk) units
    are split into contiguous ranges, tiles span two workgroups and are
    combined through the partial-sum slots."""
    monkeypatch.setenv("MDCN_WIN_CTAS", str(ctas))
    pr = SMALL[name]
    print("window split", name, dtype, ctas, flush=True)
    inp = workloads.generate(pr, dtype, seed=20)
    assert_tiles_split(pr, inp, monkeypatch)
    got = run_gpu(pr, inp, mdcn.MDCN_PATH_WINDOW).double().numpy()
    ref = oracle_full(pr, inp)
    ok, err, bound = within_tolerance(got, ref, dtype)
    assert ok, (ctas, name, dtype, error_report(got, ref))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_window_split_least_workspace(dtype, monkeypatch):
    """Split tiles with the least workspace: one image per launch, so the
    forward makes several launches, each publishing with its own flag value
    (epoch 1, 2, ...) into the same slots.  (An image has 4 tiles of 8
    chunks; 3 workgroups cut two of them.)"""
    monkeypatch.setenv("MDCN_WIN_CTAS", "3")
    pr = Problem(N=3, C=128, Co=64, H=32, W=32, offset_dist=("normal", 2.0))
    inp = workloads.generate(pr, dtype, seed=23)
    op = make_op(pr, mdcn.MDCN_PATH_WINDOW)
    dims = [pr.N, pr.C, pr.H, pr.W] + list(inp["offset"].shape) + list(inp["mask"].shape) + \
        list(inp["weight"].shape)
    code = mdcn.dtype_code(workloads.DTYPES[dtype])
    _, least = mdcn.mdcn_workspace_bytes(op, code, dims)
    assert "chunk=1" in mdcn.mdcn_describe_plan(op, code, dims, least)
    assert_tiles_split(pr, inp, monkeypatch, workspace_bytes=least)
    tr = mdcn.Trace(64)
    got = run_gpu(pr, inp, mdcn.MDCN_PATH_WINDOW, workspace_bytes=least, trace=tr)
    assert len([n for n, _ in tr.read() if n == "window_gather_gemm"]) == pr.N
    ok, err, bound = within_tolerance(got.double().numpy(), oracle_full(pr, inp), dtype)
    assert ok, error_report(got.double().numpy(), oracle_full(pr, inp))


def test_window_handover_giveup_is_reported(monkeypatch):
    """A workgroup that finishes a tile begun by another waits for that one's
    partial sums for a bounded number of polls.  With the bound forced to
    zero from the host (MDCN_WIN_SPIN_LIMIT=0) every such wait gives up at
    once: the kernels still exit normally, the affected tiles come out NaN
    and mdcn_forward_check reports MDCN_E_SYNC.  The next forward on the same
    workspace, with the normal bound, is clean again."""
    # 4 output tiles of 8 chunks each over 3 workgroups: range boundaries
    # fall inside tiles, so tiles are split
    pr = Problem(N=1, C=128, Co=64, H=32, W=32, offset_dist=("normal", 2.0))
    inp = workloads.generate(pr, "f16", seed=24)
    g = to_dev(inp)
    op = make_op(pr, mdcn.MDCN_PATH_WINDOW)
    dims = mdcn.dims_of(g["x"], g["offset"], g["mask"], g["weight"])
    nbytes, _ = mdcn.mdcn_workspace_bytes(op, mdcn.MDCN_F16, dims)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    monkeypatch.setenv("MDCN_WIN_CTAS", "3")
    monkeypatch.setenv("MDCN_WIN_SPIN_LIMIT", "0")
    out = mdcn.forward(op, g["x"], g["offset"], g["mask"], g["weight"], g["bias"],
                       workspace=ws)
    stream = torch.cuda.current_stream().cuda_stream
    st = mdcn.mdcn_forward_check(op, mdcn.MDCN_F16, dims, ws.data_ptr(), ws.numel(), stream)
    assert st == mdcn.MDCN_E_SYNC
    bad = torch.isnan(out).cpu()
    assert bool(bad.any()) and not bool(bad.all())
    with pytest.raises(mdcn.MdcnError) as e:
        mdcn.forward(op, g["x"], g["offset"], g["mask"], g["weight"], g["bias"],
                     workspace=ws, check=True)
    assert e.value.status == mdcn.MDCN_E_SYNC
    monkeypatch.delenv("MDCN_WIN_SPIN_LIMIT")
    out = mdcn.forward(op, g["x"], g["offset"], g["mask"], g["weight"], g["bias"],
                       workspace=ws, check=True)
    got = out.cpu().double().numpy()
    assert np.isfinite(got).all()
    ok, err, bound = within_tolerance(got, oracle_full(pr, inp), "f16")
    assert ok, error_report(got, oracle_full(pr, inp))


@pytest.mark.parametrize("path,dtype", [(mdcn.MDCN_PATH_DIRECT, "f32"),
                                        (mdcn.MDCN_PATH_GATHER_GEMM, "f32"),
                                        (mdcn.MDCN_PATH_FUSED, "f16"),
                                        (mdcn.MDCN_PATH_WINDOW, "f16")])
def test_nonfinite_pixel_off_image_corners(path, dtype):
    """x[n][c][0][0] is NaN (x[n][c][0][1] is +inf) and the samples sit on
    the top-left border, many with corners off the image.  A corner off the
    image reads 0 and never that pixel, so an output is non-finite exactly
    where the definition makes it so: where some tap really reaches one of
    those pixels (the oracle's non-finite pattern), and finite elsewhere."""
    pr = Problem(N=2, C=64, Co=32, H=12, W=12, offset_dist=("normal", 1.0))
    inp = workloads.generate(pr, dtype, seed=26)
    x = inp["x"].clone()
    x[:, :, 0, 0] = float("nan")
    x[:, :, 0, 1] = float("inf")
    off = inp["offset"].clone()
    off[:, 0::2] = -0.5 - off[:, 0::2].abs()              # every sample moves up
    msk = (inp["mask"].float().clamp(0.2, 1.0)).to(inp["mask"].dtype)   # no zero mask
    inp = dict(inp, x=x, offset=off.to(inp["offset"].dtype), mask=msk)
    got = run_gpu(pr, inp, path).double().numpy()
    ref = oracle_full(pr, inp)
    bad_ref = ~np.isfinite(ref)
    assert bad_ref.any() and not bad_ref.all()
    assert np.array_equal(~np.isfinite(got), bad_ref)
    fin = ~bad_ref
    ok, err, bound = within_tolerance(got[fin], ref[fin], dtype)
    assert ok, float((err - bound).max())


def test_forward_check_other_paths():
    """Paths without a hand-over wait always report MDCN_OK."""
    pr = SMALL["multi_tile_dg2"]
    inp = workloads.generate(pr, "f32", seed=25)
    for path in (mdcn.MDCN_PATH_GATHER_GEMM, mdcn.MDCN_PATH_DIRECT):
        run_gpu(pr, inp, path)


def test_window_split_matches_unsplit(monkeypatch):
    """Splitting a tile between workgroups only changes the fp32 summation
    order: the result stays within a few fp16 ulps of the unsplit one."""
    pr = SMALL["window_multi_tile"]
    inp = workloads.generate(pr, "f16", seed=22)
    a = run_gpu(pr, inp, mdcn.MDCN_PATH_WINDOW).double()
    monkeypatch.setenv("MDCN_WIN_CTAS", "11")
    b = run_gpu(pr, inp, mdcn.MDCN_PATH_WINDOW).double()
    assert float((a - b).abs().max()) <= 2e-3


@pytest.mark.parametrize("name", ["ocdnet_n4_c256_160x160", "deep_n16_c512_40x40"])
def test_window_workload_sampled(name):
    """Full-size fp16 workloads on the windowed kernel (one workgroup per CU,
    tiles split between workgroups), sampled outputs against the oracle."""
    pr, _ = workloads.WORKLOADS[name]
    print("window workload", name, flush=True)
    inp = workloads.generate(pr, "f16", seed=0)
    got = run_gpu(pr, inp, mdcn.MDCN_PATH_WINDOW)
    idx = sample_indices(tuple(got.shape), 4096, seed=12)
    ref = oracle.forward_points(inp["x"], inp["offset"], inp["mask"], inp["weight"],
                                inp["bias"], idx, **pr.attrs())
    g = got.reshape(-1)[torch.from_numpy(idx)].double().numpy()
    rms = float(np.sqrt(np.mean(np.asarray(ref, dtype=np.float64) ** 2)))
    ok, err, bound = within_tolerance(g, ref, "f16", rms=rms)
    assert ok, (name, error_report(g, ref), float((err / bound).max()))
    assert torch.isfinite(got).all()
