"""GPU parity of the windowed FP8 path (MDCN_PATH_WINDOW_FP8) against the
oracle's FP8 mode (oracle.forward_fp8: each modulated bilinear sample and
each scaled weight row rounded to E4M3, exact sums, one rounding of
2^-e * sum + bias to the output type).

The windowed kernel computes every sample in fp32 from its LDS window (or,
for a sample whose corners leave the window, from global memory), saturates
and rounds it to E4M3, and sums four taps of 16 channels per 64-deep FP8
matrix instruction (the ninth tap of a chunk on the 16-deep one).  The same
two tolerances as the FP8 gather + GEMM path apply:
- grid inputs (workloads.generate_grid): every sample is an E4M3 number and
  every product a small multiple of a power of two, which the FP8 matrix
  instructions sum exactly, so the result is the oracle's up to the output
  rounding (one unit in the last place of fp16/bf16);
- random inputs: the dtype's tolerance plus 2^-11 * S, S the oracle's sum of
  absolute scaled products of the output (the instruction's own summing
  error, below 2^-12 * S, and a sample whose fp32 and exact values straddle
  an E4M3 rounding midpoint).
Covered: several tiles with ragged edges, partial output-channel tiles,
groups, strides and dilations, samples through the global-memory fallback,
every tile shape, tiles split between workgroups (hand-overs through the
workspace), the least workspace (one image per launch), saturation, a zero
mask, 30 seeded random problems the windowed kernel takes, and the two
benchmark workloads at full size (grid inputs exactly, random inputs within
tolerance, in the launch configuration the benchmark times).
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
WFP8 = mdcn.MDCN_PATH_WINDOW_FP8

CASES = {
    # Co = 288: a partial second output-channel tile; 37 x 37 pixels: ragged
    # 16 x 16 tiles; 2 chunks
    "multi_tile": Problem(N=2, C=32, Co=288, H=37, W=37, offset_dist=("normal", 3.0)),
    # stride (2, 1), dilation (1, 2), 2 groups inside 2 offset groups, Mg = 48
    "grouped": Problem(N=2, C=64, Co=96, H=23, W=19, stride=(2, 1), padding=(1, 2),
                       dilation=(1, 2), groups=2, deformable_groups=2,
                       offset_dist=("normal", 2.0)),
    # offsets up to 20 px: many samples off the image or outside the window
    # (the global-memory fallback)
    "far_offsets": Problem(N=1, C=16, Co=32, H=30, W=30, offset_dist=("uniform", 20.0),
                           mask_dist=("uniform_zeros", 0.1)),
    # 3 chunks (an odd count: the window buffers alternate unevenly), 13 x 21
    "three_chunks": Problem(N=2, C=48, Co=64, H=13, W=21, offset_dist=("normal", 2.0)),
    # 4 output tiles per image of 8 chunks each (split between workgroups
    # below)
    "split_chunks": Problem(N=2, C=128, Co=64, H=32, W=32, offset_dist=("normal", 2.0)),
}


def make_op(pr, path=WFP8):
    return mdcn.mdcn_create(pr.stride, pr.padding, pr.dilation, pr.groups,
                            pr.deformable_groups, path=path)


def run(pr, inp, path=WFP8, workspace_bytes=None, trace=None):
    g = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    ws = None
    if workspace_bytes is not None:
        ws = torch.empty(max(workspace_bytes, 1), dtype=torch.uint8, device=DEV)
    # check: mdcn_forward_check reports a hand-over wait that gave up
    out = mdcn.forward(make_op(pr, path), g["x"], g["offset"], g["mask"], g["weight"],
                       g["bias"], workspace=ws, trace=trace, check=True)
    torch.cuda.synchronize()
    return out.cpu().double().numpy()


def ulp(r, dtype):
    """One unit in the last place of r in the output type (subnormals included)."""
    if dtype == "f16":
        return np.spacing(np.abs(r).astype(np.float16)).astype(np.float64)
    a = np.maximum(np.abs(r), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def fp8_ref(pr, inp):
    return oracle.forward_fp8(inp["x"], inp["offset"], inp["mask"], inp["weight"], inp["bias"],
                              **pr.attrs())


def assert_grid_exact(got, ref, dtype, what):
    err = np.abs(got - ref)
    assert (err <= ulp(ref, dtype)).all(), (what, dtype, float(err.max()),
                                           error_report(got, ref))


def assert_random_close(got, ref, asum, dtype, what, rms=None):
    _, err, bound = within_tolerance(got, ref, dtype, rms=rms)
    bound = bound + 2.0 ** -11 * asum
    assert (err <= bound).all(), (what, dtype, float((err / bound).max()),
                                  error_report(got, ref))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_window_fp8_grid_inputs_exact(name, dtype):
    pr = CASES[name]
    print("window fp8 grid", name, dtype, flush=True)
    inp = workloads.generate_grid(pr, dtype, seed=1)
    ref, _ = fp8_ref(pr, inp)
    tr = mdcn.Trace(16)
    got = run(pr, inp, trace=tr)
    assert [n for n, _ in tr.read()] == ["prep_blocks_fp8", "window_gather_gemm_fp8"]
    assert_grid_exact(got, ref, dtype, name)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_window_fp8_random_inputs(name, dtype):
    pr = CASES[name]
    print("window fp8 random", name, dtype, flush=True)
    inp = workloads.generate(pr, dtype, seed=2)
    ref, asum = fp8_ref(pr, inp)
    got = run(pr, inp)
    assert_random_close(got, ref, asum, dtype, name)


@pytest.mark.parametrize("tile,margin", [(0, 8), (1, 2), (2, 8), (3, 3)])
@pytest.mark.parametrize("name", ["multi_tile", "far_offsets", "three_chunks"])
def test_window_fp8_every_tile(tile, margin, name, monkeypatch):
    """Each 256-pixel tile shape (MDCN_WIN_TILE; MDCN_WIN_WIDE=0 keeps the
    groups of more than 256 channels on them) with a narrow margin (many
    samples through the fallback) or the default one (MDCN_WIN_MARGIN)."""
    monkeypatch.setenv("MDCN_WIN_WIDE", "0")
    monkeypatch.setenv("MDCN_WIN_TILE", str(tile))
    monkeypatch.setenv("MDCN_WIN_MARGIN", str(margin))
    pr = CASES[name]
    print("window fp8 tile", name, tile, margin, flush=True)
    inp = workloads.generate_grid(pr, "f16", seed=3)
    ref, _ = fp8_ref(pr, inp)
    assert_grid_exact(run(pr, inp), ref, "f16", (name, tile, margin))


@pytest.mark.parametrize("ctas,name,dtype", [(3, "split_chunks", "f16"),
                                             (7, "split_chunks", "bf16"),
                                             (11, "multi_tile", "f16"),
                                             (3, "grouped", "bf16")])
def test_window_fp8_split_tiles(ctas, name, dtype, monkeypatch):
    """Fewer workgroups than tiles (MDCN_WIN_CTAS): tiles split between two
    workgroups pass their first chunks' sums through the workspace; a forced
    give-up (MDCN_WIN_SPIN_LIMIT=0) shows that some tile really is split.
    (256-pixel tiles: MDCN_WIN_WIDE=0; the wide ones are split below.)"""
    monkeypatch.setenv("MDCN_WIN_WIDE", "0")
    monkeypatch.setenv("MDCN_WIN_CTAS", str(ctas))
    pr = CASES[name]
    print("window fp8 split", name, dtype, ctas, flush=True)
    inp = workloads.generate_grid(pr, dtype, seed=4)
    monkeypatch.setenv("MDCN_WIN_SPIN_LIMIT", "0")
    with pytest.raises(mdcn.MdcnError) as e:
        run(pr, inp)
    assert e.value.status == mdcn.MDCN_E_SYNC
    monkeypatch.delenv("MDCN_WIN_SPIN_LIMIT")
    ref, _ = fp8_ref(pr, inp)
    assert_grid_exact(run(pr, inp), ref, dtype, (name, ctas))
    rnd = workloads.generate(pr, dtype, seed=5)
    ref, asum = fp8_ref(pr, rnd)
    assert_random_close(run(pr, rnd), ref, asum, dtype, (name, ctas))


def test_window_fp8_least_workspace(monkeypatch):
    """One image per launch (the least workspace), with split tiles: the
    weight is quantized once, in the first launch's set-up, and every later
    image's x goes to 8-channel blocks in a launch of its own."""
    monkeypatch.setenv("MDCN_WIN_CTAS", "3")
    pr = Problem(N=3, C=128, Co=64, H=32, W=32, offset_dist=("normal", 2.0))
    inp = workloads.generate_grid(pr, "f16", seed=6)
    op = make_op(pr)
    dims = [pr.N, pr.C, pr.H, pr.W] + list(inp["offset"].shape) + list(inp["mask"].shape) + \
        list(inp["weight"].shape)
    _, least = mdcn.mdcn_workspace_bytes(op, mdcn.MDCN_F16, dims)
    assert "chunk=1" in mdcn.mdcn_describe_plan(op, mdcn.MDCN_F16, dims, least)
    tr = mdcn.Trace(64)
    got = run(pr, inp, workspace_bytes=least, trace=tr)
    names = [n for n, _ in tr.read()]
    assert names.count("prep_blocks_fp8") == 1 and names[0] == "prep_blocks_fp8"
    assert names.count("window_gather_gemm_fp8") == pr.N
    assert names.count("to_channel_blocks") == pr.N - 1
    ref, _ = fp8_ref(pr, inp)
    assert_grid_exact(got, ref, "f16", "least workspace")
    assert np.array_equal(got, run(pr, inp))


def test_window_fp8_agrees_with_gather_gemm_fp8():
    """Both FP8 paths round the same samples and weights; they differ only in
    the order of the fp32 sums (and in a sample whose fp32 value lies on an
    E4M3 rounding midpoint, which both compute identically in fp32)."""
    pr = CASES["grouped"]
    inp = workloads.generate(pr, "f16", seed=7)
    a = run(pr, inp)
    b = run(pr, inp, path=mdcn.MDCN_PATH_GATHER_GEMM_FP8)
    ref, asum = fp8_ref(pr, inp)
    _, err, bound = within_tolerance(a, b, "f16")
    assert (np.abs(a - b) <= bound + 2.0 ** -11 * asum).all()


def test_window_fp8_zero_mask_and_saturation():
    """A zero mask gives the bias exactly; samples beyond 448 saturate to 448
    as in the oracle (the converter alone would give NaN above 464)."""
    pr = CASES["multi_tile"]
    inp = workloads.generate(pr, "f16", seed=8)
    got = run(pr, dict(inp, mask=torch.zeros_like(inp["mask"])))
    want = np.broadcast_to(inp["bias"].double().numpy()[None, :, None, None], got.shape)
    assert np.array_equal(got, want)
    g = workloads.generate_grid(pr, "f16", seed=9)
    g["x"] = (g["x"].float() * 400.0).to(torch.float16)   # samples up to 1200
    ref, asum = fp8_ref(pr, g)
    got = run(pr, g)
    assert np.isfinite(got).all()
    assert_random_close(got, ref, asum, "f16", "saturation")


def sample_indices(pr, size, seed):
    """4096 random outputs plus the first and last row and column of the
    first and last channel of the first and last image (flat indices)."""
    N, Co, (Ho, Wo) = pr.N, pr.Co, pr.out_hw()
    rng = np.random.default_rng(seed)
    idx = [rng.integers(0, size, 4096)]
    for n in (0, N - 1):
        for co in (0, Co - 1):
            base = (n * Co + co) * Ho * Wo
            idx.append(base + np.arange(Wo))
            idx.append(base + (Ho - 1) * Wo + np.arange(Wo))
            idx.append(base + np.arange(Ho) * Wo)
            idx.append(base + np.arange(Ho) * Wo + Wo - 1)
    return np.unique(np.concatenate(idx))


@pytest.mark.parametrize("wl", ["ocdnet_n4_c256_160x160", "deep_n16_c512_40x40"])
def test_window_fp8_workload_full_size(wl):
    """The benchmark workloads at full size in the launch configuration the
    benchmark times (one workgroup per CU, tiles split between workgroups):
    grid inputs match the oracle exactly on sampled outputs, random inputs
    within the FP8 tolerance."""
    pr = workloads.WORKLOADS[wl][0]
    print("window fp8 full size", wl, flush=True)
    g = workloads.generate_grid(pr, "f16", seed=10)
    got = run(pr, g).reshape(-1)
    idx = sample_indices(pr, got.size, 11)
    ref, _ = oracle.forward_points_fp8(g["x"], g["offset"], g["mask"], g["weight"], g["bias"],
                                       idx, **pr.attrs())
    assert_grid_exact(got[idx], ref, "f16", wl)
    r = workloads.generate(pr, "f16", seed=0)
    got = run(pr, r).reshape(-1)
    ref, asum = oracle.forward_points_fp8(r["x"], r["offset"], r["mask"], r["weight"], r["bias"],
                                          idx, **pr.attrs())
    rms = float(np.sqrt(np.mean(ref ** 2)))
    assert_random_close(got[idx], ref, asum, "f16", wl, rms=rms)


def _random_cases(seed, count):
    """Problems the windowed kernel takes: 3x3, C/group a multiple of 16,
    offset groups that hold whole groups; strides, paddings, dilations,
    output channels, image sizes and offset spreads drawn at random (draws
    whose window does not fit are dropped by asking the planner)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        groups = int(rng.choice([1, 1, 2]))
        cg = int(rng.choice([16, 32, 48]))
        dg = int(rng.choice([d for d in (1, 2) if groups % d == 0]))
        pr = Problem(N=int(rng.integers(1, 3)), C=groups * cg,
                     Co=groups * int(rng.choice([8, 40, 96, 272])),
                     H=int(rng.integers(6, 40)), W=int(rng.integers(6, 40)),
                     stride=(int(rng.choice([1, 1, 2])), int(rng.choice([1, 2]))),
                     padding=(int(rng.integers(0, 3)), int(rng.integers(0, 3))),
                     dilation=(int(rng.choice([1, 1, 2])), int(rng.choice([1, 2]))),
                     groups=groups, deformable_groups=dg, bias=bool(rng.random() < 0.7),
                     offset_dist=(("normal", float(rng.choice([0.5, 2.0, 4.0])))
                                  if rng.random() < 0.8 else ("uniform", 12.0)),
                     mask_dist=(("uniform_zeros", 0.1) if rng.random() < 0.3
                                else ("sigmoid_normal",)))
        ho, wo = pr.out_hw()
        if ho < 1 or wo < 1:
            continue
        shapes = pr.shapes()
        dims = [int(v) for k in ("x", "offset", "mask", "weight") for v in shapes[k]]
        try:
            mdcn.mdcn_workspace_bytes(make_op(pr), mdcn.MDCN_F16, dims)
        except mdcn.MdcnError:
            continue                                  # no window fits this problem
        dtype = str(rng.choice(["f16", "bf16"]))
        out.append(pytest.param(pr, dtype, id=f"r{len(out)}-{dtype}"))
    return out


@pytest.mark.parametrize("pr,dtype", _random_cases(5151, 30))
def test_window_fp8_random_problems(pr, dtype):
    print("window fp8 random problem", pr, dtype, flush=True)
    g = workloads.generate_grid(pr, dtype, seed=12)
    ref, _ = fp8_ref(pr, g)
    assert_grid_exact(run(pr, g), ref, dtype, "grid")
    r = workloads.generate(pr, dtype, seed=13)
    ref, asum = fp8_ref(pr, r)
    assert_random_close(run(pr, r), ref, asum, dtype, "random")


# ---- wide tiles: groups of more than 256 output channels run 128-pixel x
# 512-channel tiles, the two waves of a SIMD sharing 32 pixels (each blends
# two of a group's four taps, or four of tap 8's eight channels, and passes
# its E4M3 bytes to the other through LDS).  The same tolerances apply: the
# samples, weights and sums are the same as on the 256-pixel tiles.
WIDE_CASES = {
    # Mg = 288: one 512-row tile with rows past Mg unused; 37 x 37 pixels
    "multi_tile": CASES["multi_tile"],
    # Mg = 512 exactly, 2 chunks, 21 x 19 pixels
    "full_rows": Problem(N=2, C=32, Co=512, H=21, W=19, offset_dist=("normal", 2.0)),
    # Mg = 640: a full and a partial channel tile, 3 chunks
    "two_row_tiles": Problem(N=1, C=48, Co=640, H=17, W=23, offset_dist=("normal", 3.0)),
    # 2 groups (Mg = 320) in 2 offset groups, stride (2, 1), dilation (1, 2)
    "grouped": Problem(N=2, C=64, Co=640, H=23, W=19, stride=(2, 1), padding=(1, 2),
                       dilation=(1, 2), groups=2, deformable_groups=2,
                       offset_dist=("normal", 2.0)),
    # offsets up to 20 px: the global-memory fallback on every local tap of
    # both waves of a pair (tap 8: each wave's half of the channels)
    "far_offsets": Problem(N=1, C=16, Co=320, H=24, W=26, offset_dist=("uniform", 20.0),
                           mask_dist=("uniform_zeros", 0.1)),
}


def _tile_of(pr, dtype):
    shapes = pr.shapes()
    dims = [int(v) for k in ("x", "offset", "mask", "weight") for v in shapes[k]]
    d = mdcn.mdcn_describe_plan(make_op(pr), mdcn.MDCN_F16 if dtype == "f16" else mdcn.MDCN_BF16,
                                dims)
    return int(d.split("tile=")[1].split()[0])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("name", sorted(WIDE_CASES))
def test_window_fp8_wide_grid_exact(name, dtype):
    pr = WIDE_CASES[name]
    print("window fp8 wide grid", name, dtype, flush=True)
    assert _tile_of(pr, dtype) in (4, 5, 6)
    inp = workloads.generate_grid(pr, dtype, seed=21)
    ref, _ = fp8_ref(pr, inp)
    tr = mdcn.Trace(16)
    got = run(pr, inp, trace=tr)
    assert [n for n, _ in tr.read()] == ["prep_blocks_fp8", "window_gather_gemm_fp8"]
    assert_grid_exact(got, ref, dtype, name)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("name", sorted(WIDE_CASES))
def test_window_fp8_wide_random(name, dtype):
    pr = WIDE_CASES[name]
    print("window fp8 wide random", name, dtype, flush=True)
    inp = workloads.generate(pr, dtype, seed=22)
    ref, asum = fp8_ref(pr, inp)
    assert_random_close(run(pr, inp), ref, asum, dtype, name)


@pytest.mark.parametrize("tile,margin", [(4, 8), (5, 2), (6, 8), (6, 2)])
@pytest.mark.parametrize("name", ["multi_tile", "two_row_tiles", "far_offsets"])
def test_window_fp8_wide_every_tile(tile, margin, name, monkeypatch):
    """Each wide tile shape with the widest margin that fits (at most the
    one asked) or a narrow one (many samples through the fallback)."""
    monkeypatch.setenv("MDCN_WIN_TILE", str(tile))
    monkeypatch.setenv("MDCN_WIN_MARGIN", str(margin))
    pr = WIDE_CASES[name]
    print("window fp8 wide tile", name, tile, margin, flush=True)
    assert _tile_of(pr, "f16") == tile
    inp = workloads.generate_grid(pr, "f16", seed=23)
    ref, _ = fp8_ref(pr, inp)
    assert_grid_exact(run(pr, inp), ref, "f16", (name, tile, margin))
    rnd = workloads.generate(pr, "bf16", seed=24)
    ref, asum = fp8_ref(pr, rnd)
    assert_random_close(run(pr, rnd), ref, asum, "bf16", (name, tile, margin))


@pytest.mark.parametrize("ctas,name,dtype", [(7, "full_rows", "f16"),
                                             (7, "two_row_tiles", "bf16"),
                                             (6, "grouped", "f16")])
def test_window_fp8_wide_split_tiles(ctas, name, dtype, monkeypatch):
    """Wide tiles split between workgroups (MDCN_WIN_CTAS; MDCN_WIN_SEG_X4=0
    balances chunks alone, so these few whole tiles do not stay whole); a
    forced give-up shows that some tile really is split."""
    monkeypatch.setenv("MDCN_WIN_CTAS", str(ctas))
    monkeypatch.setenv("MDCN_WIN_SEG_X4", "0")
    pr = WIDE_CASES[name]
    print("window fp8 wide split", name, dtype, ctas, flush=True)
    inp = workloads.generate_grid(pr, dtype, seed=25)
    monkeypatch.setenv("MDCN_WIN_SPIN_LIMIT", "0")
    with pytest.raises(mdcn.MdcnError) as e:
        run(pr, inp)
    assert e.value.status == mdcn.MDCN_E_SYNC
    monkeypatch.delenv("MDCN_WIN_SPIN_LIMIT")
    ref, _ = fp8_ref(pr, inp)
    assert_grid_exact(run(pr, inp), ref, dtype, (name, ctas))
    rnd = workloads.generate(pr, dtype, seed=26)
    ref, asum = fp8_ref(pr, rnd)
    assert_random_close(run(pr, rnd), ref, asum, dtype, (name, ctas))


@pytest.mark.parametrize("name", ["multi_tile", "two_row_tiles", "grouped"])
def test_window_fp8_narrow_tiles_on_wide_groups(name, monkeypatch):
    """MDCN_WIN_WIDE=0: the same groups on the 256-pixel tiles (each tile
    run once per 256-channel half).  On grid inputs both tilings sum exactly,
    so they agree bit for bit as well as with the oracle."""
    pr = WIDE_CASES[name]
    print("window fp8 narrow on wide groups", name, flush=True)
    inp = workloads.generate_grid(pr, "f16", seed=27)
    wide = run(pr, inp)
    monkeypatch.setenv("MDCN_WIN_WIDE", "0")
    assert _tile_of(pr, "f16") in (0, 1, 2, 3)
    narrow = run(pr, inp)
    ref, _ = fp8_ref(pr, inp)
    assert_grid_exact(narrow, ref, "f16", name)
    assert np.array_equal(wide, narrow)
