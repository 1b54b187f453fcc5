"""The fused forward in one launch (opt-in: MDCN_FUSED_ONE=1).

When asked for, a problem that takes the fused gather-GEMM path with the
whole batch in one chunk and a grid of at most one workgroup per CU runs as a
single kernel: its workgroups move x to the NHWC copy and repack the weight
themselves, meet at a bounded grid barrier, and then run the fused GEMM.  The
arithmetic is that of the two-launch forward (prep kernel + fused kernel), so
the two agree bit for bit; both are compared with the oracle.

Covered here: which kernels a traced forward records, bit equality with the
two-launch forward (MDCN_FUSED_ONE=0) on small and full-size problems, every
dtype, the fallback a workgroup takes when it gives up waiting (forced for
every workgroup with MDCN_FUSED_ONE_SPIN=0), new inputs through the same
workspace (nothing stale is read through the caches), and a captured forward,
which keeps the two launches.
"""
import pytest
import torch

from helpers import ensure_built, error_report, within_tolerance

ensure_built()
from modulated_deformable_convolution_amd import mdcn, workloads  # noqa: E402
from modulated_deformable_convolution_amd.workloads import Problem  # noqa: E402
from oracle import oracle  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

STRIDED = workloads.WORKLOADS["strided_grouped_n2_c128_co256_128x128"][0]

SMALL = {
    # grouped, strided, dilated, 3x2 kernel, 4 offset groups, Mg = 48
    "grouped": Problem(N=2, C=128, Co=96, H=17, W=15, kh=3, kw=2, stride=(2, 1),
                       padding=(2, 1), dilation=(2, 1), groups=2, deformable_groups=4,
                       offset_dist=("normal", 1.5)),
    # Co = 160 (rows of a partial weight tile), 3 x 169 pixels (ragged
    # columns and a ragged last pixel tile of the transpose)
    "multi_tile": Problem(N=3, C=64, Co=160, H=13, W=13, deformable_groups=2,
                          offset_dist=("normal", 2.0)),
    # C = 192: a partial 64-channel tile of the transpose; group 1 spans
    # offset groups 0 and 1
    "misaligned_groups": Problem(N=2, C=192, Co=96, H=9, W=11, groups=3, deformable_groups=2,
                                 offset_dist=("normal", 2.0)),
    # H*W = 256 and C a multiple of 64: x moves in 16-byte chunks (the
    # others above move element by element)
    "aligned_strided": Problem(N=2, C=128, Co=96, H=16, W=16, stride=(2, 2), padding=(2, 2),
                               dilation=(2, 2), groups=2, deformable_groups=4,
                               offset_dist=("normal", 2.0)),
    # 5x5 taps
    "k5x5": Problem(N=2, C=64, Co=64, H=11, W=10, kh=5, kw=5, padding=(2, 2),
                    offset_dist=("normal", 2.0)),
}


def _dev(inp):
    return {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}


def _op(pr):
    return mdcn.mdcn_create(pr.stride, pr.padding, pr.dilation, pr.groups,
                            pr.deformable_groups, path=mdcn.MDCN_PATH_FUSED)


def _forward(pr, g, workspace=None, trace=None):
    out = mdcn.forward(_op(pr), g["x"], g["offset"], g["mask"], g["weight"], g["bias"],
                       workspace=workspace, trace=trace, check=True)
    torch.cuda.synchronize()
    return out


@pytest.fixture(autouse=True)
def _one_launch_on(monkeypatch):
    monkeypatch.setenv("MDCN_FUSED_ONE", "1")


def _two_launch(pr, g, monkeypatch):
    with monkeypatch.context() as m:
        m.setenv("MDCN_FUSED_ONE", "0")
        tr = mdcn.Trace(16)
        out = _forward(pr, g, trace=tr)
        assert [n for n, _ in tr.read()] == ["prep_nhwc", "fused_gather_gemm"]
    return out


def _oracle(pr, inp):
    return oracle.forward(inp["x"], inp["offset"], inp["mask"], inp["weight"], inp["bias"],
                          **pr.attrs())


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("name", list(SMALL))
def test_one_launch_matches_two_launches_and_oracle(name, dtype, monkeypatch):
    pr = SMALL[name]
    print("case", name, dtype, flush=True)
    inp = workloads.generate(pr, dtype, seed=41)
    g = _dev(inp)
    tr = mdcn.Trace(16)
    one = _forward(pr, g, trace=tr)
    assert [n for n, _ in tr.read()] == ["fused_one_launch"]
    two = _two_launch(pr, g, monkeypatch)
    assert torch.equal(one, two)
    ref = _oracle(pr, inp)
    got = one.cpu().double().numpy()
    ok, err, bound = within_tolerance(got, ref, dtype)
    assert ok, (name, dtype, error_report(got, ref))


@pytest.mark.parametrize("name,dtype", [("grouped", "bf16"), ("multi_tile", "f32"),
                                        ("misaligned_groups", "f16"),
                                        ("aligned_strided", "bf16"), ("aligned_strided", "f32")])
def test_fallback_when_the_wait_gives_up(name, dtype, monkeypatch):
    """With no polls allowed every workgroup gives up at once and moves all
    of x and the whole weight itself: slower, and the same result."""
    pr = SMALL[name]
    print("case", name, dtype, flush=True)
    inp = workloads.generate(pr, dtype, seed=42)
    g = _dev(inp)
    two = _two_launch(pr, g, monkeypatch)
    with monkeypatch.context() as m:
        m.setenv("MDCN_FUSED_ONE_SPIN", "0")
        tr = mdcn.Trace(16)
        late = _forward(pr, g, trace=tr)
        assert [n for n, _ in tr.read()] == ["fused_one_launch"]
    assert torch.equal(late, two)


def test_new_inputs_through_the_same_workspace(monkeypatch):
    """Forwards on different x, weights, offsets and masks through one
    workspace buffer: each result is that of its own inputs (no NHWC copy or
    packed weight of an earlier call is read through a cache)."""
    pr = SMALL["grouped"]
    op = _op(pr)
    shapes = pr.shapes()
    dims = [int(v) for k in ("x", "offset", "mask", "weight") for v in shapes[k]]
    full, _ = mdcn.mdcn_workspace_bytes(op, mdcn.MDCN_BF16, dims)
    ws = torch.empty(full, dtype=torch.uint8, device=DEV)
    outs, refs = [], []
    for seed in (43, 44, 45, 46):
        inp = workloads.generate(pr, "bf16", seed=seed)
        g = _dev(inp)
        outs.append(_forward(pr, g, workspace=ws).clone())
        refs.append(_two_launch(pr, g, monkeypatch))
    for a, b in zip(outs, refs):
        assert torch.equal(a, b)
    assert not torch.equal(outs[0], outs[1])


def test_full_size_strided_grouped(monkeypatch):
    """The strided/dilated/grouped bf16 configuration (256 workgroups, one
    per CU): one kernel, the same output as the two-launch forward, for two
    input sets in a row."""
    for seed in (0, 7):
        inp = workloads.generate(STRIDED, "bf16", seed=seed)
        g = _dev(inp)
        tr = mdcn.Trace(16)
        one = _forward(STRIDED, g, trace=tr)
        assert [n for n, _ in tr.read()] == ["fused_one_launch"]
        two = _two_launch(STRIDED, g, monkeypatch)
        assert torch.equal(one, two)


def test_captured_forward_keeps_two_launches():
    """Under stream capture the forward records the two-launch sequence (a
    replayed one-launch kernel would reuse its barrier ticket); replays with
    new x match eager forwards."""
    pr = SMALL["grouped"]
    inp = workloads.generate(pr, "bf16", seed=47)
    g = _dev(inp)
    op = _op(pr)
    static_out = torch.empty(mdcn.mdcn_output_shape(op, mdcn.dims_of(g["x"], g["offset"],
                                                                     g["mask"], g["weight"])),
                             dtype=g["x"].dtype, device=DEV)
    ws_bytes, _ = mdcn.mdcn_workspace_bytes(op, mdcn.MDCN_BF16,
                                            mdcn.dims_of(g["x"], g["offset"], g["mask"],
                                                         g["weight"]))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mdcn.forward(op, g["x"], g["offset"], g["mask"], g["weight"], g["bias"], out=static_out,
                     workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mdcn.forward(op, g["x"], g["offset"], g["mask"], g["weight"], g["bias"], out=static_out,
                     workspace=ws)
    torch.cuda.synchronize()
    for seed in (48, 49, 50):
        new = workloads.generate(pr, "bf16", seed=seed)
        g["x"].copy_(new["x"].to(DEV))
        graph.replay()
        torch.cuda.synchronize()
        replayed = static_out.clone()
        eager = _forward(pr, g)
        assert torch.equal(replayed, eager)
