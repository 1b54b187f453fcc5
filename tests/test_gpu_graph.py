"""The forward captured into a HIP graph and replayed.

For problems whose kernels take a few microseconds (the tiny and the
strided/grouped configurations), launching the forward's kernels one by one
costs more than the kernels themselves; a caller captures `mdcn_forward` into
a graph once and replays it.  The forward issues only kernel launches on the
caller's stream (no allocation, no memset, no synchronisation; the window
path's hand-over flags are cleared by a kernel), so it can be captured.

Each test captures one forward per path, replays it several times with eager
work between the replays and new input values written into the captured
buffers, and checks every replay against an eager forward on the same values
(bit for bit: the same kernels on the same data) and, for small problems,
against the oracle.
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

CASES = [
    ("tiny", workloads.TINY, "f32", mdcn.MDCN_PATH_AUTO),
    ("strided_grouped", workloads.WORKLOADS["strided_grouped_n2_c128_co256_128x128"][0], "bf16",
     mdcn.MDCN_PATH_AUTO),
    ("gather_gemm", Problem(N=2, C=32, Co=48, H=15, W=13, deformable_groups=2,
                            offset_dist=("normal", 2.0)), "f16", mdcn.MDCN_PATH_GATHER_GEMM),
    ("window", Problem(N=2, C=32, Co=288, H=37, W=37, offset_dist=("normal", 3.0)), "f16",
     mdcn.MDCN_PATH_WINDOW),
    # the same with 7 workgroups (MDCN_WIN_CTAS): 3 of its 24 tiles split
    # between two of them, partial sums handed over through the workspace on
    # every replay
    ("window_split", Problem(N=2, C=32, Co=288, H=37, W=37, offset_dist=("normal", 3.0)), "f16",
     mdcn.MDCN_PATH_WINDOW),
    ("depthwise", Problem(N=2, C=24, Co=48, H=13, W=13, groups=24, deformable_groups=3,
                          offset_dist=("uniform", 8.0), mask_dist=("uniform_zeros", 0.1)),
     "f32", mdcn.MDCN_PATH_DEPTHWISE),
    # 3x3 depthwise, one output per channel: the persistent kernel with two
    # channel blocks per workgroup (MDCN_DW_PERSISTENT_BLOCKS), its loader
    # waves staging the second block on every replay
    ("depthwise_persistent", Problem(N=2, C=16, Co=16, H=30, W=35, groups=16,
                                     deformable_groups=2, offset_dist=("uniform", 12.0),
                                     mask_dist=("uniform_zeros", 0.1)),
     "f32", mdcn.MDCN_PATH_DEPTHWISE),
    ("gather_gemm_fp8", Problem(N=2, C=32, Co=48, H=15, W=13, deformable_groups=2,
                                offset_dist=("normal", 2.0)), "f16",
     mdcn.MDCN_PATH_GATHER_GEMM_FP8),
    # the windowed FP8 kernel, whole tiles and (MDCN_WIN_CTAS=7) split ones
    ("window_fp8", Problem(N=2, C=32, Co=288, H=37, W=37, offset_dist=("normal", 3.0)), "bf16",
     mdcn.MDCN_PATH_WINDOW_FP8),
    ("window_fp8_split", Problem(N=2, C=32, Co=288, H=37, W=37, offset_dist=("normal", 3.0)),
     "f16", mdcn.MDCN_PATH_WINDOW_FP8),
]


def _dev(inp):
    return {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}


@pytest.mark.parametrize("name,pr,dtype,path", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(name, pr, dtype, path, monkeypatch):
    if name in ("window_split", "window_fp8_split"):
        monkeypatch.setenv("MDCN_WIN_CTAS", "7")
    if name == "depthwise_persistent":
        monkeypatch.setenv("MDCN_DW_PERSISTENT_BLOCKS", "2")
    op = mdcn.mdcn_create(pr.stride, pr.padding, pr.dilation, pr.groups, pr.deformable_groups,
                          path=path)
    inputs = [workloads.generate(pr, dtype, seed=s) for s in (0, 1, 2)]
    g = _dev(inputs[0])
    shapes = pr.shapes()
    dims = [int(v) for k in ("x", "offset", "mask", "weight") for v in shapes[k]]
    code = mdcn.dtype_code(workloads.DTYPES[dtype])
    nbytes, _ = mdcn.mdcn_workspace_bytes(op, code, dims)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV)
    out = torch.empty(mdcn.mdcn_output_shape(op, dims), dtype=g["x"].dtype, device=DEV)

    # eager references, one per input set, each with its own buffers
    eager = []
    for inp in inputs:
        e = _dev(inp)
        eager.append(mdcn.forward(op, e["x"], e["offset"], e["mask"], e["weight"], e["bias"]))
    torch.cuda.synchronize()

    # capture (after an eager call on the same buffers: the kernels' one-time
    # set-up is done outside the capture)
    mdcn.forward(op, g["x"], g["offset"], g["mask"], g["weight"], g["bias"], out=out,
                 workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            mdcn.forward(op, g["x"], g["offset"], g["mask"], g["weight"], g["bias"], out=out,
                         workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(6):
        k = rep % 3
        # new values into the captured buffers, then unrelated eager work
        for key in ("x", "offset", "mask", "weight", "bias"):
            if g[key] is not None:
                g[key].copy_(inputs[k][key].to(DEV))
        out.fill_(float("nan"))
        scratch = torch.randn(1 << 16, device=DEV).sum()
        graph.replay()
        scratch.item()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[k]), f"{name}: replay {rep} differs from the eager forward"
        stream = torch.cuda.current_stream().cuda_stream
        assert mdcn.mdcn_forward_check(op, code, dims, ws.data_ptr(), ws.numel(),
                                       stream) == mdcn.MDCN_OK

    if name in ("tiny", "gather_gemm", "depthwise", "depthwise_persistent"):
        inp = inputs[2]
        ref = oracle.forward(inp["x"], inp["offset"], inp["mask"], inp["weight"], inp["bias"],
                             **pr.attrs())
        ok, err, bound = within_tolerance(out.cpu().double().numpy(), np.asarray(ref), dtype)
        assert ok, f"{name}: max error {err.max():.3g}, worst margin {(err - bound).max():.3g}"
