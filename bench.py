"""Benchmark of the modulated deformable convolution forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--dtype f16]

A step is one mdcn_forward call (every kernel of the path) on one batch of
seeded synthetic input of the named workload, already resident in device
memory.  W untimed steps, then K timed steps bracketed by device
synchronisation; then K more steps with per-kernel HIP events (the library's
tracing entry point, on the launch stream) for the kernel durations the
roofline figures use; then the CPU oracle on a bounded sample of the same
workload.  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "modulated deform-conv fwd effective GFLOP/s + HBM GB/s, % roofline, 1 GPU"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3, "fp8": 5000.0}
# fp32 FMAs on the vector ALUs without packed math (the kernels are built with
# packed fp32 off): 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz; the
# published 157.3 TF/s vector figure counts two-wide packed FMAs
VALU_FP32_TFLOPS = 78.6
ELEM = {"f32": 4, "f16": 2, "bf16": 2}
DEFAULT_WORKLOAD = "ocdnet_n4_c256_160x160"

# HBM traffic per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
# (scaled by 2.0 / 1.0, the factors a plain copy of known size gives; see
# profiles/*memory_counters.md), valid only for the kernel sources they were
# taken on (sha256 of the listed files, first 16 hex digits).
MEASURED_TRAFFIC = {
    ('deform_gather_fp8', 'ocdnet_n4_c256_160x160', 'f16'): {
        "bytes": (40450 * 2 + 230400) * 1024,
        "sources": ('gather.hip', 'device_common.h', 'plan.cpp', 'plan.h'),
        "sha": "116efe5da826d87e",
    },
    ('gemm_fp8_bias', 'ocdnet_n4_c256_160x160', 'f16'): {
        "bytes": (119933 * 2 + 51200) * 1024,
        "sources": ('gemm.hip', 'mfma_common.h', 'device_common.h', 'plan.cpp'),
        "sha": "4acbc1ebd6152ab1",
    },
    ('window_gather_gemm', 'ocdnet_n4_c256_160x160', 'f16'): {
        "bytes": (124405 * 2 + 116836) * 1024,
        "sources": ('window.hip', 'mfma_common.h', 'device_common.h', 'plan.cpp', 'plan.h'),
        "sha": "93a731dbcdfce33a",
    },
    ('window_gather_gemm', 'deep_n16_c512_40x40', 'f16'): {
        "bytes": (32163 * 2 + 25709) * 1024,
        "sources": ('window.hip', 'mfma_common.h', 'device_common.h', 'plan.cpp', 'plan.h'),
        "sha": "93a731dbcdfce33a",
    },
    ('window_gather_gemm_fp8', 'ocdnet_n4_c256_160x160', 'f16'): {
        "bytes": (114914 * 2 + 116890) * 1024,
        "sources": ('window.hip', 'mfma_common.h', 'device_common.h', 'plan.cpp', 'plan.h'),
        "sha": "93a731dbcdfce33a",
    },
    ('window_gather_gemm_fp8', 'deep_n16_c512_40x40', 'f16'): {
        "bytes": (22923 * 2 + 25602) * 1024,
        "sources": ('window.hip', 'mfma_common.h', 'device_common.h', 'plan.cpp', 'plan.h'),
        "sha": "93a731dbcdfce33a",
    },
    ('fused_gather_gemm', 'ocdnet_n4_c256_160x160', 'f16'): {
        "bytes": (53920 * 2 + 51200) * 1024,
        "sources": ('fused.hip', 'mfma_common.h', 'device_common.h', 'plan.cpp', 'plan.h'),
        "sha": "53dfca86e4afcaff",
    },
    ('gemm_bias', 'ocdnet_n4_c256_160x160', 'f16'): {
        "bytes": (119950 * 2 + 25600) * 1024,
        "sources": ('gemm.hip', 'mfma_common.h', 'device_common.h', 'plan.cpp'),
        "sha": "4acbc1ebd6152ab1",
    },
    ('deform_gather', 'ocdnet_n4_c256_160x160', 'f16'): {
        "bytes": (23283 * 2 + 230400) * 1024,
        "sources": ('gather.hip', 'device_common.h', 'plan.cpp'),
        "sha": "a7330ce3959e9adb",
    },
    ('depthwise_direct', 'depthwise_n8_c256_96x96', 'f32'): {
        "bytes": (47349 * 2 + 73728) * 1024,
        "sources": ('depthwise.hip', 'device_common.h'),
        "sha": "6edca1bd9b79c9cc",
    },
}


def sources_sha(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "modulated_deformable_convolution_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_model(pr, dtype, plan_chunk, plan_geo=False):
    """Algorithmic bytes and flops of one launch of each kernel, for a launch
    over `cnt` images.  Bytes count each tensor a kernel must touch once."""
    e = ELEM[dtype]
    Ho, Wo = pr.out_hw()
    P = Ho * Wo
    K = pr.kh * pr.kw
    Cg, Mg, G = pr.C // pr.groups, pr.Co // pr.groups, pr.groups
    Kg = Cg * K
    Kp = (Kg + 63) // 64 * 64
    dg = pr.deformable_groups
    x_img = pr.C * pr.H * pr.W * e
    off_img = 2 * dg * K * P * e
    msk_img = dg * K * P * e
    out_img = pr.Co * P * e
    w_bytes = pr.Co * Cg * K * e
    bias_bytes = pr.Co * e if pr.bias else 0
    col_img = G * P * Kp * e
    Kp8 = (Kg + 127) // 128 * 128          # FP8 path: one byte per value, 128-byte K steps
    col_img8 = G * P * Kp8
    wq_bytes = pr.Co * Kp8 + 4 * pr.Co     # E4M3 weight and fp32 row scales
    wqw_bytes = pr.Co * (Cg // 16) * 144 + 4 * pr.Co   # windowed FP8: E4M3 chunk blocks, scales

    def per_launch(name, cnt):
        if name == "pack_weight":
            return dict(bytes=w_bytes + pr.Co * Kp * e, flops=0)
        if name == "pack_weight_steps":
            return dict(bytes=2 * w_bytes, flops=0)
        if name in ("to_nhwc", "to_channel_blocks"):
            return dict(bytes=2 * cnt * x_img, flops=0)
        if name in ("prep_nhwc", "prep_blocks"):
            # the weight repacked and the first chunk's x moved, in one launch
            first = min(plan_chunk, pr.N)
            wb = w_bytes + pr.Co * Kp * e if name == "prep_nhwc" else 2 * w_bytes
            return dict(bytes=wb + 2 * first * x_img, flops=0)
        if name == "deform_gather":
            # x read once, offsets and masks read once, columns written once
            return dict(bytes=cnt * (x_img + off_img + msk_img + col_img),
                        flops=0)
        if name == "gemm_bias":
            return dict(bytes=cnt * (col_img + out_img) + pr.Co * Kp * e + bias_bytes,
                        flops=2 * cnt * pr.Co * Kg * P)
        if name == "fused_one_launch":
            # the whole forward: x (NCHW), offsets, masks and the weight read
            # once, output written once (the NHWC copy and the packed weight
            # it makes on the way are not counted)
            return dict(bytes=cnt * (x_img + off_img + msk_img + out_img) + w_bytes + bias_bytes,
                        flops=2 * cnt * pr.Co * Kg * P)
        if name in ("fused_gather_gemm", "window_gather_gemm"):
            # x (NHWC copy), offsets and masks read once, output written once
            return dict(bytes=cnt * (x_img + off_img + msk_img + out_img) + pr.Co * Kp * e
                        + bias_bytes, flops=2 * cnt * pr.Co * Kg * P)
        if name == "prep_blocks_fp8":
            # the weight rounded to E4M3 chunk blocks and the first chunk's x
            # moved to 8-channel blocks, in one launch
            first = min(plan_chunk, pr.N)
            return dict(bytes=w_bytes + wqw_bytes + 2 * first * x_img, flops=0)
        if name == "window_gather_gemm_fp8":
            # as window_gather_gemm, with the E4M3 weight
            return dict(bytes=cnt * (x_img + off_img + msk_img + out_img) + wqw_bytes
                        + bias_bytes, flops=2 * cnt * pr.Co * Kg * P)
        if name == "prep_nhwc_fp8":
            # the weight rounded to E4M3 and the first chunk's x moved, in one launch
            first = min(plan_chunk, pr.N)
            return dict(bytes=w_bytes + wq_bytes + 2 * first * x_img, flops=0)
        if name == "deform_gather_fp8":
            return dict(bytes=cnt * (x_img + off_img + msk_img + col_img8), flops=0)
        if name == "gemm_fp8_bias":
            return dict(bytes=cnt * (col_img8 + out_img) + wq_bytes + bias_bytes,
                        flops=2 * cnt * pr.Co * Kg * P)
        if name == "direct":
            # one launch over every image: x, offsets, masks and weight read
            # once, output written once
            return dict(bytes=cnt * (x_img + off_img + msk_img + out_img) + w_bytes + bias_bytes,
                        flops=2 * cnt * pr.Co * Kg * P)
        if name == "depthwise_geometry":
            # offsets and masks read once, a 16-byte record per offset group, tap
            # and pixel written once
            return dict(bytes=cnt * (off_img + msk_img + 16 * dg * K * P), flops=0)
        if name == "depthwise_direct":
            # with the geometry (staged kernel): x and the geometry read
            # once, output written once; without it (plain kernel): x,
            # offsets and masks
            geo_in = 16 * dg * K * P if plan_geo else off_img + msk_img
            return dict(bytes=cnt * (x_img + geo_in + out_img) + w_bytes + bias_bytes,
                        flops=2 * cnt * pr.Co * Kg * P)
        raise KeyError(name)
    return per_launch


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--dtype", default=None, help="f32 | f16 | bf16 (default: the workload's "
                    "lowest-precision dtype)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", default="auto", choices=["auto", "gather_gemm", "fused",
                                                       "window", "depthwise", "direct",
                                                       "gather_gemm_fp8", "window_fp8"],
                    help="computation path (default: the library's choice; gather_gemm_fp8 "
                         "and window_fp8 compute with E4M3 operands, a reduced-precision "
                         "result)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph that holds one captured forward (the "
                         "launch mode for small problems) instead of eager forwards")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (mdcn_backward, fp32) instead of the forward")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-mebibyte device buffer --steps times (a plain copy "
                         "of known size, to scale memory-traffic counters) and exit")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on exactly one GPU; --gpus %d (WORLD_SIZE %d) is not "
              "supported. The forward shards by image with no collective; only the one-GPU "
              "figure is measured." % (args.gpus, world), file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from modulated_deformable_convolution_amd import mdcn, workloads

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"copy_bytes": n, "steps": args.steps, "ms": dt * 1e3,
                          "gbs_read_plus_write": 2 * n / dt / 1e9}))
        return 0

    if not os.path.exists(mdcn.LIBRARY):
        from modulated_deformable_convolution_amd import build
        build.build()

    pr, dtypes = workloads.WORKLOADS[args.workload]
    dtype = args.dtype or ("f16" if "f16" in dtypes else "bf16" if "bf16" in dtypes else dtypes[0])
    if args.backward:
        return bench_backward(args, pr)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    inp = workloads.generate(pr, dtype, seed=0)
    g = {k: (v.to(dev) if v is not None else None) for k, v in inp.items()}
    path = {"auto": mdcn.MDCN_PATH_AUTO, "gather_gemm": mdcn.MDCN_PATH_GATHER_GEMM,
            "fused": mdcn.MDCN_PATH_FUSED, "window": mdcn.MDCN_PATH_WINDOW,
            "depthwise": mdcn.MDCN_PATH_DEPTHWISE, "direct": mdcn.MDCN_PATH_DIRECT,
            "gather_gemm_fp8": mdcn.MDCN_PATH_GATHER_GEMM_FP8,
            "window_fp8": mdcn.MDCN_PATH_WINDOW_FP8}[args.path]
    fp8 = args.path in ("gather_gemm_fp8", "window_fp8")
    op = mdcn.mdcn_create(pr.stride, pr.padding, pr.dilation, pr.groups, pr.deformable_groups,
                          path=path)
    code = mdcn.dtype_code(g["x"].dtype)
    dims = mdcn.dims_of(g["x"], g["offset"], g["mask"], g["weight"])
    ws_bytes, _ = mdcn.mdcn_workspace_bytes(op, code, dims)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    out = torch.empty(mdcn.mdcn_output_shape(op, dims), dtype=g["x"].dtype, device=dev)
    plan = mdcn.mdcn_describe_plan(op, code, dims)
    stream = torch.cuda.current_stream(dev)

    def step(trace=None):
        mdcn.forward(op, g["x"], g["offset"], g["mask"], g["weight"], g["bias"], out=out,
                     workspace=ws, stream=stream.cuda_stream, trace=trace)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timed = step
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                mdcn.forward(op, g["x"], g["offset"], g["mask"], g["weight"], g["bias"],
                             out=out, workspace=ws)
        stream.wait_stream(side)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        timed = graph.replay
    t0 = time.perf_counter()
    for _ in range(args.steps):
        timed()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # Per-call device time, warm (back to back) and cold (a 1 GiB scrub
    # buffer written between calls, outside the events, so that the 256 MB
    # Infinity Cache and the L2 hold none of the inputs): events on the
    # stream the forward runs on; median, p10, p90.
    def per_call_ms(scrub):
        times = []
        for i in range(args.steps):
            if scrub is not None:
                scrub.fill_(i & 255)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        q = np.percentile(np.asarray(times), [50, 10, 90])
        return {"median_ms": round(float(q[0]), 5), "p10_ms": round(float(q[1]), 5),
                "p90_ms": round(float(q[2]), 5)}
    warm_calls = per_call_ms(None)
    scrub = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold_calls = per_call_ms(scrub)
    cold_calls["scrub_bytes"] = scrub.numel()
    del scrub

    # Per-kernel device time: HIP events around every launch, on the stream
    # the kernels run on.
    trace = mdcn.Trace(capacity=64 * args.steps + 64)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        step(trace)
    torch.cuda.synchronize()
    per_kernel = {}
    for name, ms in trace.read():
        d = per_kernel.setdefault(name, [0, 0.0])
        d[0] += 1
        d[1] += ms
    chunk = 1
    for tok in plan.split():
        if tok.startswith("chunk="):
            chunk = int(tok.split("=")[1])
    model = kernel_model(pr, dtype, chunk, plan_geo="depthwise_geometry" in per_kernel)
    kernels = {}
    for name, (count, total_ms) in per_kernel.items():
        avg_ms = total_ms / count
        launches_per_step = count / args.steps
        cnt = (pr.N / max(1, launches_per_step)
               if name in ("direct", "to_nhwc", "to_channel_blocks", "deform_gather", "gemm_bias",
                           "fused_gather_gemm", "fused_one_launch", "window_gather_gemm",
                           "window_gather_gemm_fp8", "depthwise_geometry",
                           "depthwise_direct", "deform_gather_fp8", "gemm_fp8_bias")
               else 0)
        m = model(name, cnt)
        kernels[name] = dict(launches_per_step=launches_per_step, avg_ms=avg_ms,
                             ms_per_step=total_ms / args.steps,
                             algo_bytes_per_launch=m["bytes"],
                             algo_flops_per_launch=m["flops"],
                             gbs=m["bytes"] / (avg_ms * 1e-3) / 1e9,
                             tflops=m["flops"] / (avg_ms * 1e-3) / 1e12)
    dominant = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dominant]
    peak_tf = MFMA_PEAK_TFLOPS["fp8" if fp8 else dtype]
    t_hbm = dk["algo_bytes_per_launch"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = dk["algo_flops_per_launch"] / (peak_tf * 1e12)
    uses_mfma = dominant in ("gemm_bias", "fused_gather_gemm", "fused_one_launch",
                             "window_gather_gemm", "window_gather_gemm_fp8", "gemm_fp8_bias")
    if uses_mfma and t_mfma > t_hbm:
        roofline = dict(bound="mfma", achieved=round(dk["tflops"], 2), peak=peak_tf,
                        unit="TFLOP/s", frac=round(dk["tflops"] / peak_tf, 4), traffic=None)
    else:
        roofline = dict(bound="hbm", achieved=round(dk["gbs"], 1), peak=HBM_PEAK_GBS,
                        unit="GB/s", frac=round(dk["gbs"] / HBM_PEAK_GBS, 4), traffic=None)
    roofline["kernel"] = dominant
    meas = MEASURED_TRAFFIC.get((dominant, args.workload, dtype))
    if meas and sources_sha(meas["sources"]) == meas["sha"]:
        roofline["traffic"] = meas["bytes"]

    flops = pr.flops()
    value = flops / (ms_per_step * 1e-3) / 1e9
    e = ELEM[dtype]
    Ho, Wo = pr.out_hw()
    K = pr.kh * pr.kw
    min_bytes = e * (pr.N * pr.C * pr.H * pr.W + pr.N * 3 * pr.deformable_groups * K * Ho * Wo
                     + pr.Co * (pr.C // pr.groups) * K + (pr.Co if pr.bias else 0)
                     + pr.N * pr.Co * Ho * Wo)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(pr, inp, args.cpu_seconds)
        cpu["cpu_model"] = cpu_model()
        cpu["other_configs"] = cpu_baseline_other_configs(min(2.0, args.cpu_seconds / 4))

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if fp8 else dtype,
        "data": "synthetic (seeded; OCDNet-shaped stand-in, no dataset or weights)",
        "config": {"workload": args.workload, "N": pr.N, "C": pr.C, "Co": pr.Co,
                   "H": pr.H, "W": pr.W, "kernel": [pr.kh, pr.kw], "stride": list(pr.stride),
                   "padding": list(pr.padding), "dilation": list(pr.dilation),
                   "group": pr.groups, "deformable_group": pr.deformable_groups,
                   "bias": pr.bias, "io_dtype": dtype, "accumulate": "f32",
                   "operands": "e4m3 (reduced precision)" if fp8 else dtype,
                   "parallelism": "single GPU",
                   "launch": "graph replay" if args.graph else "eager"},
        "hbm_gbs_effective": round(min_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "per_call": {"warm": warm_calls, "cold": cold_calls},
        "plan": plan,
        "roofline": roofline,
        "kernels": {k: {kk: (round(vv, 6) if isinstance(vv, float) else vv)
                        for kk, vv in v.items()} for k, v in kernels.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))
    return 0


def backward_model(pr):
    """Algorithmic bytes and flops of one launch of each backward kernel
    (fp32; the per-image kernels cover one image)."""
    e = 4
    Ho, Wo = pr.out_hw()
    P = Ho * Wo
    K = pr.kh * pr.kw
    Cg, G, dg = pr.C // pr.groups, pr.groups, pr.deformable_groups
    Kg = Cg * K
    Kp = (Kg + 63) // 64 * 64
    x_img = pr.C * pr.H * pr.W * e
    om_img = 3 * dg * K * P * e
    table = {
        "bwd_zero": dict(bytes=x_img, flops=0),        # per image: the NHWC grad_x buffer
        "pack_weight": dict(bytes=pr.Co * Kg * e + pr.Co * Kp * e, flops=0),
        "bwd_to_nchw": dict(bytes=2 * x_img, flops=0),
        "bwd_bias": dict(bytes=pr.N * pr.Co * P * e + pr.Co * e, flops=0),
        "to_nhwc": dict(bytes=2 * x_img, flops=0),
        "deform_gather": dict(bytes=x_img + om_img + G * P * Kp * e, flops=0),
        "bwd_weight_gemm": dict(bytes=pr.Co * P * e + G * P * Kp * e + pr.Co * Kp * e,
                                flops=2 * pr.Co * Kg * P),
        "bwd_col_gemm": dict(bytes=pr.Co * Kp * e + pr.Co * P * e + G * P * Kp * e,
                             flops=2 * pr.Co * Kg * P),
        "bwd_sample": dict(bytes=2 * x_img + 2 * om_img + G * P * Kp * e, flops=0),
        "bwd_weight_out": dict(bytes=2 * pr.Co * Kg * e, flops=0),
    }
    return table


def bench_backward(args, pr):
    """The backward pass on the workload's shapes in fp32: gradients of all
    five inputs from a random grad_out.  One JSON line like the forward's;
    `value` is 2x the forward's effective flops (the two contractions) per
    second."""
    import torch
    from modulated_deformable_convolution_amd import mdcn, workloads
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = workloads.generate(pr, "f32", seed=0)
    g = {k: (v.to(dev) if v is not None else None) for k, v in inp.items()}
    ho, wo = pr.out_hw()
    go = torch.randn((pr.N, pr.Co, ho, wo), generator=torch.Generator().manual_seed(1)).to(dev)
    op = mdcn.mdcn_create(pr.stride, pr.padding, pr.dilation, pr.groups, pr.deformable_groups)
    dims = mdcn.dims_of(g["x"], g["offset"], g["mask"], g["weight"])
    wsb = mdcn.mdcn_backward_workspace_bytes(op, mdcn.MDCN_F32, dims)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(g["x"]), torch.empty_like(g["offset"]), torch.empty_like(g["mask"]),
            torch.empty_like(g["weight"]), torch.empty(pr.Co, device=dev)]
    stream = torch.cuda.current_stream(dev)

    def step(trace=None):
        st = mdcn.mdcn_backward(op, mdcn.MDCN_F32, dims, g["x"].data_ptr(),
                                g["offset"].data_ptr(), g["mask"].data_ptr(),
                                g["weight"].data_ptr(), go.data_ptr(),
                                *[t.data_ptr() for t in outs], pr.Co, ws.data_ptr(), ws.numel(),
                                stream.cuda_stream, trace)
        if st != mdcn.MDCN_OK:
            raise mdcn.MdcnError(st, "mdcn_backward")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    trace = mdcn.Trace(capacity=(8 * pr.N + 8) * args.steps + 64)
    for _ in range(args.steps):
        step(trace)
    torch.cuda.synchronize()
    per = {}
    for name, ms in trace.read():
        d = per.setdefault(name, [0, 0.0])
        d[0] += 1
        d[1] += ms
    model = backward_model(pr)
    kernels = {}
    for name, (count, total) in per.items():
        avg = total / count
        m = model[name]
        kernels[name] = dict(launches_per_step=count / args.steps, avg_ms=round(avg, 6),
                             ms_per_step=round(total / args.steps, 6),
                             algo_bytes_per_launch=m["bytes"], algo_flops_per_launch=m["flops"],
                             gbs=round(m["bytes"] / (avg * 1e-3) / 1e9, 1),
                             tflops=round(m["flops"] / (avg * 1e-3) / 1e12, 3))
    dominant = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dominant]
    # the two contractions run on the fp32 MFMA GEMM for one group with Co a
    # multiple of 32 (the weight gradient also needs Ho*Wo a multiple of 32),
    # else on a VALU kernel (fp32 FMAs, no packed math: half the published
    # 157.3 TF/s vector peak, which counts packed fp32)
    ho, wo = pr.out_hw()
    on_mfma = {"bwd_col_gemm": pr.groups == 1 and pr.Co % 32 == 0,
               "bwd_weight_gemm": pr.groups == 1 and pr.Co % 32 == 0 and (ho * wo) % 32 == 0}
    if dk["algo_flops_per_launch"] and on_mfma.get(dominant, False):
        roofline = dict(bound="mfma", achieved=dk["tflops"], peak=MFMA_PEAK_TFLOPS["f32"],
                        unit="TFLOP/s", frac=round(dk["tflops"] / MFMA_PEAK_TFLOPS["f32"], 4),
                        traffic=None, kernel=dominant)
    elif dk["algo_flops_per_launch"]:
        roofline = dict(bound="alu", achieved=dk["tflops"], peak=VALU_FP32_TFLOPS,
                        unit="TFLOP/s", frac=round(dk["tflops"] / VALU_FP32_TFLOPS, 4),
                        traffic=None, kernel=dominant)
    else:
        roofline = dict(bound="hbm", achieved=dk["gbs"], peak=HBM_PEAK_GBS, unit="GB/s",
                        frac=round(dk["gbs"] / HBM_PEAK_GBS, 4), traffic=None, kernel=dominant)
    flops = 2 * pr.flops()
    line = {
        "metric": "backward effective GFLOP/s (2 x forward flops per backward)",
        "value": round(flops / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded; OCDNet-shaped stand-in, no dataset or weights)",
        "config": {"workload": args.workload, "pass": "backward", "N": pr.N, "C": pr.C,
                   "Co": pr.Co, "H": pr.H, "W": pr.W, "kernel": [pr.kh, pr.kw],
                   "group": pr.groups, "deformable_group": pr.deformable_groups},
        "roofline": roofline, "kernels": kernels, "cpu_baseline": None,
    }
    print(json.dumps(line))
    return 0


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(pr, inp, target_s, threads=None):
    """The oracle, untouched, on a bounded random sample of the same
    workload's outputs; scaled to effective GFLOP/s.  threads: OpenMP threads
    (None: the runtime's default, every core)."""
    import numpy as np
    from oracle import oracle
    default_threads = oracle.max_threads()
    oracle.set_threads(threads or default_threads)
    Ho, Wo = pr.out_hw()
    total = pr.N * pr.Co * Ho * Wo
    Kg = (pr.C // pr.groups) * pr.kh * pr.kw
    rng = np.random.default_rng(0)
    attrs = pr.attrs()
    # inputs converted once (not timed)
    x = inp["x"].double().numpy()
    off = inp["offset"].double().numpy()
    msk = inp["mask"].double().numpy()
    w = inp["weight"].double().numpy()
    b = inp["bias"].double().numpy() if inp["bias"] is not None else None
    n = 256
    elapsed = 0.0
    while True:
        idx = rng.choice(total, size=min(n, total), replace=False)
        t0 = time.perf_counter()
        oracle.forward_points(x, off, msk, w, b, idx, **attrs)
        elapsed = time.perf_counter() - t0
        if elapsed >= target_s or n >= total:
            break
        n = min(total, int(n * max(2.0, min(16.0, 1.2 * target_s / max(elapsed, 1e-3)))))
    reps = 1
    if elapsed < 0.2:
        # the whole output takes too little time to measure once: repeat it
        reps = max(1, int(math.ceil(0.2 / max(elapsed, 1e-5))))
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.forward_points(x, off, msk, w, b, idx, **attrs)
        elapsed = (time.perf_counter() - t0) / reps
    flops = 2.0 * len(idx) * Kg
    used = oracle.max_threads()
    oracle.set_threads(default_threads)
    return {"value": round(flops / elapsed / 1e9, 3), "unit": "GFLOP/s",
            "cores": used, "kind": "oracle",
            "sample": "%d random output elements of the same workload (seed 0), %.3f s%s" %
                      (len(idx), elapsed, (" (mean of %d runs)" % reps) if reps > 1 else "")}


def cpu_baseline_other_configs(target_s):
    """The oracle on the tiny, strided/grouped and depthwise configurations,
    on every core and on one thread (bounded samples, seed 0, each
    configuration's own dtype)."""
    from modulated_deformable_convolution_amd import workloads
    out = {}
    for name in ("tiny_n1_c4_8x8", "strided_grouped_n2_c128_co256_128x128",
                 "depthwise_n8_c256_96x96"):
        pr, dtypes = workloads.WORKLOADS[name]
        inp = workloads.generate(pr, dtypes[0], seed=0)
        out[name] = {"dtype": dtypes[0],
                     "all_cores": cpu_baseline(pr, inp, target_s),
                     "one_thread": cpu_baseline(pr, inp, target_s, threads=1)}
    return out


if __name__ == "__main__":
    sys.exit(main())
