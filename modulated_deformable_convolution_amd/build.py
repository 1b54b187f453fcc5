"""Build libmdcn.so (the C-ABI library with its gfx950 HIP kernels) in-tree.

    python -m modulated_deformable_convolution_amd.build

compiles every source under csrc/ with hipcc for gfx950 and links
modulated_deformable_convolution_amd/libmdcn.so.  Object files go to _build/
(ignored by git).
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libmdcn.so")

SOURCES = ["plan.cpp", "api.cpp", "prep.hip", "gather.hip", "gemm.hip", "depthwise.hip",
           "fused.hip", "window.hip", "direct.hip", "backward.hip", "noalloc.hip"]
HEADERS = ["plan.h", "launch.h", "device_common.h", "mfma_common.h", "entry.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # No packed-fp32 instructions anywhere (v_pk_{add,mul,fma}_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
    "-Wall", "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile all sources and link the library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    # Every symbol must resolve (a kernel whose host stub went missing shows
    # up here as an undefined symbol, not later at import).
    import ctypes
    ctypes.CDLL(tmp, mode=os.RTLD_NOW | os.RTLD_LOCAL)
    os.replace(tmp, LIBRARY)
    if verbose:
        print("built", LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
