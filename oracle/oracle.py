"""CPU oracle for the modulated deformable 2-D convolution forward (DCNv2).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the GPU library and its binding never
do.  The arithmetic lives in ``mdcn_oracle.c`` (plain C, double precision,
one output element at a time, straight from the definition on the page
"TensorRT 插件解析：modulatedDeformConvPlugin 可变形卷积插件的原理、参数与使用指南",
§二, §三 and §五 steps 1-3).  This module only compiles that file with gcc,
loads it with ctypes and marshals arrays.

Inputs are converted to float64 exactly: every fp32, fp16 and bf16 value is
representable in float64, so the oracle sees the very values the GPU reads.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "mdcn_oracle.c")
LIBRARY = os.path.join(_HERE, "libmdcn_oracle.so")

_lock = threading.Lock()
_lib = None


def compile_library(source: str = SOURCE, output: str = LIBRARY, extra_flags=()) -> str:
    """Build the oracle shared library with gcc (-O2, OpenMP, no fast-math);
    extra_flags: e.g. sanitizer options for a checking build."""
    tmp = output + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off"] + list(extra_flags) + [
           source, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, output)
    return output


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int64)
    lib.mdcn_oracle_forward.argtypes = [dp, dp, dp, dp, dp, ip, dp]
    lib.mdcn_oracle_forward.restype = ctypes.c_int
    lib.mdcn_oracle_points.argtypes = [dp, dp, dp, dp, dp, ip, ctypes.c_int64, ip, dp]
    lib.mdcn_oracle_points.restype = ctypes.c_int
    lib.mdcn_oracle_points_fp8.argtypes = [dp, dp, dp, dp, dp, ip, ctypes.c_int64, ip, dp, dp,
                                           dp, dp]
    lib.mdcn_oracle_points_fp8.restype = ctypes.c_int
    lib.mdcn_oracle_e4m3_array.argtypes = [dp, ctypes.c_int64, dp]
    lib.mdcn_oracle_e4m3_array.restype = None
    lib.mdcn_oracle_fp8_row_exponent.argtypes = [dp, ctypes.c_int64]
    lib.mdcn_oracle_fp8_row_exponent.restype = ctypes.c_int
    lib.mdcn_oracle_backward.argtypes = [dp, dp, dp, dp, dp, ip, dp, dp, dp, dp, dp]
    lib.mdcn_oracle_backward.restype = ctypes.c_int
    lib.mdcn_oracle_max_threads.argtypes = []
    lib.mdcn_oracle_max_threads.restype = ctypes.c_int
    lib.mdcn_oracle_set_threads.argtypes = [ctypes.c_int]
    lib.mdcn_oracle_set_threads.restype = None
    return lib


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load (building first if absent) the oracle library.

    With ``path`` given, that exact file is loaded, which lets a test load a
    deliberately altered build of the oracle."""
    global _lib
    if path is None:
        # a checking build (e.g. under sanitizers) in place of the default one
        path = os.environ.get("MDCN_ORACLE_LIBRARY") or None
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(LIBRARY) or (
                    os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)):
                compile_library()
            _lib = _bind(ctypes.CDLL(LIBRARY))
        return _lib


def max_threads(lib: ctypes.CDLL | None = None) -> int:
    return int((lib or load_library()).mdcn_oracle_max_threads())


def set_threads(n: int, lib: ctypes.CDLL | None = None) -> None:
    """OpenMP threads for the following calls (timing only; results do not
    depend on it)."""
    (lib or load_library()).mdcn_oracle_set_threads(int(n))


def _f64(a) -> np.ndarray:
    if a is None:
        return None
    if hasattr(a, "detach"):  # a torch tensor
        a = a.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _pair(v):
    if isinstance(v, int):
        return (v, v)
    return (int(v[0]), int(v[1]))


def problem(x_shape, offset_shape, weight_shape, stride, padding, dilation,
            groups, deformable_groups) -> np.ndarray:
    """The 17-value problem description the C functions take.

    Output spatial size comes from the offset tensor's dims 2 and 3
    [plugin guide §二, getOutputShapes]."""
    N, C, H, W = x_shape
    Co, _, kh, kw = weight_shape
    Ho, Wo = offset_shape[2], offset_shape[3]
    sh, sw = _pair(stride)
    ph, pw = _pair(padding)
    dh, dw = _pair(dilation)
    return np.array([N, C, H, W, Co, kh, kw, Ho, Wo, sh, sw, ph, pw, dh, dw,
                     groups, deformable_groups], dtype=np.int64)


def forward(x, offset, mask, weight, bias=None, stride=1, padding=0, dilation=1,
            groups=1, deformable_groups=1, lib: ctypes.CDLL | None = None) -> np.ndarray:
    """Every output element, float64, shape [N, Co, Ho, Wo]."""
    lib = lib or load_library()
    x, offset, mask, weight, bias = map(_f64, (x, offset, mask, weight, bias))
    p = problem(x.shape, offset.shape, weight.shape, stride, padding, dilation,
                groups, deformable_groups)
    out = np.empty((x.shape[0], weight.shape[0], offset.shape[2], offset.shape[3]),
                   dtype=np.float64)
    rc = lib.mdcn_oracle_forward(_ptr(x), _ptr(offset), _ptr(mask), _ptr(weight),
                                 _ptr(bias), p.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                 _ptr(out))
    if rc != 0:
        raise ValueError("oracle: unsupported problem %s" % (p.tolist(),))
    return out


def forward_points(x, offset, mask, weight, bias, flat_indices, stride=1, padding=0,
                   dilation=1, groups=1, deformable_groups=1,
                   lib: ctypes.CDLL | None = None) -> np.ndarray:
    """Selected output elements (flat indices into [N, Co, Ho, Wo]), float64."""
    lib = lib or load_library()
    x, offset, mask, weight, bias = map(_f64, (x, offset, mask, weight, bias))
    p = problem(x.shape, offset.shape, weight.shape, stride, padding, dilation,
                groups, deformable_groups)
    idx = np.ascontiguousarray(np.asarray(flat_indices, dtype=np.int64))
    out = np.empty(idx.shape, dtype=np.float64)
    rc = lib.mdcn_oracle_points(_ptr(x), _ptr(offset), _ptr(mask), _ptr(weight),
                                _ptr(bias), p.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                idx.size, idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                _ptr(out))
    if rc != 0:
        raise ValueError("oracle: unsupported problem or index out of range")
    return out


# --- FP8 compute mode (F1-F3 in mdcn_oracle.c) --------------------------------

def e4m3(values, lib: ctypes.CDLL | None = None) -> np.ndarray:
    """Each value rounded to the nearest OCP E4M3 number (ties to even,
    saturating at +-448), as float64."""
    lib = lib or load_library()
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float64))
    out = np.empty_like(v)
    lib.mdcn_oracle_e4m3_array(_ptr(v.reshape(-1)), v.size, _ptr(out.reshape(-1)))
    return out


def fp8_row_exponent(row, lib: ctypes.CDLL | None = None) -> int:
    """The exponent e of one weight row: the largest integer with
    max|row| * 2^e <= 448 (0 for an all-zero row)."""
    lib = lib or load_library()
    r = np.ascontiguousarray(np.asarray(row, dtype=np.float64).reshape(-1))
    return int(lib.mdcn_oracle_fp8_row_exponent(_ptr(r), r.size))


def forward_points_fp8(x, offset, mask, weight, bias, flat_indices, stride=1, padding=0,
                       dilation=1, groups=1, deformable_groups=1,
                       lib: ctypes.CDLL | None = None):
    """Selected output elements in the FP8 compute mode, float64, and for each
    the sum of the absolute scaled products (the contraction's magnitude)."""
    lib = lib or load_library()
    x, offset, mask, weight, bias = map(_f64, (x, offset, mask, weight, bias))
    p = problem(x.shape, offset.shape, weight.shape, stride, padding, dilation,
                groups, deformable_groups)
    idx = np.ascontiguousarray(np.asarray(flat_indices, dtype=np.int64))
    out = np.empty(idx.shape, dtype=np.float64)
    asum = np.empty(idx.shape, dtype=np.float64)
    qw = np.empty(weight.size, dtype=np.float64)
    scale = np.empty(weight.shape[0], dtype=np.float64)
    rc = lib.mdcn_oracle_points_fp8(_ptr(x), _ptr(offset), _ptr(mask), _ptr(weight),
                                    _ptr(bias), p.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                    idx.size, idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                    _ptr(qw), _ptr(scale), _ptr(out), _ptr(asum))
    if rc != 0:
        raise ValueError("oracle: unsupported problem or index out of range")
    return out, asum


def forward_fp8(x, offset, mask, weight, bias=None, stride=1, padding=0, dilation=1,
                groups=1, deformable_groups=1, lib: ctypes.CDLL | None = None):
    """Every output element in the FP8 compute mode, shape [N, Co, Ho, Wo],
    and the matching sums of absolute scaled products."""
    N, Co = x.shape[0], weight.shape[0]
    Ho, Wo = offset.shape[2], offset.shape[3]
    idx = np.arange(N * Co * Ho * Wo, dtype=np.int64)
    out, asum = forward_points_fp8(x, offset, mask, weight, bias, idx, stride, padding,
                                   dilation, groups, deformable_groups, lib=lib)
    shape = (N, Co, Ho, Wo)
    return out.reshape(shape), asum.reshape(shape)


# --- backward (B1-B3 in mdcn_oracle.c) ----------------------------------------

def backward(x, offset, mask, weight, grad_out, with_bias=True, stride=1, padding=0,
             dilation=1, groups=1, deformable_groups=1, lib: ctypes.CDLL | None = None):
    """Gradients of sum(grad_out * out) with respect to x, offset, mask,
    weight and (with_bias) bias, float64, as a dict."""
    lib = lib or load_library()
    x, offset, mask, weight, grad_out = map(_f64, (x, offset, mask, weight, grad_out))
    p = problem(x.shape, offset.shape, weight.shape, stride, padding, dilation,
                groups, deformable_groups)
    out = {"x": np.empty_like(x), "offset": np.empty_like(offset), "mask": np.empty_like(mask),
           "weight": np.empty_like(weight),
           "bias": np.empty(weight.shape[0]) if with_bias else None}
    rc = lib.mdcn_oracle_backward(_ptr(x), _ptr(offset), _ptr(mask), _ptr(weight),
                                  _ptr(grad_out), p.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                  _ptr(out["x"]), _ptr(out["offset"]), _ptr(out["mask"]),
                                  _ptr(out["weight"]), _ptr(out["bias"]))
    if rc != 0:
        raise ValueError("oracle: unsupported problem %s" % (p.tolist(),))
    return out
