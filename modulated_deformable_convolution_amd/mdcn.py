"""Python binding of libmdcn.so (include/mdcn.h): argument marshalling only.

The functions named ``mdcn_*`` mirror the C entry points one to one and take
plain integers (device pointers as ints, the stream as an int handle).
``forward`` is a convenience on top that takes torch tensors, which are used
only as device memory; every step of the computation runs in the library's
HIP kernels.  There is no CPU fallback: without the built library, or without
a gfx950 GPU, these calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmdcn.so")

# mdcn_status
MDCN_OK = 0
MDCN_E_NULL = 1
MDCN_E_ATTR = 2
MDCN_E_SHAPE = 3
MDCN_E_DTYPE = 4
MDCN_E_WORKSPACE = 5
MDCN_E_LAUNCH = 6
MDCN_E_DEVICE = 7
MDCN_E_ALIAS = 8
MDCN_E_PATH = 9
MDCN_E_INTERNAL = 10
MDCN_E_SYNC = 11

# mdcn_dtype
MDCN_F32 = 0
MDCN_F16 = 1
MDCN_BF16 = 2

# mdcn_path
MDCN_PATH_AUTO = 0
MDCN_PATH_GATHER_GEMM = 1
MDCN_PATH_DEPTHWISE = 2
MDCN_PATH_FUSED = 3
MDCN_PATH_WINDOW = 4
MDCN_PATH_DIRECT = 5
MDCN_PATH_GATHER_GEMM_FP8 = 6
MDCN_PATH_WINDOW_FP8 = 7

EXPORTED = [
    "mdcn_create", "mdcn_create_with_path", "mdcn_destroy", "mdcn_output_shape",
    "mdcn_workspace_bytes", "mdcn_forward", "mdcn_trace_create", "mdcn_trace_destroy",
    "mdcn_trace_reset", "mdcn_forward_traced", "mdcn_trace_count", "mdcn_trace_read",
    "mdcn_kernel_name", "mdcn_status_string", "mdcn_abi_version", "mdcn_describe_plan",
    "mdcn_backward_workspace_bytes", "mdcn_backward", "mdcn_backward_traced",
    "mdcn_forward_check", "mdcn_forward_noalloc",
]

# bytes of the device array mdcn_forward_noalloc works in (include/mdcn.h)
MDCN_NOALLOC_SCRATCH_BYTES = 128 << 20


class MdcnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


_lock = threading.Lock()
_lib = None

_vp = ctypes.c_void_p
_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)
_szp = ctypes.POINTER(ctypes.c_size_t)


def _bind(lib):
    sig = {
        "mdcn_create": ([_i32p, _i32p, _i32p, ctypes.c_int32, ctypes.c_int32,
                         ctypes.POINTER(_vp)], ctypes.c_int),
        "mdcn_create_with_path": ([_i32p, _i32p, _i32p, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int, ctypes.POINTER(_vp)], ctypes.c_int),
        "mdcn_destroy": ([_vp], None),
        "mdcn_output_shape": ([_vp, _i64p, _i64p], ctypes.c_int),
        "mdcn_workspace_bytes": ([_vp, ctypes.c_int, _i64p, _szp, _szp], ctypes.c_int),
        "mdcn_forward": ([_vp, ctypes.c_int, _i64p, _vp, _vp, _vp, _vp, _vp, ctypes.c_int64,
                          _vp, _vp, ctypes.c_size_t, _vp], ctypes.c_int),
        "mdcn_forward_check": ([_vp, ctypes.c_int, _i64p, _vp, ctypes.c_size_t, _vp],
                               ctypes.c_int),
        "mdcn_forward_noalloc": ([_vp, ctypes.c_int, _i64p, _vp, _vp, _vp, _vp, _vp,
                                  ctypes.c_int64, _vp, _vp], ctypes.c_int),
        "mdcn_forward_traced": ([_vp, ctypes.c_int, _i64p, _vp, _vp, _vp, _vp, _vp,
                                 ctypes.c_int64, _vp, _vp, ctypes.c_size_t, _vp, _vp],
                                ctypes.c_int),
        "mdcn_backward_workspace_bytes": ([_vp, ctypes.c_int, _i64p, _szp], ctypes.c_int),
        "mdcn_backward": ([_vp, ctypes.c_int, _i64p, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                           _vp, _vp, ctypes.c_int64, _vp, ctypes.c_size_t, _vp], ctypes.c_int),
        "mdcn_backward_traced": ([_vp, ctypes.c_int, _i64p, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _vp, _vp, ctypes.c_int64, _vp, ctypes.c_size_t, _vp, _vp],
                                 ctypes.c_int),
        "mdcn_trace_create": ([ctypes.c_int32, ctypes.POINTER(_vp)], ctypes.c_int),
        "mdcn_trace_destroy": ([_vp], None),
        "mdcn_trace_reset": ([_vp], ctypes.c_int),
        "mdcn_trace_count": ([_vp, _i32p], ctypes.c_int),
        "mdcn_trace_read": ([_vp, ctypes.c_int32, _i32p, ctypes.POINTER(ctypes.c_float)],
                            ctypes.c_int),
        "mdcn_kernel_name": ([ctypes.c_int32], ctypes.c_char_p),
        "mdcn_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "mdcn_abi_version": ([], ctypes.c_int32),
        "mdcn_describe_plan": ([_vp, ctypes.c_int, _i64p, ctypes.c_size_t, ctypes.c_char_p,
                                ctypes.c_size_t], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


def library():
    """The loaded libmdcn.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIBRARY):
                raise RuntimeError(
                    "libmdcn.so is not built (expected at %s); build it with "
                    "`python -m modulated_deformable_convolution_amd.build`" % LIBRARY)
            _lib = _bind(ctypes.CDLL(LIBRARY))
        return _lib


def status_string(status: int) -> str:
    return library().mdcn_status_string(status).decode()


def _check(status: int, where: str):
    if status != MDCN_OK:
        raise MdcnError(status, where)


def _pair(v):
    if isinstance(v, int):
        return (v, v)
    return (int(v[0]), int(v[1]))


def _arr(t, vals):
    return (t * len(vals))(*vals)


# ---------------------------------------------------------------- handles

class Op:
    """Owns an mdcn_op handle."""

    def __init__(self, handle: int, attrs: dict):
        self.handle = handle
        self.attrs = attrs
        # forward()'s per-shape set-up: (dtype code, shapes) -> (ctypes dims,
        # output shape), so that repeated calls skip it
        self.calls = {}

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and _lib is not None:
            _lib.mdcn_destroy(h)


def mdcn_create(stride, padding, dilation, group, deformable_group,
                path: int = MDCN_PATH_AUTO) -> Op:
    lib = library()
    s, p, d = _pair(stride), _pair(padding), _pair(dilation)
    h = _vp()
    st = lib.mdcn_create_with_path(_arr(ctypes.c_int32, s), _arr(ctypes.c_int32, p),
                                   _arr(ctypes.c_int32, d), int(group), int(deformable_group),
                                   int(path), ctypes.byref(h))
    _check(st, "mdcn_create")
    return Op(h.value, dict(stride=s, padding=p, dilation=d, group=group,
                            deformable_group=deformable_group, path=path))


def mdcn_output_shape(op: Op, dims) -> tuple:
    out = (ctypes.c_int64 * 4)()
    _check(library().mdcn_output_shape(op.handle, _arr(ctypes.c_int64, dims), out),
           "mdcn_output_shape")
    return tuple(out)


def mdcn_workspace_bytes(op: Op, dtype: int, dims) -> tuple:
    b, mb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(library().mdcn_workspace_bytes(op.handle, int(dtype), _arr(ctypes.c_int64, dims),
                                          ctypes.byref(b), ctypes.byref(mb)),
           "mdcn_workspace_bytes")
    return b.value, mb.value


def mdcn_describe_plan(op: Op, dtype: int, dims, workspace_bytes: int = 0) -> str:
    buf = ctypes.create_string_buffer(512)
    _check(library().mdcn_describe_plan(op.handle, int(dtype), _arr(ctypes.c_int64, dims),
                                        int(workspace_bytes), buf, 512), "mdcn_describe_plan")
    return buf.value.decode()


def mdcn_forward(op: Op, dtype: int, dims, x: int, offset: int, mask: int, weight: int,
                 bias: int, bias_len: int, out: int, workspace: int, workspace_bytes: int,
                 stream: int, trace: "Trace | None" = None) -> int:
    """Raw entry point; returns the status code (does not raise)."""
    lib = library()
    d = _arr(ctypes.c_int64, dims)
    args = (op.handle, int(dtype), d, x or None, offset or None, mask or None, weight or None,
            bias or None, int(bias_len), out or None, workspace or None, int(workspace_bytes),
            stream or None)
    if trace is None:
        return lib.mdcn_forward(*args)
    return lib.mdcn_forward_traced(*args, trace.handle)


def mdcn_forward_check(op: Op, dtype: int, dims, workspace: int, workspace_bytes: int,
                       stream: int) -> int:
    """Raw entry point; returns the status code (does not raise)."""
    return library().mdcn_forward_check(op.handle, int(dtype), _arr(ctypes.c_int64, dims),
                                        workspace or None, int(workspace_bytes), stream or None)


def mdcn_forward_noalloc(op: Op, dtype: int, dims, x: int, offset: int, mask: int, weight: int,
                         bias: int, bias_len: int, out: int, stream: int) -> int:
    """Raw entry point; returns the status code (does not raise)."""
    return library().mdcn_forward_noalloc(
        op.handle, int(dtype), _arr(ctypes.c_int64, dims), x or None, offset or None,
        mask or None, weight or None, bias or None, int(bias_len), out or None, stream or None)


def mdcn_backward_workspace_bytes(op: Op, dtype: int, dims) -> int:
    lib = library()
    d = _arr(ctypes.c_int64, dims)
    b = ctypes.c_size_t()
    _check(lib.mdcn_backward_workspace_bytes(op.handle, int(dtype), d, ctypes.byref(b)),
           "mdcn_backward_workspace_bytes")
    return b.value


def mdcn_backward(op: Op, dtype: int, dims, x: int, offset: int, mask: int, weight: int,
                  grad_out: int, grad_x: int, grad_offset: int, grad_mask: int,
                  grad_weight: int, grad_bias: int, bias_len: int, workspace: int,
                  workspace_bytes: int, stream: int, trace: "Trace | None" = None) -> int:
    """Raw entry point; returns the status code (does not raise)."""
    lib = library()
    d = _arr(ctypes.c_int64, dims)
    args = (op.handle, int(dtype), d, x or None, offset or None, mask or None, weight or None,
            grad_out or None, grad_x or None, grad_offset or None, grad_mask or None,
            grad_weight or None, grad_bias or None, int(bias_len), workspace or None,
            int(workspace_bytes), stream or None)
    if trace is None:
        return lib.mdcn_backward(*args)
    return lib.mdcn_backward_traced(*args, trace.handle)


def mdcn_kernel_name(kernel_id: int) -> str:
    return library().mdcn_kernel_name(int(kernel_id)).decode()


def mdcn_abi_version() -> int:
    return int(library().mdcn_abi_version())


class Trace:
    """Owns an mdcn_trace: HIP event pairs around each traced kernel launch."""

    def __init__(self, capacity: int = 256):
        lib = library()
        h = _vp()
        _check(lib.mdcn_trace_create(int(capacity), ctypes.byref(h)), "mdcn_trace_create")
        self.handle = h.value

    def reset(self):
        _check(library().mdcn_trace_reset(self.handle), "mdcn_trace_reset")

    def read(self) -> list:
        """[(kernel name, milliseconds)] for every recorded launch (waits)."""
        lib = library()
        n = ctypes.c_int32()
        _check(lib.mdcn_trace_count(self.handle, ctypes.byref(n)), "mdcn_trace_count")
        out = []
        for i in range(n.value):
            kid, ms = ctypes.c_int32(), ctypes.c_float()
            _check(lib.mdcn_trace_read(self.handle, i, ctypes.byref(kid), ctypes.byref(ms)),
                   "mdcn_trace_read")
            out.append((mdcn_kernel_name(kid.value), ms.value))
        return out

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and _lib is not None:
            _lib.mdcn_trace_destroy(h)


# ---------------------------------------------------------------- tensor convenience

_DTYPE_CODES = {}


def dtype_code(torch_dtype) -> int:
    if not _DTYPE_CODES:
        import torch
        _DTYPE_CODES.update({torch.float32: MDCN_F32, torch.float16: MDCN_F16,
                             torch.bfloat16: MDCN_BF16})
    code = _DTYPE_CODES.get(torch_dtype)
    if code is None:
        raise MdcnError(MDCN_E_DTYPE, "dtype_code")
    return code


def dims_of(x, offset, mask, weight) -> list:
    """The dims[16] array of include/mdcn.h from four 4-D tensors."""
    dims = []
    for t in (x, offset, mask, weight):
        if t.dim() != 4:
            raise MdcnError(MDCN_E_SHAPE, "dims_of")
        dims.extend(int(v) for v in t.shape)
    return dims


def _alloc_stream(stream, device, allocates):
    """(handle, context) for a launch on `stream` (an int handle or None =
    torch's current stream): buffers torch allocates for the call are made
    inside the context, so the caching allocator ties them to the stream the
    kernels run on and cannot hand them out while those kernels still use
    them.  The context is only built when the call allocates on a stream
    other than torch's current one (switching streams costs tens of
    microseconds per call)."""
    import contextlib
    import torch
    if stream is not None and not allocates:
        return int(stream), contextlib.nullcontext()
    current = torch.cuda.current_stream(device).cuda_stream
    if stream is None:
        return current, contextlib.nullcontext()
    stream = int(stream)
    if stream == current:
        return stream, contextlib.nullcontext()
    if stream == 0:
        return 0, torch.cuda.stream(torch.cuda.default_stream(device))
    return stream, torch.cuda.stream(torch.cuda.ExternalStream(stream, device=device))


def forward(op: Op, x, offset, mask, weight, bias=None, out=None, workspace=None,
            stream=None, trace: Trace | None = None, check: bool = False):
    """Run mdcn_forward on torch device tensors; allocates `out` (and the
    workspace) with torch when not given, on the stream the forward runs on.
    With check, waits for the forward and raises if a bounded wait inside it
    gave up (mdcn_forward_check).  Raises MdcnError on failure."""
    import torch
    tensors = [x, offset, mask, weight] + ([bias] if bias is not None else [])
    for t in tensors:
        if not t.is_cuda or not t.is_contiguous() or t.dtype != x.dtype:
            raise MdcnError(MDCN_E_SHAPE if t.is_cuda else MDCN_E_NULL, "forward: tensors must "
                            "be contiguous device tensors of one dtype")
    code = dtype_code(x.dtype)
    key = (code, x.shape, offset.shape, mask.shape, weight.shape)
    call = op.calls.get(key)
    if call is None:
        dims = dims_of(x, offset, mask, weight)
        call = (dims, _arr(ctypes.c_int64, dims), mdcn_output_shape(op, dims))
        if len(op.calls) >= 64:
            op.calls.clear()
        op.calls[key] = call
    dims, dims_c, shape = call
    stream, ctx = _alloc_stream(stream, x.device, out is None or workspace is None)
    with ctx:
        if out is None:
            out = torch.empty(shape, dtype=x.dtype, device=x.device)
        elif tuple(out.shape) != shape or out.dtype != x.dtype or not out.is_contiguous():
            raise MdcnError(MDCN_E_SHAPE, "forward: out")
        if workspace is None:
            nbytes, _ = mdcn_workspace_bytes(op, code, dims)
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
        args = (op.handle, code, dims_c, x.data_ptr(), offset.data_ptr(), mask.data_ptr(),
                weight.data_ptr(), bias.data_ptr() if bias is not None else None,
                int(bias.numel()) if bias is not None else 0, out.data_ptr(),
                workspace.data_ptr() or None, workspace.numel(), stream or None)
        lib = _lib or library()
        st = (lib.mdcn_forward(*args) if trace is None
              else lib.mdcn_forward_traced(*args, trace.handle))
        _check(st, "mdcn_forward")
        if check:
            _check(mdcn_forward_check(op, code, dims, workspace.data_ptr(), workspace.numel(),
                                      stream), "mdcn_forward_check")
    return out


def backward(op: Op, x, offset, mask, weight, grad_out, with_bias=True, workspace=None,
             stream=None, trace: Trace | None = None):
    """Run mdcn_backward (fp32) on torch device tensors: returns a dict of
    gradients x, offset, mask, weight and (with_bias) bias, allocated with
    torch.  Raises MdcnError on failure."""
    import torch
    for t in (x, offset, mask, weight, grad_out):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != x.dtype:
            raise MdcnError(MDCN_E_SHAPE if t.is_cuda else MDCN_E_NULL, "backward: tensors "
                            "must be contiguous device tensors of one dtype")
    code = dtype_code(x.dtype)
    dims = dims_of(x, offset, mask, weight)
    if tuple(grad_out.shape) != mdcn_output_shape(op, dims):
        raise MdcnError(MDCN_E_SHAPE, "backward: grad_out")
    stream, ctx = _alloc_stream(stream, x.device, True)
    with ctx:
        if workspace is None:
            workspace = torch.empty(mdcn_backward_workspace_bytes(op, code, dims),
                                    dtype=torch.uint8, device=x.device)
        g = {"x": torch.empty_like(x), "offset": torch.empty_like(offset),
             "mask": torch.empty_like(mask), "weight": torch.empty_like(weight),
             "bias": torch.empty(weight.shape[0], dtype=x.dtype, device=x.device) if with_bias
             else None}
        st = mdcn_backward(op, code, dims, x.data_ptr(), offset.data_ptr(), mask.data_ptr(),
                           weight.data_ptr(), grad_out.data_ptr(), g["x"].data_ptr(),
                           g["offset"].data_ptr(), g["mask"].data_ptr(), g["weight"].data_ptr(),
                           g["bias"].data_ptr() if with_bias else 0,
                           int(weight.shape[0]) if with_bias else 0, workspace.data_ptr(),
                           workspace.numel(), stream, trace)
        _check(st, "mdcn_backward")
    return g
