"""The C ABI library on the host: it loads, exports every declared symbol, and
its validation, shape, workspace and planning rules behave as include/mdcn.h
states.  No kernel is launched: every forward here either fails validation
before touching a device or has nothing to do."""
import os
import re

import pytest

from helpers import ensure_built

ensure_built()
from modulated_deformable_convolution_amd import mdcn  # noqa: E402

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "mdcn.h")

# dims of the OCDNet-like stage: x, offset, mask, weight
DIMS = [4, 256, 160, 160, 4, 18, 160, 160, 4, 9, 160, 160, 256, 256, 3, 3]


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(mdcn_[a-z_]+)\s*\(", text)))


def test_abi_version():
    assert mdcn.mdcn_abi_version() == 2


def test_every_declared_symbol_is_exported():
    lib = mdcn.library()
    names = declared_functions()
    assert len(names) >= 15
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(mdcn.EXPORTED) == names


@pytest.mark.parametrize("kw,code", [
    (dict(stride=(0, 1)), mdcn.MDCN_E_ATTR),
    (dict(stride=(1, -2)), mdcn.MDCN_E_ATTR),
    (dict(dilation=(0, 1)), mdcn.MDCN_E_ATTR),
    (dict(padding=(-1, 0)), mdcn.MDCN_E_ATTR),
    (dict(group=0), mdcn.MDCN_E_ATTR),
    (dict(deformable_group=-1), mdcn.MDCN_E_ATTR),
    (dict(path=9), mdcn.MDCN_E_PATH),
])
def test_create_rejects(kw, code):
    args = dict(stride=1, padding=0, dilation=1, group=1, deformable_group=1)
    args.update(kw)
    with pytest.raises(mdcn.MdcnError) as e:
        mdcn.mdcn_create(**args)
    assert e.value.status == code


def test_create_null_out():
    import ctypes
    lib = mdcn.library()
    one = (ctypes.c_int32 * 2)(1, 1)
    assert lib.mdcn_create(one, one, one, 1, 1, None) == mdcn.MDCN_E_NULL
    assert lib.mdcn_create(None, one, one, 1, 1, ctypes.byref(ctypes.c_void_p())) == \
        mdcn.MDCN_E_NULL


def test_destroy_null_is_safe():
    mdcn.library().mdcn_destroy(None)
    mdcn.library().mdcn_trace_destroy(None)


def test_output_shape_rule():
    op = mdcn.mdcn_create(1, 1, 1, 1, 1)
    assert mdcn.mdcn_output_shape(op, DIMS) == (4, 256, 160, 160)
    # spatial size comes from offset dims 2 and 3, not from a formula
    d = list(DIMS)
    d[6:8] = [100, 37]
    d[10:12] = [100, 37]
    assert mdcn.mdcn_output_shape(op, d) == (4, 256, 100, 37)
    op2 = mdcn.mdcn_create(2, 2, 2, 2, 4)
    d3 = [2, 128, 128, 128, 2, 72, 64, 64, 2, 36, 64, 64, 256, 64, 3, 3]
    assert mdcn.mdcn_output_shape(op2, d3) == (2, 256, 64, 64)


def _bad(i, v, base=DIMS):
    d = list(base)
    d[i] = v
    return d


@pytest.mark.parametrize("dims", [
    _bad(0, -1),                 # negative dim
    _bad(1, 0),                  # C == 0
    _bad(2, 0),                  # H == 0
    _bad(12, 0),                 # Co == 0
    _bad(14, 0),                 # kh == 0
    _bad(4, 3),                  # offset.d0 != x.d0
    _bad(8, 5),                  # mask.d0 != x.d0
    _bad(10, 159),               # mask.d2 != offset.d2
    _bad(11, 161),               # mask.d3 != offset.d3
    _bad(5, 1),                  # offset.d1 < 2
    _bad(5, 20),                 # offset.d1 != 2*dg*kh*kw
    _bad(9, 8),                  # mask.d1 != dg*kh*kw
    _bad(13, 128),               # weight.d1 * group != C
    _bad(2, 1 << 24),            # spatial extent beyond 2^24
    _bad(6, 1 << 24),            # output extent beyond 2^24
])
def test_shape_bindings(dims):
    op = mdcn.mdcn_create(1, 1, 1, 1, 1)
    with pytest.raises(mdcn.MdcnError) as e:
        mdcn.mdcn_output_shape(op, dims)
    assert e.value.status == mdcn.MDCN_E_SHAPE
    st = mdcn.mdcn_forward(op, mdcn.MDCN_F32, dims, 16, 32, 48, 64, 0, 0, 1 << 40,
                           1 << 41, 1 << 30, 0)
    assert st == mdcn.MDCN_E_SHAPE


def test_group_divisibility():
    # C = 6 with group 4: not divisible
    op = mdcn.mdcn_create(1, 1, 1, 4, 1)
    d = [1, 6, 8, 8, 1, 18, 8, 8, 1, 9, 8, 8, 8, 1, 3, 3]
    with pytest.raises(mdcn.MdcnError) as e:
        mdcn.mdcn_output_shape(op, d)
    assert e.value.status == mdcn.MDCN_E_SHAPE
    # Co % group != 0
    op = mdcn.mdcn_create(1, 1, 1, 2, 1)
    d = [1, 6, 8, 8, 1, 18, 8, 8, 1, 9, 8, 8, 7, 3, 3, 3]
    with pytest.raises(mdcn.MdcnError):
        mdcn.mdcn_output_shape(op, d)
    # C % deformable_group != 0
    op = mdcn.mdcn_create(1, 1, 1, 1, 4)
    d = [1, 6, 8, 8, 1, 72, 8, 8, 1, 36, 8, 8, 8, 6, 3, 3]
    with pytest.raises(mdcn.MdcnError):
        mdcn.mdcn_output_shape(op, d)


def test_forward_validation_codes():
    op = mdcn.mdcn_create(1, 1, 1, 1, 1)
    F32 = mdcn.MDCN_F32
    big = 1 << 40
    # bad dtype
    assert mdcn.mdcn_forward(op, 9, DIMS, 16, 32, 48, 64, 0, 0, big, big * 2, 1 << 32, 0) == \
        mdcn.MDCN_E_DTYPE
    # bias length must equal weight.d0
    assert mdcn.mdcn_forward(op, F32, DIMS, 16, 32, 48, 64, 80, 255, big, big * 2, 1 << 32,
                             0) == mdcn.MDCN_E_SHAPE
    # null input pointer
    assert mdcn.mdcn_forward(op, F32, DIMS, 0, 32, 48, 64, 0, 0, big, big * 2, 1 << 32, 0) == \
        mdcn.MDCN_E_NULL
    # missing or small workspace on the gather + GEMM path
    assert mdcn.mdcn_forward(op, F32, DIMS, 16, 32, 48, 64, 0, 0, big, 0, 0, 0) == \
        mdcn.MDCN_E_WORKSPACE
    _, min_b = mdcn.mdcn_workspace_bytes(op, F32, DIMS)
    assert mdcn.mdcn_forward(op, F32, DIMS, 16, 32, 48, 64, 0, 0, big, big * 2, min_b - 1,
                             0) == mdcn.MDCN_E_WORKSPACE
    # output overlapping an input
    x_bytes = 4 * 256 * 160 * 160 * 4
    assert mdcn.mdcn_forward(op, F32, DIMS, big, big * 2, big * 3, big * 4, 0, 0,
                             big + x_bytes - 4, big * 5, 1 << 32, 0) == mdcn.MDCN_E_ALIAS
    # workspace overlapping the output
    assert mdcn.mdcn_forward(op, F32, DIMS, big, big * 2, big * 3, big * 4, 0, 0, big * 5,
                             big * 5 + 64, 1 << 32, 0) == mdcn.MDCN_E_ALIAS
    # null op / dims
    lib = mdcn.library()
    assert lib.mdcn_forward(None, 0, None, None, None, None, None, None, 0, None, None, 0,
                            None) == mdcn.MDCN_E_NULL


def test_depthwise_path_needs_one_channel_per_group():
    op = mdcn.mdcn_create(1, 1, 1, 1, 1, path=mdcn.MDCN_PATH_DEPTHWISE)
    with pytest.raises(mdcn.MdcnError) as e:
        mdcn.mdcn_workspace_bytes(op, mdcn.MDCN_F32, DIMS)
    assert e.value.status == mdcn.MDCN_E_PATH


def test_empty_problems_are_noops():
    op = mdcn.mdcn_create(1, 1, 1, 1, 1)
    d = list(DIMS)
    d[0] = d[4] = d[8] = 0          # N == 0
    assert mdcn.mdcn_forward(op, mdcn.MDCN_F32, d, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) == mdcn.MDCN_OK
    assert mdcn.mdcn_workspace_bytes(op, mdcn.MDCN_F32, d) == (0, 0)
    d = list(DIMS)
    d[6] = d[10] = 0                # Ho == 0
    assert mdcn.mdcn_forward(op, mdcn.MDCN_F32, d, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) == mdcn.MDCN_OK


def test_workspace_sizes_and_chunking():
    op = mdcn.mdcn_create(1, 1, 1, 1, 1)
    op = mdcn.mdcn_create(1, 1, 1, 1, 1, path=mdcn.MDCN_PATH_GATHER_GEMM)
    # f16: 2 images of 2304 x 25600 halves of columns fit the 256 MiB budget
    b, mb = mdcn.mdcn_workspace_bytes(op, mdcn.MDCN_F16, DIMS)
    col_img = 2304 * 25600 * 2
    xt_img = 256 * 160 * 160 * 2
    wp = 256 * 2304 * 2
    assert mb == 256 + wp + col_img + xt_img          # 256: alignment slack
    assert b == 256 + wp + 2 * (col_img + xt_img)
    assert "chunk=2" in mdcn.mdcn_describe_plan(op, mdcn.MDCN_F16, DIMS)
    # less workspace: one image per chunk
    assert "chunk=1" in mdcn.mdcn_describe_plan(op, mdcn.MDCN_F16, DIMS, mb)
    # f32: one image per chunk (236 MB of columns)
    assert "chunk=1" in mdcn.mdcn_describe_plan(op, mdcn.MDCN_F32, DIMS)
    # depthwise problem on the automatic path: the sampling geometry of each
    # image (a 16-byte record per tap and pixel), all 8 images at once
    dw = mdcn.mdcn_create(1, 1, 1, 256, 1)
    d5 = [8, 256, 96, 96, 8, 18, 96, 96, 8, 9, 96, 96, 256, 1, 3, 3]
    geo_img = 9 * 96 * 96 * 16
    assert mdcn.mdcn_workspace_bytes(dw, mdcn.MDCN_F32, d5) == (256 + 8 * geo_img,
                                                                256 + geo_img)
    plan = mdcn.mdcn_describe_plan(dw, mdcn.MDCN_F32, d5)
    assert "depthwise" in plan and "chunk=8" in plan
    assert "chunk=3" in mdcn.mdcn_describe_plan(dw, mdcn.MDCN_F32, d5, 256 + 3 * geo_img + 5)
    with pytest.raises(mdcn.MdcnError) as e:
        mdcn.mdcn_describe_plan(dw, mdcn.MDCN_F32, d5, geo_img)
    assert e.value.status == mdcn.MDCN_E_WORKSPACE
    # a plane too large for LDS (304 x 304 entries of 4 bytes with the ring):
    # the plain kernel, no workspace
    big = [1, 16, 300, 300, 1, 18, 300, 300, 1, 9, 300, 300, 16, 1, 3, 3]
    dwb = mdcn.mdcn_create(1, 1, 1, 16, 1)
    assert mdcn.mdcn_workspace_bytes(dwb, mdcn.MDCN_F32, big) == (0, 0)
    # ... and the gather + GEMM path can be forced for it
    dwg = mdcn.mdcn_create(1, 1, 1, 256, 1, path=mdcn.MDCN_PATH_GATHER_GEMM)
    assert mdcn.mdcn_workspace_bytes(dwg, mdcn.MDCN_F32, d5)[0] > 0


def test_fused_path_plan():
    # automatic choice for the OCDNet-like stage: the windowed kernel (its
    # 16x16 tiles cover 160x160 exactly and all 256 output channels);
    # the fused kernel takes all 4 images, packed weight + NHWC x only
    auto = mdcn.mdcn_create(1, 1, 1, 1, 1)
    assert mdcn.mdcn_describe_plan(auto, mdcn.MDCN_F16, DIMS).startswith("path=window")
    op = mdcn.mdcn_create(1, 1, 1, 1, 1, path=mdcn.MDCN_PATH_FUSED)
    desc = mdcn.mdcn_describe_plan(op, mdcn.MDCN_F16, DIMS)
    assert desc.startswith("path=fused") and "chunk=4" in desc
    # f32 is not windowed: the automatic choice is the fused kernel
    assert mdcn.mdcn_describe_plan(auto, mdcn.MDCN_F32, DIMS).startswith("path=fused")
    opw = mdcn.mdcn_create(1, 1, 1, 1, 1, path=mdcn.MDCN_PATH_WINDOW)
    assert mdcn.mdcn_describe_plan(opw, mdcn.MDCN_F16, DIMS).startswith("path=window")
    b, mb = mdcn.mdcn_workspace_bytes(op, mdcn.MDCN_F16, DIMS)
    assert b == 256 + 256 * 2304 * 2 + 4 * 256 * 160 * 160 * 2
    assert mb == 256 + 256 * 2304 * 2 + 256 * 160 * 160 * 2
    # the windowed kernel: the same packed weight and x (in 8-channel blocks),
    # plus a 256 KiB partial-sum slot and a flag per workgroup (at most 256;
    # 100 tiles per image) and the status word after the flags, 256-byte aligned
    wp, ximg, slot = 256 * 2304 * 2, 256 * 160 * 160 * 2, 256 * 256 * 4
    assert mdcn.mdcn_workspace_bytes(opw, mdcn.MDCN_F16, DIMS) == (
        256 + wp + 4 * ximg + 256 * slot + 1280, 256 + wp + ximg + 100 * slot + 512)
    assert mdcn.mdcn_workspace_bytes(auto, mdcn.MDCN_F16, DIMS) == \
        mdcn.mdcn_workspace_bytes(opw, mdcn.MDCN_F16, DIMS)
    # 40x40 in flat tiles: 1600 of 1792 pixels (89%) -> windowed; tiles that
    # are not nearly full keep the fused kernel: 13x21 (273 of 512 pixels),
    # or 128 output channels in 256-row tiles
    d40 = [16, 512, 40, 40, 16, 18, 40, 40, 16, 9, 40, 40, 512, 512, 3, 3]
    assert mdcn.mdcn_describe_plan(auto, mdcn.MDCN_F16, d40).startswith("path=window")
    d13 = [2, 256, 13, 21, 2, 18, 13, 21, 2, 9, 13, 21, 256, 256, 3, 3]
    assert mdcn.mdcn_describe_plan(auto, mdcn.MDCN_F16, d13).startswith("path=fused")
    assert mdcn.mdcn_describe_plan(opw, mdcn.MDCN_F16, d13).startswith("path=window")
    d128 = [4, 256, 160, 160, 4, 18, 160, 160, 4, 9, 160, 160, 128, 256, 3, 3]
    assert mdcn.mdcn_describe_plan(auto, mdcn.MDCN_F16, d128).startswith("path=fused")
    # not eligible: C/group = 36 is not a multiple of 64 -> gather + GEMM
    opg = mdcn.mdcn_create(1, 1, 1, 1, 1, path=mdcn.MDCN_PATH_FUSED)
    d = [1, 36, 64, 64, 1, 18, 64, 64, 1, 9, 64, 64, 8, 36, 3, 3]
    with pytest.raises(mdcn.MdcnError) as e:
        mdcn.mdcn_workspace_bytes(opg, mdcn.MDCN_F16, d)
    assert e.value.status == mdcn.MDCN_E_PATH
    assert mdcn.mdcn_describe_plan(auto, mdcn.MDCN_F16, d).startswith("path=gather_gemm")


def _fused_dims(n, c, h, w, co, k, dg, g):
    """dims[16] of a stride-1, pad-(k//2) problem with a k x k kernel."""
    kk = k * k
    return [n, c, h, w, n, 2 * dg * kk, h, w, n, dg * kk, h, w, co, c // g, k, k]


def _tile_of(desc):
    return int(desc.split("tile=")[1].split()[0])


def test_fused_tile_fits_lds():
    """The fused kernel keeps a per-tile geometry table in LDS (32 bytes per
    offset group, tap and output column) beside two operand stages of
    2 * (BM + BN) * 128 bytes; only tiles that fit in 160 KiB are chosen."""
    f16 = mdcn.MDCN_F16
    # C = 256, dg = 1, 3x3: 9 * 128 * 32 = 36 KiB + 96 KiB -> the 256 x 128 tile
    op = mdcn.mdcn_create(1, 1, 1, 1, 1, path=mdcn.MDCN_PATH_FUSED)
    assert _tile_of(mdcn.mdcn_describe_plan(op, f16, DIMS)) == 0
    # C/dg = 32 with C/group = 64: two offset groups per group, 72 KiB of table:
    # 256 x 128 (168 KiB) does not fit, 256 x 64 (80 + 36 KiB) does
    op2 = mdcn.mdcn_create(1, 1, 1, 1, 2, path=mdcn.MDCN_PATH_FUSED)
    d = _fused_dims(4, 64, 64, 64, 256, 3, 2, 1)
    assert _tile_of(mdcn.mdcn_describe_plan(op2, f16, d)) == 2
    # 5x5 kernel, Co = 64: 25 * 128 * 32 = 100 KiB + 64 KiB does not fit at
    # 128 columns; 128 x 64 (48 + 50 KiB) does
    op5 = mdcn.mdcn_create(1, 2, 1, 1, 1, path=mdcn.MDCN_PATH_FUSED)
    d5 = _fused_dims(4, 64, 64, 64, 64, 5, 1, 1)
    assert _tile_of(mdcn.mdcn_describe_plan(op5, f16, d5)) == 3
    # C/dg = 8 with C/group = 64: eight offset groups, 144 KiB of table even
    # at 64 columns: not eligible
    op8 = mdcn.mdcn_create(1, 1, 1, 1, 8, path=mdcn.MDCN_PATH_FUSED)
    d8 = _fused_dims(2, 64, 16, 16, 64, 3, 8, 1)
    with pytest.raises(mdcn.MdcnError) as e:
        mdcn.mdcn_workspace_bytes(op8, f16, d8)
    assert e.value.status == mdcn.MDCN_E_PATH
    # C/dg = 4 halves: a 16-byte chunk would straddle offset groups
    op16 = mdcn.mdcn_create(1, 1, 1, 1, 16, path=mdcn.MDCN_PATH_FUSED)
    d16 = _fused_dims(2, 64, 16, 16, 64, 3, 16, 1)
    with pytest.raises(mdcn.MdcnError) as e:
        mdcn.mdcn_workspace_bytes(op16, f16, d16)
    assert e.value.status == mdcn.MDCN_E_PATH
    # ... but 4 fp32 channels are one chunk; 16 offset groups of 4 over
    # C/group = 64 f32 is 16 * 9 * 64 * 32 = 288 KiB of table: not eligible either
    with pytest.raises(mdcn.MdcnError):
        mdcn.mdcn_workspace_bytes(op16, mdcn.MDCN_F32, d16)
    # a misaligned group (C/group = 64, C/dg = 96) spans up to two offset groups
    opm = mdcn.mdcn_create(1, 1, 1, 3, 2, path=mdcn.MDCN_PATH_FUSED)
    dm = _fused_dims(2, 192, 16, 16, 96, 3, 2, 3)
    assert mdcn.mdcn_describe_plan(opm, f16, dm).startswith("path=fused")


def test_contraction_padding():
    # Kg = 4*9 = 36 pads to 64 (on the gather + GEMM path)
    op = mdcn.mdcn_create(1, 1, 1, 1, 1, path=mdcn.MDCN_PATH_GATHER_GEMM)
    d1 = [1, 4, 8, 8, 1, 18, 8, 8, 1, 9, 8, 8, 4, 4, 3, 3]
    assert "Kp=64" in mdcn.mdcn_describe_plan(op, mdcn.MDCN_F32, d1)


def test_direct_path_plan():
    """Problems of at most 2^20 multiply-adds take the one-launch direct
    kernel (no workspace); larger ones keep the other paths; it can be forced
    on any problem whose outputs fit a 32-bit thread index."""
    auto = mdcn.mdcn_create(1, 1, 1, 1, 1)
    tiny = [1, 4, 8, 8, 1, 18, 8, 8, 1, 9, 8, 8, 4, 4, 3, 3]          # 9216 MACs
    assert mdcn.mdcn_describe_plan(auto, mdcn.MDCN_F32, tiny).startswith("path=direct")
    assert mdcn.mdcn_workspace_bytes(auto, mdcn.MDCN_F32, tiny) == (0, 0)
    # 2^20 MACs exactly: direct; one more output channel: not
    edge = _fused_dims(1, 4, 32, 32, 28, 3, 1, 1)     # 1 * 28 * 1024 * 4 * 9 = 1032192
    assert mdcn.mdcn_describe_plan(auto, mdcn.MDCN_F32, edge).startswith("path=direct")
    over = _fused_dims(1, 4, 32, 32, 32, 3, 1, 1)     # 1179648 MACs
    assert not mdcn.mdcn_describe_plan(auto, mdcn.MDCN_F32, over).startswith("path=direct")
    opd = mdcn.mdcn_create(1, 1, 1, 1, 1, path=mdcn.MDCN_PATH_DIRECT)
    assert mdcn.mdcn_describe_plan(opd, mdcn.MDCN_F16, DIMS).startswith("path=direct")
    assert mdcn.mdcn_workspace_bytes(opd, mdcn.MDCN_F16, DIMS) == (0, 0)


def test_status_strings():
    for code in range(11):
        assert mdcn.status_string(code)
    assert mdcn.status_string(99) == "unknown status"
    assert mdcn.mdcn_kernel_name(3) == "gemm_bias"


def test_forward_without_gpu_reports_device():
    """With valid arguments and no GPU present, the call fails cleanly with
    MDCN_E_DEVICE instead of launching.  (Skipped where a GPU exists: the
    pointers here are not real.)"""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    op = mdcn.mdcn_create(1, 1, 1, 1, 1)
    big = 1 << 40
    st = mdcn.mdcn_forward(op, mdcn.MDCN_F32, DIMS, big, big * 2, big * 3, big * 4, 0, 0,
                           big * 5, big * 6, 1 << 32, 0)
    assert st == mdcn.MDCN_E_DEVICE


def _win_desc(op, dtype, dims):
    d = mdcn.mdcn_describe_plan(op, dtype, dims)
    return d, int(d.split("tile=")[1].split()[0]), int(d.split("margin=")[1].split()[0])


def test_window_path_plan():
    """The windowed fused kernel: fp16/bf16, 3x3, C/group a multiple of 16
    inside one offset group; the tile with the fewest padded output pixels,
    the widest margin (at most 8) whose window (at most 1280 input positions)
    fits its LDS buffer."""
    op = mdcn.mdcn_create(1, 1, 1, 1, 1, path=mdcn.MDCN_PATH_WINDOW)
    # OCDNet-like stage: 16 x 16 tiles, window 35 x 35 (margin 8)
    d, tile, margin = _win_desc(op, mdcn.MDCN_F16, DIMS)
    assert d.startswith("path=window") and tile == 0 and margin == 8
    # a wide, short output (8 x 64): 8 x 32 tiles pad least
    d, tile, margin = _win_desc(op, mdcn.MDCN_BF16, _fused_dims(1, 32, 8, 64, 64, 3, 1, 1))
    assert tile == 1 and margin >= 2
    # tall and narrow (64 x 8): 32 x 8 tiles
    d, tile, margin = _win_desc(op, mdcn.MDCN_BF16, _fused_dims(1, 32, 64, 8, 64, 3, 1, 1))
    assert tile == 2 and margin >= 2
    # 9 x 70: 16 x 16 tiles (16 x 80 padded pixels) pad least; a flat tile's
    # window would need 70 + 2 + 2 + 2m columns (at most 62 fit a row of the
    # zero area)
    assert _win_desc(op, mdcn.MDCN_BF16, _fused_dims(1, 32, 9, 70, 64, 3, 1, 1))[1] == 0
    # narrow images: flat tiles (256 consecutive pixels in raster order).
    # 40 x 40: 7 flat tiles pad 1600 to 1792 pixels (16 x 16 tiles: 2304);
    # a run of 256 pixels spans up to 8 rows, so the window is
    # (8 - 1 + 2 + 2 + 2m) x (40 - 1 + 2 + 2 + 2m) <= 1280: margin 6
    d40 = [16, 512, 40, 40, 16, 18, 40, 40, 16, 9, 40, 40, 512, 512, 3, 3]
    d, tile, margin = _win_desc(op, mdcn.MDCN_F16, d40)
    assert tile == 3 and margin == 6
    # 37 x 37: 1369 pixels in 6 flat tiles (1536) against 2304 in 16 x 16 tiles
    d, tile, margin = _win_desc(op, mdcn.MDCN_F16, _fused_dims(2, 32, 37, 37, 288, 3, 1, 1))
    assert tile == 3 and margin == 6
    # 64 x 8: flat tiles pad as little as 32 x 8 ones, with the same margin:
    # the first listed tile stays
    assert _win_desc(op, mdcn.MDCN_BF16, _fused_dims(1, 32, 64, 8, 64, 3, 1, 1))[1] == 2
    # stride (2, 1): a 16 x 16 tile's window spans 30 + 2 + 2 + 2m rows and
    # 15 + 2 + 2 + 2m columns, at most 1280 positions: margin 5; with stride
    # and dilation 2 no tile fits
    ops = mdcn.mdcn_create((2, 1), 1, 1, 2, 1, path=mdcn.MDCN_PATH_WINDOW)
    ds = [2, 64, 64, 64, 2, 18, 32, 64, 2, 9, 32, 64, 64, 32, 3, 3]
    d, tile, margin = _win_desc(ops, mdcn.MDCN_F16, ds)
    assert tile == 0 and margin == 5
    opd = mdcn.mdcn_create(2, 2, 2, 2, 1, path=mdcn.MDCN_PATH_WINDOW)
    with pytest.raises(mdcn.MdcnError) as e:
        mdcn.mdcn_workspace_bytes(opd, mdcn.MDCN_F16, ds)
    assert e.value.status == mdcn.MDCN_E_PATH
    # not eligible: fp32, a 5x5 kernel, C/group = 8, a group spanning two
    # offset groups
    for dtype, g, dg, dims in [(mdcn.MDCN_F32, 1, 1, DIMS),
                               (mdcn.MDCN_F16, 1, 1, _fused_dims(1, 32, 12, 12, 32, 5, 1, 1)),
                               (mdcn.MDCN_F16, 2, 1, _fused_dims(1, 16, 12, 12, 32, 3, 1, 2)),
                               (mdcn.MDCN_F16, 2, 4, _fused_dims(1, 64, 12, 12, 32, 3, 4, 2))]:
        opx = mdcn.mdcn_create(1, 1, 1, g, dg, path=mdcn.MDCN_PATH_WINDOW)
        with pytest.raises(mdcn.MdcnError) as e:
            mdcn.mdcn_workspace_bytes(opx, dtype, dims)
        assert e.value.status == mdcn.MDCN_E_PATH
    # a group inside one offset group (C/group = 32, C/dg = 64) is eligible
    opx = mdcn.mdcn_create(1, 1, 1, 4, 2, path=mdcn.MDCN_PATH_WINDOW)
    assert _win_desc(opx, mdcn.MDCN_F16, _fused_dims(1, 128, 12, 12, 64, 3, 2, 4))[0].startswith(
        "path=window")
    # margin and tile overrides (tuning)
    import os
    os.environ["MDCN_WIN_MARGIN"] = "3"
    os.environ["MDCN_WIN_TILE"] = "1"
    try:
        _, tile, margin = _win_desc(op, mdcn.MDCN_F16, DIMS)
        assert tile == 1 and margin == 3
    finally:
        del os.environ["MDCN_WIN_MARGIN"], os.environ["MDCN_WIN_TILE"]


def test_fp8_path_plan():
    """The FP8 path: E4M3 weight (Kp = Kg padded to 128 bytes) plus one fp32
    scale per output channel, x in NHWC of the input dtype, E4M3 columns;
    all 4 images of the OCDNet-like stage fit the 256 MiB column budget.
    Never the automatic choice."""
    op = mdcn.mdcn_create(1, 1, 1, 1, 1, path=mdcn.MDCN_PATH_GATHER_GEMM_FP8)
    b, mb = mdcn.mdcn_workspace_bytes(op, mdcn.MDCN_F16, DIMS)
    col_img = 2304 * 25600                        # one byte per column value
    xt_img = 256 * 160 * 160 * 2
    wq = 256 * 2304 + 256 * 4                     # weight bytes + row scales (aligned)
    assert mb == 256 + wq + col_img + xt_img
    assert b == 256 + wq + 4 * (col_img + xt_img)
    desc = mdcn.mdcn_describe_plan(op, mdcn.MDCN_F16, DIMS)
    assert desc.startswith("path=gather_gemm_fp8") and "chunk=4" in desc and "Kp=2304" in desc
    # a contraction that is not a multiple of 128: padded (Kg = 9 * 20 = 180)
    d = [1, 20, 16, 16, 1, 18, 16, 16, 1, 9, 16, 16, 8, 20, 3, 3]
    assert "Kp=256" in mdcn.mdcn_describe_plan(op, mdcn.MDCN_F32, d)
    assert "Kp=192" in mdcn.mdcn_describe_plan(
        mdcn.mdcn_create(1, 1, 1, 1, 1, path=mdcn.MDCN_PATH_GATHER_GEMM), mdcn.MDCN_F16, d)
    # every dtype; the automatic choice never takes it
    for dt in (mdcn.MDCN_F32, mdcn.MDCN_BF16):
        assert mdcn.mdcn_describe_plan(op, dt, DIMS).startswith("path=gather_gemm_fp8")
    auto = mdcn.mdcn_create(1, 1, 1, 1, 1)
    for dt in (mdcn.MDCN_F32, mdcn.MDCN_F16, mdcn.MDCN_BF16):
        assert "fp8" not in mdcn.mdcn_describe_plan(auto, dt, DIMS)
        assert "fp8" not in mdcn.mdcn_describe_plan(auto, dt, d)
    names = [mdcn.mdcn_kernel_name(i) for i in range(16)]
    assert {"prep_nhwc_fp8", "deform_gather_fp8", "gemm_fp8_bias"} <= set(names)


def test_window_fp8_path_plan(monkeypatch):
    """The windowed FP8 path: the window path's tiles, margin, chunking and
    partial-sum slots, with the 16-bit step-major weight replaced by the E4M3
    chunk blocks (144 bytes per output channel and 16-channel chunk) and one
    fp32 scale per output channel; on groups of more than 256 output channels
    the wide tiles (128 pixels x 512 channels, windows of at most 1024
    positions).  Eligible where the window path is; never the automatic
    choice."""
    op = mdcn.mdcn_create(1, 1, 1, 1, 1, path=mdcn.MDCN_PATH_WINDOW_FP8)
    win = mdcn.mdcn_create(1, 1, 1, 1, 1, path=mdcn.MDCN_PATH_WINDOW)
    for dt in (mdcn.MDCN_F16, mdcn.MDCN_BF16):
        b, mb = mdcn.mdcn_workspace_bytes(op, dt, DIMS)
        bw, mbw = mdcn.mdcn_workspace_bytes(win, dt, DIMS)
        w16 = 256 * 2304 * 2
        w8 = 16 * 256 * 144 + 256 * 4             # chunk blocks + row scales (aligned)
        assert b == bw - w16 + w8 and mb == mbw - w16 + w8
        d, tile, margin = _win_desc(op, dt, DIMS)
        assert d.startswith("path=window_fp8") and tile == 0 and margin == 8
    d40 = [16, 512, 40, 40, 16, 18, 40, 40, 16, 9, 40, 40, 512, 512, 3, 3]
    # 40x40, Mg = 512: flat 128-pixel tiles, 5 rows of 40 output pixels ->
    # a window of (4 + 2 + 2 + 2m) x (39 + 2 + 2 + 2m) <= 1024 positions:
    # m = 5 (18 x 53); 13 tiles of one image, 16 images -> 208 slots
    d, tile, margin = _win_desc(op, mdcn.MDCN_F16, d40)
    assert d.startswith("path=window_fp8") and tile == 6 and margin == 5
    assert "slots=208" in d
    # MDCN_WIN_WIDE=0: the 256-pixel tiles (flat, 8 rows: m = 6), each image
    # 7 tiles x 2 channel halves -> 224 slots
    monkeypatch.setenv("MDCN_WIN_WIDE", "0")
    d, tile, margin = _win_desc(op, mdcn.MDCN_F16, d40)
    assert tile == 3 and margin == 6 and "slots=224" in d
    monkeypatch.delenv("MDCN_WIN_WIDE")
    # a forced wide tile: 8 x 16 (window (7+4+2m) x (15+4+2m): m = 8, 27 x 35)
    monkeypatch.setenv("MDCN_WIN_TILE", "4")
    d, tile, margin = _win_desc(op, mdcn.MDCN_F16, d40)
    assert tile == 4 and margin == 8
    # a narrow tile asked for a wide problem is not one of the wide tiles:
    # the planner's own choice
    monkeypatch.setenv("MDCN_WIN_TILE", "0")
    d, tile, margin = _win_desc(op, mdcn.MDCN_F16, d40)
    assert tile == 6 and margin == 5
    monkeypatch.delenv("MDCN_WIN_TILE")
    # more than 256 but not 512 output channels per group: wide as well
    # (one 512-row tile, rows past Mg unused); 256: the narrow tiles
    d384 = [2, 64, 24, 24, 2, 18, 24, 24, 2, 9, 24, 24, 384, 64, 3, 3]
    d, tile, margin = _win_desc(op, mdcn.MDCN_BF16, d384)
    assert tile in (4, 5, 6)
    d256 = [2, 64, 24, 24, 2, 18, 24, 24, 2, 9, 24, 24, 256, 64, 3, 3]
    d, tile, margin = _win_desc(op, mdcn.MDCN_BF16, d256)
    assert tile in (0, 1, 2, 3)
    # the 16-bit window path never takes them
    d, tile, margin = _win_desc(win, mdcn.MDCN_F16, d40)
    assert tile in (0, 1, 2, 3)
    # the window path's limits: fp32 and a 5x5 kernel are refused
    for dtype, dims in [(mdcn.MDCN_F32, DIMS),
                        (mdcn.MDCN_F16, _fused_dims(1, 32, 12, 12, 32, 5, 1, 1))]:
        with pytest.raises(mdcn.MdcnError) as e:
            mdcn.mdcn_workspace_bytes(op, dtype, dims)
        assert e.value.status == mdcn.MDCN_E_PATH
    auto = mdcn.mdcn_create(1, 1, 1, 1, 1)
    for dims in (DIMS, d40):
        assert "fp8" not in mdcn.mdcn_describe_plan(auto, mdcn.MDCN_F16, dims)
    assert mdcn.mdcn_kernel_name(24) == "prep_blocks_fp8"
    assert mdcn.mdcn_kernel_name(25) == "window_gather_gemm_fp8"
    assert mdcn.mdcn_kernel_name(26) == "?"


def test_backward_entry_points():
    """Inputs and gradients in the dtype, fp32 arithmetic; the workspace holds
    the packed weight and one image's NHWC x (dtype), its fp32 gradient
    accumulator (NHWC, and NCHW for fp16/bf16), its fp32 columns and their
    gradient, the weight-gradient accumulator, and the buckets of grad_x's
    gather (counts, starts, scan block totals, up to four 8-byte entries per
    sample)."""
    op = mdcn.mdcn_create(1, 1, 1, 1, 1)
    hw = 256 * 160 * 160
    col = 25600 * 2304 * 4            # columns and their gradient (fp32)
    acc = 256 * 2304 * 4
    b = mdcn.mdcn_backward_workspace_bytes(op, mdcn.MDCN_F32, DIMS)
    # fp32 with one group and Co % 32 == 0: the column gradient on the MFMA
    # GEMM, with grad_out [P][Co] and the packed weight [Kp][Co] transposed
    mfma = 25600 * 256 * 4 + 2304 * 256 * 4

    def al(v):
        return (v + 255) // 256 * 256
    cells = 160 * 160
    bins = al(cells * 4) + al((cells + 1) * 4) + al(4097 * 4) + al(4 * 9 * 25600 * 8)
    assert b == 256 + 256 * 2304 * 4 + hw * 4 + hw * 4 + 2 * col + acc + mfma + bins
    for dt in (mdcn.MDCN_F16, mdcn.MDCN_BF16):
        b16 = mdcn.mdcn_backward_workspace_bytes(op, dt, DIMS)
        assert b16 == 256 + 256 * 2304 * 2 + hw * 2 + 2 * hw * 4 + 2 * col + acc + bins
    with pytest.raises(mdcn.MdcnError) as e:
        mdcn.mdcn_backward_workspace_bytes(op, 7, DIMS)
    assert e.value.status == mdcn.MDCN_E_DTYPE
    # missing pointers and a short workspace are refused before any launch
    assert mdcn.mdcn_backward(op, mdcn.MDCN_F32, DIMS, 0, 1, 1, 1, 1, 1, 1, 1, 1, 0, 0, 1, b,
                              0) == mdcn.MDCN_E_NULL
    assert mdcn.mdcn_backward(op, mdcn.MDCN_F32, DIMS, 1, 1, 1, 1, 1, 1, 1, 1, 1, 0, 0, 1,
                              b - 1, 0) == mdcn.MDCN_E_WORKSPACE
    assert mdcn.mdcn_backward(op, mdcn.MDCN_F32, DIMS, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 5, 1,
                              b, 0) == mdcn.MDCN_E_SHAPE         # bias_len != Co
    names = [mdcn.mdcn_kernel_name(i) for i in range(23)]
    assert {"bwd_zero", "bwd_bias", "bwd_weight_gemm", "bwd_col_gemm", "bwd_sample",
            "bwd_to_nchw", "bwd_weight_out"} <= set(names)
