"""The CPU oracle against closed forms, identities and hand-worked values.

No GPU is involved.  See closed_forms.py for what each check computes and why
it is independent of the oracle's own loop.  The mutation test at the end
plants a plausible mistake in a copy of the oracle's C source (on the CPU),
builds it, and requires that at least one check notices.
"""
import json
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import closed_forms as cf
from oracle import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_1x2_kernel.json")


@pytest.fixture(scope="module")
def lib():
    return oracle.load_library()


@pytest.fixture(scope="module")
def fixture():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("idx", range(len(cf.PROBLEMS)))
@pytest.mark.parametrize("name", list(cf.CHECKS_PER_PROBLEM))
def test_closed_form(lib, name, idx):
    err = cf.CHECKS_PER_PROBLEM[name](lib, cf.PROBLEMS[idx])
    assert cf.passes(name, err), (name, idx, err)


def test_bilinear_function(lib):
    err = cf.check_bilinear_function(lib)
    assert err <= cf.TOL, err


def test_hand_worked_example(lib, fixture):
    assert cf.check_hand_example(lib, fixture) == 0.0


def test_output_shape_follows_offset_dims(lib):
    """Output dims are [x.d0, weight.d0, offset.d2, offset.d3], whatever the
    conv formula would give."""
    g = torch.Generator().manual_seed(5)
    x = torch.randn(3, 4, 9, 11, generator=g, dtype=torch.float64)
    w = torch.randn(5, 4, 3, 3, generator=g, dtype=torch.float64)
    off = torch.randn(3, 18, 4, 6, generator=g, dtype=torch.float64)
    m = torch.rand(3, 9, 4, 6, generator=g, dtype=torch.float64)
    out = oracle.forward(x, off, m, w, None, stride=2, padding=1, lib=lib)
    assert out.shape == (3, 5, 4, 6)


def test_points_agree_with_full_forward(lib):
    pr = cf.PROBLEMS[0]
    x, w, b, m = cf.random_tensors(pr, 7)
    g = torch.Generator().manual_seed(8)
    K = pr["kh"] * pr["kw"]
    off = torch.randn(pr["N"], 2 * pr["dg"] * K, pr["Ho"], pr["Wo"], generator=g,
                      dtype=torch.float64) * 2
    kw = dict(stride=pr["stride"], padding=pr["padding"], dilation=pr["dilation"],
              groups=pr["groups"], deformable_groups=pr["dg"], lib=lib)
    full = oracle.forward(x, off, m, w, b, **kw)
    idx = np.random.default_rng(0).choice(full.size, size=50, replace=False)
    pts = oracle.forward_points(x, off, m, w, b, idx, **kw)
    assert np.array_equal(pts, full.reshape(-1)[idx])


def test_rejects_bad_problems(lib):
    x = np.zeros((1, 3, 4, 4))
    w = np.zeros((2, 3, 3, 3))
    off = np.zeros((1, 18, 4, 4))
    m = np.zeros((1, 9, 4, 4))
    with pytest.raises(ValueError):
        oracle.forward(x, off, m, w, None, groups=2, lib=lib)   # 3 % 2 != 0
    with pytest.raises(ValueError):
        oracle.forward_points(x, off, m, w, None, [10 ** 6], lib=lib)


# ---------------------------------------------------------------- mutation test

# (what the oracle says, a plausible mistake in its place)
MUTANTS = {
    "corner_transposed": ("(1.0 - fy) * fx         * pixel_or_zero(X, H, W, y0, x0 + 1)",
                          "(1.0 - fy) * fx         * pixel_or_zero(X, H, W, y0 + 1, x0)"),
    "corner_term_dropped": ("+ fy         * fx         * pixel_or_zero(X, H, W, y0 + 1, x0 + 1);",
                            ";"),
    "fraction_swapped": ("double fy = h - hf;", "double fy = w - wf;"),
    "pad_sign": ("(ho * p[P_SH] - p[P_PH] + i * p[P_DH])", "(ho * p[P_SH] + p[P_PH] + i * p[P_DH])"),
    "dilation_axes_swapped": ("i * p[P_DH]", "i * p[P_DW]"),
    "stride_axes_swapped": ("wo * p[P_SW]", "wo * p[P_SH]"),
    "offset_pair_index": ("q * 2 * K + 2 * k;", "q * 2 * K + k;"),
    "offset_h_w_swapped": ("const double dh = offset[off_h_ch * HoWo + pix];",
                           "const double dh = offset[off_w_ch * HoWo + pix];"),
    "mask_group_major": ("n * DG * K + q * K + k;", "n * DG * K + k * DG + q;"),
    "offset_group_modulo": ("const int64_t q = c / Cdg;", "const int64_t q = c % DG;"),
    "truncate_not_floor": ("double hf = floor(h);", "double hf = trunc(h);"),
    "bias_dropped": ("acc += bias[co];", "acc += 0.0;"),
    "weight_taps_transposed": ("weight[((co * Cg + cl) * kh + i) * kw + j]",
                               "weight[((co * Cg + cl) * kw + j) * kh + i]"),
    "early_exit_too_tight": ("h > -1.0 &&", "h > 0.0 &&"),
    "group_base_dropped": ("const int64_t c = g * Cg + cl;", "const int64_t c = cl;"),
    "pixel_transposed": ("const int64_t pix = ho * Wo + wo;", "const int64_t pix = wo * Ho + ho;"),
    "mask_ignored": ("bilinear_zero(plane, H, W, h, w) * m;", "bilinear_zero(plane, H, W, h, w);"),
    "early_exit_right_edge": ("w < (double)W)", "w < (double)W - 1.0)"),
}


BACKWARD_MARK = " * Backward pass:"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, fixture):
    before, after = MUTANTS[name]
    with open(oracle.SOURCE) as f:
        src = f.read()
    # these checks exercise the forward: plant the mistake in the forward's
    # code (the backward section, with similar lines, follows it)
    cut = src.index(BACKWARD_MARK)
    head, tail = src[:cut], src[cut:]
    assert head.count(before) == 1, "mutation anchor not found once: %r" % before
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.c")
        with open(path, "w") as f:
            f.write(head.replace(before, after) + tail)
        so = oracle.compile_library(path, os.path.join(d, "libmutant.so"))
        lib = oracle.load_library(so)
        try:
            res = cf.all_checks(lib, fixture)
        except (ValueError, RuntimeError, IndexError) as e:  # a crash is also a catch
            res = {"raised": repr(e)}
            return
        failing = [k for k, v in res.items() if not cf.passes(k, v)]
    assert failing, "mutant %s passed every check" % name
