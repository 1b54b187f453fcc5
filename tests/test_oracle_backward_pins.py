"""The oracle's backward pass (mdcn_oracle_backward, readings B1-B3) against
routes that do not go through it:

- the forward (pinned in test_oracle_pins.py) is linear in x, in the mask,
  in the weight and in the bias separately, so for any direction d the
  gradient must satisfy the adjoint identity
  <grad, d> = <grad_out, forward with that input replaced by d, no bias>
  (bias: <grad_b, d> = <grad_out, forward with zero weight and bias d>);
- the offsets enter nonlinearly: the directional derivative <grad_offset, d>
  must match a central finite difference of <grad_out, forward(offset)>, at
  offsets kept away from integer sample coordinates (where the bilinear
  sample has a kink) and from the window edges;
- at exact integer sample coordinates (inside the image) reading B1 takes
  the derivative from above: a one-sided difference along directions that
  move every coordinate up must match.
A mutation test plants plausible mistakes in a copy of the backward code
and requires that one of these checks notices.  No GPU is involved.
"""
import os
import shutil
import tempfile

import numpy as np
import pytest

from oracle import oracle

ATTRS = dict(stride=(1, 2), padding=(1, 2), dilation=(2, 1), groups=2, deformable_groups=2)


def problem(seed):
    rng = np.random.default_rng(seed)
    N, C, Co, H, W, kh, kw = 2, 4, 6, 7, 8, 3, 2
    Ho, Wo = 5, 6
    G, DG = ATTRS["groups"], ATTRS["deformable_groups"]
    K = kh * kw
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((Co, C // G, kh, kw))
    m = rng.uniform(0.2, 1.0, (N, DG * K, Ho, Wo))
    off = rng.uniform(-2.5, 2.5, (N, 2 * DG * K, Ho, Wo))
    # keep every sample coordinate at least 0.05 from an integer (the bilinear
    # sample's kinks) so that central differences see a smooth function
    frac = off - np.floor(off)
    off = np.where(frac < 0.05, off + 0.05, np.where(frac > 0.95, off - 0.05, off))
    go = rng.standard_normal((N, Co, Ho, Wo))
    return x, off, m, w, go


def dot(a, b):
    return float(np.sum(np.asarray(a) * np.asarray(b)))


def check_adjoint(lib):
    """Largest relative violation of the adjoint identities (x, mask, weight, bias)."""
    worst = 0.0
    for seed in range(3):
        x, off, m, w, go = problem(seed)
        g = oracle.backward(x, off, m, w, go, **ATTRS, lib=lib)
        rng = np.random.default_rng(50 + seed)
        for name in ("x", "mask", "weight", "bias"):
            if name == "bias":
                d = rng.standard_normal(w.shape[0])
                f = oracle.forward(x, off, m, np.zeros_like(w), d, **ATTRS, lib=lib)
                lhs = dot(g["bias"], d)
            else:
                d = rng.standard_normal({"x": x, "mask": m, "weight": w}[name].shape)
                args = dict(x=x, offset=off, mask=m, weight=w)
                args[name] = d
                f = oracle.forward(args["x"], args["offset"], args["mask"], args["weight"], None,
                                   **ATTRS, lib=lib)
                lhs = dot(g[name], d)
            rhs = dot(go, f)
            worst = max(worst, abs(lhs - rhs) / max(abs(rhs), 1e-12))
    return worst


def check_offset_fd(lib):
    """Largest relative mismatch of <grad_offset, d> with a central difference."""
    worst = 0.0
    for seed in range(3):
        x, off, m, w, go = problem(seed)
        g = oracle.backward(x, off, m, w, go, **ATTRS, lib=lib)
        rng = np.random.default_rng(90 + seed)
        d = rng.standard_normal(off.shape)
        eps = 1e-5          # moves no coordinate across a kink (0.05 away, |d| < 5)
        lp = dot(go, oracle.forward(x, off + eps * d, m, w, None, **ATTRS, lib=lib))
        lm = dot(go, oracle.forward(x, off - eps * d, m, w, None, **ATTRS, lib=lib))
        fd = (lp - lm) / (2 * eps)
        an = dot(g["offset"], d)
        worst = max(worst, abs(fd - an) / max(abs(an), 1e-9))
        # and one offset channel at a time (h and w separately)
        for ch in (0, 1, 5):
            dd = np.zeros_like(off)
            dd[:, ch] = rng.standard_normal(dd[:, ch].shape)
            lp = dot(go, oracle.forward(x, off + eps * dd, m, w, None, **ATTRS, lib=lib))
            lm = dot(go, oracle.forward(x, off - eps * dd, m, w, None, **ATTRS, lib=lib))
            fd = (lp - lm) / (2 * eps)
            an = dot(g["offset"], dd)
            worst = max(worst, abs(fd - an) / max(abs(an), 1e-9))
    return worst


def integer_problem(seed):
    """problem(seed) with every sample coordinate an exact integer inside the
    image ([0, H-1] x [0, W-1]): the offsets move each anchor to the nearest
    integer point, clamped onto the image."""
    x, off, m, w, go = problem(seed)
    N, _, H, W = x.shape
    kh, kw = w.shape[2], w.shape[3]
    K = kh * kw
    sh, sw = ATTRS["stride"]
    ph, pw = ATTRS["padding"]
    dh, dw = ATTRS["dilation"]
    Ho, Wo = off.shape[2], off.shape[3]
    ho = np.arange(Ho)[:, None]
    wo = np.arange(Wo)[None, :]
    out = np.empty_like(off)
    for ch in range(off.shape[1]):
        k = (ch % (2 * K)) // 2
        i, j = k // kw, k % kw
        if ch % 2 == 0:
            anchor = (ho * sh - ph + i * dh) * np.ones((1, Wo))
            lim = H - 1
        else:
            anchor = (wo * sw - pw + j * dw) * np.ones((Ho, 1))
            lim = W - 1
        target = np.clip(anchor[None] + np.round(off[:, ch]), 0, lim)
        out[:, ch] = target - anchor[None]
    return x, out, m, w, go


def check_integer_one_sided(lib):
    """At exact integer sample coordinates the bilinear sample has a kink;
    reading B1 differentiates on the cell floor() selects, i.e. from above.
    A one-sided difference along directions that move every coordinate up
    must match <grad_offset, d> there."""
    worst = 0.0
    for seed in range(3):
        x, off, m, w, go = integer_problem(seed)
        g = oracle.backward(x, off, m, w, go, **ATTRS, lib=lib)
        rng = np.random.default_rng(130 + seed)
        l0 = dot(go, oracle.forward(x, off, m, w, None, **ATTRS, lib=lib))
        eps = 1e-7
        dirs = [rng.uniform(0.1, 1.0, off.shape)]
        for ch in (0, 1, 4):           # one offset channel at a time: h, w, another tap's h
            dd = np.zeros_like(off)
            dd[:, ch] = rng.uniform(0.1, 1.0, dd[:, ch].shape)
            dirs.append(dd)
        for d in dirs:
            lp = dot(go, oracle.forward(x, off + eps * d, m, w, None, **ATTRS, lib=lib))
            fd = (lp - l0) / eps
            an = dot(g["offset"], d)
            worst = max(worst, abs(fd - an) / max(abs(an), 1e-9))
    return worst


def check_off_image(lib):
    """Samples beyond the window give zero gradients for offset and mask."""
    x, off, m, w, go = problem(7)
    off = off + 100.0
    g = oracle.backward(x, off, m, w, go, **ATTRS, lib=lib)
    return float(np.abs(g["offset"]).max() + np.abs(g["mask"]).max() + np.abs(g["x"]).max()
                 + np.abs(g["weight"]).max())


def all_checks(lib):
    return {"adjoint": check_adjoint(lib), "offset_fd": check_offset_fd(lib),
            "integer_one_sided": check_integer_one_sided(lib),
            "off_image": check_off_image(lib)}


LIMITS = {"adjoint": 1e-10, "offset_fd": 1e-6, "integer_one_sided": 1e-5, "off_image": 0.0}


def passes(name, v):
    return v <= LIMITS[name]


@pytest.fixture(scope="module")
def lib():
    return oracle.load_library()


def test_adjoint_identities(lib):
    assert passes("adjoint", check_adjoint(lib))


def test_offset_gradient_matches_finite_differences(lib):
    assert passes("offset_fd", check_offset_fd(lib))


def test_offset_gradient_at_integer_coordinates_is_from_above(lib):
    x, off, m, w, go = integer_problem(0)
    assert np.array_equal(off, np.round(off))   # really on the kinks
    assert passes("integer_one_sided", check_integer_one_sided(lib))


def test_off_image_samples_have_no_gradient(lib):
    assert passes("off_image", check_off_image(lib))


def test_bias_gradient_closed_form(lib):
    x, off, m, w, go = problem(3)
    g = oracle.backward(x, off, m, w, go, **ATTRS, lib=lib)
    assert np.allclose(g["bias"], go.sum(axis=(0, 2, 3)), rtol=1e-13, atol=1e-13)
    assert oracle.backward(x, off, m, w, go, with_bias=False, **ATTRS, lib=lib)["bias"] is None


MUTANTS = {
    "dh_columns_swapped": ("*dh = (1.0 - b) * (v10 - v00) + b * (v11 - v01);",
                           "*dh = (1.0 - b) * (v01 - v00) + b * (v11 - v10);"),
    "dw_sign": ("*dw = (1.0 - a) * (v01 - v00) + a * (v11 - v10);",
                "*dw = (1.0 - a) * (v00 - v01) + a * (v11 - v10);"),
    "offset_grad_without_mask": ("goff[oh] += gwt * m * dh;", "goff[oh] += gwt * dh;"),
    "offset_h_w_swapped": ("goff[oh] += gwt * m * dh;\n                                goff[ow] += gwt * m * dw;",
                           "goff[oh] += gwt * m * dw;\n                                goff[ow] += gwt * m * dh;"),
    "mask_grad_with_mask": ("gmask[mi] += gwt * v;", "gmask[mi] += gwt * v * m;"),
    "weight_grad_without_mask": ("gw[wi] += g * v * m;", "gw[wi] += g * v;"),
    "scatter_corner_swapped": ("cx[4] = {x0, x0 + 1, x0, x0 + 1};", "cx[4] = {x0 + 1, x0, x0, x0 + 1};"),
    "scatter_without_mask": ("scatter_corners(gx + (n * C + c) * H * W, H, W, h, w, gwt * m);",
                             "scatter_corners(gx + (n * C + c) * H * W, H, W, h, w, gwt);"),
    "scatter_weights_transposed": ("(1.0 - a) * b, a * (1.0 - b), a * b};",
                                   "a * (1.0 - b), (1.0 - a) * b, a * b};"),
    "bias_grad_dropped": ("        gb[co] += g;", "        gb[co] += 0.0;"),
    # at an integer coordinate, the cell below (derivative from below); the
    # same value and the same derivative everywhere else
    "derivative_from_below": ("        return 0.0;\n    const double hf = floor(h), wf = floor(w);",
                              "        return 0.0;\n    const double hf = ceil(h) - 1.0, wf = ceil(w) - 1.0;"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    before, after = MUTANTS[name]
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(before) == 1, "mutation anchor not found once: %r" % before
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(before, after))
        so = oracle.compile_library(path, os.path.join(d, "libmutant.so"))
        lib = oracle.load_library(so)
        res = all_checks(lib)
        try:
            x, off, m, w, go = problem(3)
            g = oracle.backward(x, off, m, w, go, **ATTRS, lib=lib)
            res["bias_closed_form"] = float(np.abs(g["bias"] - go.sum(axis=(0, 2, 3))).max())
        except ValueError:
            res["bias_closed_form"] = 1.0
        failing = [k for k, v in res.items() if not (v <= LIMITS.get(k, 1e-12))]
    assert failing, "mutant %s passed every check: %s" % (name, res)
