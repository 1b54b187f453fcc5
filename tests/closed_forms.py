"""Closed forms that pin the CPU oracle to something other than itself.

Every check here computes the expected output of a special case of the
modulated deformable convolution by a different route than the oracle's
per-element loop: torch's float64 ``conv2d`` (a library routine) on shifted,
zero-extended copies of the image, exact algebraic identities, and
hand-worked numbers.  The special cases follow the operator's definition on
the page "TensorRT 插件解析：modulatedDeformConvPlugin 可变形卷积插件的原理、参数与使用指南":
  - §二: layouts of x, offset, mask, weight, bias; output dims
    [x.d0, weight.d0, offset.d2, offset.d3];
  - §三: group and deformable_group split channels into contiguous blocks;
  - §五 step 1: sample point = anchor (out*stride - pad) + tap*dilation +
    offset, bilinear interpolation, 0 outside the image, times the mask;
  - §五 steps 2-3: contraction per group, then the optional bias.

Each ``check_*`` function takes the loaded oracle library and returns the
largest absolute deviation from the closed form, so the same checks can be run
against deliberately altered oracle builds (the mutation test).
"""
from __future__ import annotations

import math

import torch
import torch.nn.functional as F

from oracle import oracle


# ---------------------------------------------------------------- problems

def conv_out_len(n, k, s, p, d):
    return (n + 2 * p - d * (k - 1) - 1) // s + 1


def make_problem(N=2, C=4, Co=6, H=7, W=9, kh=2, kw=3, stride=(2, 1), padding=(1, 2),
                 dilation=(2, 1), groups=2, dg=2, Ho=None, Wo=None):
    Ho = Ho if Ho is not None else conv_out_len(H, kh, stride[0], padding[0], dilation[0])
    Wo = Wo if Wo is not None else conv_out_len(W, kw, stride[1], padding[1], dilation[1])
    return dict(N=N, C=C, Co=Co, H=H, W=W, kh=kh, kw=kw, stride=stride, padding=padding,
                dilation=dilation, groups=groups, dg=dg, Ho=Ho, Wo=Wo)


# A spread of small problems: kh != kw, H != W, Ho != Wo, asymmetric stride,
# padding and dilation, several groups and offset groups, and an output grid
# smaller than the conv formula gives.
PROBLEMS = [
    make_problem(),
    make_problem(N=1, C=6, Co=3, H=8, W=5, kh=3, kw=2, stride=(1, 2), padding=(2, 0),
                 dilation=(1, 2), groups=3, dg=3),
    make_problem(N=2, C=4, Co=4, H=6, W=6, kh=3, kw=3, stride=(1, 1), padding=(1, 1),
                 dilation=(1, 1), groups=1, dg=1),
    make_problem(N=1, C=8, Co=8, H=5, W=7, kh=1, kw=3, stride=(1, 1), padding=(0, 1),
                 dilation=(1, 3), groups=8, dg=4),
    make_problem(N=2, C=4, Co=2, H=9, W=7, kh=3, kw=3, stride=(2, 2), padding=(2, 2),
                 dilation=(2, 2), groups=2, dg=4, Ho=3, Wo=2),
]


def random_tensors(pr, seed, bias=True):
    g = torch.Generator().manual_seed(seed)
    K = pr["kh"] * pr["kw"]
    x = torch.randn(pr["N"], pr["C"], pr["H"], pr["W"], generator=g, dtype=torch.float64)
    w = torch.randn(pr["Co"], pr["C"] // pr["groups"], pr["kh"], pr["kw"], generator=g,
                    dtype=torch.float64)
    b = torch.randn(pr["Co"], generator=g, dtype=torch.float64) if bias else None
    m = torch.rand(pr["N"], pr["dg"] * K, pr["Ho"], pr["Wo"], generator=g,
                   dtype=torch.float64) + 0.25
    return x, w, b, m


def run_oracle(lib, pr, x, off, m, w, b):
    return torch.from_numpy(oracle.forward(
        x, off, m, w, b, stride=pr["stride"], padding=pr["padding"],
        dilation=pr["dilation"], groups=pr["groups"], deformable_groups=pr["dg"], lib=lib))


def anchors(pr):
    """Integer anchor rows [Ho, kh] and columns [Wo, kw] of every tap."""
    ah = (torch.arange(pr["Ho"])[:, None] * pr["stride"][0] - pr["padding"][0]
          + torch.arange(pr["kh"])[None, :] * pr["dilation"][0])
    aw = (torch.arange(pr["Wo"])[:, None] * pr["stride"][1] - pr["padding"][1]
          + torch.arange(pr["kw"])[None, :] * pr["dilation"][1])
    return ah.double(), aw.double()


# ---------------------------------------------------------------- conv-based closed forms

def shifted_canvas(x, pr, a, b):
    """Zero-extended image re-indexed so that a padding-0 conv with the same
    stride and dilation reads pixel (anchor + tap*dilation + (a, b)):
    Y[u][v] = x[u - ph + a][v - pw + b], 0 where that pixel is off the image."""
    _, _, H, W = x.shape
    Hc = (pr["Ho"] - 1) * pr["stride"][0] + (pr["kh"] - 1) * pr["dilation"][0] + 1
    Wc = (pr["Wo"] - 1) * pr["stride"][1] + (pr["kw"] - 1) * pr["dilation"][1] + 1
    top, left = -pr["padding"][0] + a, -pr["padding"][1] + b
    pad_t, pad_l = max(0, -top), max(0, -left)
    pad_b, pad_r = max(0, top + Hc - H), max(0, left + Wc - W)
    xp = F.pad(x, (pad_l, pad_r, pad_t, pad_b))
    return xp[:, :, top + pad_t: top + pad_t + Hc, left + pad_l: left + pad_l + Wc]


class ShiftConv:
    """conv2d of channel block q of x, shifted by (a, b), with tap (i, j) of
    the weight only; cached because the closed forms reuse them."""

    def __init__(self, x, w, pr):
        self.x, self.w, self.pr, self.cache = x, w, pr, {}
        cdg = x.shape[1] // pr["dg"]
        self.blocks = []
        for q in range(pr["dg"]):
            t = torch.zeros_like(x)
            t[:, q * cdg:(q + 1) * cdg] = x[:, q * cdg:(q + 1) * cdg]
            self.blocks.append(t)

    def __call__(self, q, i, j, a, b):
        key = (q, i, j, a, b)
        if key not in self.cache:
            wk = torch.zeros_like(self.w)
            wk[:, :, i, j] = self.w[:, :, i, j]
            y = shifted_canvas(self.blocks[q], self.pr, a, b)
            out = F.conv2d(y, wk, None, stride=self.pr["stride"], padding=0,
                           dilation=self.pr["dilation"], groups=self.pr["groups"])
            self.cache[key] = out[:, :, :self.pr["Ho"], :self.pr["Wo"]]
        return self.cache[key]


def offsets_from_values(pr, vh, vw):
    """Offset tensor [N, 2*dg*K, Ho, Wo] from per-(n, q, k, ho, wo) values:
    channel q*2K + 2k holds the row offset, q*2K + 2k + 1 the column offset."""
    N, dg, K = vh.shape[0], pr["dg"], pr["kh"] * pr["kw"]
    off = torch.zeros(N, 2 * dg * K, pr["Ho"], pr["Wo"], dtype=torch.float64)
    for q in range(dg):
        for k in range(K):
            off[:, q * 2 * K + 2 * k] = vh[:, q, k]
            off[:, q * 2 * K + 2 * k + 1] = vw[:, q, k]
    return off


def selected_shift_sum(x, w, b, pr, values, sel_h, sel_w, mask):
    """Expected output when every offset is taken from the list ``values``.

    sel_h / sel_w [N, dg, K, Ho, Wo] index ``values`` per offset group, tap and
    output pixel.  A value v = floor(v) + f is the blend (1-f)*shift(floor v) +
    f*shift(floor v + 1) along its axis, so every sample is a weighted sum of
    four integer-shifted one-tap convolutions of its channel block."""
    sc = ShiftConv(x, w, pr)
    K, kw = pr["kh"] * pr["kw"], pr["kw"]
    out = torch.zeros(x.shape[0], w.shape[0], pr["Ho"], pr["Wo"], dtype=torch.float64)
    for q in range(pr["dg"]):
        for k in range(K):
            i, j = divmod(k, kw)
            for ra, va in enumerate(values):
                for rb, vb in enumerate(values):
                    sel = ((sel_h[:, q, k] == ra) & (sel_w[:, q, k] == rb)).double()
                    if not bool(sel.any()):
                        continue
                    fa, fb = math.floor(va), math.floor(vb)
                    al, be = va - fa, vb - fb
                    val = 0
                    for da, wa in ((0, 1.0 - al), (1, al)):
                        for db, wb in ((0, 1.0 - be), (1, be)):
                            if wa * wb != 0.0:
                                val = val + (wa * wb) * sc(q, i, j, fa + da, fb + db)
                    out += val * (sel * mask[:, q * K + k])[:, None]
    if b is not None:
        out += b[None, :, None, None]
    return out


# ---------------------------------------------------------------- checks

def check_plain_conv(lib, pr, seed=0):
    """offset = 0, mask = 1: the operator is an ordinary grouped convolution."""
    x, w, b, _ = random_tensors(pr, seed)
    K = pr["kh"] * pr["kw"]
    off = torch.zeros(pr["N"], 2 * pr["dg"] * K, pr["Ho"], pr["Wo"], dtype=torch.float64)
    m = torch.ones(pr["N"], pr["dg"] * K, pr["Ho"], pr["Wo"], dtype=torch.float64)
    got = run_oracle(lib, pr, x, off, m, w, b)
    ref = F.conv2d(x, w, b, stride=pr["stride"], padding=pr["padding"],
                   dilation=pr["dilation"], groups=pr["groups"])[:, :, :pr["Ho"], :pr["Wo"]]
    return float((got - ref).abs().max())


def _check_selected(lib, pr, seed, values):
    x, w, b, m = random_tensors(pr, seed)
    g = torch.Generator().manual_seed(seed + 1000)
    shape = (pr["N"], pr["dg"], pr["kh"] * pr["kw"], pr["Ho"], pr["Wo"])
    sel_h = torch.randint(0, len(values), shape, generator=g)
    sel_w = torch.randint(0, len(values), shape, generator=g)
    vv = torch.tensor(values, dtype=torch.float64)
    off = offsets_from_values(pr, vv[sel_h], vv[sel_w])
    got = run_oracle(lib, pr, x, off, m, w, b)
    ref = selected_shift_sum(x, w, b, pr, values, sel_h, sel_w, m)
    return float((got - ref).abs().max())


def check_integer_offsets(lib, pr, seed=0):
    """Integer offsets and masks varying per pixel, tap and offset group:
    each sample is one pixel of the zero-extended image."""
    return _check_selected(lib, pr, seed, [-3.0, -1.0, 0.0, 2.0])


def check_fractional_offsets(lib, pr, seed=0):
    """Fractional offsets (negative ones included, which need floor, not
    truncation) varying per pixel, tap and offset group."""
    return _check_selected(lib, pr, seed, [-2.75, -0.5, 0.25, 1.625])


def check_zero_mask(lib, pr, seed=0):
    """mask = 0 everywhere: the output is the bias, exactly."""
    x, w, b, _ = random_tensors(pr, seed)
    g = torch.Generator().manual_seed(seed + 3000)
    K = pr["kh"] * pr["kw"]
    off = torch.randn(pr["N"], 2 * pr["dg"] * K, pr["Ho"], pr["Wo"], generator=g,
                      dtype=torch.float64) * 2
    m = torch.zeros(pr["N"], pr["dg"] * K, pr["Ho"], pr["Wo"], dtype=torch.float64)
    got = run_oracle(lib, pr, x, off, m, w, b)
    return float((got - b[None, :, None, None]).abs().max())


def check_off_image(lib, pr, seed=0):
    """Every sample off the image -- far away, or exactly on one of the lines
    h = -1, h = H, w = -1, w = W, where each corner is either off the image or
    has weight 0: the output is the bias, exactly."""
    x, w, b, m = random_tensors(pr, seed)
    H, W, K = pr["H"], pr["W"], pr["kh"] * pr["kw"]
    ah, aw = anchors(pr)                       # [Ho, kh], [Wo, kw]
    big = float(4 * (H + W + 16))
    # (target row, target column) as functions of the anchors
    cases = [
        (lambda r: r + big, lambda c: c + 0.0),
        (lambda r: r - big, lambda c: c + 0.3),
        (lambda r: r + 0.4, lambda c: c + big),
        (lambda r: r - 0.2, lambda c: c - big),
        (lambda r: torch.full_like(r, -1.0), lambda c: c + 0.6),
        (lambda r: torch.full_like(r, float(H)), lambda c: c - 0.5),
        (lambda r: r + 0.7, lambda c: torch.full_like(c, -1.0)),
        (lambda r: r - 0.1, lambda c: torch.full_like(c, float(W))),
    ]
    worst = 0.0
    for th, tw in cases:
        vh = torch.zeros(pr["N"], pr["dg"], K, pr["Ho"], pr["Wo"], dtype=torch.float64)
        vw = torch.zeros_like(vh)
        for k in range(K):
            i, j = divmod(k, pr["kw"])
            r = ah[:, i][:, None].expand(pr["Ho"], pr["Wo"])
            c = aw[:, j][None, :].expand(pr["Ho"], pr["Wo"])
            vh[:, :, k] = th(r) - r
            vw[:, :, k] = tw(c) - c
        off = offsets_from_values(pr, vh, vw)
        got = run_oracle(lib, pr, x, off, m, w, b)
        worst = max(worst, float((got - b[None, :, None, None]).abs().max()))
    return worst


def check_bilinear_function(lib, seed=0):
    """Bilinear interpolation reproduces f(h, w) = a + b*h + c*w + d*h*w
    exactly inside [0, H-1] x [0, W-1]; in the one-pixel rim outside the
    image the zero extension scales the edge value linearly down to 0.  A 1x1
    kernel with unit weight on one channel makes the output the sample itself
    times the mask."""
    g = torch.Generator().manual_seed(seed)
    H, W, Ho, Wo = 6, 9, 5, 7
    a, bb, c, d = 0.7, -1.3, 0.45, 0.2
    hh = torch.arange(H, dtype=torch.float64)[:, None]
    ww = torch.arange(W, dtype=torch.float64)[None, :]
    img = (a + bb * hh + c * ww + d * hh * ww)[None, None]
    pr = dict(stride=(1, 1), padding=(0, 0), dilation=(1, 1), groups=1, dg=1)
    sh = torch.rand(Ho, Wo, generator=g, dtype=torch.float64) * (H + 0.98) - 0.99
    sw = torch.rand(Ho, Wo, generator=g, dtype=torch.float64) * (W + 0.98) - 0.99
    off = torch.stack([sh - torch.arange(Ho, dtype=torch.float64)[:, None],
                       sw - torch.arange(Wo, dtype=torch.float64)[None, :]])[None]
    m = torch.rand(1, 1, Ho, Wo, generator=g, dtype=torch.float64)
    got = run_oracle(lib, pr, img, off, m, torch.ones(1, 1, 1, 1, dtype=torch.float64),
                     None)[0, 0]

    def rim(s, n):  # (edge factor, coordinate clamped into the image)
        if s < 0:
            return s + 1.0, 0.0
        if s > n - 1:
            return float(n) - s, float(n - 1)
        return 1.0, s

    ref = torch.empty(Ho, Wo, dtype=torch.float64)
    for u in range(Ho):
        for v in range(Wo):
            fh, ch = rim(float(sh[u, v]), H)
            fw, cw = rim(float(sw[u, v]), W)
            ref[u, v] = fh * fw * (a + bb * ch + c * cw + d * ch * cw) * float(m[0, 0, u, v])
    return float((got - ref).abs().max())


def check_linearity(lib, pr, seed=0):
    """out - bias is linear in x, in the weight and in the mask."""
    x, w, b, m = random_tensors(pr, seed)
    x2, w2, _, m2 = random_tensors(pr, seed + 1)
    g = torch.Generator().manual_seed(seed + 4000)
    K = pr["kh"] * pr["kw"]
    off = torch.randn(pr["N"], 2 * pr["dg"] * K, pr["Ho"], pr["Wo"], generator=g,
                      dtype=torch.float64) * 1.5
    al, be = 0.75, -1.25

    def o(xx, ww, mm):
        return run_oracle(lib, pr, xx, off, mm, ww, b) - b[None, :, None, None]
    e1 = (o(al * x + be * x2, w, m) - (al * o(x, w, m) + be * o(x2, w, m))).abs().max()
    e2 = (o(x, al * w + be * w2, m) - (al * o(x, w, m) + be * o(x, w2, m))).abs().max()
    e3 = (o(x, w, al * m + be * m2) - (al * o(x, w, m) + be * o(x, w, m2))).abs().max()
    return float(max(e1, e2, e3))


def check_hand_example(lib, fixture):
    """Values worked out by hand, stored under tests/golden/."""
    pr = dict(stride=tuple(fixture["stride"]), padding=tuple(fixture["padding"]),
              dilation=tuple(fixture["dilation"]), groups=fixture["groups"],
              dg=fixture["deformable_groups"])
    t = {k: torch.tensor(fixture[k], dtype=torch.float64)
         for k in ("x", "offset", "mask", "weight")}
    b = torch.tensor(fixture["bias"], dtype=torch.float64) if fixture.get("bias") else None
    got = run_oracle(lib, pr, t["x"], t["offset"], t["mask"], t["weight"], b)
    ref = torch.tensor(fixture["expected"], dtype=torch.float64)
    if got.shape != ref.shape:
        return float("inf")
    return float((got - ref).abs().max())


CHECKS_PER_PROBLEM = {
    "plain_conv": check_plain_conv,
    "integer_offsets": check_integer_offsets,
    "fractional_offsets": check_fractional_offsets,
    "zero_mask": check_zero_mask,
    "off_image": check_off_image,
    "linearity": check_linearity,
}

# Checks that involve no rounding: their deviation must be exactly 0.
EXACT = ("zero_mask", "off_image")
TOL = 1e-10


def all_checks(lib, fixture):
    """Run every check; returns {name: max abs deviation}."""
    res = {}
    for idx, pr in enumerate(PROBLEMS):
        for name, fn in CHECKS_PER_PROBLEM.items():
            res["%s_%d" % (name, idx)] = fn(lib, pr)
    res["bilinear_function"] = check_bilinear_function(lib)
    res["hand_example"] = check_hand_example(lib, fixture)
    return res


def passes(name, err):
    if any(name.startswith(e) for e in EXACT):
        return err == 0.0
    return err <= TOL
