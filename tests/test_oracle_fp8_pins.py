"""The oracle's FP8 compute mode (mdcn_oracle.c, F1-F3) against what the E4M3
format and the mathematics fix, independently of the oracle's own code:

- the quantizer against a brute-force nearest search over the 254 finite
  E4M3 values, each decoded from its bit fields (sign, 4 exponent bits with
  bias 7, 3 mantissa bits; exponent 0 subnormal; S.1111.111 NaN), ties to
  the even code, saturation at +-448;
- the row exponent against its defining inequality;
- the FP8 forward equal to the (separately pinned) exact forward when every
  weight and every column value is an E4M3 number already;
- the FP8 forward within the rounding bound of the format around the exact
  forward on random problems, and not trivially close to it;
- a hand-worked example (tests/golden/fp8_hand_worked_1x1.json).
No GPU is involved.  A mutation test plants plausible mistakes in a copy of
the oracle's FP8 code and requires that one of these checks notices.
"""
import json
import os
import shutil
import tempfile
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_hand_worked_1x1.json")


def e4m3_decode(code):
    """Value of an 8-bit E4M3 code from its bit fields."""
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    v = m * 2.0 ** -9 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


CODES = [c for c in range(256) if not np.isnan(e4m3_decode(c))]
VALUES = np.array([e4m3_decode(c) for c in CODES])


def brute_round(v):
    """Nearest finite E4M3 value, ties to the even code, |v| >= 448 -> +-448."""
    if np.isnan(v):
        return v
    if abs(v) >= 448:
        return np.copysign(448.0, v)
    best = None
    for c, y in zip(CODES, VALUES):
        if (c >> 7) != (1 if np.signbit(v) else 0):
            continue                  # the sign bit follows v (so -0.0 stays -0.0)
        d = abs(y - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
            best = (d, c, y)
    return best[2]


def check_quantizer(lib):
    """Largest disagreement of oracle.e4m3 with the brute-force rounding."""
    rng = np.random.default_rng(11)
    pos = np.sort(VALUES[VALUES > 0])
    mids = (pos[1:] + pos[:-1]) / 2
    vals = np.concatenate([
        VALUES, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
        rng.standard_normal(3000) * 10.0 ** rng.integers(-4, 3, 3000),
        [447.9, 448.0, 448.1, 464.0, 470.0, 479.0, 1e6, np.inf, -np.inf, 2.0 ** -10, 2.0 ** -11, 0.0]])
    vals = np.concatenate([vals, -vals])
    got = oracle.e4m3(vals, lib=lib)
    want = np.array([brute_round(v) for v in vals])
    bad = ~((got == want) & (np.signbit(got) == np.signbit(want)))
    return int(bad.sum()), vals[bad][:5]


def check_exponent(lib):
    """Number of rows whose exponent breaks max*2^e <= 448 < max*2^(e+1)."""
    rng = np.random.default_rng(12)
    bad = 0
    for t in range(300):
        row = rng.standard_normal(int(rng.integers(1, 40))) * 10.0 ** rng.uniform(-6, 4)
        e = oracle.fp8_row_exponent(row, lib=lib)
        mx = np.max(np.abs(row))
        if not (mx * 2.0 ** e <= 448 < mx * 2.0 ** (e + 1)):
            bad += 1
    for row, want in (([0.0, 0.0], 0), ([0.875], 9), ([-0.875], 9), ([448.0], 0),
                      ([449.0], -1), ([2.0 ** -20], 28)):
        bad += oracle.fp8_row_exponent(row, lib=lib) != want
    return bad


def small_problem(seed, exact):
    """A small problem; with exact=True every weight is an E4M3 value times
    2^-7 and every column value is an E4M3 value (integer offsets, masks in
    {0, 0.5, 1}, image values E4M3 numbers of magnitude >= 2^-5)."""
    rng = np.random.default_rng(seed)
    N, C, Co, H, W, kh, kw, G, DG = 2, 6, 4, 7, 8, 3, 3, 2, 3
    Ho, Wo = 5, 6
    K = kh * kw
    big = VALUES[(np.abs(VALUES) >= 2.0 ** -5) & (np.abs(VALUES) <= 224)]
    if exact:
        x = rng.choice(big, (N, C, H, W))
        w = rng.choice(VALUES[np.abs(VALUES) <= 64], (Co, C // G, kh, kw)) * 2.0 ** -7
        off = rng.integers(-3, 4, (N, 2 * DG * K, Ho, Wo)).astype(np.float64)
        m = rng.choice([0.0, 0.5, 1.0], (N, DG * K, Ho, Wo))
    else:
        x = rng.standard_normal((N, C, H, W))
        w = rng.standard_normal((Co, C // G, kh, kw)) * 0.1
        off = rng.standard_normal((N, 2 * DG * K, Ho, Wo)) * 1.5
        m = rng.uniform(0, 1, (N, DG * K, Ho, Wo))
    b = rng.standard_normal(Co)
    kw_ = dict(stride=(1, 2), padding=(1, 1), dilation=(1, 1), groups=G, deformable_groups=DG)
    return (x, off, m, w, b), kw_


def check_exact_inputs(lib):
    """Relative disagreement of forward_fp8 with forward when no rounding happens."""
    worst = 0.0
    for seed in range(3):
        args, kw = small_problem(seed, exact=True)
        ref = oracle.forward(*args, **kw, lib=lib)
        got, _ = oracle.forward_fp8(*args, **kw, lib=lib)
        worst = max(worst, float(np.max(np.abs(got - ref)) / np.max(np.abs(ref))))
    return worst


def rounding_bound(args, kw, lib):
    """Per output: sum over the contraction of the worst rounding of each
    product, with |q(a) - a| <= 2^-4 |a| + 2^-10 for |a| < 448 (half the
    spacing: 2^-4 relative for normals, 2^-10 absolute for subnormals), the
    weight's absolute term scaled back by 2^-e of its row."""
    x, off, m, w, b = args
    ax = np.abs(x)
    bound_args = (ax, off, np.abs(m), np.ones_like(w), None)
    # sum |w| |v| and sum |v| per output come from the exact oracle on |x|, |m|
    # (a bilinear sample of |x| bounds |sample of x|), with |w| and with ones
    s_wv = oracle.forward(ax, off, np.abs(m), np.abs(w), None, **kw, lib=lib)
    s_v = oracle.forward(*bound_args, **kw, lib=lib)
    G = kw["groups"]
    Co, Cg, kh, kw_ = w.shape
    ew = np.array([oracle.fp8_row_exponent(w[c], lib=lib) for c in range(Co)])
    aw = 2.0 ** -10 * 2.0 ** -ew                       # absolute term of the weights
    # sum |w| over one row, times the columns' absolute term
    s_w = np.abs(w).reshape(Co, -1).sum(1)
    cnt = Cg * kh * kw_
    r = 2.0 ** -4
    # |qw qv - w v| <= (r|w| + aw)(|v|(1 + r) + 2^-10) + |w|(r|v| + 2^-10)
    bound = ((2 * r + r * r) * s_wv + aw[None, :, None, None] * (1 + r) * s_v
             + (r + 1) * 2.0 ** -10 * s_w[None, :, None, None]
             + aw[None, :, None, None] * 2.0 ** -10 * cnt)
    return bound


def check_rounding_bound(lib):
    """(largest error / bound, largest error / output scale) on random problems."""
    worst, largest = 0.0, 0.0
    for seed in range(3):
        args, kw = small_problem(100 + seed, exact=False)
        ref = oracle.forward(*args, **kw, lib=lib)
        got, _ = oracle.forward_fp8(*args, **kw, lib=lib)
        bound = rounding_bound(args, kw, lib)
        worst = max(worst, float(np.max(np.abs(got - ref) / bound)))
        largest = max(largest, float(np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref ** 2))))
    return worst, largest


def check_hand_example(lib, fx):
    got, _ = oracle.forward_fp8(np.array(fx["x"]), np.array(fx["offset"]), np.array(fx["mask"]),
                                np.array(fx["weight"]), np.array(fx["bias"]),
                                stride=fx["stride"], padding=fx["padding"],
                                dilation=fx["dilation"], groups=fx["groups"],
                                deformable_groups=fx["deformable_groups"], lib=lib)
    want = np.vectorize(lambda s: float(Fraction(s)))(np.array(fx["expected_fraction"]))
    return float(np.max(np.abs(got - want)))


def check_abs_sum(lib):
    """forward_fp8's second result is 2^-e * sum |q(w) q(col)|.  With exact
    inputs q is the identity, and with integer offsets each sample is one
    corner, so |col| = |x| |m| at that corner: the result then equals the
    exact forward of |x|, |m|, |w| without bias."""
    args, kw = small_problem(5, exact=True)
    x, off, m, w, b = args
    _, asum = oracle.forward_fp8(*args, **kw, lib=lib)
    want = oracle.forward(np.abs(x), off, np.abs(m), np.abs(w), None, **kw, lib=lib)
    return float(np.max(np.abs(asum - want)) / np.max(want))


def all_checks(lib, fx):
    nq, _ = check_quantizer(lib)
    worst, largest = check_rounding_bound(lib)
    return {"quantizer": nq, "exponent": check_exponent(lib),
            "exact_inputs": check_exact_inputs(lib), "rounding_bound": worst,
            "not_trivial": largest, "hand": check_hand_example(lib, fx),
            "abs_sum": check_abs_sum(lib)}


def passes(name, v):
    if name in ("quantizer", "exponent"):
        return v == 0
    if name in ("exact_inputs", "abs_sum"):
        return v <= 1e-12
    if name == "rounding_bound":
        return v <= 1.0
    if name == "not_trivial":
        return v >= 1e-3          # quantization must change the result visibly
    if name == "hand":
        return v <= 1e-15
    raise KeyError(name)


@pytest.fixture(scope="module")
def lib():
    return oracle.load_library()


@pytest.fixture(scope="module")
def fixture():
    with open(GOLDEN) as f:
        return json.load(f)


def test_quantizer_matches_brute_force(lib):
    n, examples = check_quantizer(lib)
    assert n == 0, examples


def test_known_e4m3_values(lib):
    vals = [448.0, 2.0 ** -9, 2.0 ** -6, 1.0, 240.0, -3.5]
    assert list(oracle.e4m3(vals, lib=lib)) == vals
    assert e4m3_decode(0x7E) == 448.0 and e4m3_decode(0x01) == 2.0 ** -9
    assert e4m3_decode(0x38) == 1.0 and np.isnan(e4m3_decode(0x7F))
    assert np.isnan(oracle.e4m3([np.nan], lib=lib)[0])
    assert list(oracle.e4m3([np.inf, -1e9], lib=lib)) == [448.0, -448.0]


def test_row_exponent(lib):
    assert check_exponent(lib) == 0


def test_equals_exact_forward_on_representable_inputs(lib):
    assert passes("exact_inputs", check_exact_inputs(lib))


def test_within_format_rounding_bound(lib):
    worst, largest = check_rounding_bound(lib)
    assert worst <= 1.0, worst
    assert largest >= 1e-3, largest


def test_hand_worked_example(lib, fixture):
    assert check_hand_example(lib, fixture) <= 1e-15


def test_abs_sum(lib):
    assert passes("abs_sum", check_abs_sum(lib))


def test_points_agree_with_full_forward(lib):
    args, kw = small_problem(9, exact=False)
    full, fs = oracle.forward_fp8(*args, **kw, lib=lib)
    idx = np.random.default_rng(0).choice(full.size, size=40, replace=False)
    pts, ps = oracle.forward_points_fp8(*args, idx, **kw, lib=lib)
    assert np.array_equal(pts, full.reshape(-1)[idx]) and np.array_equal(ps, fs.reshape(-1)[idx])


# (what the oracle says, a plausible mistake in its place)
MUTANTS = {
    "ties_away": ("return copysign(nearbyint(a / step) * step, v);",
                  "return copysign(round(a / step) * step, v);"),
    "truncating": ("return copysign(nearbyint(a / step) * step, v);",
                   "return copysign(floor(a / step) * step, v);"),
    "mantissa_bits_4": ("step = ldexp(1.0, ex - 1 - 3);", "step = ldexp(1.0, ex - 1 - 4);"),
    "subnormal_step": ("step = 0x1p-9;", "step = 0x1p-10;"),
    "no_saturation": ("if (a >= 448.0)", "if (a >= 480.0)"),
    "exponent_off_by_one": ("int e = (f <= 0.875) ? 9 - ex : 8 - ex;",
                            "int e = (f <= 0.875) ? 10 - ex : 9 - ex;"),
    "exponent_threshold": ("int e = (f <= 0.875) ? 9 - ex : 8 - ex;",
                           "int e = (f < 0.75) ? 9 - ex : 8 - ex;"),
    "scale_not_undone": ("acc *= scale[co];", "acc *= 1.0;"),
    "abs_sum_unscaled": ("*abs_sum = scale ? sa * scale[co] : sa;", "*abs_sum = sa;"),
    "column_not_rounded": ("const double col = scale ? mdcn_oracle_e4m3(val) : val;",
                           "const double col = val;"),
    "mask_after_rounding": ("const double col = scale ? mdcn_oracle_e4m3(val) : val;",
                            "const double col = scale ? mdcn_oracle_e4m3(val / m) * m : val;"),
    "weight_not_rounded": ("qw[co * Cg * K + t] = mdcn_oracle_e4m3(ldexp(row[t], e));",
                           "qw[co * Cg * K + t] = ldexp(row[t], e);"),
    "fp8_bias_dropped": ("    if (bias)\n        acc += bias[co];",
                         "    if (bias)\n        acc += scale ? 0.0 : bias[co];"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, fixture):
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
        res = all_checks(lib, fixture)
        failing = [k for k, v in res.items() if not passes(k, v)]
    assert failing, "mutant %s passed every check: %s" % (name, res)
