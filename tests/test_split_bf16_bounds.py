"""Host checks of the numerical reading of the backward's split GEMM (fp32
operands on the bf16 matrix cores): each fp32 value a is hi + mid + lo, three
bf16 values each rounded to nearest even from the remainder, and a product
a*b is taken as the six terms hi*hi + mid*hi + hi*mid + mid*mid + hi*lo +
lo*hi.  The claims checked here, on the arithmetic itself (numpy, no GPU):
the split loses at most 2^-25 |a| (normal range), the remainders are exact in
fp32, and the six-term product is within 2^-22 |a b| of the exact product.
"""
import numpy as np
import pytest


def bf16_rne(x):
    """fp32 -> bf16 (kept as fp32 with the low 16 bits zero), round to
    nearest even, for finite values."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)


def split3(a):
    a = np.asarray(a, dtype=np.float32)
    hi = bf16_rne(a)
    r = (a - hi).astype(np.float32)
    mid = bf16_rne(r)
    t = (r - mid).astype(np.float32)
    lo = bf16_rne(t)
    return hi, mid, lo, r, t


def test_rounding_is_nearest_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even -> 1; 1 + 3*2^-8
    # halfway between 1 + 2^-7 and 1 + 2^-6: even -> 1 + 2^-6
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -1.5],
                 dtype=np.float32)
    assert bf16_rne(x).tolist() == [1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -1.5]


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -60, 2.0 ** 60])
def test_split_reconstructs_within_2_pow_minus_25(scale):
    rng = np.random.default_rng(7)
    a = (rng.standard_normal(200000) * scale).astype(np.float32)
    a = np.concatenate([a, np.float32(scale) * np.array([1, -1, 1 + 2.0 ** -23, 3.0], np.float32)])
    hi, mid, lo, r, t = split3(a)
    a64 = a.astype(np.float64)
    # the remainders are exact in fp32
    assert np.array_equal(r.astype(np.float64), a64 - hi.astype(np.float64))
    assert np.array_equal(t.astype(np.float64), r.astype(np.float64) - mid.astype(np.float64))
    rec = hi.astype(np.float64) + mid.astype(np.float64) + lo.astype(np.float64)
    assert (np.abs(rec - a64) <= 2.0 ** -25 * np.abs(a64)).all()


def test_six_term_product_within_2_pow_minus_22():
    rng = np.random.default_rng(8)
    a = rng.standard_normal(200000).astype(np.float32)
    b = rng.standard_normal(200000).astype(np.float32)
    ah, am, al, _, _ = (v.astype(np.float64) for v in split3(a))
    bh, bm, bl, _, _ = (v.astype(np.float64) for v in split3(b))
    six = ah * bh + am * bh + ah * bm + am * bm + ah * bl + al * bh
    exact = a.astype(np.float64) * b.astype(np.float64)
    assert (np.abs(six - exact) <= 2.0 ** -22 * np.abs(exact)).all()
    # and the dropped terms are what the error is: a plausible mistake (a
    # term dropped from the six) breaks the bound
    five = six - am * bm
    assert not (np.abs(five - exact) <= 2.0 ** -22 * np.abs(exact)).all()
