"""Pins for the oracle's binary16 decode and its fp64 -> fp16 rounding.

The rounding the oracle applies once per output (the float16 cast in the
tutorial's epilogue, "1. WGMMA", section "The Full Kernel", read as IEEE 754
round-to-nearest-even) is checked against two things that do not share its
code: numpy's float64 -> float16 conversion, and exact rational rounding.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests._exact import POS_VALUES, round_fraction_to_f16_bits


def test_decode_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.signbit(oracle.f16_to_f64(0x8000)) and not np.signbit(oracle.f16_to_f64(0))


def _encode_many(xs):
    return np.array([oracle.f64_to_f16(float(x)) for x in xs], dtype=np.uint16)


def test_encode_every_midpoint_and_neighbours():
    """Every midpoint between adjacent finite fp16 values (all the ties), and
    the doubles just either side of it."""
    vals = np.array([float(v) for v in POS_VALUES])
    mids = (vals[:-1] + vals[1:]) / 2.0  # exact in fp64 (one more bit)
    xs = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf), vals])
    xs = np.concatenate([xs, -xs])
    got = _encode_many(xs)
    ref = xs.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_encode_random_doubles_match_numpy():
    rng = np.random.default_rng(7)
    mant = rng.random(20000) + 1.0
    expo = rng.integers(-30, 16, size=20000)
    xs = mant * np.exp2(expo) * np.where(rng.random(20000) < 0.5, -1.0, 1.0)
    got = _encode_many(xs)
    with np.errstate(over="ignore"):  # values past 65504 round to inf, as they should
        ref = xs.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize(
    "x, expect_bits",
    [
        (1.0 + 2.0**-11, 0x3C00),            # tie between 1 and 1+2^-10 -> even (1)
        (1.0 + 3 * 2.0**-11, 0x3C02),        # tie between 1+2^-10 and 1+2^-9 -> even
        (2.0**-25, 0x0000),                  # half the smallest subnormal -> 0
        (3 * 2.0**-25, 0x0002),              # tie between 1 and 2 subnormal units -> 2
        (2.0**-14 - 2.0**-25, 0x0400),       # top subnormal tie rounds up to the smallest normal
        (65504.0, 0x7BFF),
        (65519.999, 0x7BFF),
        (65520.0, 0x7C00),                   # tie to the (even) overflow -> inf
        (-65520.0, 0xFC00),
        (1e300, 0x7C00),
        (-0.0, 0x8000),
        (-(2.0**-26), 0x8000),               # rounds to negative zero
        (float("inf"), 0x7C00),
    ],
)
def test_encode_constructed_cases(x, expect_bits):
    got = oracle.f64_to_f16(x)
    assert got == expect_bits
    if np.isfinite(x) and x != 0.0:  # Fraction has no infinities and no -0
        assert got == round_fraction_to_f16_bits(Fraction(x))


def test_encode_nan_stays_nan():
    bits = oracle.f64_to_f16(float("nan"))
    assert (bits & 0x7C00) == 0x7C00 and (bits & 0x3FF) != 0


def test_encode_matches_exact_rational_rounding():
    """Rationals that are exact doubles but not fp16, rounded by exact comparison."""
    rng = np.random.default_rng(11)
    for _ in range(3000):
        e = int(rng.integers(-26, 17))
        num = int(rng.integers(1, 2**20))
        x = Fraction(num, 2**20) * Fraction(2) ** e
        if rng.random() < 0.5:
            x = -x
        assert oracle.f64_to_f16(float(x)) == round_fraction_to_f16_bits(x)
