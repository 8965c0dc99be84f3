"""Exact rational helpers the oracle tests check against.

Independent of the oracle's C code: binary16 values come from numpy's own
float16 -> float64 conversion (a library routine), sums are exact
``fractions.Fraction`` arithmetic, and rounding picks the nearer of the two
neighbouring representable values by exact comparison, ties to the even bit
pattern (IEEE 754 roundTiesToEven).
"""
from __future__ import annotations

import bisect
from fractions import Fraction

import numpy as np

_all_bits = np.arange(0, 0x7C00, dtype=np.uint16)  # +0 .. 65504, all finite non-negative
_all_vals = _all_bits.view(np.float16).astype(np.float64)
POS_VALUES = [Fraction(float(v)) for v in _all_vals]  # strictly increasing
POS_BITS = [int(b) for b in _all_bits]
OVERFLOW_AT = Fraction(65520)  # 65504 + half of the 32-wide last spacing


def f16_fraction(bits: int) -> Fraction:
    """Exact value of a finite binary16 bit pattern (via numpy's decoder)."""
    return Fraction(float(np.array([bits], dtype=np.uint16).view(np.float16)[0].astype(np.float64)))


def round_fraction_to_f16_bits(x: Fraction) -> int:
    """Round an exact rational to binary16, nearest, ties to even; returns bits."""
    sign = 0x8000 if x < 0 else 0
    ax = -x if x < 0 else x
    if ax >= OVERFLOW_AT:
        return sign | 0x7C00
    i = bisect.bisect_left(POS_VALUES, ax)
    if i < len(POS_VALUES) and POS_VALUES[i] == ax:
        return sign | POS_BITS[i]
    lo, hi = i - 1, i  # POS_VALUES[lo] < ax < POS_VALUES[hi]
    if hi == len(POS_VALUES):  # between 65504 and the overflow midpoint
        return sign | POS_BITS[-1]
    dlo = ax - POS_VALUES[lo]
    dhi = POS_VALUES[hi] - ax
    if dlo < dhi:
        pick = lo
    elif dhi < dlo:
        pick = hi
    else:
        pick = lo if POS_BITS[lo] % 2 == 0 else hi
    return sign | POS_BITS[pick]


def exact_gemm_bits(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """fp16(A @ B^T) with exact rational sums; tiny shapes only."""
    m, k = a_bits.shape
    n = b_bits.shape[0]
    av = [[f16_fraction(int(a_bits[i, j])) for j in range(k)] for i in range(m)]
    bv = [[f16_fraction(int(b_bits[i, j])) for j in range(k)] for i in range(n)]
    out = np.zeros((m, n), dtype=np.uint16)
    for i in range(m):
        for j in range(n):
            s = sum((av[i][t] * bv[j][t] for t in range(k)), Fraction(0))
            out[i, j] = round_fraction_to_f16_bits(s)
    return out
