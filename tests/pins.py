"""Expected values and tolerances shared by the oracle pins and the parity tests.

Nothing here calls the HIP library.
"""
from __future__ import annotations

import numpy as np


def eighths_exact_bits(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """fp16(A @ B^T) for inputs in {-8..8}/8, computed exactly.

    8A and 8B are integer matrices with entries in [-8, 8], so 64 * C is an
    integer of magnitude <= 64 K; with K < 2^46 every partial sum is exact
    in fp64 whatever order a BLAS uses.  C = (64 C) / 64 is then exact in
    fp64 and numpy rounds it to fp16 (nearest, ties to even) in one step.
    """
    ai = a.astype(np.float64) * 8.0
    bi = b.astype(np.float64) * 8.0
    assert np.array_equal(ai, np.round(ai)) and np.array_equal(bi, np.round(bi))
    assert np.abs(ai).max(initial=0) <= 8 and np.abs(bi).max(initial=0) <= 8
    c64 = (ai @ bi.T) / 64.0
    return c64.astype(np.float16).view(np.uint16)


def f16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of binary16 at |x|: 2^(max(floor(log2|x|), -14) - 10); 2^-24 at 0."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.where(ax > 0, np.maximum(e, -14), -14)
    return np.exp2(e - 10)


def ulp_tolerance(ref: np.ndarray, k: int) -> np.ndarray:
    """|err| allowed for random-normal/uniform inputs: 2 fp16 ulp of |C| plus
    1e-2 * sqrt(K) * 2^-11, the ulp taken at the oracle's fp16 value."""
    return 2.0 * f16_ulp(ref) + 1e-2 * np.sqrt(k) * 2.0**-11


def check_ulp(got: np.ndarray, ref: np.ndarray, k: int) -> tuple[bool, float, tuple]:
    """(ok, worst error/tolerance ratio, index of the worst element)."""
    g = got.astype(np.float64)
    r = ref.astype(np.float64)
    err = np.abs(g - r)
    err = np.where(np.isnan(err), np.inf, err)
    ratio = err / ulp_tolerance(r, k)
    if ratio.size == 0:
        return True, 0.0, ()
    idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    return bool(np.all(ratio <= 1.0)), float(ratio[idx]), idx


def check_rel(got: np.ndarray, ref: np.ndarray, tol: float = 1e-3) -> tuple[bool, float, tuple]:
    """The day-78 gate: |gpu - ref| / max(|ref|, 1) <= tol."""
    g = got.astype(np.float64)
    r = ref.astype(np.float64)
    rel = np.abs(g - r) / np.maximum(np.abs(r), 1.0)
    rel = np.where(np.isnan(rel), np.inf, rel)
    if rel.size == 0:
        return True, 0.0, ()
    idx = np.unravel_index(int(np.argmax(rel)), rel.shape)
    return bool(np.all(rel <= tol)), float(rel[idx]), idx
