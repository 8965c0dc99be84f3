"""Pins for the second oracle function: the day-78 listing's reference
(\"wgmma_gemm.cu\", gemmCpu): D = A * B with A [M,K], B [K,N] row-major,
summed in fp64 over increasing k and left unrounded, plus sum |A B|.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from dense_fp16_gemm_f16_amd import inputs
from tests._exact import f16_fraction
from tests.test_oracle_gemm import _rand_f16


@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (3, 4, 5), (7, 2, 16), (5, 9, 33)])
def test_brute_force_exact_rationals(m, n, k):
    # |x| in [2^-6, 2^6): all partial sums are exact in fp64 (see the NT pins)
    rng = np.random.default_rng(500 + m * 100 + n * 10 + k)
    a = _rand_f16(rng, (m, k), -6, 6)
    b = _rand_f16(rng, (k, n), -6, 6)
    d, dabs = oracle.gemm_f16_nn_f64(a, b)
    for i in range(m):
        for j in range(n):
            prods = [f16_fraction(int(a.view(np.uint16)[i, t])) * f16_fraction(int(b.view(np.uint16)[t, j]))
                     for t in range(k)]
            assert Fraction(d[i, j]) == sum(prods, Fraction(0))
            assert Fraction(dabs[i, j]) == sum((abs(x) for x in prods), Fraction(0))


def test_equals_the_nt_oracle_on_transposed_b():
    rng = np.random.default_rng(8)
    a = rng.standard_normal((31, 200)).astype(np.float16)
    b = rng.standard_normal((200, 45)).astype(np.float16)
    d, _ = oracle.gemm_f16_nn_f64(a, b)
    assert np.array_equal(d, oracle.gemm_f16_nt_f64(a, b.T.copy()))


def test_day78_workload_exact_integer_gemm():
    """256^3 from the listing's LCG, B filled as [K,N]: 64 D is an exact integer GEMM."""
    a, b = inputs.workload_inputs("gemm_nn_256_eighths")
    assert b.shape == (256, 256)
    d, dabs = oracle.gemm_f16_nn_f64(a, b)
    exact = ((a.astype(np.float64) * 8) @ (b.astype(np.float64) * 8)) / 64.0
    assert np.array_equal(d, exact)
    assert np.array_equal(dabs, (np.abs(a.astype(np.float64) * 8) @ np.abs(b.astype(np.float64) * 8)) / 64.0)


def test_identity_and_rows():
    rng = np.random.default_rng(9)
    b = rng.standard_normal((40, 23)).astype(np.float16)
    d, _ = oracle.gemm_f16_nn_f64(np.eye(40, dtype=np.float16), b)
    assert np.array_equal(d, b.astype(np.float64))
    a = rng.standard_normal((17, 40)).astype(np.float16)
    d, _ = oracle.gemm_f16_nn_f64(a, np.eye(40, dtype=np.float16))
    assert np.array_equal(d, a.astype(np.float64))
    full, fabs_ = oracle.gemm_f16_nn_f64(a, b)
    part, pabs = oracle.gemm_f16_nn_f64(a, b, rows=[16, 0, 3])
    assert np.array_equal(part, full[[16, 0, 3]]) and np.array_equal(pabs, fabs_[[16, 0, 3]])


def test_degenerate():
    d, dabs = oracle.gemm_f16_nn_f64(np.zeros((3, 0), np.float16), np.zeros((0, 4), np.float16))
    assert d.shape == (3, 4) and np.all(d == 0) and np.all(dabs == 0)
