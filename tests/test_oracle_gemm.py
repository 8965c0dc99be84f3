"""Pins for the GEMM oracle C = fp16(sum_k A[m,k] * B[n,k]).

Each check compares the oracle with something that does not share its code:
exact rational sums on tiny shapes, closed forms that follow from C = A * B^T
(the tutorial "1. WGMMA", section "The Full Kernel": A viewed [m,k], B viewed
[n,k], B transposed into the product), and an exact integer GEMM on the
{-8..8}/8 inputs of "wgmma_gemm.cu" (day 78), where every partial sum is a
multiple of 1/64 and no summation order can round.
"""
import os

import numpy as np
import pytest

import oracle
from dense_fp16_gemm_f16_amd import inputs
from tests import pins
from tests._exact import exact_gemm_bits


def _rand_f16(rng, shape, lo_exp, hi_exp, zero_frac=0.1):
    """Random finite fp16 values with |x| in [2^lo_exp, 2^hi_exp), some zeros."""
    mant = rng.integers(0, 1024, size=shape)
    e = rng.integers(lo_exp, hi_exp, size=shape)
    x = (1.0 + mant / 1024.0) * np.exp2(e)
    x *= np.where(rng.random(shape) < 0.5, -1.0, 1.0)
    x[rng.random(shape) < zero_frac] = 0.0
    return x.astype(np.float16)


SHAPES = [(1, 1, 1), (2, 3, 5), (7, 9, 4), (8, 8, 16), (3, 5, 17), (9, 2, 31), (4, 4, 33), (15, 16, 8)]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_brute_force_exact_rationals(m, n, k):
    # |x| in [2^-6, 2^6): every partial sum of <= 33 products is a multiple
    # of 2^-32 below 2^18, so the fp64 sum is exact and only the final
    # rounding is tested; ties do occur and must go to even.
    rng = np.random.default_rng(1000 + m * 100 + n * 10 + k)
    a = _rand_f16(rng, (m, k), -6, 6)
    b = _rand_f16(rng, (n, k), -6, 6)
    got = oracle.gemm_f16_nt(a, b).view(np.uint16)
    assert np.array_equal(got, exact_gemm_bits(a.view(np.uint16), b.view(np.uint16)))


@pytest.mark.parametrize("m,n,k", [(3, 4, 9), (5, 2, 16)])
def test_brute_force_subnormal_operands(m, n, k):
    rng = np.random.default_rng(77 + k)
    sub = (rng.integers(-1023, 1024, size=(m, k)) * 2.0**-24).astype(np.float16)  # subnormal or 0
    b = _rand_f16(rng, (n, k), -6, 6)
    got = oracle.gemm_f16_nt(sub, b).view(np.uint16)
    assert np.array_equal(got, exact_gemm_bits(sub.view(np.uint16), b.view(np.uint16)))


def test_constructed_ties_round_to_even():
    # 1 + 2^-11 is a tie between 1 and 1 + 2^-10 -> 1; 1 + 3*2^-11 -> 1 + 2^-9.
    a = np.array([[1.0, 2.0**-11], [1.0, 3 * 2.0**-11]], dtype=np.float16)
    b = np.array([[1.0, 1.0]], dtype=np.float16)
    got = oracle.gemm_f16_nt(a, b).view(np.uint16)
    assert got[0, 0] == 0x3C00 and got[1, 0] == 0x3C02


def test_overflow_to_inf_and_sign():
    a = np.array([[255.875, 255.875], [-255.875, 255.875]], dtype=np.float16)  # 2*255.875^2 = 130,944.03
    b = np.array([[255.875, 255.875]], dtype=np.float16)
    got = oracle.gemm_f16_nt(a, b).view(np.uint16)
    assert got[0, 0] == 0x7C00 and got[1, 0] == 0x0000


def test_identity_closed_forms():
    rng = np.random.default_rng(3)
    n, k = 37, 48
    b = rng.standard_normal((n, k)).astype(np.float16)
    eye = np.eye(k, dtype=np.float16)
    # A = I (M = K): C = B^T exactly, whatever B holds
    assert np.array_equal(oracle.gemm_f16_nt(eye, b).view(np.uint16), b.T.copy().view(np.uint16))
    a = rng.standard_normal((29, k)).astype(np.float16)
    # B = I (N = K): C = A exactly
    assert np.array_equal(oracle.gemm_f16_nt(a, eye).view(np.uint16), a.view(np.uint16))


@pytest.mark.parametrize("k", [1, 256, 1000, 2048, 4096, 8192])
def test_all_ones_gives_k(k):
    a = np.ones((3, k), dtype=np.float16)
    b = np.ones((5, k), dtype=np.float16)
    c = oracle.gemm_f16_nt(a, b)
    assert np.all(c == np.float16(k))


def test_one_hot_rows_select_columns_of_b():
    rng = np.random.default_rng(5)
    m, n, k = 40, 23, 64
    p = rng.integers(0, k, size=m)
    a = np.zeros((m, k), dtype=np.float16)
    a[np.arange(m), p] = 1.0
    b = rng.standard_normal((n, k)).astype(np.float16)
    c = oracle.gemm_f16_nt(a, b)
    assert np.array_equal(c.view(np.uint16), b[:, p].T.copy().view(np.uint16))


def test_a_sum_of_zeros_is_positive_zero():
    # C is a sum that starts at +0: with every product -0 (1 * -0 and
    # 0 * negative numbers) it stays +0, since +0 + (-0) = +0 under
    # round-to-nearest; a sum started at -0 would give -0
    a = np.array([[1.0, 0.0, 0.0], [0.0, 0.0, 0.0]], dtype=np.float16)
    b = np.array([[-0.0, -1.0, -2.0], [0.0, 1.0, 2.0]], dtype=np.float16)
    c = oracle.gemm_f16_nt(a, b).view(np.uint16)
    assert c.tolist() == [[0x0000, 0x0000], [0x0000, 0x0000]]


def test_row_sums_and_rank_one():
    rng = np.random.default_rng(6)
    k = 64
    b = (rng.integers(-8, 9, size=(11, k)) / 8.0).astype(np.float16)
    a = np.ones((4, k), dtype=np.float16)
    c = oracle.gemm_f16_nt(a, b).astype(np.float64)
    assert np.array_equal(c, np.tile(b.astype(np.float64).sum(axis=1), (4, 1)))
    av = (rng.integers(-8, 9, size=7) / 8.0)
    bv = (rng.integers(-8, 9, size=9) / 8.0)
    a1 = np.repeat(av[:, None], k, axis=1).astype(np.float16)
    b1 = np.repeat(bv[:, None], k, axis=1).astype(np.float16)
    c1 = oracle.gemm_f16_nt(a1, b1).astype(np.float64)
    assert np.array_equal(c1, k * np.outer(av, bv))


@pytest.mark.parametrize("name", ["gemm_256_eighths", "gemm_5000x3000x1000_eighths"])
def test_eighths_workloads_exact_integer_gemm(name):
    """{-8..8}/8 inputs: 64 * C is an integer GEMM, exact in fp64 in any order."""
    a, b = inputs.workload_inputs(name)
    got = oracle.gemm_f16_nt(a, b).view(np.uint16)
    assert np.array_equal(got, pins.eighths_exact_bits(a, b))


def test_rows_and_threads_do_not_change_results():
    rng = np.random.default_rng(9)
    a = rng.standard_normal((33, 130)).astype(np.float16)
    b = rng.standard_normal((17, 130)).astype(np.float16)
    full = oracle.gemm_f16_nt(a, b, nthreads=1).view(np.uint16)
    assert np.array_equal(full, oracle.gemm_f16_nt(a, b, nthreads=5).view(np.uint16))
    rows = [32, 0, 7, 7, 19]
    assert np.array_equal(oracle.gemm_f16_nt_rows(a, b, rows, nthreads=3).view(np.uint16), full[rows])


def test_unrounded_variant_rounds_to_the_same_bits():
    rng = np.random.default_rng(10)
    a = rng.standard_normal((20, 300)).astype(np.float16)
    b = rng.standard_normal((21, 300)).astype(np.float16)
    c64 = oracle.gemm_f16_nt_f64(a, b)
    c = oracle.gemm_f16_nt(a, b).view(np.uint16)
    assert np.array_equal(c64.astype(np.float16).view(np.uint16), c)
    # and fp64 agrees with an fp64 library matmul to within its own rounding
    ref = a.astype(np.float64) @ b.astype(np.float64).T
    assert np.max(np.abs(c64 - ref)) < 1e-9


def test_degenerate_sizes():
    a = np.zeros((4, 0), dtype=np.float16)
    b = np.zeros((3, 0), dtype=np.float16)
    c = oracle.gemm_f16_nt(a, b)
    assert c.shape == (4, 3) and np.all(c.view(np.uint16) == 0)
    assert oracle.gemm_f16_nt(np.zeros((0, 5), np.float16), np.ones((3, 5), np.float16)).shape == (0, 3)
    assert oracle.gemm_f16_nt(np.ones((2, 5), np.float16), np.zeros((0, 5), np.float16)).shape == (2, 0)


def test_lcg_matches_sequential_definition():
    """The vectorised generator against the recurrence run one step at a time."""
    state = inputs.LCG_SEED
    seq = []
    for _ in range(5000):
        state = (state * 1664525 + 1013904223) & 0xFFFFFFFF
        seq.append(((state >> 24) % 17 - 8) / 8.0)
    got = inputs.lcg_eighths(5000).astype(np.float64)
    assert np.array_equal(got, np.array(seq))
    # every value in {-8..8}/8 occurs; -1 is the one with 16/256 weight
    vals = inputs.lcg_eighths(200000).astype(np.float64)
    assert set(np.unique(vals * 8).astype(int)) == set(range(-8, 9))


def test_no_double_rounding_via_fp32():
    """1 + 2^-11 + 2^-30 lies just above a tie: one rounding gives 1 + 2^-10;
    rounding to fp32 first would land on the tie and go to 1."""
    a = np.array([[1.0, 2.0**-11, 2.0**-15]], dtype=np.float16)
    b = np.array([[1.0, 1.0, 2.0**-15]], dtype=np.float16)
    assert oracle.gemm_f16_nt(a, b).view(np.uint16)[0, 0] == 0x3C01


def test_threads_that_cannot_start_run_inline():
    """With the address space capped, most of 64 requested threads cannot get
    a stack: their row ranges run on the calling thread instead, the threads
    that did start are joined, and C is the same as with one thread."""
    import subprocess
    import sys
    import textwrap

    code = textwrap.dedent("""
        import resource, sys
        import numpy as np
        import oracle
        rng = np.random.default_rng(5)
        a = (rng.integers(-8, 9, (192, 40)) / 8).astype(np.float16)
        b = (rng.integers(-8, 9, (24, 40)) / 8).astype(np.float16)
        one = oracle.gemm_f16_nt(a, b, nthreads=1)
        one_nn = oracle.gemm_f16_nn_f64(a, np.ascontiguousarray(b.T), nthreads=1)
        vm = [int(l.split()[1]) for l in open('/proc/self/status') if l.startswith('VmSize')][0] * 1024
        cap = vm + 40 * 2**20   # room for a few 8 MiB thread stacks, not 63
        resource.setrlimit(resource.RLIMIT_AS, (cap, cap))
        many = oracle.gemm_f16_nt(a, b, nthreads=64)
        many_nn = oracle.gemm_f16_nn_f64(a, np.ascontiguousarray(b.T), nthreads=64)
        ok = np.array_equal(one.view(np.uint16), many.view(np.uint16))
        ok = ok and all(np.array_equal(x, y) for x, y in zip(one_nn, many_nn))
        print("ok" if ok else "mismatch")
    """)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, PYTHONPATH=root)
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip() == "ok"
