"""CPU oracle for C = A * B^T (fp16 in, fp64 sum, one fp16 rounding).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP
library never loads it and it never loads the HIP library.

The arithmetic lives in ``gemm_ref.c`` (plain C, built with gcc); this module
only marshals numpy arrays of binary16 bit patterns (``uint16``) into it.
``raster.py`` holds the oracle for the tile scheduler.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_ref.c")
_LIB_PATH = os.path.join(_HERE, "libgemm_ref.so")
_lib = None


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile ``gemm_ref.c`` with gcc (no fast-math, no FMA contraction: the
    k-sum must stay a plain ordered sequence of fp64 multiplies and adds)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
           "-ffp-contract=off", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class Oracle:
    """ctypes handle on one build of ``gemm_ref.c`` (the default build, or a
    test's deliberately broken copy)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_f64_to_f16.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_f16.restype = ctypes.c_uint16
        lib.oracle_gemm_f16_nt.argtypes = [i64, i64, i64, p, p, p, ctypes.c_int]
        lib.oracle_gemm_f16_nt.restype = ctypes.c_int
        lib.oracle_gemm_f16_nt_rows.argtypes = [i64, i64, i64, p, p, p, i64, p, ctypes.c_int]
        lib.oracle_gemm_f16_nt_rows.restype = ctypes.c_int
        lib.oracle_gemm_f16_nt_f64.argtypes = [i64, i64, i64, p, p, p, ctypes.c_int]
        lib.oracle_gemm_f16_nt_f64.restype = ctypes.c_int
        lib.oracle_gemm_f16_nn_f64.argtypes = [i64, i64, i64, p, p, p, i64, p, p, ctypes.c_int]
        lib.oracle_gemm_f16_nn_f64.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def f16_to_f64(self, bits: int) -> float:
        return self.lib.oracle_f16_to_f64(int(bits) & 0xFFFF)

    def f64_to_f16(self, x: float) -> int:
        return int(self.lib.oracle_f64_to_f16(float(x)))

    def gemm_f16_nt(self, a, b, nthreads=None):
        """C = fp16(A @ B^T) with A [M,K], B [N,K]; returns float16 [M,N]."""
        a, b = _bits(a), _bits(b)
        m, k = a.shape
        n, kb = b.shape
        if kb != k:
            raise ValueError("K mismatch")
        c = np.zeros((m, n), dtype=np.uint16)
        _check(self.lib.oracle_gemm_f16_nt(m, n, k, a.ctypes.data, b.ctypes.data, c.ctypes.data,
                                           nthreads or default_threads()))
        return c.view(np.float16)

    def gemm_f16_nt_rows(self, a, b, rows, nthreads=None):
        """Rows ``rows`` of C = fp16(A @ B^T); returns float16 [len(rows), N]."""
        a, b = _bits(a), _bits(b)
        m, k = a.shape
        n, kb = b.shape
        if kb != k:
            raise ValueError("K mismatch")
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        c = np.zeros((r.size, n), dtype=np.uint16)
        _check(self.lib.oracle_gemm_f16_nt_rows(m, n, k, a.ctypes.data, b.ctypes.data,
                                                r.ctypes.data, r.size, c.ctypes.data,
                                                nthreads or default_threads()))
        return c.view(np.float16)

    def gemm_f16_nt_f64(self, a, b, nthreads=None):
        """The unrounded fp64 sums of A @ B^T; returns float64 [M,N]."""
        a, b = _bits(a), _bits(b)
        m, k = a.shape
        n, kb = b.shape
        if kb != k:
            raise ValueError("K mismatch")
        c = np.zeros((m, n), dtype=np.float64)
        _check(self.lib.oracle_gemm_f16_nt_f64(m, n, k, a.ctypes.data, b.ctypes.data,
                                               c.ctypes.data, nthreads or default_threads()))
        return c


    def gemm_f16_nn_f64(self, a, b, rows=None, nthreads=None):
        """D = A @ B (A [M,K], B [K,N]) in fp64, unrounded, and sum |A[m,k] B[k,n]|.

        Returns (d, dabs), float64 [len(rows) or M, N]."""
        a, b = _bits(a), _bits(b)
        m, k = a.shape
        kb, n = b.shape
        if kb != k:
            raise ValueError("K mismatch")
        if rows is None:
            r_ptr, nrows = None, m
        else:
            r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
            r_ptr, nrows = r.ctypes.data, r.size
        d = np.zeros((nrows, n), dtype=np.float64)
        dabs = np.zeros((nrows, n), dtype=np.float64)
        _check(self.lib.oracle_gemm_f16_nn_f64(m, n, k, a.ctypes.data, b.ctypes.data, r_ptr, nrows,
                                               d.ctypes.data, dabs.ctypes.data,
                                               nthreads or default_threads()))
        return d, dabs


def _load() -> Oracle:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = Oracle(_LIB_PATH)
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def f16_to_f64(bits: int) -> float:
    return _load().f16_to_f64(bits)


def f64_to_f16(x: float) -> int:
    return _load().f64_to_f16(x)


def _bits(x: np.ndarray) -> np.ndarray:
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    if x.dtype != np.uint16:
        raise TypeError("expected binary16 data (float16 or uint16 bit patterns)")
    return np.ascontiguousarray(x)


def _check(rc: int) -> None:
    if rc != 0:
        raise RuntimeError(f"oracle returned {rc}")


def gemm_f16_nt(a: np.ndarray, b: np.ndarray, nthreads: int | None = None) -> np.ndarray:
    """C = fp16(A @ B^T) with A [M,K], B [N,K]; returns float16 [M,N]."""
    return _load().gemm_f16_nt(a, b, nthreads)


def gemm_f16_nt_rows(a: np.ndarray, b: np.ndarray, rows, nthreads: int | None = None) -> np.ndarray:
    """Rows ``rows`` of C = fp16(A @ B^T); returns float16 [len(rows), N]."""
    return _load().gemm_f16_nt_rows(a, b, rows, nthreads)


def gemm_f16_nt_f64(a: np.ndarray, b: np.ndarray, nthreads: int | None = None) -> np.ndarray:
    """The unrounded fp64 sums of A @ B^T; returns float64 [M,N]."""
    return _load().gemm_f16_nt_f64(a, b, nthreads)


def gemm_f16_nn_f64(a: np.ndarray, b: np.ndarray, rows=None, nthreads: int | None = None):
    """The day-78 listing's reference: D = A @ B with B [K,N], fp64, unrounded,
    plus sum |A B|; returns (d, dabs)."""
    return _load().gemm_f16_nn_f64(a, b, rows, nthreads)
