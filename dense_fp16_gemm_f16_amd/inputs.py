"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws numbers; it holds none of the GEMM's arithmetic.  Both
the HIP path and the CPU oracle are fed the same binary16 arrays made here.

Workloads (shapes and value distributions):

* ``gemm_256_eighths``      M=N=K=256, entries from {-8..8}/8 via the day-78
  listing's LCG ("wgmma_gemm.cu", the input loop in ``main``): state <- state *
  1664525 + 1013904223 (mod 2^32), seed 20260901, value ((state >> 24) % 17 -
  8) / 8.  A's M*K values come first (row-major), then B's N*K values in
  row-major [N,K] order.  Every value is exact in fp16.
* ``gemm_4096_normal``      M=N=K=4096, i.i.d. N(0,1) rounded to fp16.
* ``gemm_8192_uniform``     M=N=K=8192, i.i.d. uniform[-1,1] rounded to fp16.
* ``gemm_16384x4096x2048_normal05``  i.i.d. N(0, 0.5) read as standard
  deviation 0.5, rounded to fp16.
* ``gemm_5000x3000x1000_eighths``    ragged, {-8..8}/8 through the same LCG.
* ``gemm_1024x8192x8192_uniform``    one GPU's share of the 8192^3 GEMM when
  eight GPUs split M (each takes 1024 rows of A and C and all of B),
  uniform[-1,1] with its own seed.

The float distributions use numpy's PCG64 generator in float32 and round to
fp16 with numpy's round-to-nearest-even conversion.

Workloads of the second contract, D = A * B with B [K,N] row-major and an
fp32 D (the day-78 listing's own), carry ``b_layout == "kn"``: their B is
drawn as a [K,N] row-major array (for the LCG: A's M*K values, then B's K*N
values in [K,N] order, exactly as that listing fills its inputs).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

LCG_SEED = 20260901
_LCG_A = 1664525
_LCG_C = 1013904223


@dataclass(frozen=True)
class Workload:
    name: str
    m: int
    n: int
    k: int
    dist: str  # "eighths" | "normal" | "uniform" | "normal05"
    seed: int
    b_layout: str = "nk"  # "nk": B is [N,K] (C = A B^T); "kn": B is [K,N] (D = A B)

    @property
    def flops(self) -> int:
        return 2 * self.m * self.n * self.k


WORKLOADS = {
    w.name: w
    for w in (
        Workload("gemm_256_eighths", 256, 256, 256, "eighths", LCG_SEED),
        Workload("gemm_4096_normal", 4096, 4096, 4096, "normal", 4096),
        Workload("gemm_8192_uniform", 8192, 8192, 8192, "uniform", 8192),
        Workload("gemm_16384x4096x2048_normal05", 16384, 4096, 2048, "normal05", 2048),
        Workload("gemm_5000x3000x1000_eighths", 5000, 3000, 1000, "eighths", LCG_SEED),
        Workload("gemm_1024x8192x8192_uniform", 1024, 8192, 8192, "uniform", 1024),
        Workload("gemm_nn_256_eighths", 256, 256, 256, "eighths", LCG_SEED, "kn"),
        Workload("gemm_nn_5000x3000x1000_eighths", 5000, 3000, 1000, "eighths", LCG_SEED, "kn"),
        Workload("gemm_nn_8192_uniform", 8192, 8192, 8192, "uniform", 8192, "kn"),
    )
}


def lcg_states(count: int, seed: int = LCG_SEED) -> np.ndarray:
    """The LCG's states s_1..s_count (s_i = a*s_{i-1} + c mod 2^32), vectorised.

    s_i = a^i * s_0 + c * (1 + a + ... + a^(i-1)); uint64 arithmetic wraps
    mod 2^64, which keeps every residue mod 2^32 intact.
    """
    if count <= 0:
        return np.zeros(0, dtype=np.uint32)
    with np.errstate(over="ignore"):
        powers = np.cumprod(np.full(count, _LCG_A, dtype=np.uint64))  # a^1 .. a^count
        geo = np.empty(count, dtype=np.uint64)  # 1 + a + ... + a^(i-1)
        geo[0] = 1
        if count > 1:
            geo[1:] = 1 + np.cumsum(powers[:-1])
        states = powers * np.uint64(seed) + np.uint64(_LCG_C) * geo
    return (states & np.uint64(0xFFFFFFFF)).astype(np.uint32)


def lcg_eighths(count: int, seed: int = LCG_SEED) -> np.ndarray:
    """``count`` values ((state >> 24) % 17 - 8) / 8 as float16."""
    top = (lcg_states(count, seed) >> np.uint32(24)).astype(np.int64)
    return ((top % 17 - 8).astype(np.float32) / np.float32(8.0)).astype(np.float16)


def make_inputs(m: int, n: int, k: int, dist: str, seed: int,
                b_layout: str = "nk") -> tuple[np.ndarray, np.ndarray]:
    """A [m,k] and B ([n,k], or [k,n] for b_layout "kn") as C-contiguous float16 arrays."""
    b_shape = (n, k) if b_layout == "nk" else (k, n)
    if dist == "eighths":
        v = lcg_eighths(m * k + n * k, seed)
        return v[: m * k].reshape(m, k).copy(), v[m * k:].reshape(b_shape).copy()
    rng = np.random.default_rng(seed)
    if dist == "normal":
        a = rng.standard_normal((m, k), dtype=np.float32)
        b = rng.standard_normal(b_shape, dtype=np.float32)
    elif dist == "normal05":
        a = rng.standard_normal((m, k), dtype=np.float32) * np.float32(0.5)
        b = rng.standard_normal(b_shape, dtype=np.float32) * np.float32(0.5)
    elif dist == "uniform":
        a = rng.random((m, k), dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
        b = rng.random(b_shape, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return a.astype(np.float16), b.astype(np.float16)


def workload_inputs(name: str) -> tuple[np.ndarray, np.ndarray]:
    w = WORKLOADS[name]
    return make_inputs(w.m, w.n, w.k, w.dist, w.seed, w.b_layout)
