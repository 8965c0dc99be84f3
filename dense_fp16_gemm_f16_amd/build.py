"""Build the GEMM library in-tree with hipcc for gfx950: libgemm_f16.so.

The kernels are compiled per block tile (csrc/tile_*.hip, each instantiating
the templates of csrc/kernels.h) and the host side (csrc/gemm_f16.hip) on its
own, all in parallel, then linked into one shared library.

build_ceiling() builds the MFMA-rate probe libmfma_ceiling.so, a measurement
tool that is not part of the library (tune.py --ceiling builds it on demand).
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgemm_f16.so")
OBJ_DIR = os.path.join(HERE, "_build")
CEILING_SRC = os.path.join(CSRC, "mfma_ceiling.hip")
CEILING_LIB = os.path.join(HERE, "libmfma_ceiling.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 ops are kept out of the generated code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources() -> list[str]:
    """Translation units of libgemm_f16.so: the host side, one per block tile and one
    per block tile of the ring kernel's variants."""
    return ([os.path.join(CSRC, "gemm_f16.hip")] + sorted(glob.glob(os.path.join(CSRC, "tile_*.hip")))
            + sorted(glob.glob(os.path.join(CSRC, "ring_*.hip"))))


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), file=sys.stderr, flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False, extra: list[str] | None = None, jobs: int | None = None) -> str:
    """Compile every translation unit (in parallel) and link libgemm_f16.so."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJ_DIR, os.path.splitext(os.path.basename(s))[0] + ".o") for s in srcs]
    cmds = [[_hipcc(), *HIPCC_FLAGS, *(extra or []), "-I", INCLUDE, "-I", CSRC, "-c", s, "-o", o]
            for s, o in zip(srcs, objs)]
    jobs = jobs or min(len(cmds), 16, os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


def build_ceiling(verbose: bool = False) -> str:
    """The MFMA-rate probe (measurement tool, not part of the library)."""
    tmp = CEILING_LIB + ".tmp"
    _run([_hipcc(), *HIPCC_FLAGS, "-shared", "-I", CSRC, CEILING_SRC, "-o", tmp], verbose)
    os.replace(tmp, CEILING_LIB)
    return CEILING_LIB


if __name__ == "__main__":
    print(build(verbose=True))
