"""Build the GEMM library in-tree with hipcc for gfx950: libgemm_f16.so.

The kernels are compiled per block tile (csrc/tile_*.hip, each instantiating
the templates of csrc/kernels.h) and the host side (csrc/gemm_f16.hip) on its
own, all in parallel, then linked into one shared library.

build_ceiling() builds the MFMA-rate probe libmfma_ceiling.so, and
build_trace() the timestamp-traced copy of the library, libgemm_f16_trace.so
(the same sources with -DGEMM_F16_TRACE), and build_poison() the debug copy
whose kernels fill their LDS with NaN before the first load,
libgemm_f16_poison.so (-DGEMM_F16_POISON_LDS): measurement and debug tools
that are not part of the library (tune.py --ceiling, trace.py and the tests
use them).
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
TRACE_LIB = os.path.join(HERE, "libgemm_f16_trace.so")
TRACE_OBJ_DIR = os.path.join(HERE, "_build_trace")
TRACE_KT_LIB = os.path.join(HERE, "libgemm_f16_trace_kt.so")
TRACE_KT_OBJ_DIR = os.path.join(HERE, "_build_trace_kt")
POISON_LIB = os.path.join(HERE, "libgemm_f16_poison.so")
POISON_OBJ_DIR = os.path.join(HERE, "_build_poison")
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


def _build_lib(lib: str, obj_dir: str, flags: list[str], verbose: bool, jobs: int | None) -> str:
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(obj_dir, os.path.splitext(os.path.basename(s))[0] + ".o") for s in srcs]
    cmds = [[_hipcc(), *HIPCC_FLAGS, *flags, "-I", INCLUDE, "-I", CSRC, "-c", s, "-o", o]
            for s, o in zip(srcs, objs)]
    jobs = jobs or min(len(cmds), 16, os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = lib + ".tmp"
    _run([_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, extra: list[str] | None = None, jobs: int | None = None) -> str:
    """Compile every translation unit (in parallel) and link libgemm_f16.so."""
    return _build_lib(LIB, OBJ_DIR, list(extra or []), verbose, jobs)


def build_trace(verbose: bool = False, jobs: int | None = None, ktiles: bool = False) -> str:
    """The timestamp-traced copy of the library (measurement tool); ktiles:
    the copy that also stamps the K-tiles around the first tile change."""
    if ktiles:
        return _build_lib(TRACE_KT_LIB, TRACE_KT_OBJ_DIR, ["-DGEMM_F16_TRACE", "-DGEMM_F16_TRACE_KTILES"], verbose, jobs)
    return _build_lib(TRACE_LIB, TRACE_OBJ_DIR, ["-DGEMM_F16_TRACE"], verbose, jobs)


def build_ceiling(verbose: bool = False) -> str:
    """The MFMA-rate probe (measurement tool, not part of the library)."""
    tmp = CEILING_LIB + ".tmp"
    _run([_hipcc(), *HIPCC_FLAGS, "-shared", "-I", CSRC, CEILING_SRC, "-o", tmp], verbose)
    os.replace(tmp, CEILING_LIB)
    return CEILING_LIB


def build_poison(verbose: bool = False, jobs: int | None = None) -> str:
    """The debug copy of the library whose kernels poison their LDS with NaN."""
    return _build_lib(POISON_LIB, POISON_OBJ_DIR, ["-DGEMM_F16_POISON_LDS"], verbose, jobs)


if __name__ == "__main__":
    if "--trace" in sys.argv[1:]:
        print(build_trace(verbose=True, ktiles="--ktiles" in sys.argv[1:]))
    elif "--poison" in sys.argv[1:]:
        print(build_poison(verbose=True))
    else:
        print(build(verbose=True))
