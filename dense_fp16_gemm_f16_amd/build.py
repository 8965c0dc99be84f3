"""Build the HIP libraries in-tree with hipcc for gfx950: libgemm_f16.so (the
GEMM) and libmfma_ceiling.so (the MFMA-rate probe the roofline is read
against)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "gemm_f16.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgemm_f16.so")
CEILING_SRC = os.path.join(HERE, "csrc", "mfma_ceiling.hip")
CEILING_LIB = os.path.join(HERE, "libmfma_ceiling.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed fp32 ops are kept out of the generated code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc(src: str, out: str, verbose: bool, extra: list[str] | None) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *(extra or []), "-I", INCLUDE, src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    _hipcc(CEILING_SRC, CEILING_LIB, verbose, extra)
    return _hipcc(SRC, LIB, verbose, extra)


if __name__ == "__main__":
    print(build(verbose=True))
