"""Builds the C programs that call the library's C ABI with no Python in
the process.  ``gemm_from_c`` (needs a GPU) is built here, ahead of the GPU
tests that run it; the host-only check is built by its CPU test.

Both link the library (and the GPU program also the C oracle and the HIP
runtime) through run paths relative to the binary, so the tree can move.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(ROOT, "dense_fp16_gemm_f16_amd")
ORACLE_DIR = os.path.join(ROOT, "oracle")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
GPU_PROGRAM = os.path.join(HERE, "gemm_from_c")

WARN = ["-std=c11", "-O2", "-Wall", "-Wextra", "-Werror"]


def _rpath(*dirs: str) -> list[str]:
    rel = [os.path.join("$ORIGIN", os.path.relpath(d, HERE)) for d in dirs]
    return ["-Wl,-rpath," + ":".join(rel + [os.path.join(ROCM, "lib")])]


def host_command(out: str) -> list[str]:
    """gcc line for abi_host.c (host entry points only)."""
    return (["gcc", "-std=c99", "-pedantic", "-O2", "-Wall", "-Wextra", "-Werror", "-I", INCLUDE,
             os.path.join(HERE, "abi_host.c"), "-L", LIB_DIR, "-lgemm_f16",
             "-Wl,-rpath," + LIB_DIR, "-Wl,-rpath-link," + os.path.join(ROCM, "lib"), "-o", out])


def build(verbose: bool = False) -> str:
    """Compiles gemm_from_c.c (the library and the oracle must be built)."""
    tmp = GPU_PROGRAM + ".tmp"
    cmd = (["gcc"] + WARN + ["-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-I", os.path.join(ROCM, "include"),
                             os.path.join(HERE, "gemm_from_c.c"), "-L", LIB_DIR, "-lgemm_f16",
                             "-L", ORACLE_DIR, "-lgemm_ref", "-L", os.path.join(ROCM, "lib"), "-lamdhip64"]
           + _rpath(LIB_DIR, ORACLE_DIR) + ["-o", tmp])
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, GPU_PROGRAM)
    return GPU_PROGRAM


if __name__ == "__main__":
    print(build(verbose=True))
