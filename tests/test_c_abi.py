"""The library called from C programs, with no Python in their process
(tests/c_abi/): the header compiles as C, the host entry points behave as
documented, and on the GPU both contracts match the C oracle bit for bit
on exact inputs."""
import os
import subprocess

import pytest

from tests.c_abi import build as c_build


def test_header_and_host_entry_points_from_c(tmp_path):
    exe = str(tmp_path / "abi_host")
    subprocess.run(c_build.host_command(exe), check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"


@pytest.mark.gpu
def test_both_contracts_from_c_match_the_oracle():
    if not os.path.exists(c_build.GPU_PROGRAM):
        pytest.fail(f"{c_build.GPU_PROGRAM} is not built (python tests/c_abi/build.py, or __graft_entry__.build())")
    print("case: tests/c_abi/gemm_from_c", flush=True)
    r = subprocess.run([c_build.GPU_PROGRAM], capture_output=True, text=True, timeout=240)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().endswith("ok")
