"""The device code of the built library: every gfx950 kernel fits its
registers (no VGPR spills, no scratch) and carries no packed-fp32 VALU
instructions.  Reads the code objects of libgemm_f16.so (built here); no GPU.
"""
import os
import re
import subprocess
import tempfile

import pytest

import dense_fp16_gemm_f16_amd as g
from tests import _codeobj

OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"


@pytest.fixture(scope="module")
def records():
    if not os.path.exists(g.LIB_PATH):
        pytest.fail(f"{g.LIB_PATH} is not built")
    recs = _codeobj.kernel_records(g.LIB_PATH)
    assert recs, "no gfx950 kernels found in the library"
    return recs


def test_every_gemm_kernel_is_present(records):
    names = " ".join(r[".name"] for r in records)
    for kind in ("gemm_f16_kernel", "gemm_f16_direct_kernel", "gemm_f16_direct_ahead_kernel",
                 "gemm_f16_persistent_kernel", "fill_zero_kernel"):
        assert kind in names, kind
    assert len({r[".name"] for r in records}) == len(records), "a kernel is compiled into two code objects"


def test_no_kernel_spills_or_uses_scratch(records):
    bad = [(r[".name"], r[".vgpr_spill_count"], r[".private_segment_fixed_size"]) for r in records
           if r[".vgpr_spill_count"] or r[".private_segment_fixed_size"] or r.get(".uses_dynamic_stack")]
    assert not bad, bad


def test_lds_fits_the_cu(records):
    for r in records:
        assert r[".group_segment_fixed_size"] <= 160 * 1024, r[".name"]


@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="llvm-objdump not installed")
def test_no_packed_fp32_instructions():
    with open(g.LIB_PATH, "rb") as f:
        blob = f.read()
    found, mfma = [], 0
    with tempfile.TemporaryDirectory() as d:
        for i, (triple, obj) in enumerate(_codeobj._bundles(blob)):
            if "gfx950" not in triple:
                continue
            path = os.path.join(d, f"co{i}.o")
            with open(path, "wb") as f:
                f.write(obj)
            asm = subprocess.run([OBJDUMP, "-d", path], capture_output=True, text=True, check=True).stdout
            mfma += asm.count("v_mfma")
            found += re.findall(r"\bv_pk_(?:fma|mul|add)_f32\b", asm)
    assert mfma > 0
    assert not found, sorted(set(found))
