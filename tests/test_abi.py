"""The C-ABI library loads, exports what include/gemm_f16.h declares, and its
host logic (argument checks, status strings, tile scheduler, tile choice)
behaves as documented.  No GPU is needed: every call here returns before the
library makes its first HIP call.
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import dense_fp16_gemm_f16_amd as g
from oracle import raster

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_f16.h")


def _declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_f16_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    declared = _declared_functions()
    assert declared == sorted(g.EXPORTS)
    L = g.lib()
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings():
    for code in (g.OK, g.EINVAL, g.ENULL, g.EALIGN, g.EDEVICE, g.EHIP, g.EOVERLAP):
        s = g.status_string(code)
        assert s and s != "unknown status"
    assert g.status_string(-99) == "unknown status"


FAKE_A, FAKE_B, FAKE_C = 0x10000000, 0x20000000, 0x30000000  # never dereferenced


@pytest.mark.parametrize(
    "args, expect",
    [
        ((-1, 4, 4, FAKE_A, FAKE_B, FAKE_C), g.EINVAL),
        ((4, -1, 4, FAKE_A, FAKE_B, FAKE_C), g.EINVAL),
        ((4, 4, -1, FAKE_A, FAKE_B, FAKE_C), g.EINVAL),
        ((4, 4, 1 << 22, FAKE_A, FAKE_B, FAKE_C), g.EINVAL),
        ((1 << 31, 4, 4, FAKE_A, FAKE_B, FAKE_C), g.EINVAL),
        ((1 << 30, 4, 4, FAKE_A, FAKE_B, FAKE_C), g.EINVAL),
        ((4, 1 << 30, 4, FAKE_A, FAKE_B, FAKE_C), g.EINVAL),
        ((1 << 24, 1 << 23, 4, FAKE_A, FAKE_B, FAKE_C), g.EINVAL),
        ((4, 4, 4, 0, FAKE_B, FAKE_C), g.ENULL),
        ((4, 4, 4, FAKE_A, 0, FAKE_C), g.ENULL),
        ((4, 4, 4, FAKE_A, FAKE_B, 0), g.ENULL),
        ((4, 4, 4, FAKE_A + 1, FAKE_B, FAKE_C), g.EALIGN),
        ((4, 4, 4, FAKE_A, FAKE_B, FAKE_C + 1), g.EALIGN),
        ((4, 4, 4, FAKE_A, FAKE_B, FAKE_A + 8), g.EOVERLAP),
        ((4, 4, 4, FAKE_A, FAKE_B, FAKE_B - 8), g.EOVERLAP),
        ((0, 4, 4, FAKE_A, FAKE_B, FAKE_C), g.OK),   # empty: nothing launched
        ((4, 0, 4, FAKE_A, FAKE_B, FAKE_C), g.OK),
        ((0, 0, 0, 0, 0, 0), g.OK),
    ],
)
def test_argument_checks_return_before_any_hip_call(args, expect):
    assert g.lib().gemm_f16_nt(*args, None) == expect


@pytest.mark.parametrize("opt", [(10, 0, -1), (-1, 0, -1), (0, -1, -1), (0, 0, 2), (0, 0, -2)])
def test_bad_options_rejected(opt):
    assert g.gemm_f16_nt_raw(8, 8, 8, FAKE_A, FAKE_B, FAKE_C, 0, *opt) == g.EINVAL


@pytest.mark.parametrize("nm,nn", [(1, 1), (3, 5), (8, 8), (32, 32), (64, 16), (20, 12), (17, 31)])
@pytest.mark.parametrize("sw", [1, 3, 4, 8])
@pytest.mark.parametrize("xcd", [0, 1])
def test_tile_coord_matches_the_oracle(nm, nn, sw, xcd):
    grid = nm * nn
    seen = set()
    for pid in range(grid):
        logical = raster.xcd_remap(pid, grid, 8) if xcd else pid
        expect = raster.swizzle_tile_coord(logical, nm, nn, sw)
        got = g.tile_coord(pid, nm, nn, sw, xcd)
        assert got == expect
        seen.add(got)
    assert len(seen) == grid


@pytest.mark.parametrize("nm,nn", [(46341, 46341), (65536, 65536), (3, 2**30 + 7), (2**31 - 1, 1), (2**31, 1)])
@pytest.mark.parametrize("xcd", [0, 1])
def test_tile_coord_at_the_32_bit_boundary(nm, nn, xcd):
    """Grids below 2^31 tiles run the kernels' 32-bit arithmetic, larger ones
    (which the GEMM entry points refuse) the 64-bit one; both match the
    oracle at the ends of the grid and in between."""
    grid = nm * nn
    for sw in (1, 4, 7):
        for pid in sorted({0, 1, 7, 8, grid // 3, grid // 2 + 5, grid - 9, grid - 8, grid - 1}):
            if not 0 <= pid < grid:
                continue
            logical = raster.xcd_remap(pid, grid, 8) if xcd else pid
            assert g.tile_coord(pid, nm, nn, sw, xcd) == raster.swizzle_tile_coord(logical, nm, nn, sw)


def test_tile_coord_rejects_bad_input():
    for args in [(-1, 4, 4, 1, 0), (16, 4, 4, 1, 0), (0, 4, 4, 0, 0), (0, 0, 4, 1, 0),
                 (0, 1 << 40, 1 << 40, 1, 0), (0, 1 << 62, 4, 1, 0), (0, 3, 1 << 62, 1, 0)]:
        with pytest.raises(g.GemmError):
            g.tile_coord(*args)


def test_select_tile():
    assert g.select_tile(8192, 8192, 8192) == g.TILE_256x256
    assert g.select_tile(4096, 4096, 4096) == g.TILE_256x256   # 256 tiles: one per CU
    assert g.select_tile(256, 256, 256) == g.TILE_64x64
    assert g.select_tile(5000, 3000, 1000) in g.TILES
    # short K: the per-tile cost dominates and a 128-row or -column tile wins
    # over 256x256 (4096^2 x 256 measured 16.0 us on 128x256, 16.4 on 256x256)
    assert g.select_tile(4096, 4096, 256) in (g.TILE_128x256, g.TILE_256x128, g.TILE_128x128)
    # a rectangular tile lies with its long side along the shorter dimension
    assert g.select_tile(8192, 1024, 1024) == g.TILE_128x256
    assert g.select_tile(1024, 8192, 1024) == g.TILE_256x128
    assert g.select_tile(16384, 4096, 256) == g.TILE_128x256
    # K % 8 != 0 would run the 256x256 tile as 128x256: never chosen
    assert g.select_tile(4096, 4096, 4095) != g.TILE_256x256
    with pytest.raises(g.GemmError):
        g.select_tile(-1, 4, 4)


def _busiest_xcd_panels(nm, nn, sw, remap):
    grid = nm * nn
    most = 0
    for x in range(8):
        rows, cols = set(), set()
        for pid in range(x, grid, 8):
            logical = raster.xcd_remap(pid, grid, 8) if remap else pid
            mb, nb = raster.swizzle_tile_coord(logical, nm, nn, sw)
            rows.add(mb)
            cols.add(nb)
        most = max(most, len(rows) + len(cols))
    return most


def test_select_xcd_keeps_dispatch_order_only_where_it_costs_no_panels():
    # a grid that fills the 256 CUs once: the dispatch order when it gives no
    # XCD more operand panels than the remap
    for nm in (1, 2, 4, 8, 16, 32, 64, 128, 256):
        nn = 256 // nm
        for sw in (1, 2, 4, 8):
            want = 0 if _busiest_xcd_panels(nm, nn, sw, False) <= _busiest_xcd_panels(nm, nn, sw, True) else 1
            assert g.select_xcd(nm, nn, sw, 256) == want, (nm, nn, sw)
    assert g.select_xcd(16, 16, 4, 256) == 0   # 12 panels either way (4096^2 on 256x256)
    assert g.select_xcd(8, 32, 4, 256) == 0
    assert g.select_xcd(32, 8, 4, 256) == 1    # 18 panels without the remap, 12 with it
    assert g.select_xcd(4, 64, 4, 256) == 1
    # anything but exactly one full round keeps the remap
    for nm, nn, cus in [(20, 12, 256), (12, 12, 256), (32, 32, 256), (16, 16, 304), (16, 16, 0), (2, 2, 4096)]:
        assert g.select_xcd(nm, nn, 4, cus) == 1, (nm, nn, cus)
    # the answer is per shape, not left over from the previous call
    assert [g.select_xcd(*a) for a in [(16, 16, 4, 256), (32, 8, 4, 256), (16, 16, 4, 256)]] == [0, 1, 0]
    for args in [(0, 4, 4, 256), (4, 0, 4, 256), (4, 4, 0, 256), (4, 4, 4, -1), (1 << 16, 1 << 15, 4, 256),
                 (1 << 40, 1 << 40, 4, 256)]:
        with pytest.raises(g.GemmError):
            g.select_xcd(*args)


def test_python_wrapper_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    a = torch.zeros(4, 8, dtype=torch.float16)
    with pytest.raises(ValueError):
        g.gemm_f16_nt(a, a)
    with pytest.raises(TypeError):
        g.gemm_f16_nt(a.float(), a.float())


@pytest.mark.parametrize(
    "args, expect",
    [
        ((4, 4, 4, FAKE_A, FAKE_B, FAKE_C + 2), g.EALIGN),          # fp32 output needs 4-byte alignment
        ((4, 1 << 25, 4, FAKE_A, FAKE_B, FAKE_C), g.EINVAL),
        ((4, 4, 4, FAKE_A, FAKE_B, FAKE_A + 16), g.EOVERLAP),
        ((0, 4, 4, FAKE_A, FAKE_B, FAKE_C), g.OK),
        ((4, 4, 4, 0, FAKE_B, FAKE_C), g.ENULL),
    ],
)
def test_nn_argument_checks(args, expect):
    assert g.lib().gemm_f16_nn_f32(*args, None) == expect


def test_nn_rejects_the_16x16_tile():
    assert g.gemm_f16_nn_f32_raw(8, 8, 8, FAKE_A, FAKE_B, FAKE_C, 0, g.TILE_128x128_M16) == g.EINVAL


# The device gate: GEMM_F16_TEST_ARCH, read when the library loads, stands in
# for the device's architecture name, so the refusal runs on any host.  Only
# names that must be refused are tried: an accepted one would go on to launch.
@pytest.mark.parametrize("arch", ["gfx942", "gfx90a", "gfx9500", "gfx95", "gfx951", "", "gfx1100"])
def test_device_gate_refuses_other_architectures(arch):
    code = (
        "import dense_fp16_gemm_f16_amd as g\n"
        f"A, B, C = {FAKE_A}, {FAKE_B}, {FAKE_C}\n"
        "print(g.lib().gemm_f16_nt(4, 4, 4, A, B, C, None), g.lib().gemm_f16_nn_f32(4, 4, 4, A, B, C, None),"
        " g.lib().gemm_f16_nt(4, 4, 0, A, B, C, None), g.status_string(g.EDEVICE))\n"
    )
    env = dict(os.environ, GEMM_F16_TEST_ARCH=arch, PYTHONPATH=ROOT)
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, check=True)
    nt, nn, k0, msg = out.stdout.split(maxsplit=3)
    assert (int(nt), int(nn), int(k0)) == (g.EDEVICE, g.EDEVICE, g.EDEVICE)
    assert "gfx950" in msg


def test_argument_errors_come_before_the_device_gate():
    code = (
        "import dense_fp16_gemm_f16_amd as g\n"
        f"print(g.lib().gemm_f16_nt(-1, 4, 4, {FAKE_A}, {FAKE_B}, {FAKE_C}, None),"
        f" g.lib().gemm_f16_nt(0, 4, 4, {FAKE_A}, {FAKE_B}, {FAKE_C}, None))\n"
    )
    env = dict(os.environ, GEMM_F16_TEST_ARCH="gfx942", PYTHONPATH=ROOT)
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, check=True)
    assert [int(x) for x in out.stdout.split()] == [g.EINVAL, g.OK]


@pytest.mark.parametrize("tile,variant,k,a_off", [
    (0, 1, 64, 0),                    # variants need an explicit block tile
    (3, 1, 64, 0),                    # ... of 256x256, 256x128, 128x256 or 128x128
    (g.TILE_256x256, 2, 64, 0),       # 3 stages of block_k 64 do not fit 256x256's LDS
    (g.TILE_256x256, 6, 64, 0),       # loader waves: the MFMA waves' 128x128 would not fit
    (g.TILE_256x128, 7, 64, 0),       # 3 stages with loader waves: 128x128 only
    (g.TILE_128x128, 1, 96, 0),       # K a multiple of block_k 64
    (g.TILE_128x128, 3, 48, 0),       # ... of block_k 32
    (g.TILE_128x128, 1, 0, 0),        # K > 0
    (g.TILE_128x128, 1, 64, 8),       # 16-byte aligned operands
    (g.TILE_128x128, 8, 64, 0),       # no variant 8
    (g.TILE_128x128, -1, 64, 0),
])
def test_bad_variants_rejected(tile, variant, k, a_off):
    assert g.gemm_f16_nt_raw(8, 8, k, FAKE_A + a_off, FAKE_B, FAKE_C, 0, tile, 0, -1, variant) == g.EINVAL


def test_variants_are_for_the_first_contract():
    opt = g.Options(g.TILE_128x128, 0, -1, 1)
    assert g.lib().gemm_f16_nn_f32_ex(8, 8, 64, FAKE_A, FAKE_B, FAKE_C, None, ctypes.byref(opt)) == g.EINVAL
