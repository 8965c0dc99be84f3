"""Pins for the tile-scheduler oracle (oracle/raster.py).

The worked example of "4. Pipeline Abstraction and Two Consumer Warp Groups"
(section "Tile Rasterization") is stored in tests/golden/ with its citation.
"""
import json
import os

import pytest

from oracle import raster

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "raster_worked_example.json")


def test_worked_example_strip_counts():
    with open(GOLDEN) as f:
        g = json.load(f)
    nm, nn, active, sw = g["num_m_blocks"], g["num_n_blocks"], g["active_blocks"], g["swizzle_size"]
    plain = [raster.plain_2d_coord(p, nm, nn) for p in range(active)]
    swz = [raster.swizzle_tile_coord(p, nm, nn, sw) for p in range(active)]
    pa, pb = raster.strips_touched(plain)
    sa, sb = raster.strips_touched(swz)
    assert (pa, pb, pa + pb) == (g["plain_2d"]["a_strips"], g["plain_2d"]["b_strips"], g["plain_2d"]["total"])
    assert (sa, sb, sa + sb) == (g["swizzled"]["a_strips"], g["swizzled"]["b_strips"], g["swizzled"]["total"])
    assert round(100 * (1 - (sa + sb) / (pa + pb))) == g["reduction_percent"]
    assert sorted(swz) == sorted((m, n) for m in range(4) for n in range(4))  # the 4 x 4 square


@pytest.mark.parametrize("nm", [1, 2, 3, 7, 8, 13])
@pytest.mark.parametrize("nn", [1, 2, 5, 8, 9, 31])
@pytest.mark.parametrize("sw", [1, 2, 3, 4, 8, 40])
def test_swizzle_is_a_bijection(nm, nn, sw):
    coords = [raster.swizzle_tile_coord(p, nm, nn, sw) for p in range(nm * nn)]
    assert sorted(coords) == [(m, n) for m in range(nm) for n in range(nn)]


def test_swizzle_one_is_the_plain_grid():
    for p in range(6 * 5):
        assert raster.swizzle_tile_coord(p, 6, 5, 1) == raster.plain_2d_coord(p, 6, 5)


def test_narrow_last_group_is_row_major():
    # 3 tile-columns with groups of 2: the last group is 1 wide and walks down M
    got = [raster.swizzle_tile_coord(p, 4, 3, 2) for p in range(12)]
    assert got[8:] == [(0, 2), (1, 2), (2, 2), (3, 2)]
    assert got[:4] == [(0, 0), (0, 1), (1, 0), (1, 1)]


@pytest.mark.parametrize("grid", [1, 7, 8, 9, 240, 256, 1023, 1024])
def test_xcd_remap_bijection_and_contiguity(grid):
    logical = [raster.xcd_remap(p, grid, 8) for p in range(grid)]
    assert sorted(logical) == list(range(grid))
    for x in range(8):
        run = [logical[p] for p in range(grid) if p % 8 == x]
        assert run == list(range(run[0], run[0] + len(run))) if run else True
