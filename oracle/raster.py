"""Oracle for the block-tile scheduler (swizzled tile rasterization).

TEST INFRASTRUCTURE ONLY: only ``tests/``, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library's scheduler.

Source: "4. Pipeline Abstraction and Two Consumer Warp Groups" (Tilus Hopper
matmul tutorial), section "Tile Rasterization".  The page describes a 1D grid
in which the N axis of the tile grid is cut into groups of ``swizzle_size``
tile-columns; tiles inside one group are handed out in row-major order (along
n first, then down m); when the number of tile-columns is not a multiple of
``swizzle_size`` the final group is narrower, and the mapping stays a
bijection.  ``swizzle_size == 1`` degenerates to a plain grid that walks down
M first (the page's "plain 2D grid" where blockIdx.x walks M).

The XCD-contiguous remap below is not on the pages: it is this library's
addition for a chip whose workgroups are dispatched round-robin over 8
dies, each with its own L2.  It is stated here from its definition so the
tests can check the product's composed mapping against it.
"""
from __future__ import annotations


def swizzle_tile_coord(pid: int, num_m: int, num_n: int, swizzle: int) -> tuple[int, int]:
    """Logical tile index ``pid`` -> (m_block, n_block), per the page's grouping."""
    if not (0 <= pid < num_m * num_n):
        raise ValueError("pid out of range")
    if swizzle < 1:
        raise ValueError("swizzle must be >= 1")
    tiles_per_group = num_m * swizzle
    group = pid // tiles_per_group
    first_n = group * swizzle
    width = min(swizzle, num_n - first_n)  # the last group may be narrower
    within = pid - group * tiles_per_group
    m_block = within // width
    n_block = first_n + within % width
    return m_block, n_block


def plain_2d_coord(pid: int, num_m: int, num_n: int) -> tuple[int, int]:
    """The page's plain 2D grid: blockIdx.x walks down M first."""
    return pid % num_m, pid // num_m


def xcd_remap(pid: int, grid: int, num_xcd: int) -> int:
    """Dispatch index -> logical index so that each die gets a contiguous run.

    Dispatch index ``pid`` lands on die ``pid % num_xcd``.  Die x receives
    ``grid // num_xcd + (x < grid % num_xcd)`` workgroups; its j-th workgroup
    (j = pid // num_xcd) gets logical index (start of die x's run) + j.
    """
    if not (0 <= pid < grid):
        raise ValueError("pid out of range")
    q, r = divmod(grid, num_xcd)
    x = pid % num_xcd
    start = x * q + min(x, r)
    return start + pid // num_xcd


def strips_touched(coords) -> tuple[int, int]:
    """Distinct A row-strips and B column-strips used by a set of tiles."""
    ms = {m for m, _ in coords}
    ns = {n for _, n in coords}
    return len(ms), len(ns)
