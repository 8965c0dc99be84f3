"""The fitting tool's copy of the automatic tile choice (tune.model_choice)
against the library's own (gemm_f16_select_tile), with the coefficients the
library is built with, read from its source: the tool's reported choices
are the library's."""
import os
import re

import pytest

import dense_fp16_gemm_f16_amd as g
from dense_fp16_gemm_f16_amd import tune

SRC = os.path.join(os.path.dirname(g.__file__), "csrc", "gemm_f16.hip")


def library_coefficients():
    with open(SRC) as f:
        text = f.read()
    rows = re.findall(r"\{GEMM_F16_TILE_(\w+), (\d+), (\d+), ([\d.]+), ([\d.]+), ([\d.]+)\}", text)
    coef = {}
    for name, bm, bn, c, a, b in rows:
        tile = getattr(g, "TILE_" + name)
        assert tune.MODEL_TILES[tile] == (int(bm), int(bn))
        coef[tile] = (float(c), float(a), float(b))
    assert set(coef) == set(tune.MODEL_TILES)
    return coef


SIDES = [64, 200, 512, 1000, 1024, 1536, 2048, 3000, 4096, 5000, 6144, 8192, 16384]


@pytest.mark.parametrize("k", [8, 100, 256, 1000, 1024, 4095, 4096, 8192])
def test_tool_and_library_choose_the_same_tile(k):
    coef = library_coefficients()
    for m in SIDES:
        for n in SIDES:
            assert tune.model_choice(coef, m, n, k, 256) == g.select_tile(m, n, k), (m, n, k)
