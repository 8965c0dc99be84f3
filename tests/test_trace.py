"""The timestamp-traced build: its summary arithmetic (CPU) and, on the GPU,
that tracing leaves C bit-identical and every wave records its words."""
import os

import numpy as np
import pytest

from dense_fp16_gemm_f16_amd import build, trace


def _words(waves):
    """Trace words for a list of per-wave dicts (workgroup-major, 4 waves each)."""
    w = np.zeros((trace.TRACE_BLOCKS * 4, trace.TRACE_WORDS), dtype=np.uint64)
    for i, d in enumerate(waves):
        row = w[i]
        for j, key in enumerate(("t0", "t1", "rel", "acq", "acq_first", "tl", "te", "r0", "re", "tiles")):
            row[j] = d.get(key, 0)
        for j, v in enumerate(d.get("tile_start", [])):
            row[10 + j] = v
        row[16] = d.get("xcc", 0)
        for j, v in enumerate(d.get("kt_stamps", [])):
            row[20 + j] = v
    return w


def test_summary_of_a_made_up_trace():
    # two workgroups (8 waves) on XCCs 0 and 1; K = 1024 -> 16 K-tiles per tile
    # and 2 tiles per workgroup; clock 2 GHz on XCC 0 and 1 GHz on XCC 1
    waves = []
    for wg in range(2):
        clk = 2.0 if wg == 0 else 1.0
        for wave in range(4):
            t0 = 1_000_000 + 7 * wave
            cycles = 100_000
            ticks = int(cycles / clk / 10)  # 100 MHz ticks
            waves.append(dict(t0=t0, t1=t0 + 4_000, tl=t0 + 4_000 + 80_000, te=t0 + cycles,
                              rel=32 * 50, acq=32 * 25, acq_first=2 * 300, tiles=2,
                              r0=500 + wg, re=500 + wg + ticks, xcc=wg,
                              tile_start=[t0 + 4_000, t0 + 44_000],
                              # low 32 bits, wrapping between the second and third
                              kt_stamps=[2**32 - 5_500, 2**32 - 3_000, 0, 2_500]))
    s = trace.summarize(_words(waves), 1024)
    assert s["waves"] == 8
    assert s["k_tiles_per_tile"] == 16
    assert s["cycles"]["prologue"]["median"] == 4_000
    assert s["cycles"]["k_loop"]["median"] == 80_000
    assert s["cycles"]["epilogue"]["median"] == 16_000
    assert s["k_loop_cycles_per_ktile"]["median"] == 80_000 / 32
    assert s["cycles"]["mfma_issue"]["median"] == 32 * 2048
    assert s["mfma_share_of_k_loop"]["median"] == pytest.approx(32 * 2048 / 80_000, abs=1e-3)
    assert s["barrier_wait_cycles_per_ktile"]["release"]["median"] == 50
    assert s["barrier_wait_cycles_per_ktile"]["acquire"]["median"] == 25
    assert s["acquire_wait_first_ktile_of_tile_cycles"]["median"] == 300
    assert s["tile_cycles"][0]["median"] == 40_000
    change = s["first_tile_change_cycles"]
    assert change["last_ktile_of_tile_1_and_change"]["median"] == 2_500
    assert change["ktile_0_of_tile_2"]["median"] == 3_000
    assert change["ktile_1_of_tile_2"]["median"] == 2_500
    assert s["xcc"]["0"]["clock_ghz"] == pytest.approx(2.0, rel=1e-3)
    assert s["xcc"]["1"]["clock_ghz"] == pytest.approx(1.0, rel=1e-3)
    # XCC 1 starts one tick later and runs twice as long
    assert s["xcc"]["0"]["end_us_max"] == pytest.approx(50.0, abs=0.011)  # 100k cycles at 2 GHz
    assert s["xcc"]["1"]["end_us_max"] == pytest.approx(100.01, abs=0.011)
    assert s["start_spread_us"] == pytest.approx(0.01)


def test_summary_refuses_an_empty_trace():
    with pytest.raises(ValueError):
        trace.summarize(np.zeros((trace.TRACE_BLOCKS * 4, trace.TRACE_WORDS), dtype=np.uint64), 256)


@pytest.mark.gpu
@pytest.mark.parametrize("m,n,k", [(1000, 1000, 1000), (4608, 4096, 256), (2304, 2048, 512)])
def test_traced_build_matches_the_library(m, n, k):
    """The 256x256 tile through the traced build: the fragment-ahead kernel
    (16 tiles, K ragged; 72 tiles) and the stream kernel (288 tiles, more than
    the CUs): C bit-identical to the library's, every wave's words written."""
    if not os.path.exists(build.TRACE_LIB):
        pytest.skip("libgemm_f16_trace.so is not built (python -m dense_fp16_gemm_f16_amd.build --trace)")
    import torch

    import dense_fp16_gemm_f16_amd as g
    from dense_fp16_gemm_f16_amd import inputs

    lib = trace.load()
    a_np, b_np = inputs.make_inputs(m, n, k, "uniform", 11)
    a = torch.from_numpy(a_np).cuda()
    b = torch.from_numpy(b_np).cuda()
    c_ref = torch.empty((m, n), dtype=torch.float16, device="cuda")
    c = torch.full((m, n), float("nan"), dtype=torch.float16, device="cuda")
    assert g.gemm_f16_nt_raw(m, n, k, a.data_ptr(), b.data_ptr(), c_ref.data_ptr(), 0, g.TILE_256x256) == g.OK
    words = trace.run(lib, a, b, c, m, n, k, 3, 0)
    assert torch.equal(c.view(torch.int16), c_ref.view(torch.int16))
    tiles = -(-m // 256) * -(-n // 256)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    s = trace.summarize(words, k)
    assert s["waves"] == 4 * min(tiles, cus)
    assert s["tiles_per_workgroup"]["max"] == -(-tiles // min(tiles, cus))
    assert s["cycles"]["k_loop"]["min"] > 0 and s["cycles"]["epilogue"]["min"] > 0
    assert 0.3 < s["clock_ghz"]["median"] < 3.0
