"""Offline sweep of block tile and rasterization options on one GPU.

    python -m dense_fp16_gemm_f16_amd.tune [--shapes M,N,K ...] [--rounds 3]
    python -m dense_fp16_gemm_f16_amd.tune --data      # operand values vs time
    python -m dense_fp16_gemm_f16_amd.tune --ceiling   # MFMA rate, no HBM traffic
    python -m dense_fp16_gemm_f16_amd.tune --graph 100 # eager launches vs one HIP graph
    python -m dense_fp16_gemm_f16_amd.tune --fit SWEEP.jsonl [...]  # refit the tile model

For every shape (default: the five benchmark workloads) it times each block
tile (and, for the default tile, a few swizzle widths) with HIP events,
interleaving the candidates over several rounds and taking the median, on
uniform[-1,1] fp16 operands.  One JSON line per (shape, option), then one
line per shape naming the fastest option.  The automatic tile choice in the
library (gemm_f16_select_tile) is meant to agree with these results.
"""
from __future__ import annotations

import argparse
import json
import math
import statistics
import sys

import dense_fp16_gemm_f16_amd as g
from dense_fp16_gemm_f16_amd import inputs


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--shapes", nargs="*", default=None, help="M,N,K triples")
    ap.add_argument("--rounds", type=int, default=3)
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--swizzles", default="1,4,8")
    ap.add_argument("--variants", action="store_true",
                    help="also time the kernel variants (block_k 32/64, 2-4 LDS stages, loader waves) "
                         "on every block tile they fit, default rasterization")
    ap.add_argument("--data", action="store_true",
                    help="instead: time the automatic configuration on one shape (default 8192^3) "
                         "with different operand values (zeros, ones, {-8..8}/8, U[0,1], U[-1,1], N(0,1))")
    ap.add_argument("--ceiling", action="store_true",
                    help="instead: the sustained v_mfma_f32_32x32x16_f16 and v_mfma_f32_16x16x32_f16 rates of the device with no "
                         "global memory traffic (libmfma_ceiling.so), on random and on zero operands")
    ap.add_argument("--hold", type=float, default=0.0, metavar="SECONDS",
                    help="with --data or --ceiling: run each operand set (or probe variant) back to back "
                         "for this long and print its wall-clock start and end (to line up with power and "
                         "clock samples)")
    ap.add_argument("--fit", nargs="+", default=None, metavar="SWEEP",
                    help="instead (no GPU): fit the automatic tile choice's model to sweep files of this "
                         "tool (the geometric mean over the files), print its coefficients and its choice "
                         "against the fastest tile on every shape")
    ap.add_argument("--graph", type=int, default=0, metavar="N",
                    help="instead: time N GEMMs of each shape (default 256^3, 1024^3, 2048^3) launched "
                         "eagerly and replayed from one captured HIP graph")
    a = ap.parse_args(argv)
    if a.fit:
        return fit_model(a.fit)
    import torch

    if a.graph:
        return graph_sweep(a, torch)
    if a.data:
        return data_sweep(a, torch)
    if a.ceiling:
        return ceiling(a, torch)

    shapes = ([tuple(int(x) for x in s.split(",")) for s in a.shapes] if a.shapes else
              [(w.m, w.n, w.k) for w in inputs.WORKLOADS.values()])
    swz = [int(x) for x in a.swizzles.split(",")]
    gen = torch.Generator(device="cuda").manual_seed(0)
    stream = torch.cuda.current_stream()
    for (m, n, k) in shapes:
        A = (torch.rand((m, k), device="cuda", generator=gen) * 2 - 1).half()
        B = (torch.rand((n, k), device="cuda", generator=gen) * 2 - 1).half()
        C = torch.empty((m, n), device="cuda", dtype=torch.float16)
        auto = g.select_tile(m, n, k)
        opts = [(t, 0, -1, 0) for t in sorted(g.TILES)] + [(auto, s, x, 0) for s in swz for x in (0, 1)]
        if a.variants:
            for v, (bk, _, _) in sorted(g.VARIANTS.items()):
                for t in sorted(g.TILES):
                    if k % bk == 0 and g.gemm_f16_nt_raw(0, 0, k, 16, 16, 16, 0, t, 0, -1, v) == g.OK:
                        opts.append((t, 0, -1, v))
        times = {o: [] for o in opts}
        for _ in range(a.rounds):
            for o in opts:
                def run():
                    rc = g.gemm_f16_nt_raw(m, n, k, A.data_ptr(), B.data_ptr(), C.data_ptr(),
                                           stream.cuda_stream, *o)
                    if rc != g.OK:
                        raise g.GemmError(rc)
                for _ in range(2):
                    run()
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(a.reps)]
                for e0, e1 in ev:
                    e0.record(stream)
                    run()
                    e1.record(stream)
                torch.cuda.synchronize()
                times[o].append(statistics.median(e0.elapsed_time(e1) for e0, e1 in ev))
        best = None
        for o in opts:
            us = statistics.median(times[o]) * 1e3
            tf = 2.0 * m * n * k / (us * 1e-6) / 1e12
            print(json.dumps({"shape": [m, n, k], "tile": o[0], "swizzle": o[1], "xcd": o[2], "variant": o[3],
                              "us": round(us, 2), "tflops": round(tf, 1),
                              "auto": o[0] == auto and o[3] == 0}), flush=True)
            if best is None or us < best[1]:
                best = (o, us)
        print(json.dumps({"shape": [m, n, k], "best": best[0], "best_us": round(best[1], 2),
                          "auto_tile": auto}), flush=True)
        del A, B, C
    return 0


def data_sweep(a, torch) -> int:
    """The MFMA clock depends on the operand bits: same kernel, different values."""
    m, n, k = (tuple(int(x) for x in a.shapes[0].split(",")) if a.shapes else (8192, 8192, 8192))
    gen = torch.Generator(device="cuda").manual_seed(1)
    makers = {
        "zeros": lambda s: torch.zeros(s, device="cuda", dtype=torch.float16),
        "ones": lambda s: torch.ones(s, device="cuda", dtype=torch.float16),
        "eighths": lambda s: (torch.randint(-8, 9, s, device="cuda", generator=gen) / 8).half(),
        "uniform[0,1]": lambda s: torch.rand(s, device="cuda", generator=gen).half(),
        "uniform[-1,1]": lambda s: (torch.rand(s, device="cuda", generator=gen) * 2 - 1).half(),
        "normal": lambda s: torch.randn(s, device="cuda", generator=gen).half(),
    }
    C = torch.empty((m, n), device="cuda", dtype=torch.float16)
    stream = torch.cuda.current_stream()
    data = {name: (f((m, k)), f((n, k))) for name, f in makers.items()}
    if a.hold > 0:
        return hold_sweep(a, torch, m, n, k, data, C, stream)
    times = {name: [] for name in data}
    for _ in range(a.rounds):
        for name, (A, B) in data.items():
            def run():
                rc = g.gemm_f16_nt_raw(m, n, k, A.data_ptr(), B.data_ptr(), C.data_ptr(), stream.cuda_stream)
                if rc != g.OK:
                    raise g.GemmError(rc)
            for _ in range(2):
                run()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(a.reps)]
            for e0, e1 in ev:
                e0.record(stream)
                run()
                e1.record(stream)
            torch.cuda.synchronize()
            times[name].append(statistics.median(e0.elapsed_time(e1) for e0, e1 in ev))
    for name, t in times.items():
        us = statistics.median(t) * 1e3
        print(json.dumps({"shape": [m, n, k], "operands": name, "us": round(us, 1),
                          "tflops": round(2.0 * m * n * k / (us * 1e-6) / 1e12, 1)}), flush=True)
    return 0


def hold_sweep(a, torch, m, n, k, data, C, stream) -> int:
    """Each operand set back to back for a.hold seconds, synchronising every
    50 launches; one JSON line per set with its wall-clock interval."""
    import time

    for name, (A, B) in data.items():
        def run():
            rc = g.gemm_f16_nt_raw(m, n, k, A.data_ptr(), B.data_ptr(), C.data_ptr(), stream.cuda_stream)
            if rc != g.OK:
                raise g.GemmError(rc)
        for _ in range(5):
            run()
        torch.cuda.synchronize()
        t0 = time.time()
        launches = 0
        while time.time() - t0 < a.hold:
            for _ in range(50):
                run()
            torch.cuda.synchronize()
            launches += 50
        t1 = time.time()
        print(json.dumps({"shape": [m, n, k], "operands": name, "start": round(t0, 3), "end": round(t1, 3),
                          "launches": launches,
                          "tflops": round(2.0 * m * n * k * launches / (t1 - t0) / 1e12, 1)}), flush=True)
        time.sleep(1.0)  # an idle gap between sets in the samples
    return 0


def graph_sweep(a, torch) -> int:
    """Launch-bound shapes: N back-to-back GEMMs enqueued one call at a time,
    against the same N GEMMs captured once in a HIP graph and replayed.  Both
    are timed with one HIP-event pair around all N; the result is per GEMM."""
    shapes = ([tuple(int(x) for x in s.split(",")) for s in a.shapes] if a.shapes else
              [(256, 256, 256), (1024, 1024, 1024), (2048, 2048, 2048)])
    gen = torch.Generator(device="cuda").manual_seed(3)
    n_gemm = a.graph
    for (m, n, k) in shapes:
        A = (torch.rand((m, k), device="cuda", generator=gen) * 2 - 1).half()
        B = (torch.rand((n, k), device="cuda", generator=gen) * 2 - 1).half()
        C = torch.empty((m, n), device="cuda", dtype=torch.float16)
        side = torch.cuda.Stream()  # default priority

        def enqueue(stream):
            for _ in range(n_gemm):
                rc = g.gemm_f16_nt_raw(m, n, k, A.data_ptr(), B.data_ptr(), C.data_ptr(), stream.cuda_stream)
                if rc != g.OK:
                    raise g.GemmError(rc)

        with torch.cuda.stream(side):
            enqueue(side)  # warm-up, outside any capture
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                enqueue(torch.cuda.current_stream())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        res = {"eager": [], "graph": []}
        for _ in range(max(a.rounds, 3)):
            for mode in ("eager", "graph"):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                with torch.cuda.stream(side):
                    e0.record(side)
                    if mode == "eager":
                        enqueue(side)
                    else:
                        graph.replay()
                    e1.record(side)
                torch.cuda.synchronize()
                res[mode].append(e0.elapsed_time(e1) * 1e3 / n_gemm)
        for mode, t in res.items():
            us = statistics.median(t)
            print(json.dumps({"shape": [m, n, k], "mode": mode, "gemms": n_gemm, "tile": g.select_tile(m, n, k),
                              "us_per_gemm": round(us, 2), "tflops": round(2.0 * m * n * k / (us * 1e-6) / 1e12, 1)}),
                  flush=True)
        del graph, A, B, C
    return 0


def ceiling(a, torch) -> int:
    """Sustained MFMA rate on a 128x128 wave tile: v_mfma_f32_32x32x16_f16
    with fragments from LDS (variant 0) or registers (variant 1), and
    v_mfma_f32_16x16x32_f16 with tied accumulators, the same two ways
    (variants 2, 3); operands uniform[-1,1] fp16 or zeros."""
    import ctypes
    import os

    from dense_fp16_gemm_f16_amd import build

    path = build.CEILING_LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run dense_fp16_gemm_f16_amd.build.build_ceiling() "
                           "(a measurement probe, not part of the library)")
    L = ctypes.CDLL(path)
    L.mfma_ceiling_launch.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p]
    L.mfma_ceiling_flops.argtypes = [ctypes.c_int64, ctypes.c_int32]
    L.mfma_ceiling_flops.restype = ctypes.c_double
    wgs = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 60000  # ~40 ms per launch at 1.5 GHz: long enough for the clock to settle
    out = torch.empty(wgs * 256, device="cuda", dtype=torch.float32)
    gen = torch.Generator(device="cuda").manual_seed(7)
    tables = {"uniform[-1,1]": (torch.rand(4096 * 8, device="cuda", generator=gen) * 2 - 1).half(),
              "zeros": torch.zeros(4096 * 8, device="cuda", dtype=torch.float16)}
    stream = torch.cuda.current_stream()
    names = {0: "fragments from LDS", 1: "fragments in registers", 2: "fragments from LDS",
             3: "fragments in registers"}
    probes = {0: "v_mfma_f32_32x32x16_f16", 1: "v_mfma_f32_32x32x16_f16",
              2: "v_mfma_f32_16x16x32_f16 (tied)", 3: "v_mfma_f32_16x16x32_f16 (tied)"}
    for operands, t in tables.items():
        for variant in (0, 1, 2, 3):
            def run(n):
                rc = L.mfma_ceiling_launch(variant, n, wgs, t.data_ptr(), out.data_ptr(), stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"mfma_ceiling_launch returned {rc}")
            run(iters // 20)
            if a.hold > 0:
                # back to back for a.hold seconds, with the wall-clock interval
                # printed (to line up with power and clock samples)
                import time

                torch.cuda.synchronize()
                t0 = time.time()
                launches = 0
                while time.time() - t0 < a.hold:
                    run(iters)
                    torch.cuda.synchronize()
                    launches += 1
                t1 = time.time()
                tf = L.mfma_ceiling_flops(iters, wgs) * launches / (t1 - t0) / 1e12
                print(json.dumps({"probe": probes[variant] + ", 128x128 wave tile", "variant": names[variant],
                                  "operands": operands, "start": round(t0, 3), "end": round(t1, 3),
                                  "launches": launches, "tflops": round(tf, 1)}), flush=True)
                time.sleep(1.0)
                continue
            ms = []
            for _ in range(max(a.rounds, 3)):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                run(iters)
                e1.record(stream)
                torch.cuda.synchronize()
                ms.append(e0.elapsed_time(e1))
            med = statistics.median(ms)
            tf = L.mfma_ceiling_flops(iters, wgs) / (med * 1e-3) / 1e12
            print(json.dumps({"probe": probes[variant] + ", 128x128 wave tile", "variant": names[variant],
                              "operands": operands, "workgroups": wgs, "ms": round(med, 2),
                              "tflops": round(tf, 1)}), flush=True)
    return 0



# The automatic tile choice's candidates (tile id: block tile), the same list
# and order as auto_tile in csrc/gemm_f16.hip.
MODEL_TILES = {g.TILE_256x256: (256, 256), g.TILE_256x128: (256, 128), g.TILE_128x256: (128, 256),
               g.TILE_128x128: (128, 128), g.TILE_128x64: (128, 64), g.TILE_64x128: (64, 128),
               g.TILE_64x64: (64, 64)}


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def model_terms(tile: int, m: int, n: int, k: int, cus: int = 256) -> tuple[float, float, float]:
    """The model's three terms for one block tile: 1, rounds * k_tiles, tiles / cus."""
    bm, bn = MODEL_TILES[tile]
    tiles = _cdiv(m, bm) * _cdiv(n, bn)
    return 1.0, float(_cdiv(tiles, cus) * _cdiv(k, 64)), tiles / cus


def model_choice(coef: dict, m: int, n: int, k: int, cus: int = 256) -> int:
    """The tile auto_tile picks with coefficients coef {tile: (c, a, b)}: the
    smallest modelled time, then a rectangular tile turned with its long side
    along the shorter dimension unless that costs a round of tiles."""
    best, best_t = g.TILE_64x64, 1e300
    for tile in MODEL_TILES:
        if tile == g.TILE_256x256 and k % 8 != 0:
            continue
        t = sum(x * y for x, y in zip(coef[tile], model_terms(tile, m, n, k, cus)))
        if t < best_t * 0.999:
            best, best_t = tile, t
    if best in (g.TILE_256x128, g.TILE_128x256) and m != n:
        def rounds(wide):
            return _cdiv(_cdiv(m, 128 if wide else 256) * _cdiv(n, 256 if wide else 128), cus)
        wide = m > n
        if rounds(wide) <= rounds(best == g.TILE_128x256):
            best = g.TILE_128x256 if wide else g.TILE_256x128
    return best


def fit_model(paths: list[str]) -> int:
    """Least squares in relative error, per candidate tile, of the time model
    to the default-rasterization times of sweep files (geometric mean over
    the files where a shape and tile appear in all of them)."""
    import numpy as np

    runs = []
    for path in paths:
        times = {}
        with open(path) as f:
            for line in f:
                r = json.loads(line)
                if "best" in r or r.get("swizzle") != 0 or r.get("variant", 0) != 0:
                    continue
                times[(tuple(r["shape"]), r["tile"])] = r["us"]
        runs.append(times)
    keys = set(runs[0]).intersection(*runs[1:])
    mean = {key: math.exp(statistics.fmean(math.log(t[key]) for t in runs)) for key in keys}
    shapes = sorted({s for s, _ in mean})
    coef = {}
    for tile in MODEL_TILES:
        rows = [[x / mean[(s, tile)] for x in model_terms(tile, *s)] for s in shapes if (s, tile) in mean]
        coef[tile] = tuple(float(v) for v in np.linalg.lstsq(np.array(rows), np.ones(len(rows)), rcond=None)[0])
    names = {t: f"{bm}x{bn}" if t in MODEL_TILES else f"{bm}x{bn} (tile {t})" for t, (bm, bn) in g.TILES.items()}
    for tile, (c, a_, b) in coef.items():
        print(json.dumps({"tile": tile, "block": names[tile], "c": round(c, 3), "a": round(a_, 3), "b": round(b, 3)}))
    ratios = []
    for s in shapes:
        have = {t: mean[(s, t)] for t in g.TILES if (s, t) in mean}  # every tile swept, candidates or not
        fastest = min(have, key=have.get)
        pick = model_choice(coef, *s)
        ratios.append(have[pick] / have[fastest])
        print(json.dumps({"shape": list(s), "fastest": names[fastest], "fastest_us": round(have[fastest], 2),
                          "model": names[pick], "model_us": round(have[pick], 2),
                          "ratio": round(ratios[-1], 3)}))
    print(json.dumps({"shapes": len(ratios), "within_3pct": sum(r <= 1.03 for r in ratios),
                      "within_5pct": sum(r <= 1.05 for r in ratios), "worst": round(max(ratios), 3)}))
    return 0


if __name__ == "__main__":
    sys.exit(main())
