"""Per-wave timestamps of the 256x256 kernels from the traced build of the library.

    python -m dense_fp16_gemm_f16_amd.trace [--workloads NAME ...] [--shapes M,N,K ...] [--dist D]
                                            [--launches 30] [--repeat 2] [--save DIR] [--build] [--ktiles]

libgemm_f16_trace.so is the library compiled with -DGEMM_F16_TRACE
(build.build_trace(); --build rebuilds it).  Its fragment-ahead and stream
kernels record, per wave, the shader-clock counter at their start, after the
prologue's wait, after the K loop and after their last store, the 100 MHz
counter at start and end, the cycles spent waiting in the K loop's two
barriers and the XCC the wave ran on; the stream kernel also the start of
each of its first four tiles.  --ktiles uses libgemm_f16_trace_kt.so, which
also stamps the K-tiles around the stream kernel's first tile change (the
last of the first tile, the first three of the second); those stamps cost
its K loop some scalar-register spills, so the other figures come from the
plain traced build.  Each run launches the GEMM on the 256x256 tile `--launches`
times back to back (the device settles at its loaded clock) and reads the
last launch's words.

The summary splits a wave's cycles into prologue, K loop and epilogue, sets
the K loop against the MFMA issue time it holds (128 v_mfma_f32_16x16x32_f16
per wave and K-tile at 16 cycles each: 2.5 PFLOP/s over 1024 SIMDs at
2.4 GHz is 1017 flop per SIMD and cycle, and the MFMA does 16384), and gives
each XCC's clock (counter cycles over 100 MHz ticks) and end time.  Only the
256x256 block tile is traced: the other tiles' kernels write their own
translation units' copies, which this does not read.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys

import numpy as np

import dense_fp16_gemm_f16_amd as _g
from dense_fp16_gemm_f16_amd import build as _build

TRACE_BLOCKS = 2048
TRACE_WORDS = 24
MFMA_CYCLES_PER_KTILE = 128 * 16  # per wave: 8 x 8 blocks x 2 k steps, 16 cycles each
BK = 64


def summarize(words: np.ndarray, k: int) -> dict:
    """Summary of one launch's trace words ([TRACE_BLOCKS * 4, TRACE_WORDS]
    uint64, as the traced kernels write them) for a GEMM of depth k."""
    w = np.asarray(words, dtype=np.uint64).reshape(-1, TRACE_WORDS).astype(np.int64)
    w = w[w[:, 0] != 0]
    if len(w) == 0:
        raise ValueError("no wave recorded anything (not a 256x256 fragment-ahead or stream launch?)")
    t0, t1, rel, acq, acq_first, tl, te, r0, re, tiles = (w[:, i] for i in range(10))
    xcc = w[:, 16] & 0xF
    kt = -(-k // BK)
    ktiles = kt * tiles
    clock = (te - t0) / ((re - r0) * 10.0)  # counter cycles per ns
    start = r0.min()
    end_us = (re - start) / 100.0

    def q(x):
        x = np.asarray(x, dtype=np.float64)
        return {"min": round(float(x.min()), 3), "median": round(float(np.median(x)), 3),
                "max": round(float(x.max()), 3)}

    mfma = MFMA_CYCLES_PER_KTILE * ktiles
    rec = {
        "waves": int(len(w)),
        "tiles_per_workgroup": q(tiles),
        "k_tiles_per_tile": int(kt),
        "cycles": {
            "prologue": q(t1 - t0),
            "k_loop": q(tl - t1),
            "epilogue": q(te - tl),
            "total": q(te - t0),
            "mfma_issue": q(mfma),
        },
        "k_loop_cycles_per_ktile": q((tl - t1) / ktiles),
        "mfma_share_of_k_loop": q(mfma / (tl - t1)),
        "mfma_share_of_wave": q(mfma / (te - t0)),
        "barrier_wait_cycles_per_ktile": {"release": q(rel / ktiles), "acquire": q(acq / ktiles)},
        "acquire_wait_first_ktile_of_tile_cycles": q(acq_first / np.maximum(tiles, 1)),
        "start_spread_us": round(float((r0.max() - start) / 100.0), 3),
        "end_us": q(end_us),
        "clock_ghz": q(clock),
        "xcc": {},
    }
    if tiles.min() > 1:
        s = w[:, 10:14]
        n = int(min(tiles.min(), 4))
        rec["tile_cycles"] = [q(s[:, i + 1] - s[:, i]) for i in range(n - 1)]
        if kt >= 4 and (w[:, 20] != 0).all():
            kl, k0, k1, k2 = (w[:, 20 + i] for i in range(4))
            m32 = 1 << 32  # the stamps are the counter's low 32 bits
            rec["first_tile_change_cycles"] = {
                "last_ktile_of_tile_1_and_change": q((k0 - kl) % m32),
                "ktile_0_of_tile_2": q((k1 - k0) % m32),
                "ktile_1_of_tile_2": q((k2 - k1) % m32),
            }
    for x in sorted(set(xcc.tolist())):
        sel = xcc == x
        rec["xcc"][str(x)] = {"waves": int(sel.sum()), "clock_ghz": round(float(np.median(clock[sel])), 4),
                              "end_us_median": round(float(np.median(end_us[sel])), 2),
                              "end_us_max": round(float(end_us[sel].max()), 2),
                              "total_cycles_median": round(float(np.median((te - t0)[sel])), 0)}
    ends = [v["end_us_max"] for v in rec["xcc"].values()]
    rec["end_us_last_xcc_over_mean_xcc"] = round(max(ends) / (sum(ends) / len(ends)), 4)
    return rec


def load(rebuild: bool = False, ktiles: bool = False) -> ctypes.CDLL:
    path = _build.TRACE_KT_LIB if ktiles else _build.TRACE_LIB
    if rebuild or not os.path.exists(path):
        _build.build_trace(ktiles=ktiles)
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.gemm_f16_nt_ex.argtypes = [i64, i64, i64, vp, vp, vp, vp, ctypes.POINTER(_g.Options)]
    lib.gemm_f16_nt_ex.restype = ctypes.c_int
    lib.gemm_f16_trace_read.argtypes = [vp, ctypes.c_size_t]
    lib.gemm_f16_trace_read.restype = ctypes.c_int
    lib.gemm_f16_trace_clear.restype = ctypes.c_int
    return lib


def run(lib, a, b, c, m: int, n: int, k: int, launches: int, stream: int) -> np.ndarray:
    """`launches` GEMMs on the 256x256 tile (default rasterization) back to
    back on `stream`; the trace words of the last."""
    import torch

    if lib.gemm_f16_trace_clear() != 0:
        raise RuntimeError("gemm_f16_trace_clear failed")
    torch.cuda.synchronize()
    opt = _g.Options(_g.TILE_256x256, 0, -1, _g.VARIANT_DEFAULT)
    for _ in range(launches):
        rc = lib.gemm_f16_nt_ex(m, n, k, a.data_ptr(), b.data_ptr(), c.data_ptr(), stream or None, ctypes.byref(opt))
        if rc != 0:
            raise _g.GemmError(rc)
    torch.cuda.synchronize()
    buf = np.zeros(TRACE_BLOCKS * 4 * TRACE_WORDS, dtype=np.uint64)
    if lib.gemm_f16_trace_read(buf.ctypes.data, buf.nbytes) != 0:
        raise RuntimeError("gemm_f16_trace_read failed")
    return buf.reshape(TRACE_BLOCKS * 4, TRACE_WORDS)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", nargs="*", default=None,
                    help="workloads of inputs.WORKLOADS (C = A B^T ones); default: the four large benchmark ones")
    ap.add_argument("--shapes", nargs="*", default=[], help="M,N,K triples")
    ap.add_argument("--dist", default="uniform", choices=["uniform", "normal", "eighths", "zeros"],
                    help="operand values for --shapes")
    ap.add_argument("--launches", type=int, default=30)
    ap.add_argument("--repeat", type=int, default=2)
    ap.add_argument("--save", default=None, help="directory for the raw words (.npy)")
    ap.add_argument("--build", action="store_true", help="rebuild the traced library first")
    ap.add_argument("--ktiles", action="store_true",
                    help="the build that also stamps the K-tiles around the first tile change")
    a = ap.parse_args(argv)

    import torch

    from dense_fp16_gemm_f16_amd import inputs

    lib = load(a.build, a.ktiles)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    cases = []
    names = a.workloads if a.workloads is not None else [
        "gemm_4096_normal", "gemm_8192_uniform", "gemm_16384x4096x2048_normal05", "gemm_5000x3000x1000_eighths"]
    for name in names:
        w = inputs.WORKLOADS[name]
        if w.b_layout != "nk":
            raise SystemExit(f"{name}: only C = A B^T workloads are traced")
        cases.append((name, w.m, w.n, w.k, lambda w=w: inputs.workload_inputs(w.name)))
    for s in a.shapes:
        m, n, k = (int(x) for x in s.split(","))
        if a.dist == "zeros":
            make = (lambda m=m, n=n, k=k: (np.zeros((m, k), np.float16), np.zeros((n, k), np.float16)))
        else:
            make = (lambda m=m, n=n, k=k: inputs.make_inputs(m, n, k, a.dist, 7))
        cases.append((f"{m}x{n}x{k}_{a.dist}", m, n, k, make))
    for name, m, n, k, make in cases:
        a_np, b_np = make()
        A = torch.from_numpy(a_np).to(dev)
        B = torch.from_numpy(b_np).to(dev)
        C = torch.empty((m, n), dtype=torch.float16, device=dev)
        for rep in range(a.repeat):
            words = run(lib, A, B, C, m, n, k, a.launches, stream)
            if a.save:
                os.makedirs(a.save, exist_ok=True)
                np.save(os.path.join(a.save, f"trace_{name}_{rep}.npy"), words)
            print(json.dumps({"case": name, "shape": [m, n, k], "repeat": rep, "launches": a.launches,
                              **summarize(words, k)}), flush=True)
        del A, B, C
    return 0


if __name__ == "__main__":
    sys.exit(main())
