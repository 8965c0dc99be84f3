#!/usr/bin/env python3
"""Throughput of the fp16 GEMM C = fp16(A @ B^T) (fp32 accumulate) on one MI355X.

One step is one GEMM over the whole workload (default: M = N = K = 8192,
A and B i.i.d. uniform[-1,1] rounded to fp16), with A, B and C resident in
HBM before the timed region starts.  Prints one JSON line.

Timing follows the tutorials' protocol (CUDA-event timed; the Tilus pages
report the median of three fresh processes): W untimed warm-up GEMMs, then
exactly K timed GEMMs between two device synchronisations; every launch is
also bracketed by HIP events on the stream it runs on, which gives the
kernel's average duration for the roofline figure.

The CPU baseline times the oracle (plain fp64 triple loop, one fp16
rounding) on a bounded sample of the same workload -- whole rows of C -- and
the same rows double as a parity spot check of the timed output.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fp16 GEMM TFLOP/s (fp32 acc) at 8192³; % of MI355X dense fp16 MFMA peak"
PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, published
PROFILE_DIR = os.path.join(ROOT, "profiles")


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(PROFILE_DIR, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    from dense_fp16_gemm_f16_amd.profile_summary import kernel_source_hash

    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(a, b, c_gpu, w, budget_s: float):
    """Time the oracle on whole rows of C; returns (record, parity summary)."""
    import numpy as np

    import oracle

    threads = oracle.default_threads()
    rng = np.random.default_rng(12345)
    # Calibrate on one row per thread, then run random rows in batches of
    # about a quarter of the budget until the budget is spent.  The small
    # calibration call also pays for starting threads and cold caches, so
    # the batches, not the calibration, decide how many rows fit.
    t0 = time.perf_counter()
    first = oracle.gemm_f16_nt_rows(a, b, list(range(min(threads, w.m))), threads)
    t_round = max(time.perf_counter() - t0, 1e-6)  # one row on every thread
    batch = max(threads, int(budget_s / 4.0 / t_round) * threads)
    order = rng.permutation(w.m)
    row_parts, ref_parts = [], []
    dt, done = 0.0, 0
    while done < w.m and (dt < budget_s or done == 0):
        rows_b = np.sort(order[done:done + batch])
        t0 = time.perf_counter()
        ref_parts.append(oracle.gemm_f16_nt_rows(a, b, rows_b, threads))
        dt += time.perf_counter() - t0
        row_parts.append(rows_b)
        done += len(rows_b)
    rows = np.concatenate(row_parts)
    ref = np.concatenate(ref_parts)
    flops = 2.0 * len(rows) * w.n * w.k
    rec = {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{len(rows)} of {w.m} rows of C (all {w.n} columns, full K={w.k}), "
                  f"fp64 triple loop, {dt:.1f} s",
    }
    got = c_gpu[rows].astype(np.float64)
    r = ref.astype(np.float64)
    # 2 fp16 ulp of |C_oracle| + 1e-2 sqrt(K) 2^-11 (bit-exact expected on {-8..8}/8)
    ar = np.abs(r)
    e = np.where(ar > 0, np.maximum(np.floor(np.log2(np.where(ar > 0, ar, 1.0))), -14), -14)
    tol = 2.0 * np.exp2(e - 10) + 1e-2 * np.sqrt(w.k) * 2.0**-11
    if w.dist == "eighths":
        tol = np.zeros_like(tol) + 1e-300
    err = np.abs(got - r)
    err = np.where(np.isnan(err), np.inf, err)
    worst = float(np.max(err / tol)) if err.size else 0.0
    ok = worst <= 1.0
    del first
    return rec, {"rows": int(len(rows)), "ok": bool(ok), "worst_err_over_tol": round(worst, 4)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gemm_8192_uniform")
    ap.add_argument("--tile", type=int, default=0)
    ap.add_argument("--swizzle", type=int, default=0)
    ap.add_argument("--xcd", type=int, default=-1)
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--traffic-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain elementwise copy (negation) of BYTES, 3 times: the "
                         "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this GEMM has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.traffic_calibration:
        n = args.traffic_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)  # one elementwise kernel: reads and writes BYTES
        torch.cuda.synchronize()
        print(json.dumps({"traffic_calibration_bytes": n * 4}), flush=True)
        return 0

    import dense_fp16_gemm_f16_amd as g
    from dense_fp16_gemm_f16_amd import inputs

    w = inputs.WORKLOADS[args.workload]
    print(f"[bench] workload {w.name} ({w.m}x{w.n}x{w.k}, {w.dist}); generating inputs",
          file=sys.stderr, flush=True)
    a_np, b_np = inputs.workload_inputs(w.name)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    a = torch.from_numpy(a_np).to(dev)
    b = torch.from_numpy(b_np).to(dev)
    nn = w.b_layout == "kn"  # the second contract: D fp32 = A B with B [K,N]
    c = torch.empty((w.m, w.n), dtype=torch.float32 if nn else torch.float16, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    ap_, bp_, cp_ = a.data_ptr(), b.data_ptr(), c.data_ptr()

    call = g.gemm_f16_nn_f32_raw if nn else g.gemm_f16_nt_raw

    def step():
        rc = call(w.m, w.n, w.k, ap_, bp_, cp_, sp, args.tile, args.swizzle, args.xcd)
        if rc != g.OK:
            raise g.GemmError(rc)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done; timing {args.steps} steps", file=sys.stderr, flush=True)

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    durs = [s.elapsed_time(e) for s, e in zip(starts, ends)]  # ms
    avg_ms = sum(durs) / len(durs)
    med_ms = sorted(durs)[len(durs) // 2]
    ms_per_step = wall * 1e3 / args.steps
    flops = float(w.flops)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (avg_ms * 1e-3) / 1e12
    print(f"[bench] kernel avg {avg_ms * 1e3:.1f} us, median {med_ms * 1e3:.1f} us, "
          f"wall/step {ms_per_step * 1e3:.1f} us", file=sys.stderr, flush=True)

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",  # fp16 operands; the accumulation (fp32) is named in the metric
        "data": "synthetic",
        "config": {"workload": w.name, "m": w.m, "n": w.n, "k": w.k, "values": w.dist,
                   "tile": args.tile or g.select_tile(w.m, w.n, w.k)},
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_TFLOPS, 4),
            "traffic": measured_traffic(w.name),
            "kernel_avg_us": round(avg_ms * 1e3, 2),
            "kernel_median_us": round(med_ms * 1e3, 2),
        },
        "cpu_baseline": None,
    }
    if nn:
        rec["metric"] = "fp16 GEMM D = A*B (B [K,N], fp32 out) TFLOP/s; % of MI355X dense fp16 MFMA peak"
        rec["dtype"] = "f16"
    if args.cpu_budget > 0 and not nn:
        print("[bench] CPU baseline (oracle on sampled rows)", file=sys.stderr, flush=True)
        c_host = c.cpu().numpy()
        base, parity = cpu_baseline(a_np, b_np, c_host, w, args.cpu_budget)
        rec["cpu_baseline"] = base
        rec["parity_sample"] = parity
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
