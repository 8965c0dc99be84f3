#!/usr/bin/env python3
"""Throughput of the fp16 GEMM C = fp16(A @ B^T) (fp32 accumulate) on one MI355X.

One step is one GEMM over the whole workload (default: M = N = K = 8192,
A and B i.i.d. uniform[-1,1] rounded to fp16), with A, B and C resident in
HBM before the timed region starts.  Prints one JSON line.

Timing follows the tutorials' protocol (CUDA-event timed, median of three
fresh processes, "4. Pipeline Abstraction and Two Consumer Warp Groups",
section "Performance").  This process never touches the GPU: it draws the
inputs of every workload once, then starts --procs fresh child processes one
after another.  Each child first times each of the five workloads: warm-up
launches back to back for at least --config-warmup seconds (at least 5;
the clock takes milliseconds to settle after the load changes, and 0.1 s
and 0.3 s give the same figures), then 50 event-timed launches, 200 for the
launch-bound 256^3.  Then, for the headline workload, it runs W untimed
warm-up GEMMs and exactly K timed GEMMs between two device
synchronisations, every launch also bracketed by HIP events on the stream
it runs on (the kernel's average duration, for the roofline figure); then
a sustained run of back-to-back GEMMs for at least --sustain seconds, a
cold-cache figure (a 512 MiB buffer written before each launch), and last
each other workload back to back for at least --config-sustain seconds
("sustained_tflops" in `configs`, the wall-clock rate, launch gaps
included).  `value` is the median over the children of the headline's
K-step wall-clock rate; the per-workload figures are medians too.  The headline thus runs on a device at its operating
point; the first child also times the headline's first W + K steps on the
device as it comes from idle ("cold_start"), which on this power-managed
part run about a tenth slower while the clock ramps.

Afterwards this process times the oracle (plain fp64 triple loop, one fp16
rounding) on a bounded sample of the headline workload -- whole rows of C --
as the CPU baseline, and compares the first child's outputs of every
workload with the oracle: the same rows for the headline, all of C for the
others.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import subprocess
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fp16 GEMM TFLOP/s (fp32 acc) at 8192³; % of MI355X dense fp16 MFMA peak"
PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, published
PROFILE_DIR = os.path.join(ROOT, "profiles")
# the five measured workloads: M=N=K=256 {-8..8}/8, 4096^3 N(0,1), 8192^3
# uniform[-1,1], 16384x4096x2048 N(0,0.5), 5000x3000x1000 {-8..8}/8
CONFIGS = ("gemm_256_eighths", "gemm_4096_normal", "gemm_8192_uniform",
           "gemm_16384x4096x2048_normal05", "gemm_5000x3000x1000_eighths")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def ulp_tolerance(ref, k: int):
    """2 fp16 ulp of |C_oracle| + 1e-2 sqrt(K) 2^-11, ulp(x) = 2^(max(floor(log2|x|), -14) - 10)."""
    import numpy as np

    ar = np.abs(ref)
    e = np.where(ar > 0, np.maximum(np.floor(np.log2(np.where(ar > 0, ar, 1.0))), -14), -14)
    return 2.0 * np.exp2(e - 10) + 1e-2 * np.sqrt(k) * 2.0**-11


def compare(got, ref, w) -> dict:
    """Worst |err| / tolerance over the compared elements: bit-exact expected on
    {-8..8}/8 inputs (the exact sum is unique), else the ulp bound."""
    import numpy as np

    if w.dist == "eighths":
        bad = int(np.count_nonzero(got.view(np.uint16) != ref.view(np.uint16)))
        return {"elements": int(ref.size), "bit_exact": bad == 0, "mismatches": bad, "ok": bad == 0}
    g64, r64 = got.astype(np.float64), ref.astype(np.float64)
    err = np.abs(g64 - r64)
    err = np.where(np.isnan(err), np.inf, err)
    worst = float(np.max(err / ulp_tolerance(r64, w.k))) if err.size else 0.0
    return {"elements": int(ref.size), "worst_err_over_tol": round(worst, 4), "ok": worst <= 1.0}


# ---- child: one fresh process on the GPU --------------------------------------------

def child(args) -> int:
    import numpy as np
    import torch

    import dense_fp16_gemm_f16_amd as g
    from dense_fp16_gemm_f16_amd import inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    out = {"index": args.index, "configs": {}}

    def setup(name):
        w = inputs.WORKLOADS[name]
        a = torch.from_numpy(np.load(os.path.join(args.child, f"{name}_a.npy"))).to(dev)
        b = torch.from_numpy(np.load(os.path.join(args.child, f"{name}_b.npy"))).to(dev)
        nn = w.b_layout == "kn"
        c = torch.empty((w.m, w.n), dtype=torch.float32 if nn else torch.float16, device=dev)
        call = g.gemm_f16_nn_f32_raw if nn else g.gemm_f16_nt_raw
        ptrs = (a.data_ptr(), b.data_ptr(), c.data_ptr())

        def step():
            rc = call(w.m, w.n, w.k, *ptrs, sp, args.tile, args.swizzle, args.xcd)
            if rc != g.OK:
                raise g.GemmError(rc)
        return w, (a, b, c), step

    def event_timed(step, reps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for s, e in ev:
            s.record(stream)
            step()
            e.record(stream)
        torch.cuda.synchronize()
        return [s.elapsed_time(e) * 1e3 for s, e in ev]  # us

    def headline_steps():
        """W warm-up steps, then exactly K timed steps between two synchronisations."""
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
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
        return wall, [s.elapsed_time(e) * 1e3 for s, e in zip(starts, ends)]

    # every workload resident first, so no host work idles the device between
    # the measurements below
    order = [c for c in CONFIGS if c != args.workload] + [args.workload]
    setups = {name: setup(name) for name in order}
    w, bufs, step = setups[args.workload]

    # the first process, before anything else: the headline on a device that
    # was idle (its clock still ramping), for reference
    if args.index == 0:
        wall, durs = headline_steps()
        out["cold_start"] = {"wall_s": wall, "kernel_us": durs}

    # every workload: warm-up launches back to back for at least
    # --config-warmup seconds (at least 5), then 50 (256^3: 200) event-timed
    # ones; the headline workload last
    for name in order:
        cw, cbufs, cstep = setups[name]
        for _ in range(5):
            cstep()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(5):
            cstep()
        torch.cuda.synchronize()
        per_launch = (time.perf_counter() - t0) / 5
        for _ in range(int(args.config_warmup / per_launch)):
            cstep()
        out["configs"][name] = {"kernel_us": event_timed(cstep, 200 if cw.m * cw.n * cw.k < 2**26 else 50),
                                "tile": args.tile or g.select_tile(cw.m, cw.n, cw.k)}
    log(f"child {args.index}: five workloads timed")

    # the headline, right after, on a device at its operating point
    wall, durs = headline_steps()
    out["headline"] = {"workload": w.name, "wall_s": wall, "kernel_us": durs,
                       "tile": args.tile or g.select_tile(w.m, w.n, w.k)}
    log(f"child {args.index}: {w.name} {args.steps} steps, wall/step {wall / args.steps * 1e6:.1f} us, "
        f"kernel avg {statistics.mean(durs):.1f} us")

    # sustained: back-to-back GEMMs for at least --sustain seconds
    if args.sustain > 0:
        n = max(1, int(args.sustain / (wall / args.steps)) + 1)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            step()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        out["sustained"] = {"launches": n, "seconds": dt}
        log(f"child {args.index}: sustained {n} launches in {dt:.2f} s")

    # cold cache: a 512 MiB buffer written before each event-timed launch
    flush = torch.empty(512 * 2**20 // 4, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(5):
        flush.fill_(1.0)
        cold += event_timed(step, 1)
    out["cold_kernel_us"] = cold
    del flush

    # every other workload sustained too: back-to-back launches for at least
    # --config-sustain seconds each, after the headline's figures so that they
    # do not change the state the headline runs in
    if args.config_sustain > 0:
        for name in order:
            if name == args.workload:
                continue
            cw, cbufs, cstep = setups[name]
            us = statistics.median(out["configs"][name]["kernel_us"])
            n = max(1, int(args.config_sustain / (us * 1e-6)) + 1)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(n):
                cstep()
            torch.cuda.synchronize()
            out["configs"][name]["sustained"] = {"launches": n, "seconds": time.perf_counter() - t0}
        log(f"child {args.index}: other workloads sustained")

    # outputs for the parity check (first child), from a launch of its own
    if args.index == 0:
        for name in order:
            cw, cbufs, cstep = setups[name]
            cstep()
            torch.cuda.synchronize()
            np.save(os.path.join(args.child, f"{name}_c.npy"), cbufs[2].cpu().numpy())
    del setups, bufs, step
    with open(os.path.join(args.child, f"result_{args.index}.json"), "w") as f:
        json.dump(out, f)
    return 0


def profile_run(args) -> int:
    """W warm-up steps and K event-timed steps of one workload in this process,
    so that a profiler wrapped around it sees exactly those W + K launches."""
    import numpy as np
    import torch

    import dense_fp16_gemm_f16_amd as g
    from dense_fp16_gemm_f16_amd import inputs

    w = inputs.WORKLOADS[args.workload]
    a_np, b_np = inputs.workload_inputs(w.name)
    dev = torch.device("cuda:0")
    a = torch.from_numpy(a_np).to(dev)
    b = torch.from_numpy(b_np).to(dev)
    nn = w.b_layout == "kn"
    c = torch.empty((w.m, w.n), dtype=torch.float32 if nn else torch.float16, device=dev)
    stream = torch.cuda.current_stream(dev)
    call = g.gemm_f16_nn_f32_raw if nn else g.gemm_f16_nt_raw
    for i in range(args.warmup + args.steps):
        if i == args.warmup:
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        rc = call(w.m, w.n, w.k, a.data_ptr(), b.data_ptr(), c.data_ptr(), stream.cuda_stream,
                  args.tile, args.swizzle, args.xcd)
        if rc != g.OK:
            raise g.GemmError(rc)
    e1 = torch.cuda.Event(enable_timing=True)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / max(args.steps, 1)
    print(json.dumps({"workload": w.name, "steps": args.steps, "warmup": args.warmup, "us_per_step": round(us, 2),
                      "tflops": round(w.flops / (us * 1e-6) / 1e12, 1)}), flush=True)
    return 0


# ---- parent: inputs, children, oracle ------------------------------------------------

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
    oracle.gemm_f16_nt_rows(a, b, list(range(min(threads, w.m))), threads)
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
        "cpu_model": cpu_model(),
        "sample": f"{len(rows)} of {w.m} rows of C (all {w.n} columns, full K={w.k}), "
                  f"fp64 triple loop, {dt:.1f} s",
    }
    parity = compare(c_gpu[rows], ref, w)
    parity["rows"] = int(len(rows))
    return rec, parity


def summarize(args, results: list) -> dict:
    """The JSON record from the children's results (everything but the CPU
    baseline and the parity checks, which need the inputs and outputs)."""
    from dense_fp16_gemm_f16_amd import inputs

    w = inputs.WORKLOADS[args.workload]
    nn = w.b_layout == "kn"
    flops = float(w.flops)
    per_proc = []
    for r in results:
        h = r["headline"]
        per_proc.append({"value": flops * args.steps / h["wall_s"] / 1e12,
                         "ms_per_step": h["wall_s"] * 1e3 / args.steps,
                         "kernel_avg_us": statistics.mean(h["kernel_us"]),
                         "kernel_median_us": statistics.median(h["kernel_us"])})
    mid = sorted(range(len(per_proc)), key=lambda i: per_proc[i]["value"])[len(per_proc) // 2]
    med = per_proc[mid]
    avg_us = statistics.median(p["kernel_avg_us"] for p in per_proc)
    achieved = flops / (avg_us * 1e-6) / 1e12
    log(f"headline per process: " + ", ".join(f"{p['value']:.1f}" for p in per_proc) + " TFLOP/s")

    rec = {
        "metric": METRIC,
        "value": round(med["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",  # fp16 operands; the accumulation (fp32) is named in the metric
        "data": "synthetic",
        "config": {"workload": w.name, "m": w.m, "n": w.n, "k": w.k, "values": w.dist,
                   "tile": results[mid]["headline"]["tile"]},
        "timing": {"processes": len(per_proc),
                   "value_per_process": [round(p["value"], 2) for p in per_proc],
                   "statistic": "median over fresh processes of the K-step wall-clock rate"},
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_TFLOPS, 4),
            "traffic": measured_traffic(w.name),
            "kernel_avg_us": round(avg_us, 2),
            "kernel_median_us": round(statistics.median(p["kernel_median_us"] for p in per_proc), 2),
        },
        "cpu_baseline": None,
    }
    if all("sustained" in r for r in results):
        rates = [flops * r["sustained"]["launches"] / r["sustained"]["seconds"] / 1e12 for r in results]
        rec["sustained"] = {"tflops": round(statistics.median(rates), 2),
                            "tflops_per_process": [round(x, 2) for x in rates],
                            "seconds": round(statistics.median(r["sustained"]["seconds"] for r in results), 3),
                            "launches": results[0]["sustained"]["launches"]}
    cs = results[0].get("cold_start")
    if cs:
        rec["cold_start"] = {"tflops": round(flops * args.steps / cs["wall_s"] / 1e12, 2),
                             "kernel_avg_us": round(statistics.mean(cs["kernel_us"]), 2),
                             "what": f"the first process's first {args.warmup} + {args.steps} steps, "
                                     "on a device that was idle"}
    cold = statistics.median(statistics.median(r["cold_kernel_us"]) for r in results)
    rec["cold_cache"] = {"kernel_median_us": round(cold, 2), "tflops": round(flops / (cold * 1e-6) / 1e12, 2),
                         "flush": "512 MiB written before each launch"}
    cfgs = []
    for name in CONFIGS:
        cw = inputs.WORKLOADS[name]
        per = [statistics.median(r["configs"][name]["kernel_us"]) for r in results]
        us = statistics.median(per)
        tf = cw.flops / (us * 1e-6) / 1e12
        cfg = {"workload": name, "m": cw.m, "n": cw.n, "k": cw.k, "values": cw.dist,
               "tile": results[0]["configs"][name]["tile"], "kernel_median_us": round(us, 2),
               "tflops": round(tf, 1), "frac": round(tf / PEAK_TFLOPS, 4),
               "traffic": measured_traffic(name), "warmup_s": getattr(args, "config_warmup", None)}
        if name == w.name and "sustained" in rec:
            cfg["sustained_tflops"] = rec["sustained"]["tflops"]
        elif all("sustained" in r["configs"][name] for r in results):
            cfg["sustained_tflops"] = round(statistics.median(
                cw.flops * r["configs"][name]["sustained"]["launches"]
                / r["configs"][name]["sustained"]["seconds"] / 1e12 for r in results), 1)
        cfgs.append(cfg)
    rec["configs"] = cfgs
    if nn:
        rec["metric"] = "fp16 GEMM D = A*B (B [K,N], fp32 out) TFLOP/s; % of MI355X dense fp16 MFMA peak"
    return rec


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gemm_8192_uniform")
    ap.add_argument("--tile", type=int, default=0)
    ap.add_argument("--swizzle", type=int, default=0)
    ap.add_argument("--xcd", type=int, default=-1)
    ap.add_argument("--procs", type=int, default=3, help="fresh processes timed (median reported)")
    ap.add_argument("--sustain", type=float, default=1.0,
                    help="seconds of back-to-back headline GEMMs per process (0 = skip)")
    ap.add_argument("--config-sustain", type=float, default=1.0,
                    help="seconds of back-to-back launches of each other workload (0: skip)")
    ap.add_argument("--config-warmup", type=float, default=0.1,
                    help="seconds of back-to-back warm-up launches before each workload's event-timed ones")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip it and the parity checks)")
    ap.add_argument("--traffic-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain elementwise copy (negation) of BYTES, 3 times: the "
                         "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--profile", action="store_true",
                    help="for a profiler: this process alone runs the workload's W + K steps and nothing else "
                         "(no children, no other workloads, no CPU baseline)")
    ap.add_argument("--child", default=None, help=argparse.SUPPRESS)
    ap.add_argument("--index", type=int, default=0, help=argparse.SUPPRESS)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this GEMM has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2
    if args.child:
        return child(args)
    if args.profile:
        return profile_run(args)

    if args.traffic_calibration:
        import torch

        n = args.traffic_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)  # one elementwise kernel: reads and writes BYTES
        torch.cuda.synchronize()
        print(json.dumps({"traffic_calibration_bytes": n * 4}), flush=True)
        return 0

    import numpy as np

    from dense_fp16_gemm_f16_amd import inputs

    names = [args.workload] + [c for c in CONFIGS if c != args.workload]
    with tempfile.TemporaryDirectory(prefix="gemm_bench_") as tmp:
        log(f"generating inputs of {len(names)} workloads")
        data = {}
        for name in names:
            a, b = inputs.workload_inputs(name)
            np.save(os.path.join(tmp, f"{name}_a.npy"), a)
            np.save(os.path.join(tmp, f"{name}_b.npy"), b)
            data[name] = (a, b)
        results = []
        for i in range(args.procs):
            log(f"child {i}: starting a fresh process")
            cmd = [sys.executable, os.path.abspath(__file__), "--child", tmp, "--index", str(i),
                   "--steps", str(args.steps), "--warmup", str(args.warmup), "--workload", args.workload,
                   "--tile", str(args.tile), "--swizzle", str(args.swizzle), "--xcd", str(args.xcd),
                   "--sustain", str(args.sustain), "--config-sustain", str(args.config_sustain),
                   "--config-warmup", str(args.config_warmup)]
            rc = subprocess.run(cmd).returncode
            if rc != 0:
                log(f"child {i} failed with status {rc}")
                return rc if rc > 0 else 1
            with open(os.path.join(tmp, f"result_{i}.json")) as f:
                results.append(json.load(f))

        rec = summarize(args, results)
        w = inputs.WORKLOADS[args.workload]
        nn = w.b_layout == "kn"
        cfgs = rec["configs"]

        if args.cpu_budget > 0 and not nn:
            import oracle

            log("CPU baseline (oracle on sampled rows of the headline workload)")
            a, b = data[w.name]
            c_head = np.load(os.path.join(tmp, f"{w.name}_c.npy"))
            base, parity = cpu_baseline(a, b, c_head, w, args.cpu_budget)
            rec["cpu_baseline"] = base
            rec["parity_sample"] = parity
            for cfg in cfgs:
                if cfg["workload"] == w.name:
                    cfg["parity"] = parity
                    continue
                log(f"parity: {cfg['workload']} against the oracle, all of C")
                cw = inputs.WORKLOADS[cfg["workload"]]
                ca, cb = data[cfg["workload"]]
                got = np.load(os.path.join(tmp, f"{cfg['workload']}_c.npy"))
                cfg["parity"] = compare(got, oracle.gemm_f16_nt(ca, cb), cw)
            rec["parity_ok"] = all(c["parity"]["ok"] for c in cfgs)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
