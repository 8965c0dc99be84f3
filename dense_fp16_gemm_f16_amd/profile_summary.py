"""Summaries of rocprofv3 CSV output for the GEMM kernel.

    python -m dense_fp16_gemm_f16_amd.profile_summary stats DIR [--kernel gemm_f16_nt_kernel]
    python -m dense_fp16_gemm_f16_amd.profile_summary window DIR --kernel NAME [--min-us X] --skip N --count K
    python -m dense_fp16_gemm_f16_amd.profile_summary counters DIR --kernel NAME
    python -m dense_fp16_gemm_f16_amd.profile_summary traffic \\
        --gemm-fetch DIR --gemm-write DIR --copy-fetch DIR --copy-write DIR \\
        --copy-bytes N --workload NAME --out profiles/traffic_NAME.json

`stats` reads <DIR>/*_kernel_stats.csv (rocprofv3 --kernel-trace --stats
--output-format csv); `window` the kernel trace's launches by position;
`counters` the per-dispatch values of every counter in
<DIR>/*_counter_collection.csv, with the MFMA-busy share when
SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE are among them (busy cycles
summed over the 1024 SIMDs, over GPU-busy cycles summed over the 8 XCDs).  `traffic` reads <DIR>/*_counter_collection.csv of
--pmc FETCH_SIZE / --pmc WRITE_SIZE runs (values in KiB per dispatch), scales
each by the ratio of a plain copy's known bytes to what the same counter
reported for it, and writes HBM bytes per GEMM launch together with a hash
of the kernel source, so that stale counters are never reported for a
changed kernel.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def code_text(src: str) -> str:
    """The source with its comments removed and each run of white space made
    one blank: edits to comments or layout leave it unchanged.  (The sources
    hashed here have no string or character literal that holds // or /*.)"""
    return " ".join(_COMMENT.sub(" ", src).split())


def kernel_source_hash() -> str:
    """Hash of the code of every source the library is built from (the host
    side, the kernel templates, the scheduler and the per-tile units),
    comments and layout aside."""
    h = hashlib.sha256()
    names = ["gemm_f16.hip", "kernels.h", "tile_sched.h"] + sorted(
        os.path.basename(p) for p in glob.glob(os.path.join(CSRC, "tile_*.hip")) + glob.glob(os.path.join(CSRC, "ring_*.hip")))
    for name in names:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def _csv_rows(path: str) -> list:
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _one(pattern: str) -> str:
    """The one file matching `pattern`; a folder that holds several runs is
    ambiguous and raises rather than reading whichever sorts first."""
    files = sorted(glob.glob(pattern, recursive=True))
    if not files:
        raise FileNotFoundError(pattern)
    if len(files) > 1:
        raise ValueError(f"{len(files)} files match {pattern}: {files[:4]}; give one run's folder")
    return files[0]


def kernel_stats(d: str, kernel: str) -> dict:
    path = _one(os.path.join(d, "**", "*kernel_stats.csv"))
    for r in _csv_rows(path):
        if kernel in r["Name"]:
            return {"name": r["Name"], "calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                    "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3}
    raise KeyError(kernel)


def kernel_window(d: str, kernel: str, min_us: float, skip: int, count: int) -> dict:
    """Durations of the launches of `kernel` lasting at least min_us, in dispatch
    order, after the first `skip` of them: `count` launches."""
    path = _one(os.path.join(d, "**", "*kernel_trace.csv"))
    rows = [r for r in _csv_rows(path) if kernel in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    durs = [x for x in durs if x >= min_us]
    sel = durs[skip:skip + count]
    if len(sel) != count:
        raise ValueError(f"only {len(sel)} of {count} launches after skipping {skip}")
    return {"kernel": kernel, "launches": count, "avg_us": statistics.mean(sel), "median_us": statistics.median(sel),
            "min_us": min(sel), "max_us": max(sel)}


def counter_per_dispatch(d: str, kernel: str, counter: str) -> list[float]:
    path = _one(os.path.join(d, "**", "*counter_collection.csv"))
    per = {}
    for r in _csv_rows(path):
        if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
            per[int(r["Dispatch_Id"])] = per.get(int(r["Dispatch_Id"]), 0.0) + float(r["Counter_Value"])
    return [per[k] for k in sorted(per)]


def counters(d: str, kernel: str) -> dict:
    """Every counter of a --pmc run, per dispatch of `kernel`."""
    path = _one(os.path.join(d, "**", "*counter_collection.csv"))
    names = sorted({r["Counter_Name"] for r in _csv_rows(path) if kernel in r["Kernel_Name"]})
    out = {c: counter_per_dispatch(d, kernel, c) for c in names}
    if "SQ_VALU_MFMA_BUSY_CYCLES" in out and "GRBM_GUI_ACTIVE" in out:
        out["mfma_busy_share"] = [round(b / 1024.0 / (g / 8.0), 4) for b, g in
                                  zip(out["SQ_VALU_MFMA_BUSY_CYCLES"], out["GRBM_GUI_ACTIVE"])]
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s1 = sub.add_parser("stats")
    s1.add_argument("dir")
    s1.add_argument("--kernel", default="gemm_f16_nt_kernel")
    s3 = sub.add_parser("window", help="launches of one kernel from a kernel trace, selected by position")
    s3.add_argument("dir")
    s3.add_argument("--kernel", required=True)
    s3.add_argument("--min-us", type=float, default=0.0, help="only launches at least this long")
    s3.add_argument("--skip", type=int, default=0, help="matching launches to skip first")
    s3.add_argument("--count", type=int, required=True, help="matching launches to take after them")
    s4 = sub.add_parser("counters", help="per-dispatch counter values of a --pmc run")
    s4.add_argument("dir")
    s4.add_argument("--kernel", default="gemm_f16")
    s2 = sub.add_parser("traffic")
    for k in ("gemm-fetch", "gemm-write", "copy-fetch", "copy-write", "workload", "out"):
        s2.add_argument("--" + k, required=True)
    s2.add_argument("--copy-bytes", type=int, required=True)
    s2.add_argument("--kernel", default="gemm_f16_nt_kernel")
    s2.add_argument("--copy-kernel", default="copy")
    s2.add_argument("--command", default="")
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print(json.dumps(kernel_stats(a.dir, a.kernel)))
        return 0
    if a.cmd == "window":
        print(json.dumps(kernel_window(a.dir, a.kernel, a.min_us, a.skip, a.count)))
        return 0
    if a.cmd == "counters":
        print(json.dumps(counters(a.dir, a.kernel)))
        return 0
    fetch = counter_per_dispatch(a.gemm_fetch, a.kernel, "FETCH_SIZE")
    write = counter_per_dispatch(a.gemm_write, a.kernel, "WRITE_SIZE")
    cf = counter_per_dispatch(a.copy_fetch, a.copy_kernel, "FETCH_SIZE")
    cw = counter_per_dispatch(a.copy_write, a.copy_kernel, "WRITE_SIZE")
    f_scale = a.copy_bytes / (statistics.median(cf) * 1024.0)
    w_scale = a.copy_bytes / (statistics.median(cw) * 1024.0)
    fetch_b = statistics.median(fetch) * 1024.0 * f_scale
    write_b = statistics.median(write) * 1024.0 * w_scale
    rec = {
        "workload": a.workload,
        "kernel_source_sha256_16": kernel_source_hash(),
        "fetch_kib_per_dispatch": fetch,
        "write_kib_per_dispatch": write,
        "copy_bytes": a.copy_bytes,
        "copy_fetch_kib": cf,
        "copy_write_kib": cw,
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "hbm_fetch_bytes_per_launch": fetch_b,
        "hbm_write_bytes_per_launch": write_b,
        "hbm_bytes_per_launch": fetch_b + write_b,
        "command": a.command,
    }
    with open(a.out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())
