"""The profiling helpers' host logic: the source hash that ties recorded
traffic to the kernel code, and the trace-window selection."""
import csv
import os

import pytest

from dense_fp16_gemm_f16_amd import profile_summary as ps


def test_code_text_drops_comments_and_layout():
    a = "int x = 1; // one\n/* block\n comment */ int  y=2;\n"
    b = "int x = 1;\n\n\n   int  y=2; /* other words */"
    assert ps.code_text(a) == ps.code_text(b) == "int x = 1; int y=2;"
    assert ps.code_text("a/b; c*d;") == "a/b; c*d;"
    assert ps.code_text("x = 1;") != ps.code_text("x = 2;")


def _write_tree(d, kernels_h):
    os.makedirs(d, exist_ok=True)
    for name, text in {"gemm_f16.hip": "int host;\n", "kernels.h": kernels_h, "tile_sched.h": "int s;\n",
                       "tile_256x256.hip": "int t;\n", "ring_256x256.hip": "int r;\n"}.items():
        with open(os.path.join(d, name), "w") as f:
            f.write(text)


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    d = str(tmp_path)
    _write_tree(d, "int k = 1; // a comment\n")
    monkeypatch.setattr(ps, "CSRC", d)
    h0 = ps.kernel_source_hash()
    _write_tree(d, "/* reworded */\nint k = 1;\n")
    assert ps.kernel_source_hash() == h0
    _write_tree(d, "int k = 2;\n")
    assert ps.kernel_source_hash() != h0


def test_source_hash_of_the_library_is_recorded_in_the_traffic_files():
    import json
    import glob
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    files = glob.glob(os.path.join(root, "profiles", "traffic_*.json"))
    assert files
    for p in files:
        with open(p) as f:
            rec = json.load(f)
        assert len(rec["kernel_source_sha256_16"]) == 16
        assert rec["hbm_bytes_per_launch"] > 0


def test_window_picks_launches_by_position(tmp_path):
    path = tmp_path / "run_kernel_trace.csv"
    rows = []
    t = 1000
    for i, dur in enumerate([5, 500, 7, 600, 700, 800, 900]):
        rows.append({"Kernel_Name": "gemm_f16_x" if dur != 7 else "other", "Start_Timestamp": t,
                     "End_Timestamp": t + dur * 1000})
        t += dur * 1000 + 10
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)
    r = ps.kernel_window(str(tmp_path), "gemm_f16", 400, 1, 2)
    assert r["launches"] == 2 and r["min_us"] == 600 and r["max_us"] == 700


def test_a_folder_with_two_runs_is_refused(tmp_path):
    for pid in (1, 2):
        (tmp_path / f"run_{pid}_kernel_trace.csv").write_text("Kernel_Name,Start_Timestamp,End_Timestamp\n")
    with pytest.raises(ValueError, match="2 files match"):
        ps.kernel_window(str(tmp_path), "gemm_f16", 0, 0, 1)
