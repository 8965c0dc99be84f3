"""bench.py's JSON line, assembled from the child processes' results: the keys
and types of the benchmark contract, and the statistics over the processes
(no GPU: the results are made up)."""
import argparse
import json

import pytest

import bench
from dense_fp16_gemm_f16_amd import inputs

STEPS, WARMUP = 50, 10
HEADLINE = "gemm_8192_uniform"


def _process(scale, index):
    """One child's results: kernels at 1000 TFLOP/s (the headline at 1550),
    all times multiplied by `scale`."""
    res = {"index": index, "configs": {}}
    for name in bench.CONFIGS:
        us = inputs.WORKLOADS[name].flops / 1e12 / 1000.0 * 1e6 * scale
        res["configs"][name] = {"kernel_us": [us] * 50, "tile": 1,
                                "sustained": {"launches": 1000, "seconds": 1000 * us * 1e-6 * 1.25}}
    us = inputs.WORKLOADS[HEADLINE].flops / 1e12 / 1550.0 * 1e6 * scale
    res["headline"] = {"workload": HEADLINE, "wall_s": STEPS * us * 1e-6 * 1.01, "kernel_us": [us] * STEPS,
                       "tile": 1}
    res["sustained"] = {"launches": 1400, "seconds": 1400 * us * 1e-6 * 1.02}
    res["cold_kernel_us"] = [us * 1.05] * 5
    if index == 0:
        res["cold_start"] = {"wall_s": STEPS * us * 1e-6 * 1.1, "kernel_us": [us * 1.08] * STEPS}
    return res


@pytest.fixture
def record():
    args = argparse.Namespace(workload=HEADLINE, steps=STEPS, warmup=WARMUP)
    return bench.summarize(args, [_process(1.1, 0), _process(1.0, 1), _process(0.9, 2)])


def test_contract_keys_and_types(record):
    assert record["metric"] == bench.METRIC and record["unit"] == "TFLOP/s"
    assert record["n_gpus"] == 1 and record["steps"] == STEPS and record["warmup"] == WARMUP
    assert record["higher_is_better"] is True and record["scaling"] == "weak"
    assert record["vs_baseline"] is None and record["dtype"] == "f16" and record["data"] == "synthetic"
    assert record["config"]["workload"] == HEADLINE and "model" not in record["config"]
    roof = record["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert roof["frac"] == round(roof["achieved"] / 2500.0, 4)
    assert roof["traffic"] is None or roof["traffic"] > 0
    json.loads(json.dumps(record))  # one JSON-serialisable object


def test_value_is_the_median_process(record):
    # the middle process (scale 1.0) ran the K steps at 1550 / 1.01 TFLOP/s
    assert record["value"] == pytest.approx(1550 / 1.01, rel=1e-4)
    assert record["timing"]["processes"] == 3
    assert sorted(record["timing"]["value_per_process"]) == pytest.approx(
        sorted(1550 / 1.01 / s for s in (1.1, 1.0, 0.9)), rel=1e-4)
    assert record["ms_per_step"] == pytest.approx(inputs.WORKLOADS[HEADLINE].flops / 1550e12 * 1.01 * 1e3, rel=1e-4)
    # kernel times by HIP events: the median process's average
    assert record["roofline"]["achieved"] == pytest.approx(1550, rel=1e-4)


def test_sustained_cold_and_configs(record):
    assert record["sustained"]["tflops"] == pytest.approx(1550 / 1.02, rel=1e-3)
    assert record["cold_cache"]["tflops"] == pytest.approx(1550 / 1.05, rel=1e-3)
    assert record["cold_start"]["tflops"] == pytest.approx(1550 / 1.1 / 1.1, rel=1e-3)  # process 0, scale 1.1
    cfgs = {c["workload"]: c for c in record["configs"]}
    assert list(cfgs) == list(bench.CONFIGS)
    for name, c in cfgs.items():
        if name == HEADLINE:
            assert c["sustained_tflops"] == record["sustained"]["tflops"]
            continue
        assert c["tflops"] == pytest.approx(1000, rel=2e-3)
        assert c["frac"] == pytest.approx(0.4, rel=2e-3)
        assert c["sustained_tflops"] == pytest.approx(800, rel=2e-3)


def test_more_than_one_gpu_is_refused_with_a_message():
    import os
    import subprocess
    import sys

    r = subprocess.run([sys.executable, os.path.abspath(bench.__file__), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and r.stdout == ""
    assert "one GPU" in r.stderr


def test_parity_helpers_match_the_tests_bar():
    import numpy as np

    from tests import pins

    rng = np.random.default_rng(3)
    ref = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-6, 4, 2000), [0.0, 6e-8, 65504.0]])
    for k in (256, 1000, 8192):
        assert np.array_equal(bench.ulp_tolerance(ref, k), pins.ulp_tolerance(ref, k))

    w_exact = inputs.WORKLOADS["gemm_256_eighths"]
    ref16 = (rng.integers(-64, 65, 500) / 8).astype(np.float16)
    got16 = ref16.copy()
    assert bench.compare(got16, ref16, w_exact)["ok"]
    got16.view(np.uint16)[7] ^= 1
    r = bench.compare(got16, ref16, w_exact)
    assert not r["ok"] and r["mismatches"] == 1

    w_ulp = inputs.WORKLOADS["gemm_4096_normal"]
    ref16 = rng.standard_normal(500).astype(np.float16)
    tol = bench.ulp_tolerance(ref16.astype(np.float64), w_ulp.k)
    assert bench.compare(ref16.copy(), ref16, w_ulp)["worst_err_over_tol"] == 0.0
    near = (ref16.astype(np.float64) + 0.9 * tol).astype(np.float32)
    assert bench.compare(near, ref16, w_ulp)["ok"]
    far = (ref16.astype(np.float64) + 1.1 * tol).astype(np.float32)
    assert not bench.compare(far, ref16, w_ulp)["ok"]
    bad = ref16.astype(np.float32)
    bad[3] = np.nan
    assert not bench.compare(bad, ref16, w_ulp)["ok"]
