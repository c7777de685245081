"""The benchmark's one-line JSON report, from short runs of bench.py in a child
process: every field the report promises is present and self-consistent."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

from tests.gpu_helpers import announce

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
        "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline")


def run_bench(*args):
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def check_common(d, steps):
    for k in KEYS:
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["data"] == "synthetic" and d["vs_baseline"] is None
    r = d["roofline"]
    assert 0 < r["frac"] < 1 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert r["avg_launch_ms"] > 0
    return r


def test_training_step_report():
    announce("bench.py train --steps 3")
    d = run_bench("--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    r = check_common(d, 3)
    assert d["config"]["workload"] == "gpt2_124m_bf16_b12_h12_t1024" and d["dtype"] == "bf16"
    assert d["unit"] == "TFLOP/s" and r["bound"] == "mfma" and r["peak"] == 2500.0
    assert r["kernel"] == "attn_bwd_main_kernel" and r["flop_per_launch"] == 48_365_568_000
    achieved = r["flop_per_launch"] / (r["avg_launch_ms"] * 1e-3) / 1e12
    assert abs(achieved - r["achieved"]) <= 0.01 * achieved
    total = (19_346_227_200 + 48_365_568_000) / (d["ms_per_step"] * 1e-3) / 1e12
    assert abs(total - d["value"]) <= 0.01 * total
    assert "cpu_baseline" not in d
    # The shader clock the steps ran at, from the probe beside them.
    assert d["sclk_mhz"] is not None and 300.0 < d["sclk_mhz"] < 3000.0, d["sclk_mhz"]
    assert d["config"]["entry_points"] == "plain" and d["config"]["o_lo"] is False
    for part in ("fwd", "bwd"):
        assert d[part]["ms"] > 0 and d[part]["pct_peak"] > 0
    assert 0 < d["fwd"]["min_ms"] <= d["fwd"]["ms"]
    assert 0 < d["bwd"]["main_min_ms"] <= d["bwd"]["main_ms"] == r["avg_launch_ms"]
    # The default rotates over enough copies of the step's data (228 MB each
    # here) to exceed the 256 MB Infinity Cache several times over.
    assert d["config"]["data_sets"] >= 4


def test_training_step_warm_cache_option():
    announce("bench.py train --sets 1 --steps 3")
    d = run_bench("--sets", "1", "--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    check_common(d, 3)
    assert d["config"]["data_sets"] == 1


def test_decode_report():
    announce("bench.py decode --steps 3")
    d = run_bench("--mode", "decode", "--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    r = check_common(d, 3)
    assert d["unit"] == "GB/s" and r["bound"] == "hbm" and r["peak"] == 8000.0
    assert d["config"]["bytes_per_step"] == r["bytes_per_launch"] > 0
    assert d["config"]["data_sets"] >= 4


def test_all_configs_report_errors_against_the_oracle():
    announce("bench.py --all-configs --steps 2")
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--all-configs",
                        "--steps", "2", "--warmup", "1", "--reps", "1", "--settle-ms", "20",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    recs = [json.loads(ln) for ln in r.stdout.splitlines() if ln.startswith("{")]
    import bench
    assert [d["config"]["workload"] for d in recs] == list(bench.ALL_CONFIGS)
    for d in recs:
        tol = (1e-5, None) if d["dtype"] == "f32" else (2e-2, 5e-3)
        for name, e in d["errors_vs_oracle"].items():
            assert e["max_abs"] <= tol[0], (d["config"]["workload"], name, e)
            assert tol[1] is None or e["mean_abs"] <= tol[1], (d["config"]["workload"], name)
