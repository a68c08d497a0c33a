"""bench.py's JSON line on the GPU: a short run of the small workload must
print one line with the fields the benchmark contract names, a roofline
object for the dominant kernel and a positive rate."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    print(f"[case] bench.py {' '.join(args)}", flush=True)
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                         capture_output=True, text=True, cwd=ROOT, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = [ln for ln in out.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, out.stdout
    return json.loads(lines[0])


def test_bench_line_fields():
    sys.path.insert(0, ROOT)
    import bench
    rec = run_bench("--workload", "laplace_2048x1024", "--steps", "8", "--warmup", "4",
                    "--no-cpu-baseline")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline"):
        assert key in rec, key
    assert rec["metric"] == bench.METRIC and rec["unit"] == "GB/s"
    assert rec["n_gpus"] == 1 and rec["steps"] == 8 and rec["warmup"] == 4
    assert rec["value"] > 0 and rec["ms_per_step"] > 0
    assert rec["higher_is_better"] is True and rec["data"] == "synthetic"
    assert rec["config"]["workload"] == "laplace_2048x1024" and rec["config"]["block"] == 128
    # value is bf16 input bytes over the step time
    n = 2048 * 1024
    assert rec["value"] == pytest.approx(2.0 * n / (rec["ms_per_step"] * 1e-3) / 1e9, rel=1e-2)
    roof = rec["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert 0 < roof["frac"] < 1 and roof["frac"] == pytest.approx(roof["achieved"] / 8000.0,
                                                                  rel=1e-3)
    assert "cpu_baseline" not in rec
    rep = rec["repeats"]
    assert rep["n"] == 20
    assert rep["ms_per_step_min"] <= rep["ms_per_step_median"] <= rep["ms_per_step_max"]


def test_default_line_times_the_largest_workload_exactly():
    """With no workload named, the line is the four-payload X[32768,12288]
    workload at B = 256, with exactly the K timed and W warmup steps asked
    for, and the accumulate kernel (the slower one) as its roofline."""
    rec = run_bench("--steps", "3", "--warmup", "2", "--no-cpu-baseline", "--no-configs")
    cfg = rec["config"]
    assert cfg["workload"] == "gpt175b_hidden_32768x12288" and cfg["block"] == 256
    assert cfg["tokens"] == 32768 and cfg["hidden"] == 12288
    assert rec["steps"] == 3 and rec["warmup"] == 2
    assert rec["roofline"]["kernel"] == "accumulate"
    n = 32768 * 12288
    # value: the four payloads' bf16 input bytes over the step time
    assert rec["value"] == pytest.approx(4 * 2.0 * n / (rec["ms_per_step"] * 1e-3) / 1e9,
                                         rel=1e-2)
    assert 0 < rec["roofline"]["frac"] < 1
    assert "configs" not in rec
