"""bench.py's output contract.

CPU: more than one GPU is refused with a message before any device work;
the oracle baseline leg reports env-steps/s with its core count and sample.
GPU: a short run prints one JSON line carrying the fields the measurement
needs (metric, value, unit, steps, roofline with HBM traffic, CPU baseline).
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, BENCH, "--gpus", "2"], cwd=ROOT, capture_output=True,
                         text=True, timeout=120)
    assert out.returncode == 2
    assert "one GPU" in out.stderr and out.stdout == ""


def test_cpu_baseline_leg_reports_its_sample():
    import bench
    from linear_recurrence_scan_row_amd import workloads

    cfg = dict(workloads.CONFIGS["gae_8x16"])
    host = workloads.make("gae_8x16")
    r = bench.run_cpu_baseline("gae_8x16", cfg, host, 0.2)
    assert r["kind"] == "oracle" and r["unit"] == "env-steps/s" and r["cores"] == 1
    assert r["value"] > 0 and "8x16" in r["sample"]
    r2 = bench.run_cpu_baseline("gae_8x16", cfg, host, 0.2, workers=2)
    assert r2["cores"] == 2 and r2["value"] > 0
    # with the step's bytes, the byte model's GB/s: passes per second times bytes per pass
    r3 = bench.run_cpu_baseline("gae_8x16", cfg, host, 0.2, step_bytes=2848)
    assert r3["gbs"] == pytest.approx(r3["value"] / (8 * 16) * 2848 / 1e9, rel=1e-3, abs=1e-3)


@pytest.mark.gpu
def test_bench_prints_one_json_line(gpu_device):
    out = subprocess.run([sys.executable, BENCH, "--steps", "20", "--warmup", "2",
                          "--cpu-seconds", "0.5"], cwd=ROOT, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr[-3000:]
    lines = [l for l in out.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, out.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 2
    assert d["unit"] == "GB/s" and d["value"] > 0 and d["dtype"] == "f32"
    assert d["config"]["workload"] == "gae_td_4096x128"
    assert d["copy_ceiling"]["value_over_copy"] > 0
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-4)
    assert r["traffic"] is None or r["traffic"] > 0
    assert r["frac_event"] == pytest.approx(r["achieved_event"] / r["peak"], abs=1e-4)
    assert r["source"]
    # the streaming floor of the same step, and the metric's own call
    assert d["floor"]["us"] > 0 and 0 < d["floor"]["value_over_floor"]
    g = d["roofline_gae_call"]
    assert g["frac"] == pytest.approx(g["achieved"] / r["peak"], abs=1e-4)
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0 and c["gbs"] > 0
    assert d["host_cores"]["affinity"] >= 1 and d["host_cores"]["nproc"] >= 1
