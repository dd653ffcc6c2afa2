"""The benchmark script's contract: one GPU only, and the JSON line it prints
(exact step counts, the roofline and context objects)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(*args, timeout=600):
    return subprocess.run([sys.executable, BENCH, *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=timeout)


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_more_than_one_gpu_is_refused(gpus):
    r = _run("--gpus", gpus, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_json_line_contract():
    """Small run: 3 timed steps after 2 warm-up steps, in graphs of 2 steps (so
    the last timed graph holds one step)."""
    r = _run("--steps", "3", "--warmup", "2", "--steps-per-graph", "2", "--no-extra",
             "--no-detail", "--no-cpu-baseline")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    out = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline"):
        assert key in out, key
    assert out["n_gpus"] == 1 and out["steps"] == 3 and out["warmup"] == 2
    assert out["value"] > 0 and out["ms_per_step"] > 0 and out["higher_is_better"] is True
    assert out["config"]["launch"].startswith("hipGraphs of up to 2 steps")
    rf = out["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0 < rf["frac"] < 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    # per launch: the step's device time over the 8 launches of a step
    assert abs(rf["avg_launch_us"] * 8 - rf["step_device_us"]) < 0.01 * rf["step_device_us"] + 0.01
