"""The benchmark's output contract, on the smallest workload: one JSON line with the step's
metric, the roofline object of its dominant stage and the oracle's CPU baseline.  Runs
bench.py in a child process (the same way it is run on its own) with a short step count."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

from gpu_util import device, note

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line_on_the_tiny_workload():
    device()
    note("bench.py --workload tiny --steps 3 --warmup 1 --no-per-config (child process)")
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", "tiny",
                        "--steps", "3", "--warmup", "1", "--no-per-config",
                        "--cpu-swish-len", "65536"],
                       capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "stages"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "% of roofline" and 0 < d["value"] <= 100
    assert d["config"]["M"] == 256 and d["config"]["K"] == 64 and d["config"]["N"] == 128
    roof = d["roofline"]
    assert roof["bound"] in ("hbm", "mfma") and roof["unit"] in ("GB/s", "TFLOP/s")
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert 0 < roof["frac"] <= 1
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0
    for name in ("b", "w", "x", "swish_grad_fp32", "swish_grad_fp16", "swish_grad_bf16"):
        st = d["stages"][name]
        assert st["us"] > 0 and 0 < st["frac"] <= 1, (name, st)
        # the kernel span lies inside the events recorded around the call
        assert st["us"] <= st["event_us"] + 5.0, (name, st)
    assert abs(roof["avg_launch_us"] - d["stages"][roof["stage"]]["us"]) < 0.01
    for name in ("b", "w", "x"):   # the fp16 stages timed beside the step
        st = d["fp16"][name]
        assert st["us"] > 0 and 0 < st["frac"] <= 1, (name, st)
