"""The bench's one-line JSON record on the GPU: the fields, units and
roofline object it promises, from a short run of the default workload."""

import json
import os
import subprocess
import sys

import pytest

from helpers import gpu_or_skip, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_default_bench_line():
    gpu_or_skip()
    say("bench line")
    r = subprocess.run([sys.executable, "bench.py", "--steps", "5", "--warmup", "2", "--no-cpu-baseline"],
                       cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["scaling"] in ("weak", "strong")
    assert d["vs_baseline"] is None and d["data"].startswith("synthetic")
    assert d["config"]["workload"] == "llama3_8b_decode_b64_L128-2048"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    # the step moves the algorithmic bytes in ms_per_step: value x time = bytes
    step_bytes = d["decode_attention"]["step_bytes"]
    assert abs(d["value"] * 1e9 * d["ms_per_step"] * 1e-3 - step_bytes) <= 0.01 * step_bytes
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0 < rf["achieved"] < rf["peak"] and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["traffic"] is None or rf["traffic"] > rf["algorithmic_bytes_per_launch"] * 0.9
