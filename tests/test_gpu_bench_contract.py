"""bench.py on the GPU: one short run prints one JSON line with the fields
the benchmark contract asks for, the roofline of the dominant kernel
(algorithmic bytes over its measured time, against 8 TB/s) and the
measured HBM traffic of the committed counter summary."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.gpu


def test_bench_prints_one_contract_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "1", "--no-cpu-baseline", "--no-long", "--no-next",
                        "--no-rope", "--no-prefill"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["value"] > 0
    assert "workload" in d["config"]
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["peak"] == 8000.0 and rf["unit"] == "GB/s"
    assert 0 < rf["frac"] < 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    # achieved = algorithmic bytes of one call over its measured duration
    assert abs(rf["achieved"] - rf["algorithmic_bytes"] / (rf["us_per_call"] * 1e-6) / 1e9) \
        < 0.01 * rf["achieved"]
    assert rf["traffic"] is not None and rf["traffic"] > rf["algorithmic_bytes"]
