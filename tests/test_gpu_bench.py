"""bench.py end to end on the GPU, on the tiny workload: one JSON line with
every field of its contract (the metric and its unit, the step time, the
roofline entry of the dominant kernel, the CPU oracle baseline with its
core count and model, the per-kernel and per-rank figures beside the
empty-kernel floor and a same-size copy)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_on_the_tiny_workload():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "3",
                        "--warmup", "1", "--secondary", "none", "--cpu-budget", "1"],
                       cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "kernels", "per_rank"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["data"] == "synthetic"
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert "workload" in d["config"]
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and roof["unit"] == "GB/s"
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0 and cpu["sample"]
    assert cpu["single_core"]["cores"] == 1
    for name in ("pack", "combine"):
        k = d["kernels"][name]
        assert k["us_per_launch"] > 0 and k["cold_us_per_launch"] > 0 and len(k["launch"]) == 2
        assert k["copy_same_bytes"]["cold_us"] > 0 and k["of_copy_same_bytes"] > 0
        pr = d["per_rank"][name]
        assert pr["empty_kernel_us"] > 0 and pr["copy_same_bytes"]["GBps"] > 0

