"""bench.py end to end on the GPU: one JSON line with the fields the benchmark
contract asks for (metric, value, roofline, CPU baseline of the oracle, the
timed regions and the copy control), on the small workload so it runs in
seconds."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_complete_json_line():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "20", "--warmup", "2",
           "--no-other-workloads", "--cpu-seconds", "0.5"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    assert d["unit"] == "GB/s" and d["value"] > 0 and d["n_gpus"] == 1 and d["steps"] == 20
    assert d["higher_is_better"] is True and d["dtype"] == "bf16" and d["data"] == "synthetic"
    assert d["config"]["workload"] == "tiny" and d["kernel"].startswith("update_")
    rl = d["roofline"]
    assert rl["bound"] == "hbm" and rl["peak"] == 8000.0 and rl["unit"] == "GB/s"
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    assert cpu["single_thread"]["cores"] == 1
    t = d["timing"]
    assert t["steps_per_region"] == 20 and t["regions"] >= 5
    assert t["us_per_call"]["p10"] <= t["us_per_call"]["median"] <= t["us_per_call"]["p90"]
    assert abs(d["ms_per_step"] * 1e3 - t["us_per_call"]["median"]) < 1e-4  # the median is rounded to 4 places
    assert d["copy_control"]["us_per_call"] > 0 and d["copy_control"]["frac_of_copy"] > 0
    assert d["steady_state"]["steps_per_region"] == 1000
