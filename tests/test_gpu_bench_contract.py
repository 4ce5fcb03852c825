"""bench.py's output contract, on the GPU: one JSON line per mode with the
metric, value, timing, roofline and cpu_baseline fields (a one-step run
without the CPU baseline); the default mode's line also carries the other
workloads' measurements."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("mode", ["", "--layer", "--stack", "--head"])
def test_bench_prints_one_json_line(mode):
    print(f"[case] bench {mode or 'default'}", flush=True)
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "1", "--warmup", "0", "--no-cpu-baseline"]
    if mode:
        cmd.append(mode)
    out = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=600, check=True).stdout
    lines = [ln for ln in out.splitlines() if ln.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 1 and d["value"] > 0 and d["ms_per_step"] > 0
    assert d["unit"] == "tokens/s" and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert "workload" in d["config"]
    r = d["roofline"]
    assert r["bound"] in ("hbm", "mfma", "alu") and r["peak"] > 0 and 0 < r["frac"] < 1
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    if not mode:
        others = d["other_workloads"]
        assert sorted(others) == ["32b_layer", "4b_layer", "sparse_64k"]
        for name, o in others.items():
            assert o["config"]["workload"] == name and o["value"] > 0 and o["ms_per_step"] > 0
            assert 0 < o["pct_bf16_peak"] < 100 and 0 < o["roofline"]["frac"] < 1
