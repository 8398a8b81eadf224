"""Throughput regression guard: bench.py on the video, MMDiT and DiT
workloads must reach at least 85% of the last accepted GB/s on one MI355X
(box-to-box spread of the same kernels is about 3%).  Each run is bench.py
itself, in a child process, so the guard times exactly what the bench line
reports; the line's fields and roofline arithmetic are checked too."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# last accepted bench.py values (GB/s of algorithmic bytes) on MI355X
ACCEPTED_GBS = {"video_bf16": 5640.0, "mmdit_bf16": 3600.0, "dit_bf16": 3150.0}
FLOOR = 0.85


@pytest.mark.parametrize("config", list(ACCEPTED_GBS))
def test_bench_throughput_floor(config):
    print(f"[perf] bench.py --config {config}", flush=True)
    run = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", config, "--steps", "50",
                          "--no-cpu-baseline"], capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert run.returncode == 0, run.stderr[-3000:]
    line = [ln for ln in run.stdout.splitlines() if ln.startswith("{")][-1]
    res = json.loads(line)
    print(f"  {res['value']} GB/s ({res['pct_of_peak']}% of peak), {res['ms_per_step']} ms/step", flush=True)
    assert res["value"] >= FLOOR * ACCEPTED_GBS[config], (
        f"{config}: {res['value']} GB/s is below {FLOOR:.0%} of the accepted {ACCEPTED_GBS[config]} GB/s")
    # the line's contract
    for k, t in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                 ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                 ("dtype", str), ("data", str), ("config", dict), ("roofline", dict)):
        assert isinstance(res.get(k), t), f"{k}: {res.get(k)!r}"
    assert "vs_baseline" in res and res["n_gpus"] == 1 and res["steps"] == 50
    assert res["config"]["name"] == config and isinstance(res["config"]["workload"], str)
    rf = res["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3 and 0.0 < rf["frac"] < 1.0
    assert "traffic" in rf
