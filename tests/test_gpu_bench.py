"""bench.py on the GPU: one JSON line on stdout carrying the contract's
fields, the roofline object of the headline kernel and the CPU oracle
baseline, with figures that agree with one another."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

import synth

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_json_line_with_the_contract_fields():
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "5", "--warmup", "2",
           "--cpu-budget", "1"]
    print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-3000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["higher_is_better"] is True and d["vs_baseline"] is None
    assert d["config"]["workload"].startswith("c3")
    # value is the step's operations over its measured time
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert abs(d["config"]["ops_per_step"] / (d["ms_per_step"] * 1e-3) / 1e12 - d["value"]) / d["value"] < 1e-3
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s"
    assert rf["achieved"] == pytest.approx(d["value"], rel=1e-3)
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], abs=1e-4)
    assert 0 < rf["frac"] < 1
    assert rf["launch_us_mean"] == pytest.approx(d["ms_per_step"] * 1e3, rel=1e-3)
    assert rf["traffic"] is None or rf["traffic"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    # every workload measured in the same run, the headline last
    assert set(d["workloads"]) == set(synth.WORKLOADS)
    assert list(d["workloads"])[-1] == "c3"
