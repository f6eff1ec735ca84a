"""The benchmark runs every workload end to end and prints lines that keep its contract.

A short run (two timed steps after one untimed call, no CPU baseline) of every workload in a child process, so
that a workload whose setup or kernel closure breaks shows here and not only in a full benchmark run.
"""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIELDS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
          "vs_baseline", "dtype", "data", "config", "roofline")


def test_every_workload_runs():
    sys.path.insert(0, ROOT)
    import bench

    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--all", "--steps", "2", "--warmup", "1",
                          "--no-cpu"], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = [json.loads(l) for l in out.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == len(bench.WORKLOADS), out.stdout[-2000:]
    for d in lines:
        for f in FIELDS:
            assert f in d, (d["config"]["workload"], f)
        assert d["steps"] == 2 and d["warmup"] == 1 and d["n_gpus"] == 1
        assert d["value"] > 0 and d["ms_per_step"] > 0
        r = d["roofline"]
        assert r["bound"] in ("hbm", "mfma") and r["peak"] > 0 and 0 < r["frac"] < 1.0, (d["config"]["workload"], r)
