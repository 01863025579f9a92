"""Host-side checks of bench.py (no GPU): the one-GPU guard and the rule that
counter-derived traffic is reported only for the sources it was taken on."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    line = json.loads(p.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus"] == 2


def test_traffic_follows_the_recorded_sources(monkeypatch):
    rec = bench.MEASURED_TRAFFIC
    now = {name: bench.measured_traffic(name) for name in rec["bytes"]}
    # either every recorded source still matches (bytes reported) or none is reported
    assert all(v is None for v in now.values()) or now == rec["bytes"]
    changed = dict(rec, sources=dict(rec["sources"], **{"csrc/kq_gemv.hip": "0" * 16}))
    monkeypatch.setattr(bench, "MEASURED_TRAFFIC", changed)
    assert all(bench.measured_traffic(name) is None for name in rec["bytes"])
