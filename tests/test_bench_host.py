"""Host-side logic of bench.py (CPU only): the single-GPU guard, the traffic
figure's staleness check, and the oracle baseline's accounting on a tiny
workload."""

from __future__ import annotations

import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_is_dropped_when_the_kernel_source_changes(tmp_path, monkeypatch):
    src = tmp_path / "attention_wan_qk_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "k.hip").write_text("kernel v1\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec = {"k": {"wl": {"bytes_per_launch": 123, "source": "k.hip",
                        "source_sha": bench.kernel_source_sha("k.hip")}}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("k", "wl") == 123
    assert bench.measured_traffic("k", "other") is None
    (src / "k.hip").write_text("kernel v2\n")
    assert bench.measured_traffic("k", "wl") is None
    (tmp_path / "profiles" / "traffic.json").unlink()
    assert bench.measured_traffic("k", "wl") is None


def test_cpu_baseline_counts_what_it_ran():
    from attention_wan_qk_amd import synth
    from attention_wan_qk_amd.workloads import WORKLOADS
    w = WORKLOADS[0]
    q, k, v = (synth.tensor(w, t, "cpu") for t in ("q", "k", "v"))
    r = bench.cpu_baseline(w, (q, k, v), budget_s=30.0)
    rows = min(640, w.tokens)
    pairs = w.batch * w.heads
    assert f"{rows} query rows x {pairs} (batch, head) pairs" in r["sample"]
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["cores"] >= 1
    assert r["value"] > 0
    # the whole tiny problem fits the budget: the sample is the problem itself
    assert 4.0 * rows * w.tokens * w.head_dim * pairs == w.self_attn_flop()
    assert np.isclose(r["full_problem_s_extrapolated"],
                      round(w.self_attn_flop() / (r["value"] * 1e12), 1), rtol=0.05, atol=0.05)
