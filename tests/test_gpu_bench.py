"""bench.py end to end on the GPU (tiny workload): the JSON line keeps the
benchmark contract."""

from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


@pytest.mark.timeout(300)
def test_bench_json_line_on_the_tiny_workload():
    """bench.py end to end on the tiny workload: one JSON line on stdout with
    the fields of the benchmark contract and a roofline object."""
    print("[case] bench.py --workload tiny-5x8x8", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny-5x8x8",
                        "--steps", "2", "--warmup", "1", "--no-cpu-baseline",
                        "--no-measured-peaks"], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    rec = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 2 and rec["warmup"] == 1
    assert rec["value"] > 0 and rec["ms_per_step"] > 0
    assert rec["config"]["workload"] == "tiny-5x8x8" and "tiny-5x8x8" in rec["metric"]
    roof = rec["roofline"]
    assert roof["bound"] == "mfma" and roof["peak"] == 2500.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
