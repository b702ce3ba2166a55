"""The bench line's contract, on the GPT-2-shaped workload: one JSON line with the
metric, its unit and direction, the run's shape, the workload's config, the
dominant kernel's roofline entry (achieved over peak, the launches it was
measured on) and the CPU oracle baseline (its rate, unit, the cores it used,
what the sample was)."""

import json
import os
import subprocess
import sys

import pytest

from gpu_util import note, require_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(300)
def test_bench_line_carries_the_contract_fields():
    require_gpu()
    note("bench contract: python bench.py --config c2 --steps 3 --warmup 1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "c2", "--steps", "3",
                        "--warmup", "1"], capture_output=True, text=True, timeout=280, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    b = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in b, k
    assert b["n_gpus"] == 1 and b["steps"] == 3 and b["warmup"] == 1
    assert b["unit"] == "GB/s" and b["higher_is_better"] is True and b["scaling"] in ("weak", "strong")
    assert b["vs_baseline"] is None and b["data"] == "synthetic"
    assert b["value"] > 0 and b["ms_per_step"] > 0
    assert "workload" in b["config"] and b["config"]["name"] == "c2"
    rf = b["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "launches", "avg_launch_ms",
              "algorithmic_bytes_per_launch"):
        assert k in rf, k
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], abs=1e-4)
    assert rf["achieved"] == pytest.approx(rf["algorithmic_bytes_per_launch"] / (rf["avg_launch_ms"] * 1e-3) / 1e9,
                                           rel=1e-2)
    cb = b["cpu_baseline"]
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in cb, k
    assert cb["kind"] == "oracle" and cb["cores"] == 1 and cb["value"] > 0 and cb["unit"] == "GB/s"
    # the step's phases, each timed, and the partition reported once beside them
    assert {"gather_fwd", "gather_bwd", "reduce_scatter", "grad_norm", "adam", "partition_once"} <= set(b["kernels"])
