"""The benchmark's output line: bench.py run as the driver runs it (one GPU,
a few steps) on a small workload, its one JSON line checked for the fields
and relations the measurement relies on (the time base of `value` and of the
roofline, the clock settling, the oracle's CPU baseline)."""
import json
import os
import subprocess
import sys

import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [x for x in r.stdout.splitlines() if x.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def test_forward_line():
    d = run_bench("--gpus", "1", "--steps", "5", "--warmup", "2", "--settle-ms", "50",
                  "--cpu-reps", "1", "--workload", "internimage_stage_bf16")
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "roofline_alu", "cpu_baseline", "clock_settle_ms"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["config"]["workload"] == "internimage_stage_bf16"
    assert d["config"]["launch"] == "hip_graph"
    assert d["clock_settle_ms"] >= 50
    # value is the ideal bytes over the per-step time; the roofline uses the
    # same time base
    ideal = d["config"]["ideal_bytes"]
    assert d["value"] == pytest.approx(ideal / (d["ms_per_step"] * 1e-3) / 1e9, rel=1e-3)
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(d["value"], rel=1e-3)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-3)
    assert 0.0 < r["frac"] < 1.0
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0


def test_more_gpus_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0 and "one GPU" in r.stderr
