"""bench.py keeps its output contract: one JSON line with the metric, the
whole-job value, the step counts, the workload configuration, the roofline
of the dominant kernel and the oracle baseline slot; more than one GPU is
refused."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.gpu
@pytest.mark.timeout(300)
def test_short_run_prints_one_complete_json_line():
    print("[bench] short run: 3 steps, no extra workloads", flush=True)
    r = subprocess.run([sys.executable, BENCH, "--steps", "3", "--warmup", "1", "--kernel-reps", "1",
                        "--no-configs", "--no-prefill", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=280)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["unit"] == "GB/s"
    assert d["higher_is_better"] is True and d["scaling"] in ("weak", "strong")
    assert d["config"]["workload"] == "long_context_decode" and d["config"]["layers"] == 32
    roof = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert 0 < roof["frac"] < 1 and abs(roof["achieved"] / roof["peak"] - roof["frac"]) < 1e-3
    assert roof["traffic"] is None or roof["traffic"] > 0
