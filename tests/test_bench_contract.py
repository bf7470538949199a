"""bench.py's output contract: one JSON line with the fields the benchmark
record needs, and a clear refusal of more than one GPU.

The CPU test only parses arguments (the multi-GPU refusal comes before
anything touches a device); the GPU test runs two short steps of the small
workload and checks every field of the line.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, timeout):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT, capture_output=True,
                          text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"], 120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.gpu
def test_json_line_fields():
    r = _run(["--workload", "square256_bf16", "--steps", "2", "--warmup", "1", "--settle", "0",
              "--no-cpu-baseline"], 300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"] == "square256_bf16"
    rf = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in rf, key
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s"
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
