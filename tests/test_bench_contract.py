"""bench.py's output contract: one JSON line with the fields the driver reads,
a roofline object for the dominant kernel and the oracle's CPU baseline; more
than one GPU is refused with a message."""

import json
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, timeout=600):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2", timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
def test_decode_line_fields():
    r = run_bench("--steps", "8", "--warmup", "2", "--cpu-baseline-seconds", "0.5",
                  "--no-secondary")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    line = json.loads(lines[-1])
    for key, kind in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int),
                      ("steps", int), ("warmup", int), ("ms_per_step", float),
                      ("higher_is_better", bool), ("scaling", str), ("dtype", str),
                      ("data", str), ("config", dict), ("roofline", dict),
                      ("cpu_baseline", dict)):
        assert isinstance(line[key], kind), (key, line.get(key))
    assert "vs_baseline" in line and line["vs_baseline"] is None
    assert line["n_gpus"] == 1 and line["steps"] == 8 and line["warmup"] == 2
    assert line["unit"] == "GB/s" and line["higher_is_better"] is True
    assert line["config"]["workload"] == "decode"
    assert line["value"] > 0 and line["ms_per_step"] > 0
    roof = line["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-12
    assert 0 < roof["frac"] < 1
    assert roof["kernel"] == "gemm_decode_kernel"
    assert "traffic" in roof
    cpu = line["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
    assert isinstance(cpu["sample"], str) and cpu["unit"] == "GB/s"
