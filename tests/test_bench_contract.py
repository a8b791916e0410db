"""bench.py's output contract: one JSON line with the fields the driver reads,
a roofline object for the dominant kernel and the oracle's CPU baseline; more
than one GPU is refused with a message; the committed HBM-traffic record is
reported only while the kernel source it was taken on is unchanged."""

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


def _kernel_tree(tmp_path):
    """A copy of the files the traffic record is keyed on, and the record."""
    import shutil
    import bench
    for rel in set(bench.KERNEL_SOURCES) | set(bench.KV_SOURCES) | {bench.TRAFFIC_FILE}:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), dst)
    return bench


def test_traffic_stays_attached_to_its_kernel_source(tmp_path, monkeypatch):
    # the committed HBM-traffic record is used only while the kernel source it
    # was taken on is unchanged; comments and blank lines do not count
    bench = _kernel_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    with open(tmp_path / bench.TRAFFIC_FILE) as f:
        workloads = sorted(json.load(f))
    assert "decode" in workloads and "kv_cache" in workloads
    attached = {w: bench.measured_traffic(w) is not None for w in workloads}
    src = tmp_path / bench.KERNEL_SOURCES[0]
    text = src.read_text()
    src.write_text(text + "\n// a note\n\n/* another\n   note */\n")
    assert {w: bench.measured_traffic(w) is not None for w in workloads} == attached
    src.write_text(text + "\nstatic int fp8_changed_token = 0;\n")
    for w in workloads:
        if w == "kv_cache":               # keyed on the KV sources only
            assert (bench.measured_traffic(w) is not None) == attached[w]
        else:
            assert bench.measured_traffic(w) is None, w


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
    # the step's GEMM-carrying launches: the fused linear kernel for M = 1
    # and 4, the decode GEMM for M = 16 (its activation quantized before)
    assert roof["kernel"] == "gemm_decode_kernel + linear_decode_kernel"
    per = {r["M"]: r for r in roof["per_launch"]}
    assert sorted(per) == [1, 4, 16]
    assert per[1]["kernel"] == per[4]["kernel"] == "linear_decode_kernel"
    assert per[16]["kernel"] == "gemm_decode_kernel"
    us = sum(r["avg_launch_us"] for r in per.values())
    b = sum(r["algorithmic_bytes"] for r in per.values())
    assert abs(roof["achieved"] - b / (us * 1e-6) / 1e9) < 1e-6 * roof["achieved"]
    assert "traffic" in roof
    ref = line["hbm_reference"]
    assert ref["copy"]["GB/s"] > 0 and ref["read_stream"]["GB/s"] > 0
    assert ref["read_stream_decode_bytes"]["bytes_read"] == 11008 * 4096
    cpu = line["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
    assert isinstance(cpu["sample"], str) and cpu["unit"] == "GB/s"
    assert isinstance(cpu["cpu_model"], str) and cpu["cpu_model"]
    assert [r["workload"] for r in cpu["single_thread"]] == ["tiny", "decode", "prefill"]
    assert all(r["threads"] == 1 and r["GFLOP/s"] > 0 for r in cpu["single_thread"])


def test_dominant_kernel_follows_the_dispatch():
    # the roofline's kernel name is the one the library launches for the
    # workload's step: one fused launch where fp8_linear needs no workspace
    # (the tiny shape), the decode GEMM where it quantizes first (decode
    # M = 16), the hand-scheduled prefill kernel for the prefill shapes
    sys.path.insert(0, ROOT)
    import bench
    import fp8_w8a8_block_amd._lib as L
    from workloads import synth
    assert L.workspace_bytes(L.OP_LINEAR, 16, 256, 512, "block") == 0
    assert bench.dominant_kernel("tiny", False) == "linear_decode_kernel"
    assert L.workspace_bytes(L.OP_LINEAR, 16, 11008, 4096, "block") > 0
    assert bench.gemm_kernel_name(16, 4096) == "gemm_decode_kernel"
    for name in ("prefill", "mlp_down", "large"):
        c = synth.CONFIGS[name]
        assert bench.gemm_kernel_name(c["M"], c["K"]) == "gemm_prefill_asm_kernel"
        assert bench.dominant_kernel(name, False) == "gemm_prefill_asm_kernel"
