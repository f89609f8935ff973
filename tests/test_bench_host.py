"""Host-side checks of bench.py that need no GPU: the one-GPU contract, the PMC traffic
lookup (keyed by the kernel sources' hash) and the algorithmic byte constants."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_no_gpu_fails_loudly_instead_of_falling_back():
    pytest.importorskip("torch")
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    r = _run("--steps", "1", "--warmup", "0", "--no-cpu-baseline")
    assert r.returncode != 0
    assert not r.stdout.strip().startswith("{")            # no JSON line without the GPU path


def test_recorded_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    summary = tmp_path / "pmc_linear.md"
    h = bench.source_hash()
    summary.write_text("x\nTRAFFIC_JSON: " + json.dumps({"source_hash": h, "bytes_per_launch": {"g": 1234}}) + "\n")
    monkeypatch.setattr(bench, "pmc_summary_path", lambda w: str(summary))
    assert bench.recorded_traffic("linear", "g") == 1234
    assert bench.recorded_traffic("linear", "other") is None
    summary.write_text("TRAFFIC_JSON: " + json.dumps({"source_hash": "0" * 16, "bytes_per_launch": {"g": 1}}) + "\n")
    assert bench.recorded_traffic("linear", "g") is None    # kernels changed since the counters were taken
    summary.unlink()
    assert bench.recorded_traffic("linear", "g") is None


def test_source_hash_covers_every_kernel_source():
    csrc = os.path.join(ROOT, "microscaling_precision_quantization_amd", "csrc")
    kernels = sorted(f for f in os.listdir(csrc) if f.endswith(".hip") and f != "api.hip")
    listed = sorted(os.path.basename(p) for p in bench.KERNEL_SOURCES if p.endswith(".hip"))
    assert listed == kernels
    assert len(bench.source_hash()) == 16


def test_algorithmic_bytes_per_element():
    assert bench.MX_ROWCOL == 4.0625                      # 2 read + 1 + 1 + 2/32
    assert bench.MX4_ROWCOL == 3.0625                     # 2 read + 0.5 + 0.5 + 2/32
    assert bench.NV_TOKEN == 2.5625                       # 2 read + 0.5 + 1/16
    assert bench.NV_TENSOR == bench.NV_TOKEN + 2          # amax pass reads the input again
    assert bench.FP8B_ACT == 4.0625                       # 2 read + 1 + 1 + 2 * 4/128
    assert bench.HBM_PEAK_GBPS == 8000.0
    assert bench.MFMA_PEAK_TFLOPS == {"bf16": 2500.0, "fp16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}
