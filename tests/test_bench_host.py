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


def test_cpu_baseline_row_chunks_equal_the_whole_tensor_oracle():
    """The thread-pool CPU baseline splits the oracle's work into row (or column) chunks;
    the bytes must be those of one whole-tensor call."""
    import numpy as np

    import bench
    from microscaling_precision_quantization_amd import inputs
    from oracle import mxfp8 as omx
    from oracle import nvfp4 as onv
    g = np.random.default_rng(5)
    x = inputs.to_bf16_bits(g.standard_normal((96, 64)) * np.exp(g.standard_normal((96, 1))))
    for a, b in zip(bench.rows_parallel(omx.quantize_rowwise, x), omx.quantize_rowwise(x)):
        assert np.array_equal(a, b)
    for a, b in zip(bench.mx_colwise_parallel(omx, x), omx.quantize_colwise(x)):
        assert np.array_equal(a, b)
    for a, b in zip(bench.rows_parallel(onv.quantize_per_token, x), onv.quantize_per_token(x)):
        assert np.array_equal(a, b)
    for a, b in zip(bench.nv_group_parallel(onv, x, 32), onv.quantize_per_group(x, [0, 32, 64, 96])):
        assert np.array_equal(a, b)
