"""bench.py end to end on the GPU for the small workload: one JSON line with the
driver's contract fields, the step timed as HIP graph replays (and eagerly with
--no-graph), a roofline object and the CPU-oracle baseline."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "small", *args],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def test_bench_small_graph_replay_json_contract():
    d = _bench("--steps", "50", "--warmup", "10")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 50 and d["warmup"] == 10
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["data"] == "synthetic"
    assert d["step_launch"].startswith("hip_graph")
    assert d["ms_per_step_eager"] > 0
    rf = d["roofline"]
    assert rf["bound"] in ("hbm", "mfma") and 0 < rf["frac"] < 1 and rf["peak"] > 0
    assert "not bandwidth-measurable" in rf["note"]          # the launch-bound workload says so
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1


def test_bench_small_eager_flag():
    d = _bench("--steps", "20", "--warmup", "5", "--no-cpu-baseline", "--no-graph")
    assert d["step_launch"] == "eager" and d["cpu_baseline"] is None
    assert abs(d["ms_per_step"] - d["ms_per_step_eager"]) < 1e-9
