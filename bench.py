#!/usr/bin/env python3
"""Benchmark of the microscaling hot path on one MI355X.

Workload: the MXFP8 linear layer with input (2048, 2048) and out_features 8192
-- X (2048, 2048) ~ N(0, 1), W (8192, 2048) ~ N(0, 0.02), dY (2048, 8192) ~
N(0, 1e-3), BF16, seeded synthetic data. One step = MXFP8 rowwise + columnwise
quantization of X, W and dY (three launches) followed by the three block-scaled
GEMMs fprop Y = X W^T, dgrad dX = dY W and wgrad dW = dY^T X (FP32 outputs).
Inputs are resident in HBM before timing starts; four copies of the inputs are
rotated (288 MB, more than the 256 MB Infinity Cache) so steps read HBM.

Prints one JSON line. `value` is the step's GEMM work (3 x 2*2048*8192*2048
flop) per second of the whole step (quantization included), in TFLOP/s; the
quantizer GB/s and GEMM TFLOP/s are reported per kernel beside it, each with
its roofline fraction. `roofline` covers the dominant kernel (the GEMM) with
its average launch time taken from HIP events on the launch stream;
`cpu_baseline` times the CPU oracle on a bounded sample of the same step.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
    python bench.py --profile-pass     # short fixed run for rocprofv3 counters
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}
METRIC = "quantize GB/s (% HBM peak) + block-scaled GEMM TFLOPS (% MFMA peak), 1 GPU"
T, DIN, DOUT = 2048, 2048, 8192
GEMM_FLOP = 2 * T * DOUT * DIN                       # each of fprop, dgrad, wgrad
QUANT_BYTES_PER_ELEM = 2 + 1 + 1 + 2 / 32            # BF16 read + two E4M3 copies + two scale sets
QUANT_BYTES = {"x": T * DIN * QUANT_BYTES_PER_ELEM, "w": DOUT * DIN * QUANT_BYTES_PER_ELEM,
               "dy": T * DOUT * QUANT_BYTES_PER_ELEM}
GEMM_KERNEL_SOURCES = ["microscaling_precision_quantization_amd/csrc/gemm_exact.hip",
                       "microscaling_precision_quantization_amd/csrc/common.h"]
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_gemm_mxfp8_linear_2048x8192x2048.md")
N_SETS = 4


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per GEMM launch from the committed rocprofv3 PMC summary, or None
    when the summary is missing or the kernel source changed since it was taken."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    m = re.search(r"TRAFFIC_JSON:\s*(\{.*\})", open(PMC_SUMMARY).read())
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("source_hash") != source_hash(GEMM_KERNEL_SOURCES):
        return None
    return d.get("bytes_per_launch")


def make_device_inputs(torch, dev):
    import numpy as np

    from microscaling_precision_quantization_amd import inputs
    w = inputs.workload_linear_mxfp8(T, DIN, DOUT)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
    base = {k: up(v) for k, v in w.items()}
    sets = [{k: v.clone() for k, v in base.items()} for _ in range(N_SETS)]
    return w, sets


def alloc_outputs(torch, dev):
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)
    q = {
        "x": (u8(T, DIN), u8(T, DIN // 32), u8(DIN, T), u8(DIN, T // 32)),
        "w": (u8(DOUT, DIN), u8(DOUT, DIN // 32), u8(DIN, DOUT), u8(DIN, DOUT // 32)),
        "dy": (u8(T, DOUT), u8(T, DOUT // 32), u8(DOUT, T), u8(DOUT, T // 32)),
    }
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)
    c = {"y": f32(T, DOUT), "dx": f32(T, DIN), "dw": f32(DOUT, DIN)}
    return q, c


def run_step(mxq, s, q, c):
    """One pass of the hot path (used for warmup and the profiling pass)."""
    mxq.quantize_mxfp8(s["x"], out=q["x"])
    mxq.quantize_mxfp8(s["w"], out=q["w"])
    mxq.quantize_mxfp8(s["dy"], out=q["dy"])
    xr, xrs, xc, xcs = q["x"]
    wr, wrs, wc, wcs = q["w"]
    dr, drs, dc, dcs = q["dy"]
    mxq.gemm_block_scaled(mxq.MXFP8, xr, xrs, wr, wrs, out=c["y"])      # fprop  Y  = X W^T
    mxq.gemm_block_scaled(mxq.MXFP8, dr, drs, wc, wcs, out=c["dx"])     # dgrad  dX = dY W
    mxq.gemm_block_scaled(mxq.MXFP8, dc, dcs, xc, xcs, out=c["dw"])     # wgrad  dW = dY^T X


def cpu_baseline(w):
    """The CPU oracle, as it stands, on one complete step of the same workload:
    MXFP8 row+col quantization of X, W and dY, then the fprop, dgrad and wgrad
    FP64 GEMMs of the exact dequantized operands."""
    from oracle import gemm as og
    from oracle import mxfp8 as omx
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    q = {k: (omx.quantize_rowwise(w[k]), omx.quantize_colwise(w[k])) for k in ("x", "w", "dy")}
    tq = time.perf_counter() - t0
    t1 = time.perf_counter()
    deq = lambda qs: omx.dequantize_exact(*qs)
    og.gemm_tn_fp64(deq(q["x"][0]), deq(q["w"][0]))       # fprop
    og.gemm_tn_fp64(deq(q["dy"][0]), deq(q["w"][1]))      # dgrad
    og.gemm_tn_fp64(deq(q["dy"][1]), deq(q["x"][1]))      # wgrad
    tg = time.perf_counter() - t1
    step_s = tq + tg
    return {"value": round(3 * GEMM_FLOP / step_s / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"one full step: MXFP8 row+col quantize of X, W, dY ({tq:.2f} s, single-threaded NumPy) "
                      f"and the three FP64 GEMMs of dequantized operands ({tg:.2f} s, NumPy BLAS, {cores} host "
                      f"threads available)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-pass", action="store_true",
                    help="1 warmup + 2 steps, then a 512 MiB device copy used to calibrate PMC byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch

    import microscaling_precision_quantization_amd as mxq
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    mxq.binding.lib()                                    # fails loudly if libmxq.so is missing
    w, sets = make_device_inputs(torch, dev)
    q, c = alloc_outputs(torch, dev)
    torch.cuda.synchronize()

    if args.profile_pass:
        for i in range(3):
            run_step(mxq, sets[i % N_SETS], q, c)
        src = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print("profile pass done: 3 steps + 512 MiB copy")
        return

    for i in range(args.warmup):
        run_step(mxq, sets[i % N_SETS], q, c)
    torch.cuda.synchronize()

    K = args.steps
    ev = {n: [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)] for n in ("quant", "gemm")}
    per_launch = {"gemm": [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(3 * K)]}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        s = sets[i % N_SETS]
        ev["quant"][i][0].record()
        mxq.quantize_mxfp8(s["x"], out=q["x"])
        mxq.quantize_mxfp8(s["w"], out=q["w"])
        mxq.quantize_mxfp8(s["dy"], out=q["dy"])
        ev["quant"][i][1].record()
        xr, xrs, xc, xcs = q["x"]
        wr, wrs, wc, wcs = q["w"]
        dr, drs, dc, dcs = q["dy"]
        ev["gemm"][i][0].record()
        for j, (A, sA, B, sB, out) in enumerate(((xr, xrs, wr, wrs, c["y"]), (dr, drs, wc, wcs, c["dx"]),
                                                 (dc, dcs, xc, xcs, c["dw"]))):
            per_launch["gemm"][3 * i + j][0].record()
            mxq.gemm_block_scaled(mxq.MXFP8, A, sA, B, sB, out=out)
            per_launch["gemm"][3 * i + j][1].record()
        ev["gemm"][i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms_step = wall / K * 1e3
    q_ms = sum(a.elapsed_time(b) for a, b in ev["quant"]) / K
    g_ms = sum(a.elapsed_time(b) for a, b in ev["gemm"]) / K
    launch_ms = sum(a.elapsed_time(b) for a, b in per_launch["gemm"]) / (3 * K)
    quant_gbps = sum(QUANT_BYTES.values()) / (q_ms * 1e-3) / 1e9
    gemm_tflops = 3 * GEMM_FLOP / (g_ms * 1e-3) / 1e12
    achieved = GEMM_FLOP / (launch_ms * 1e-3) / 1e12

    # native scaled-FP8 matrix-core kernel on the same operands (reported beside, not in the step)
    mc_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(3 * K)]
    for i in range(2):
        mxq.gemm_mxfp8_matrix_core(q["x"][0], q["x"][1], q["w"][0], q["w"][1], out=c["y"])
    torch.cuda.synchronize()
    for i in range(K):
        for j, (A, sA, B, sB, out) in enumerate(((q["x"][0], q["x"][1], q["w"][0], q["w"][1], c["y"]),
                                                 (q["dy"][0], q["dy"][1], q["w"][2], q["w"][3], c["dx"]),
                                                 (q["dy"][2], q["dy"][3], q["x"][2], q["x"][3], c["dw"]))):
            mc_ev[3 * i + j][0].record()
            mxq.gemm_mxfp8_matrix_core(A, sA, B, sB, out=out)
            mc_ev[3 * i + j][1].record()
    torch.cuda.synchronize()
    mc_ms = sum(a.elapsed_time(b) for a, b in mc_ev) / (3 * K)
    mc_tflops = GEMM_FLOP / (mc_ms * 1e-3) / 1e12

    traffic = recorded_traffic()
    out = {
        "metric": METRIC,
        "value": round(3 * GEMM_FLOP / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "MXFP8 linear layer: X (2048,2048) N(0,1), W (8192,2048) N(0,0.02), "
                               "dY (2048,8192) N(0,1e-3); row+col quantize of X, W, dY; fprop, dgrad, wgrad",
                   "tokens": T, "in_features": DIN, "out_features": DOUT, "input_sets_rotated": N_SETS},
        "components": {
            "quantize_mxfp8_rowcol": {"GB/s": round(quant_gbps, 1), "frac_hbm": round(quant_gbps / HBM_PEAK_GBPS, 4),
                                      "ms_per_step": round(q_ms, 4), "bytes_per_step": int(sum(QUANT_BYTES.values()))},
            "gemm_block_scaled_mxfp8": {"TFLOP/s": round(gemm_tflops, 1),
                                        "frac_mfma_bf16": round(gemm_tflops / MFMA_PEAK_TFLOPS["bf16"], 4),
                                        "frac_mfma_fp8": round(gemm_tflops / MFMA_PEAK_TFLOPS["fp8"], 4),
                                        "ms_per_step": round(g_ms, 4)},
            "gemm_mxfp8_matrix_core": {"TFLOP/s": round(mc_tflops, 1),
                                       "frac_mfma_fp8": round(mc_tflops / MFMA_PEAK_TFLOPS["fp8"], 4),
                                       "ms_per_launch": round(mc_ms, 4),
                                       "note": "native scaled-FP8 MFMA; outside the step (accumulation model differs)"},
        },
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_PEAK_TFLOPS["bf16"], 4), "traffic": traffic,
                     "kernel": "exact_dense_kernel<1,...> (MXFP8 operands formed exactly in BF16, BF16 MFMA)",
                     "flop_per_launch": GEMM_FLOP, "avg_launch_ms": round(launch_ms, 4)},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(w),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
