"""Build libmxq.so (all HIP sources, gfx950) in-tree.

    python -m microscaling_precision_quantization_amd.build [--jobs N]

Every source is compiled with IEEE binary32 semantics (no fast math, no FP
contraction, correctly rounded division, denormals kept), which the bit-exact
quantizers rely on, and with packed-FP32 instructions disabled.

build_asan() links a second copy, _build/libmxq_asan.so, whose host code in
api.hip (argument validation, workspace sizing, launch set-up) is built with
AddressSanitizer; the device code is the same as in libmxq.so. It is meant for the
CPU ABI tests, run with the sanitizer runtime preloaded (ASAN_RUNTIME).
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmxq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.hip", "quant_mxfp8.hip", "quant_nvfp4.hip", "quant_fp8_block.hip", "dequant_moe.hip", "gemm_exact.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I" + os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out:
        print(out, file=sys.stderr)
    return obj


ASAN_RUNTIME = "/opt/rocm/llvm/lib/clang/{}/lib/linux/libclang_rt.asan-x86_64.so"
# host-only instrumentation: each sanitizer flag applies to the host compilation alone
ASAN_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str | None:
    """Path of the clang AddressSanitizer runtime that matches hipcc, or None."""
    import glob
    hits = sorted(glob.glob(ASAN_RUNTIME.format("*")))
    return hits[-1] if hits else None


def build_asan() -> str:
    """_build/libmxq_asan.so: api.hip with host AddressSanitizer, the kernels as built."""
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in objs):
        build(verbose=False)
    obj = os.path.join(BUILD, "api_asan.o")
    flags = [f for f in FLAGS if f != "-O3"] + ASAN_FLAGS
    r = subprocess.run([HIPCC, *flags, "-c", os.path.join(CSRC, "api.hip"), "-o", obj], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for api.hip (host sanitizer build):\n" + r.stdout + r.stderr)
    lib = os.path.join(BUILD, "libmxq_asan.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", obj, *objs, "-o", lib],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed (host sanitizer build):\n" + r.stdout + r.stderr)
    return lib


def build(jobs: int = 6, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=6)
    build(ap.parse_args().jobs)
