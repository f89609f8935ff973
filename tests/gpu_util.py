"""Helpers for the GPU parity tests: move seeded numpy inputs to the device and
results back, and the comparison criteria (bit-exact bytes; normwise 2e-5)."""

import numpy as np
import torch

from oracle import gemm as ogemm

GEMM_RTOL = 2e-5


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def assert_bytes_equal(got: np.ndarray, exp: np.ndarray, what: str):
    got = np.asarray(got)
    exp = np.asarray(exp)
    assert got.shape == exp.shape, (what, got.shape, exp.shape)
    if not np.array_equal(got, exp):
        bad = np.argwhere(got != exp)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches; first at {i}: got {got[i]!r} expected {exp[i]!r}")


def assert_gemm_close(c: np.ndarray, c_ref: np.ndarray, what: str, rtol: float = GEMM_RTOL):
    """Normwise check against the FP64 reference rounded once to binary32 (the
    output format): a reference below the FP32 range must come out as zero."""
    with np.errstate(over="ignore", under="ignore"):
        ref32 = np.asarray(c_ref, dtype=np.float64).astype(np.float32)
    err = ogemm.normwise_rel_err(c, ref32)
    assert err <= rtol, f"{what}: normwise relative error {err:.3e} > {rtol:.1e}"
    return err
