"""Reference GEMMs over dequantized operands (CPU oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Block-scaled GEMMs consume operands whose scaling blocks lie along the
reduction dimension ("Miles Blackwell RL", remio.ai, section "Un Cuantizador
Compartido Es el Mecanismo Real"), so every GEMM here is written "TN":
C[m, n] = sum_k A[m, k] * B[n, k] with both operands K-contiguous.

The reference value is the FP64 product of the exact dequantized operands
(a library matmul serves as that step). The pass criterion is the normwise
relative error ||C - C_ref||_F / ||C_ref||_F <= 2e-5; if C_ref is all zero, C
must be exactly zero.
"""

from __future__ import annotations

import numpy as np

from . import mxfp8, nvfp4

GEMM_RTOL = 2e-5


def gemm_tn_fp64(a_hat: np.ndarray, b_hat: np.ndarray) -> np.ndarray:
    """C = A_hat @ B_hat^T in FP64 (A_hat (M, K), B_hat (N, K))."""
    return np.asarray(a_hat, dtype=np.float64) @ np.asarray(b_hat, dtype=np.float64).T


def gemm_mxfp8_ref(qa, sa, qb, sb) -> np.ndarray:
    """Reference for an MXFP8 x MXFP8 GEMM: both operands K-contiguous, scales per 32 along K."""
    return gemm_tn_fp64(mxfp8.dequantize_exact(qa, sa), mxfp8.dequantize_exact(qb, sb))


def gemm_nvfp4_ref(pa, Sa, ta_rows, pb, Sb, tb_rows) -> np.ndarray:
    """Reference for an NVFP4 x NVFP4 GEMM; t's are per row of each operand (broadcast a
    per-tensor scale to every row)."""
    return gemm_tn_fp64(nvfp4.dequantize_exact(pa, Sa, ta_rows),
                        nvfp4.dequantize_exact(pb, Sb, tb_rows))


def normwise_rel_err(c, c_ref) -> float:
    """||C - C_ref||_F / ||C_ref||_F in FP64; an all-zero C_ref gives 0 when C is exactly
    zero (either sign) and +inf otherwise. Both norms are taken of the arrays divided by
    one power of two near their largest magnitude (an exact step), so squares of tiny
    or huge entries neither underflow nor overflow."""
    c = np.asarray(c, dtype=np.float64)
    c_ref = np.asarray(c_ref, dtype=np.float64)
    d = c - c_ref
    if not np.any(c_ref):
        return 0.0 if not np.any(c) else float("inf")
    big = max(float(np.max(np.abs(c_ref))), float(np.max(np.abs(d))) if d.size else 0.0)
    scale = 2.0 ** np.floor(np.log2(big))
    return float(np.linalg.norm(d / scale) / np.linalg.norm(c_ref / scale))
