"""DeepSeek-V3-style blockwise FP8 (CPU oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

What the pages fix: E4M3 elements; weights scaled in 128 x 128 blocks and
activations (and gradients) in 1 x 128 tiles; the scales are FP32 and are
applied in software around the matrix-multiply path rather than by the matrix
hardware ("Miles Blackwell MXFP8/NVFP4 RL recipes", aib.vote, second paragraph;
"Miles Blackwell RL", remio.ai, section "NVFP4 por token cuestiona el valor
predeterminado uniforme de BF16"; 7minutos.es NVFP4 page, the 12B results
paragraph, for the activation and gradient tiles).

Readings (the pages print no formula):
  * scale of a block: s = fl32(amax / 448), binary32 division of the block's
    largest magnitude by the E4M3 maximum (the block's largest element then
    lands on +-448); an all-zero block gets s = 0.
  * element: v = fl32(x / s) (binary32 division), q = RNE_sat_E4M3(v); in an
    all-zero block q = 0 with the sign of the zero kept.
  * dequantized value q * s; a GEMM over such operands is
    C[m, n] = sum over 128-K blocks kb of sA[m, kb] sB[n, kb] sum_{k in kb} qA qB,
    i.e. the product of the dequantized operands.
  * layouts: codes row-major like the input; activation scales (rows, cols/128);
    weight scales (rows/128, cols/128), both row-major. A "128 x 1" activation
    copy (tiles along the rows, for a GEMM that reduces over rows) is the 1 x 128
    quantization of the transposed tensor, stored transposed.
(parity unpinned for the choice of s = amax / 448 and for the zero-block scale;
held by closed forms, the reduction to MXFP8 on power-of-two blocks, error bounds
and invariants in tests/test_oracle_fp8_block.py.)
"""

from __future__ import annotations

import numpy as np

from .formats import E4M3_MAX, bf16_bits_to_f32, decode_e4m3, encode_e4m3

TILE = 128
f32 = np.float32


def _as_f32(x) -> np.ndarray:
    x = np.asarray(x)
    return bf16_bits_to_f32(x) if x.dtype == np.uint16 else x.astype(f32)


def block_scale(amax) -> np.ndarray:
    """s = fl32(amax / 448) (0 for amax = 0)."""
    a = np.asarray(amax, dtype=f32)
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(a > 0, a / f32(E4M3_MAX), f32(0)).astype(f32)


def quantize_with_scales(x: np.ndarray, s_elem: np.ndarray) -> np.ndarray:
    """q = RNE_sat_E4M3(fl32(x / s)) per element with its block's scale (q = signed 0 where s = 0)."""
    x = np.asarray(x, dtype=f32)
    s_elem = np.asarray(s_elem, dtype=f32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(s_elem > 0, x / s_elem, x * f32(0)).astype(f32)     # binary32 division
    return encode_e4m3(v.astype(np.float64))


def quantize_act(x) -> tuple[np.ndarray, np.ndarray]:
    """1 x 128 tiles along each row: (q (R, C) E4M3 codes, s (R, C/128) FP32)."""
    x = _as_f32(x)
    R, C = x.shape
    if C % TILE:
        raise ValueError("cols must be a multiple of 128")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    amax = np.max(np.abs(x).reshape(R, C // TILE, TILE), axis=2)
    s = block_scale(amax)
    q = quantize_with_scales(x, np.repeat(s, TILE, axis=1))
    return q, s


def quantize_act_transposed(x) -> tuple[np.ndarray, np.ndarray]:
    """128 x 1 tiles down each column, stored transposed: (q (C, R), s (C, R/128))."""
    return quantize_act(np.ascontiguousarray(_as_f32(x).T))


def quantize_weight(x) -> tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """128 x 128 blocks: (q (R, C), s (R/128, C/128), qT (C, R), sT (C/128, R/128)); the
    transposed copy holds the same codes and scales, transposed."""
    x = _as_f32(x)
    R, C = x.shape
    if R % TILE or C % TILE:
        raise ValueError("both axes must be multiples of 128")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    amax = np.max(np.abs(x).reshape(R // TILE, TILE, C // TILE, TILE), axis=(1, 3))
    s = block_scale(amax)
    s_elem = np.repeat(np.repeat(s, TILE, axis=0), TILE, axis=1)
    q = quantize_with_scales(x, s_elem)
    return q, s, np.ascontiguousarray(q.T), np.ascontiguousarray(s.T)


def dequantize_act(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Exact FP64 values q * s of a 1 x 128 operand."""
    return decode_e4m3(q) * np.repeat(np.asarray(s, dtype=np.float64), TILE, axis=1)


def dequantize_weight(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Exact FP64 values q * s of a 128 x 128-block operand."""
    S = np.repeat(np.repeat(np.asarray(s, dtype=np.float64), TILE, axis=0), TILE, axis=1)
    return decode_e4m3(q) * S
