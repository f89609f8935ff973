"""MXFP8 quantization and dequantization (CPU oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

What the pages fix:
  * every 32 consecutive E4M3 values share one E8M0 scale ("Miles Blackwell
    RL", remio.ai, section "La Compatibilidad de Miles Blackwell Ahora Abarca
    Todo el Ciclo de RL"; aib.vote summary, MXFP8 paragraph);
  * E8M0 scales are powers of two (7minutos.es NVFP4 page, section "Que es
    realmente NVFP4");
  * the scaling blocks must run along the GEMM's reduction dimension, and
    forward and backward need different orientations, so two copies are made
    from the original high-precision tensor: rowwise 1x32 blocks and
    columnwise 32x1 blocks, which are numerically different (remio.ai, section
    "Un Cuantizador Compartido Es el Mecanismo Real"; aib.vote, MXFP8
    paragraph).

Readings where the pages are silent (each listed in the design notes):
  * E8M0 exponent: the smallest power of two X with amax / X <= 448, i.e. the
    exponent is rounded up. The NVFP4-vs-MXFP4 section of the 7minutos.es page
    says power-of-two block scales can waste up to one binade and lose the top
    FP4 samples, which is what rounding the scale up does. Under this rule no
    finite input ever saturates. (parity unpinned: no page prints a worked
    MXFP8 value; the rule is held by the invariants and hand-worked closed
    forms in the tests.)
  * all-zero block -> scale code 0 (the clamp of an exponent of -inf); its
    elements encode as +-0.
  * scale code clamped to [0, 254]; 0xFF (NaN) is never produced.
  * columnwise copy stored transposed: qT[c][r] and sT[c][r // 32], so both
    copies are K-contiguous operands of a "TN" GEMM.
"""

from __future__ import annotations

import numpy as np

from .formats import (E4M3_MAX, bf16_bits_to_f32, decode_e4m3, decode_e8m0,
                      encode_e4m3)

BLOCK = 32


def e8m0_scale_for_amax(amax) -> np.ndarray:
    """Scale code s for block maxima ``amax`` (float64, >= 0).

    s = clamp(e + 127, 0, 254) with e the smallest integer such that
    amax <= 448 * 2^e; s = 0 for an all-zero block.
    """
    a = np.asarray(amax, dtype=np.float64)
    s = np.zeros(a.shape, dtype=np.int64)
    nz = a > 0
    an = a[nz]
    e = np.ceil(np.log2(an / E4M3_MAX)).astype(np.int64)       # first guess
    # Make the guess exact with exact FP64 comparisons (448 * 2^e is exact).
    e = np.where(an > np.ldexp(E4M3_MAX, e), e + 1, e)
    e = np.where(an <= np.ldexp(E4M3_MAX, e - 1), e - 1, e)
    assert np.all(an <= np.ldexp(E4M3_MAX, e)) and np.all(an > np.ldexp(E4M3_MAX, e - 1))
    s[nz] = np.clip(e + 127, 0, 254)
    return s.astype(np.uint8)


def _quantize_blocks_last_axis(x: np.ndarray):
    """x: float64 (R, C) with C % 32 == 0; blocks of 32 along the last axis."""
    R, C = x.shape
    if C % BLOCK:
        raise ValueError("blocked axis must be a multiple of 32")
    xb = x.reshape(R, C // BLOCK, BLOCK)
    amax = np.max(np.abs(xb), axis=2)
    s = e8m0_scale_for_amax(amax)
    # x * 2^(127 - s): exact in FP64 (a power-of-two product).
    scaled = np.ldexp(xb, 127 - s.astype(np.int64)[:, :, None])
    q = encode_e4m3(scaled).reshape(R, C)
    return q, s


def quantize_rowwise(x_bf16_bits: np.ndarray):
    """Rowwise 1x32 MXFP8 copy of a BF16 (R, C) tensor.

    Returns (q uint8 (R, C) E4M3 codes, s uint8 (R, C/32) E8M0 codes).
    """
    x = bf16_bits_to_f32(x_bf16_bits).astype(np.float64)
    return _quantize_blocks_last_axis(x)


def quantize_colwise(x_bf16_bits: np.ndarray):
    """Columnwise 32x1 MXFP8 copy, stored transposed.

    Blocks are 32 consecutive rows of one column of x (R, C). Returns
    (qT uint8 (C, R), sT uint8 (C, R/32)): qT[c][r] encodes x[r][c] under the
    scale sT[c][r // 32].
    """
    x = bf16_bits_to_f32(x_bf16_bits).astype(np.float64)
    R, C = x.shape
    if R % BLOCK:
        raise ValueError("rows must be a multiple of 32 for the columnwise copy")
    qT = np.empty((C, R), dtype=np.uint8)
    sT = np.empty((C, R // BLOCK), dtype=np.uint8)
    for rb in range(R // BLOCK):
        blk = x[rb * BLOCK:(rb + 1) * BLOCK, :]            # (32, C): one block per column
        amax = np.max(np.abs(blk), axis=0)                 # (C,)
        s = e8m0_scale_for_amax(amax)
        scaled = np.ldexp(blk, 127 - s.astype(np.int64)[None, :])
        qT[:, rb * BLOCK:(rb + 1) * BLOCK] = encode_e4m3(scaled).T
        sT[:, rb] = s
    return qT, sT


def dequantize_exact(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Exact FP64 value of each element: E4M3(q) * 2^(s - 127), blocks along the last axis."""
    R, C = q.shape
    vals = decode_e4m3(q).reshape(R, C // BLOCK, BLOCK)
    scale = decode_e8m0(s)[:, :, None]
    return (vals * scale).reshape(R, C)


def dequantize_f32(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """FP32 dequantization: the exact product rounded once to binary32 (overflow -> Inf)."""
    with np.errstate(over="ignore"):
        return dequantize_exact(q, s).astype(np.float32)
