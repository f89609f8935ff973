"""MXFP4 quantization and dequantization (CPU oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

What the pages fix: MXFP4 uses blocks of 32 elements, each element stored as
E2M1 (sign, 2 exponent bits, 1 mantissa bit: +-0, +-0.5, +-1, +-1.5, +-2, +-3,
+-4, +-6), with the block scale stored in UE8M0, a power of two (7minutos.es
NVFP4 page, section "Que es realmente NVFP4"). Power-of-two scales can waste up
to one binade and lose the +-4 / +-6 samples in the worst case (same page,
section "NVFP4 frente a MXFP4").

Readings (the same as for MXFP8, with the E2M1 maximum 6 in place of 448):
  * E8M0 exponent: the smallest power of two X with amax / X <= 6 (rounded up,
    which is what loses the top samples when amax / X falls in (3, 4));
    s = clamp(e + 127, 0, 254); an all-zero block gets s = 0.
  * q = RNE_sat_E2M1(x * 2^(127 - s)); the product is exact (power of two).
  * packing as NVFP4: element 2j in the low nibble of byte j.
  * columnwise copy stored transposed, as for MXFP8.
(parity unpinned for the exponent rule, as for MXFP8: held by closed forms and
invariants in the tests.)
"""

from __future__ import annotations

import numpy as np

from .formats import E2M1_MAX, bf16_bits_to_f32, decode_e2m1, decode_e8m0, encode_e2m1

BLOCK = 32


def e8m0_scale_for_amax(amax) -> np.ndarray:
    """s = clamp(e + 127, 0, 254), e the smallest integer with amax <= 6 * 2^e; 0 for amax = 0."""
    a = np.asarray(amax, dtype=np.float64)
    s = np.zeros(a.shape, dtype=np.int64)
    nz = a > 0
    an = a[nz]
    e = np.ceil(np.log2(an / E2M1_MAX)).astype(np.int64)
    e = np.where(an > np.ldexp(E2M1_MAX, e), e + 1, e)            # exact fix-ups (6 * 2^e exact)
    e = np.where(an <= np.ldexp(E2M1_MAX, e - 1), e - 1, e)
    assert np.all(an <= np.ldexp(E2M1_MAX, e)) and np.all(an > np.ldexp(E2M1_MAX, e - 1))
    s[nz] = np.clip(e + 127, 0, 254)
    return s.astype(np.uint8)


def _quantize_last_axis(x: np.ndarray):
    R, C = x.shape
    if C % BLOCK:
        raise ValueError("blocked axis must be a multiple of 32")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    xb = x.astype(np.float64).reshape(R, C // BLOCK, BLOCK)
    s = e8m0_scale_for_amax(np.max(np.abs(xb), axis=2))
    v = xb * np.ldexp(1.0, 127 - s.astype(np.int64))[:, :, None]   # exact
    q = encode_e2m1(v).reshape(R, C)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8), s


def quantize_rowwise(x_bf16_bits: np.ndarray):
    """1x32 blocks along each row: (packed (R, C/2), E8M0 (R, C/32))."""
    return _quantize_last_axis(bf16_bits_to_f32(x_bf16_bits))


def quantize_colwise(x_bf16_bits: np.ndarray):
    """32x1 blocks down each column, stored transposed: (packed (C, R/2), E8M0 (C, R/32))."""
    return _quantize_last_axis(np.ascontiguousarray(bf16_bits_to_f32(x_bf16_bits).T))


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    R, Ch = packed.shape
    out = np.empty((R, 2 * Ch), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def dequantize_exact(packed: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Exact FP64 values q * 2^(s - 127)."""
    q = decode_e2m1(unpack_codes(packed))
    return q * np.repeat(decode_e8m0(s), BLOCK, axis=1)
