"""Element and scale formats: E4M3, E2M1, E8M0, BF16 (CPU oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Definitions followed:
  * E2M1: 1 sign, 2 exponent and 1 mantissa bit; its magnitudes are exactly
    0, 0.5, 1, 1.5, 2, 3, 4, 6.  ("NVIDIA presenta una metodologia ... NVFP4",
    7minutos.es, section "Que es realmente NVFP4".)
  * UE8M0 / E8M0 scales hold only an exponent, so every scale is a power of
    two. (same page and section.)
  * E4M3: the 8-bit element of MXFP8 and the block-scale format of NVFP4
    ("Miles Blackwell RL", remio.ai, section "La Compatibilidad de Miles
    Blackwell Ahora Abarca Todo el Ciclo de RL"). The pages do not say which
    E4M3 variant; the reading taken is the OCP "fn" variant (bias 7, no
    infinities, S.1111.111 is NaN, largest finite 448).

Rounding convention (stated by the method's description, not by a page):
round to nearest, ties to the even code, saturating at the largest finite
magnitude; the sign of zero is kept.  Rounding is done in exact FP64 as
``rint(v / quantum) * quantum`` with a power-of-two quantum, which is exact
because every input here has at most 24 significant bits.
"""

from __future__ import annotations

import numpy as np

FLT_MAX = float(np.finfo(np.float32).max)

E4M3_MAX = 448.0
E2M1_MAX = 6.0


# --------------------------------------------------------------------------
# Decoding: closed forms, one code at a time.
# --------------------------------------------------------------------------

def e4m3_value(code: int) -> float:
    """Value of one OCP E4M3 byte: bias 7, subnormal (m/8)*2^-6, NaN at S.1111.111."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e2m1_value(code: int) -> float:
    """Value of one E2M1 nibble: bit 3 sign, 2-bit exponent (bias 1), 1-bit mantissa."""
    sign = -1.0 if (code >> 3) & 1 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return sign * (m / 2.0)          # subnormal: 0 or 0.5
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


def e8m0_value(code: int) -> float:
    """Value of one E8M0 byte: 2^(code-127); 0xFF is NaN."""
    if code == 0xFF:
        return float("nan")
    return 2.0 ** (code - 127)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)

# Non-negative finite magnitudes in code order (code == index).
_E4M3_POS = E4M3_TABLE[:0x7F]          # codes 0x00 .. 0x7E
_E2M1_POS = E2M1_TABLE[:8]             # codes 0x0 .. 0x7


# --------------------------------------------------------------------------
# Rounding to a small float grid.
# --------------------------------------------------------------------------

def round_to_grid(v, man_bits: int, emin: int, vmax: float) -> np.ndarray:
    """Round-to-nearest-even onto a binary float grid, saturating at ``vmax``.

    The grid has ``man_bits`` stored mantissa bits and smallest normal binade
    2^emin (below it the spacing stays 2^(emin-man_bits): subnormals).  The
    result keeps the sign of ``v`` (so a negative value that rounds to zero
    gives -0).  Inputs must be finite.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite input: NaN/Inf are outside the quantizer's domain")
    a = np.abs(v)
    _, e2 = np.frexp(a)                   # a = f * 2^e2, f in [0.5, 1)
    binade = np.maximum(e2 - 1, emin)     # floor(log2 a), clamped to the subnormal binade
    quantum = np.ldexp(1.0, binade - man_bits)
    r = np.rint(a / quantum) * quantum    # exact: quantum is a power of two
    r = np.minimum(r, vmax)
    return np.copysign(r, v)


def _encode(v, grid_pos: np.ndarray, man_bits: int, emin: int, vmax: float,
            sign_bit: int) -> np.ndarray:
    r = round_to_grid(v, man_bits, emin, vmax)
    mag = np.abs(r)
    idx = np.searchsorted(grid_pos, mag)
    if not np.all(grid_pos[np.minimum(idx, len(grid_pos) - 1)] == mag):
        raise AssertionError("rounded value is not on the grid")
    sign = np.signbit(r).astype(np.int64) << sign_bit
    return (idx.astype(np.int64) | sign)


def encode_e4m3(v) -> np.ndarray:
    """RNE, saturating conversion to OCP E4M3 codes (uint8). -0 -> 0x80."""
    return _encode(v, _E4M3_POS, 3, -6, E4M3_MAX, 7).astype(np.uint8)


def encode_e2m1(v) -> np.ndarray:
    """RNE, saturating conversion to E2M1 codes (0..15, as uint8). -0 -> 0x8."""
    return _encode(v, _E2M1_POS, 1, 0, E2M1_MAX, 3).astype(np.uint8)


def decode_e4m3(codes) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.int64)]


def decode_e2m1(codes) -> np.ndarray:
    return E2M1_TABLE[np.asarray(codes, dtype=np.int64)]


def decode_e8m0(codes) -> np.ndarray:
    return E8M0_TABLE[np.asarray(codes, dtype=np.int64)]


# --------------------------------------------------------------------------
# BF16 <-> FP32 / FP64
# --------------------------------------------------------------------------

def bf16_bits_to_f32(bits) -> np.ndarray:
    """BF16 bit patterns (uint16) -> float32 (exact: BF16 is the top half of FP32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def f32_to_bf16_bits(v) -> np.ndarray:
    """float32 -> BF16 bit patterns by round-to-nearest-even (overflow gives +-Inf;
    +-Inf stays +-Inf, e.g. an FP32 dequantization that overflowed).

    Done as a grid rounding with 7 mantissa bits and BF16's normal range
    (smallest normal 2^-126), then the exact FP32 result's top 16 bits.
    """
    v = np.asarray(v, dtype=np.float32)
    inf = np.isinf(v)
    r = round_to_grid(np.where(inf, 0.0, v).astype(np.float64), 7, -126, np.inf)
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)        # exact, or +-Inf past the BF16 range
    r32 = np.where(inf, v, r32)           # an FP32 infinity stays infinite
    return (r32.view(np.uint32) >> 16).astype(np.uint16)
