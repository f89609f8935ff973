"""MoE expert-layer stages (CPU oracle): grouped GEMM reference, SwiGLU, combine.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

NVFP4 is applied to the routed experts' weights and activations, with the rest
of the model (including shared experts, which see every token) kept in higher
precision ("Miles Blackwell RL", remio.ai, sections "La Compatibilidad ..." and
"NVFP4 por token cuestiona el valor predeterminado uniforme de BF16"). Expert
FFNs are SwiGLU, with gate and up entering one fused GEMM (remio.ai, "Un
Cuantizador Compartido Es el Mecanismo Real").

Stage-wise checking: each stage's reference consumes the device's actual input
to that stage, so a one-ulp FP32 difference upstream cannot cascade into
requantization bits downstream.
  * grouped GEMM: FP64 product of the exact dequantized operands per expert;
  * SwiGLU: h = silu(g) * u = g u / (1 + e^(-g)) of the FP32 gate/up values,
    rounded once, to nearest-even, from its exact real value to BF16 (no
    intermediate binary32 rounding). The pages name no exponential; the
    correctly rounded value is the one result that depends on none, and keeps
    approximate math out of what the FP4 quantizer consumes ("Miles Blackwell
    RL", remio.ai, section "Un Cuantizador Compartido Es el Mecanismo Real").
  * combine: y_t = sum_j w_{t,j} * O[slot(t, j)] in FP64.
Weight layout: the gate_up matrix of an expert has 2I rows, gate rows first
(0..I-1), up rows next (I..2I-1); the GEMM output row of a slot is therefore
[g_0 .. g_{I-1}, u_0 .. u_{I-1}].
"""

from __future__ import annotations

from decimal import Context, Decimal

import numpy as np

from .formats import bf16_bits_to_f32, f32_to_bf16_bits, round_to_grid


def grouped_gemm_ref(a_hat: np.ndarray, offsets, b_hat_groups) -> np.ndarray:
    """Per expert g: C[off[g]:off[g+1]] = A_hat[off[g]:off[g+1]] @ B_hat[g]^T (FP64).

    a_hat: (S, K) rows already in expert order; b_hat_groups: (G, N, K).
    """
    off = np.asarray(offsets, dtype=np.int64)
    G = len(off) - 1
    N = b_hat_groups.shape[1]
    out = np.zeros((a_hat.shape[0], N), dtype=np.float64)
    for g in range(G):
        lo, hi = off[g], off[g + 1]
        if hi > lo:
            out[lo:hi] = np.asarray(a_hat[lo:hi], np.float64) @ np.asarray(b_hat_groups[g], np.float64).T
    return out


def swiglu_ref_f64(gate_up_f32: np.ndarray) -> np.ndarray:
    """silu(g) * u = (g u) / (1 + e^(-g)) in FP64 from FP32 inputs; gate = first half of
    the columns. g u is exact in FP64; the result is within a few FP64 ulps of the real
    value (e^(-g) overflowing for g < -709 gives a signed zero, and the real value is then
    below 1e-200 in magnitude)."""
    gu = np.asarray(gate_up_f32, dtype=np.float32).astype(np.float64)
    I = gu.shape[1] // 2
    g, u = gu[:, :I], gu[:, I:]
    with np.errstate(over="ignore"):
        return (g * u) / (1.0 + np.exp(-g))


_DEC = Context(prec=90, Emax=10 ** 9, Emin=-10 ** 9)


def _swiglu_exact_above(g: float, u: float, mid: float) -> bool:
    """Is |g u / (1 + e^(-g))| above the dyadic value mid > 0?  Decided with 90-digit
    decimal arithmetic (float -> Decimal is exact). If the decimal value lands on mid
    itself, e^(-g) vanished below its precision (g > 200): the real value is then
    |g u| times 1/(1 + e^(-g)) < 1, i.e. strictly below, so the answer is False."""
    gd, ud = Decimal(g), Decimal(u)
    h = _DEC.divide(_DEC.multiply(gd, ud), _DEC.add(Decimal(1), _DEC.exp(_DEC.minus(gd))))
    return _DEC.compare(h.copy_abs(), Decimal(mid)) > 0            # copy_abs: no rounding


def swiglu_bf16_ref(gate_up_f32: np.ndarray) -> np.ndarray:
    """BF16 bits of h = g u / (1 + e^(-g)), correctly rounded (nearest, ties to even) from
    the exact value; overflow past the BF16 range gives +-Inf, a vanishing value a zero
    with the sign of g u.

    The FP64 value carries a relative error below 2^-50, so its BF16 rounding is the
    correct one unless it lies within that distance of a rounding midpoint; for those
    elements the side of the midpoint is decided exactly in decimal arithmetic."""
    gu = np.asarray(gate_up_f32, dtype=np.float32)
    h = swiglu_ref_f64(gu)
    r = round_to_grid(h, 7, -126, np.inf)                 # RNE onto the BF16 grid, in FP64
    # distance to the nearest midpoint, in units of the BF16 quantum (exact FP64 steps)
    a = np.abs(h)
    _, e2 = np.frexp(a)
    quantum = np.ldexp(1.0, np.maximum(e2 - 1, -126) - 7)
    frac = a / quantum - np.floor(a / quantum)
    near = np.argwhere((np.abs(frac - 0.5) < 2.0 ** -36) & (a > 0))
    I = gu.shape[1] // 2
    for i, j in near:
        lo = np.floor(a[i, j] / quantum[i, j]) * quantum[i, j]
        mid = lo + 0.5 * quantum[i, j]
        up = _swiglu_exact_above(float(gu[i, j]), float(gu[i, j + I]), float(mid))
        r[i, j] = np.copysign(lo + quantum[i, j] if up else lo, h[i, j])
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)                        # exact, or +-Inf past the BF16 range
    return (r32.view(np.uint32) >> 16).astype(np.uint16)


def bf16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in BF16 ulps between two BF16 bit arrays (monotone integer map)."""
    def key(b):
        b = np.asarray(b, dtype=np.uint16).astype(np.int64)
        return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b)
    return np.abs(key(a_bits) - key(b_bits))


def combine_ref(o_slots: np.ndarray, slot_of: np.ndarray, weights: np.ndarray) -> np.ndarray:
    """y[t] = sum_j weights[t, j] * o_slots[slot_of[t, j]] in FP64."""
    o = np.asarray(o_slots, dtype=np.float64)
    w = np.asarray(weights, dtype=np.float32).astype(np.float64)
    T, k = slot_of.shape
    y = np.zeros((T, o.shape[1]), dtype=np.float64)
    for j in range(k):
        y += w[:, j:j + 1] * o[slot_of[:, j]]
    return y


def bf16_to_f64(bits) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)
