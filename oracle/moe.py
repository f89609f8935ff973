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
  * SwiGLU: h = silu(g) * u computed in FP64 from the FP32 gate/up values,
    rounded to BF16; the device may differ by at most one BF16 ulp (it uses
    the hardware exponential);
  * combine: y_t = sum_j w_{t,j} * O[slot(t, j)] in FP64.
Weight layout: the gate_up matrix of an expert has 2I rows, gate rows first
(0..I-1), up rows next (I..2I-1); the GEMM output row of a slot is therefore
[g_0 .. g_{I-1}, u_0 .. u_{I-1}].
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f32, f32_to_bf16_bits


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
    """silu(g) * u in FP64 from FP32 inputs; gate = first half of the columns."""
    gu = np.asarray(gate_up_f32, dtype=np.float32).astype(np.float64)
    I = gu.shape[1] // 2
    g, u = gu[:, :I], gu[:, I:]
    return g / (1.0 + np.exp(-g)) * u


def swiglu_bf16_ref(gate_up_f32: np.ndarray) -> np.ndarray:
    """BF16 bits of the FP64 SwiGLU (rounded to FP32, then to BF16)."""
    return f32_to_bf16_bits(swiglu_ref_f64(gate_up_f32).astype(np.float32))


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
