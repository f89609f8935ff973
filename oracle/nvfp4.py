"""NVFP4 quantization (per token, per tensor, per group), random Hadamard
transform, and dequantization (CPU oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

What the pages fix:
  * NVFP4 stores E2M1 values, one E4M3 scale for every 16 values, plus a
    second FP32 scale over a larger scope so the E4M3 block scales stay in
    range; the block amax lands close to the FP4 maximum ("NVIDIA presenta una
    metodologia ... NVFP4", 7minutos.es, section "Que es realmente NVFP4";
    "Miles Blackwell RL", remio.ai, section "La Compatibilidad ...").
  * In the RL recipe the FP32 scale is computed online per token, so a token's
    bits do not depend on which other tokens share the batch (remio.ai,
    sections "La Compatibilidad ..." and "Un Cuantizador Compartido Es el
    Mecanismo Real"; aib.vote summary, per-token paragraph).
  * Gate and up projections of a SwiGLU expert are quantized together so both
    get one consistent larger scale (remio.ai, "Un Cuantizador Compartido").
  * Fast/approximate math is kept out of the FP4 quantization path (remio.ai,
    "Un Cuantizador Compartido"): every FP32 step below is an IEEE binary32
    operation with round-to-nearest-even.
  * Random Hadamard transform: 16x16 Hadamard matrix combined with a random
    +-1 sign vector, applied to the inputs of the weight-gradient GEMM only;
    it is orthogonal, so it cancels inside the dot product and the GEMM needs
    no correction (7minutos.es, section "La metodologia de formacion de
    cuatro partes").

Readings where the pages are silent (parity unpinned for the exact FP32
operation order; pinned by invariants and closed forms in the tests):
  * scope encode scale  s_enc = fl(6 * 448 / A), A the scope amax; A = 0 gives
    s_enc = 1; an overflow to +Inf gives FLT_MAX.
  * the stored FP32 scale is the decode scale t = fl(1 / s_enc).
  * block scale  S_b = E4M3_RNE_sat(fl(fl(a_b / 6) * s_enc)).
  * element      q_i = E2M1_RNE_sat(fl(x_i * r_b)),  r_b = min(fl(s_enc / S_b),
    FLT_MAX), r_b = 0 when S_b = 0. The product is rounded to FP32 first.
  * packing: element 2j in the low nibble of byte j, element 2j+1 in the high
    nibble.
  * RHT of a 16-chunk v with signs s: w = s * v, then a Sylvester-order fast
    Walsh-Hadamard transform in FP32 (stages h = 1, 2, 4, 8, butterfly
    (w_i, w_{i+h}) <- (w_i + w_{i+h}, w_i - w_{i+h}) for i with bit h clear),
    then u = fl(w * 0.25).  0.25 = 1/sqrt(16) makes the transform orthogonal.
"""

from __future__ import annotations

import numpy as np

from . import rng
from .formats import (E2M1_MAX, E4M3_MAX, FLT_MAX, bf16_bits_to_f32,
                      decode_e2m1, decode_e4m3, encode_e2m1, encode_e4m3,
                      f32_to_bf16_bits)

BLOCK = 16
f32 = np.float32


def scope_scales(amax_scope) -> tuple[np.ndarray, np.ndarray]:
    """(s_enc, t) for an array of scope maxima (FP32)."""
    A = np.asarray(amax_scope, dtype=f32)
    with np.errstate(divide="ignore", over="ignore"):
        s_enc = f32(E2M1_MAX * E4M3_MAX) / A                 # 2688 / A in binary32
    s_enc = np.where(A == 0, f32(1.0), s_enc)
    s_enc = np.where(np.isinf(s_enc), f32(FLT_MAX), s_enc).astype(f32)
    t = (f32(1.0) / s_enc).astype(f32)
    return s_enc, t


E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_stochastic(v: np.ndarray, words: np.ndarray) -> np.ndarray:
    """Stochastic rounding of FP32 values onto the E2M1 grid: each value rounds to
    one of its two nearest representable neighbours with probability set by its
    distance to them, which removes the bias round-to-nearest-even introduces
    (7minutos.es NVFP4 page, section "La metodologia de formacion de cuatro
    partes", stochastic-rounding item: gradients only).

    Reading (the page gives no procedure): m = |v|; lo = the largest grid magnitude
    <= m, hi the next one (m >= 6 saturates to 6), d = hi - lo; f = (m - lo) / d,
    exact; round up iff (word >> 8) < f * 2^24, i.e. with probability f for a
    uniform 32-bit word. The sign is copied (-0 keeps it). Returns E2M1 codes.
    """
    v = np.asarray(v, dtype=np.float32)
    m = np.abs(v).astype(np.float64)
    sat = m >= 6.0
    lo_i = np.searchsorted(E2M1_GRID, np.minimum(m, 6.0), side="right") - 1     # index of lo
    lo = E2M1_GRID[lo_i]
    hi = E2M1_GRID[np.minimum(lo_i + 1, 7)]
    d = np.where(sat, 1.0, hi - lo)
    f = np.where(sat, 0.0, (m - lo) / d)                                         # exact
    u = (np.asarray(words, dtype=np.uint32) >> np.uint32(8)).astype(np.float64)
    up = u < f * 2.0 ** 24
    code = np.where(up, lo_i + 1, lo_i).astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 3)


def quantize_with_scope_amax(x: np.ndarray, amax_rows: np.ndarray, sr_seed: int | None = None):
    """Core NVFP4 quantizer.

    x: float32 (R, C), C % 16 == 0; amax_rows: float32 (R,) -- the scope amax
    that applies to each row (the row's own max for per-token scaling, the
    tensor's max broadcast for per-tensor scaling).
    sr_seed: None for round-to-nearest-even elements; else the elements are
    rounded stochastically with the random word of element (r, c) taken from
    rng.element_words(sr_seed, r * C + c) (its index in the (R, C) output). The
    block and scope scales are the same either way.
    Returns (packed uint8 (R, C/2), S uint8 (R, C/16) E4M3 codes, t float32 (R,)).
    """
    x = np.asarray(x, dtype=f32)
    R, C = x.shape
    if C % BLOCK:
        raise ValueError("quantized axis must be a multiple of 16")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    s_enc, t = scope_scales(amax_rows)
    xb = x.reshape(R, C // BLOCK, BLOCK)
    a_b = np.max(np.abs(xb), axis=2)                          # (R, C/16) exact
    d_b = ((a_b / f32(6.0)).astype(f32) * s_enc[:, None]).astype(f32)
    S = encode_e4m3(d_b.astype(np.float64))                   # >= 0, saturating
    S_val = decode_e4m3(S).astype(f32)                        # exact in FP32
    with np.errstate(divide="ignore", over="ignore"):
        r_b = (s_enc[:, None] / S_val).astype(f32)
    r_b = np.where(S_val == 0, f32(0.0), np.minimum(r_b, f32(FLT_MAX))).astype(f32)
    prod = (xb * r_b[:, :, None]).astype(f32)                 # rounded to FP32 first
    if sr_seed is None:
        q = encode_e2m1(prod.astype(np.float64)).reshape(R, C)
    else:
        words = rng.element_words(sr_seed, np.arange(R * C, dtype=np.uint64)).reshape(R, C)
        q = e2m1_stochastic(prod.reshape(R, C), words)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return packed, S, t


def quantize_per_token(x_bf16_bits: np.ndarray, sr_seed: int | None = None):
    """Per-token NVFP4: the FP32 scale's scope is one row (token) of x (T, H)."""
    x = bf16_bits_to_f32(x_bf16_bits)
    amax = np.max(np.abs(x), axis=1).astype(f32)
    return quantize_with_scope_amax(x, amax, sr_seed)


def quantize_per_tensor(x: np.ndarray, sr_seed: int | None = None):
    """Per-tensor NVFP4 over a float32 or BF16-bits (R, C) tensor; t is a scalar."""
    x = bf16_bits_to_f32(x) if x.dtype == np.uint16 else np.asarray(x, dtype=f32)
    A = f32(np.max(np.abs(x))) if x.size else f32(0.0)
    packed, S, _ = quantize_with_scope_amax(x, np.full(x.shape[0], A, dtype=f32), sr_seed)
    return packed, S, scope_scales(np.array([A], dtype=f32))[1]


def quantize_per_group(x: np.ndarray, row_offsets):
    """Per-group NVFP4: rows [off[g], off[g+1]) of x share one FP32 scale.

    Used for stacked expert weights (one scale per expert matrix; gate and up
    rows of one expert form one group). Returns t of shape (G,).
    """
    x = bf16_bits_to_f32(x) if x.dtype == np.uint16 else np.asarray(x, dtype=f32)
    off = np.asarray(row_offsets, dtype=np.int64)
    G = len(off) - 1
    amax_rows = np.zeros(x.shape[0], dtype=f32)
    amax_g = np.zeros(G, dtype=f32)
    for g in range(G):
        blk = x[off[g]:off[g + 1]]
        amax_g[g] = np.max(np.abs(blk)) if blk.size else f32(0.0)
        amax_rows[off[g]:off[g + 1]] = amax_g[g]
    packed, S, _ = quantize_with_scope_amax(x, amax_rows)
    return packed, S, scope_scales(amax_g)[1].astype(f32)


def quantize_2d(x: np.ndarray, scope_rows: int | None = None):
    """NVFP4 weights with one E4M3 scale per 16x16 block (2D block scaling).

    The pages: standard NVFP4 scales 1x16 blocks along the dot-product axis; the
    backward pass transposes the weight, so 1x16 blocks would give the forward
    and backward passes different quantized weights and break the chain rule;
    scaling the weights in 16x16 blocks makes both passes use one quantized
    representation, while activations and gradients keep 1x16 blocks
    (7minutos.es NVFP4 page, section "La metodologia de formacion de cuatro
    partes", the 2D weight-scaling item).

    Reading (the page gives no formula): the per-block steps of the 1x16
    quantizer with the block amax taken over the 16x16 block: A = amax over the
    scope (the tensor, or each group of `scope_rows` rows = one expert matrix);
    s_enc, t as scope_scales; S_b = E4M3_RNE_sat(fl(fl(a_b / 6) * s_enc));
    r_b = min(fl(s_enc / S_b), FLT_MAX) (0 if S_b = 0); q = E2M1_RNE_sat(fl(x * r_b)).

    x: (R, C), float32 or BF16 bits, R % 16 == C % 16 == 0.
    Returns (packed (R, C/2), S_rows (R, C/16), packedT (G*C, gr/2), S_T
    (G*C, gr/16), t (G,)) with G = R / gr scope groups. S_rows repeats each 16x16
    block's code for its 16 rows (the 1x16 form a K-contiguous GEMM consumes);
    packedT / S_T hold, group after group, the transpose of each group's rows in
    the same form (for one group: the transposed tensor), with identical codes.
    """
    x = bf16_bits_to_f32(x) if x.dtype == np.uint16 else np.asarray(x, dtype=f32)
    R, C = x.shape
    if R % BLOCK or C % BLOCK:
        raise ValueError("both axes must be multiples of 16")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    gr = R if scope_rows is None else int(scope_rows)
    if gr <= 0 or R % gr or gr % BLOCK:
        raise ValueError("scope rows must divide the rows and be a multiple of 16")
    G = R // gr
    amax_g = np.array([np.max(np.abs(x[g * gr:(g + 1) * gr])) if gr * C else 0.0 for g in range(G)], dtype=f32)
    s_enc_g, t = scope_scales(amax_g)
    s_enc = np.repeat(s_enc_g, gr // BLOCK)                         # per 16-row band
    xb = x.reshape(R // BLOCK, BLOCK, C // BLOCK, BLOCK)
    a_b = np.max(np.abs(xb), axis=(1, 3))                           # (R/16, C/16) exact
    d_b = ((a_b / f32(6.0)).astype(f32) * s_enc[:, None]).astype(f32)
    S = encode_e4m3(d_b.astype(np.float64))
    S_val = decode_e4m3(S).astype(f32)
    with np.errstate(divide="ignore", over="ignore"):
        r_b = (s_enc[:, None] / S_val).astype(f32)
    r_b = np.where(S_val == 0, f32(0.0), np.minimum(r_b, f32(FLT_MAX))).astype(f32)
    prod = (xb * r_b[:, None, :, None]).astype(f32)                # rounded to FP32 first
    q = encode_e2m1(prod.astype(np.float64)).reshape(R, C)
    pack = lambda codes: (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    S_rows = np.repeat(S, BLOCK, axis=0)                            # (R, C/16)
    # transposed copy per scope group (one expert matrix each): (G, C, gr) stacked as (G*C, gr)
    qT = np.concatenate([q[g * gr:(g + 1) * gr].T for g in range(G)], axis=0)
    S_T = np.concatenate([np.repeat(S[g * gr // BLOCK:(g + 1) * gr // BLOCK].T, BLOCK, axis=0) for g in range(G)], axis=0)
    return pack(q), S_rows, pack(np.ascontiguousarray(qT)), np.ascontiguousarray(S_T), t.astype(f32)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """uint8 (R, C/2) -> E2M1 codes (R, C): low nibble first."""
    R, Ch = packed.shape
    out = np.empty((R, 2 * Ch), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def dequantize_exact(packed, S, t_rows) -> np.ndarray:
    """Exact FP64 value q * S_b * t (<= 30 significant bits, so FP64 holds it exactly)."""
    q = decode_e2m1(unpack_codes(packed))
    R, C = q.shape
    Sv = np.repeat(decode_e4m3(S), BLOCK, axis=1)
    t = np.asarray(t_rows, dtype=f32).astype(np.float64).reshape(-1, 1)
    return q * Sv * t


def dequantize_f32(packed, S, t_rows) -> np.ndarray:
    """FP32 dequantization: v = fl(fl(q * S_b) * t); q * S_b is exact in FP32."""
    q = decode_e2m1(unpack_codes(packed)).astype(f32)
    Sv = np.repeat(decode_e4m3(S), BLOCK, axis=1).astype(f32)
    t = np.asarray(t_rows, dtype=f32).reshape(-1, 1)
    with np.errstate(over="ignore"):
        return ((q * Sv).astype(f32) * t).astype(f32)


def dequantize_bf16_bits(packed, S, t_rows) -> np.ndarray:
    """BF16 dequantization: the FP32 dequantization rounded once more to BF16 (RNE)."""
    return f32_to_bf16_bits(dequantize_f32(packed, S, t_rows))


# --------------------------------------------------------------------------
# Random Hadamard transform (16-point), FP32.
# --------------------------------------------------------------------------

def rht16_rows(x: np.ndarray, signs) -> np.ndarray:
    """Apply the 16-point RHT to every 16-chunk along the LAST axis of x (FP32)."""
    x = np.asarray(x, dtype=f32)
    s = np.asarray(signs, dtype=f32).reshape(16)
    if not np.all(np.abs(s) == 1):
        raise ValueError("signs must be +-1")
    R, C = x.shape
    if C % 16:
        raise ValueError("transformed axis must be a multiple of 16")
    w = (x.reshape(R, C // 16, 16) * s).astype(f32)          # exact sign flips
    h = 1
    while h < 16:
        nxt = w.copy()
        for i in range(16):
            if i & h:
                continue
            a, b = w[..., i], w[..., i + h]
            nxt[..., i] = (a + b).astype(f32)
            nxt[..., i + h] = (a - b).astype(f32)
        w = nxt
        h *= 2
    return (w * f32(0.25)).astype(f32).reshape(R, C)


def rht_quantize_colwise_per_tensor(x_bf16_bits: np.ndarray, signs, sr_seed: int | None = None):
    """Weight-gradient operand: RHT along the rows of x (R, C) (the reduction
    axis of dW = dY^T X), then per-tensor NVFP4 with 1x16 blocks along that
    same axis, stored transposed as (C, R).
    Returns (packed (C, R/2), S (C, R/16), t (1,)).
    """
    x = bf16_bits_to_f32(x_bf16_bits)
    u = rht16_rows(np.ascontiguousarray(x.T), signs)         # (C, R): chunks along R
    return quantize_per_tensor(u, sr_seed)
