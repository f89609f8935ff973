"""Seeded synthetic inputs for the five workloads (shared by tests and bench).

This module holds input generation only -- no step of the quantize / GEMM
method. Both the device path and the CPU oracle consume the exact BF16 bit
patterns (uint16 arrays) produced here.

Conventions:
  * generator = numpy default_rng(SeedSequence([workload_id, tensor_id]));
  * samples drawn in FP64, cast to FP32, then to BF16 by round-to-nearest-even;
  * N(mu, sigma): the second parameter is the standard deviation;
  * routing logits are FP32; top-k routing picks the k largest logits (ties to
    the lower expert index); the combine weights are the softmax over all
    experts restricted to the chosen k and renormalised, listed in descending
    weight order; slots are laid out expert-major, tokens ascending inside an
    expert.

Shapes follow the workloads named by the MXFP8 linear-layer memory check
(input (2048, 2048), out_features 8192) and the MoE models the pages discuss
(Qwen3-30B-A3B-like: hidden 2048, 128 experts, intermediate 768, top-8;
DeepSeek-V3-like: hidden 7168, 256 routed + 1 shared expert, intermediate
2048, top-8).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def rng(workload: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([workload, tensor]))


def to_bf16_bits(x) -> np.ndarray:
    """FP64/FP32 -> FP32 -> BF16 bits, round-to-nearest-even (finite inputs)."""
    b = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_float(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(g: np.random.Generator, shape, std=1.0) -> np.ndarray:
    return to_bf16_bits(g.standard_normal(shape) * std)


# --------------------------------------------------------------------------
# Workload 1: small MXFP8 case (256x512 with 1% outliers x100, second operand 512x256)
# --------------------------------------------------------------------------

def outlier_normal_bf16(g: np.random.Generator, shape, frac=0.01, mult=100.0) -> np.ndarray:
    x = g.standard_normal(shape)
    n = x.size
    k = int(round(frac * n))
    idx = g.choice(n, size=k, replace=False)
    x.reshape(-1)[idx] *= mult
    return to_bf16_bits(x)


def workload_small_mxfp8():
    """X (256, 512) ~ N(0,1) with 1% of entries x100; W2 (512, 256) likewise."""
    x = outlier_normal_bf16(rng(1, 0), (256, 512))
    w2 = outlier_normal_bf16(rng(1, 1), (512, 256))
    return {"x": x, "w2": w2}


# --------------------------------------------------------------------------
# Workload 2: MXFP8 linear layer, input (2048, 2048), out_features 8192
# --------------------------------------------------------------------------

def workload_linear_mxfp8(tokens=2048, d_in=2048, d_out=8192):
    x = normal_bf16(rng(2, 0), (tokens, d_in), 1.0)
    w = normal_bf16(rng(2, 1), (d_out, d_in), 0.02)
    dy = normal_bf16(rng(2, 2), (tokens, d_out), 1e-3)
    return {"x": x, "w": w, "dy": dy}


# --------------------------------------------------------------------------
# MoE routing
# --------------------------------------------------------------------------

@dataclass
class Routing:
    topk_idx: np.ndarray      # (T, k) int32, descending weight order
    topk_w: np.ndarray        # (T, k) float32
    offsets: np.ndarray       # (G+1,) int64 slot offsets per expert
    row_index: np.ndarray     # (S,) int32 token of each slot (expert-major)
    slot_of: np.ndarray       # (T, k) int64 slot holding token t's j-th choice


def route_topk(logits: np.ndarray, k: int, pad: int = 1) -> Routing:
    """Top-k routing of FP32 logits (T, G). With pad > 1 every expert's slot range
    starts at a multiple of `pad` (its length rounded up); padding slots carry
    row_index -1 and are never named by slot_of."""
    logits = np.asarray(logits, dtype=np.float32)
    T, G = logits.shape
    # stable sort on -logit: ties keep the lower expert index first
    order = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :k]
    lg = logits.astype(np.float64)
    m = lg.max(axis=1, keepdims=True)
    p = np.exp(lg - m)
    p /= p.sum(axis=1, keepdims=True)
    pk = np.take_along_axis(p, order, axis=1)
    pk /= pk.sum(axis=1, keepdims=True)
    w = pk.astype(np.float32)
    # order is by descending logit == descending weight
    counts = np.bincount(order.reshape(-1), minlength=G)
    padded = (counts + pad - 1) // pad * pad
    offsets = np.zeros(G + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    flat_e = order.reshape(-1)
    flat_t = np.repeat(np.arange(T), k)
    flat_j = np.tile(np.arange(k), T)
    perm = np.lexsort((flat_t, flat_e))          # expert-major, token ascending
    e_sorted = flat_e[perm]
    first = np.zeros(G + 1, dtype=np.int64)
    first[1:] = np.cumsum(counts)
    slot = offsets[e_sorted] + (np.arange(T * k) - first[e_sorted])
    row_index = np.full(int(offsets[-1]), -1, dtype=np.int32)
    row_index[slot] = flat_t[perm]
    slot_of = np.empty((T, k), dtype=np.int64)
    slot_of[flat_t[perm], flat_j[perm]] = slot
    return Routing(order.astype(np.int32), w, offsets, row_index, slot_of)


# --------------------------------------------------------------------------
# Workload 3: per-token NVFP4 MoE layer, Qwen3-30B-A3B-like shapes
# --------------------------------------------------------------------------

def workload_moe_qwen3(tokens=4096, hidden=2048, experts=128, inter=768, topk=8,
                       with_weights=True):
    g = rng(3, 0)
    mag = rng(3, 1).lognormal(0.0, 1.0, size=(tokens, 1))
    x = to_bf16_bits(g.standard_normal((tokens, hidden)) * mag)
    logits = rng(3, 2).standard_normal((tokens, experts)).astype(np.float32)
    out = {"x": x, "logits": logits, "routing": route_topk(logits, topk),
           "hidden": hidden, "experts": experts, "inter": inter, "topk": topk}
    if with_weights:
        out["w_gu"] = normal_bf16(rng(3, 3), (experts, 2 * inter, hidden), 0.02)
        out["w_d"] = normal_bf16(rng(3, 4), (experts, hidden, inter), 0.02)
    return out


# --------------------------------------------------------------------------
# Workload 4: DeepSeek-V3-shaped MoE layer (routed NVFP4 experts + BF16 shared expert)
# --------------------------------------------------------------------------

def workload_moe_deepseek(tokens=16384, hidden=7168, experts=256, inter=2048, topk=8, pad=32):
    """Activations and routing on the host (numpy, as above). The expert weights and
    the synthetic upstream gradients are ~11 G and ~1.6 G values: they are drawn on
    the device by `deepseek_device_tensors`."""
    x = normal_bf16(rng(4, 0), (tokens, hidden), 1.0)
    logits = rng(4, 1).standard_normal((tokens, experts)).astype(np.float32)
    return {"x": x, "logits": logits, "routing": route_topk(logits, topk, pad=pad), "hidden": hidden,
            "experts": experts, "inter": inter, "topk": topk}


def device_normal_bf16(torch, dev, shape, std, seed):
    """N(0, std) drawn in FP32 by torch's seeded device generator (Philox), rounded
    to BF16 (RNE). Used where a host draw of the tensor would take minutes."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * std).to(torch.bfloat16)


def deepseek_device_tensors(torch, dev, w, shared=True, grads=True):
    """Routed expert weights W_gu (G*2I, H) (gate rows then up rows per expert) and
    W_d (G*H, I), ~N(0, 0.02); the shared expert's W_sgu (2I, H) and W_sd (H, I);
    synthetic upstream gradients ~N(0, 1e-3) of the routed down / gate_up outputs
    (padding slots zero) and of the shared expert's outputs. Seeds 4000 + tensor id."""
    H, G, I = w["hidden"], w["experts"], w["inter"]
    S = int(w["routing"].offsets[-1])
    T = w["x"].shape[0]
    out = {"w_gu": device_normal_bf16(torch, dev, (G * 2 * I, H), 0.02, 4002),
           "w_d": device_normal_bf16(torch, dev, (G * H, I), 0.02, 4003)}
    if shared:
        out["w_sgu"] = device_normal_bf16(torch, dev, (2 * I, H), 0.02, 4004)
        out["w_sd"] = device_normal_bf16(torch, dev, (H, I), 0.02, 4005)
    if grads:
        live = torch.from_numpy(w["routing"].row_index >= 0).to(dev)[:, None]
        out["d_o"] = device_normal_bf16(torch, dev, (S, H), 1e-3, 4006) * live
        out["d_gu"] = device_normal_bf16(torch, dev, (S, 2 * I), 1e-3, 4007) * live
        if shared:
            out["d_os"] = device_normal_bf16(torch, dev, (T, H), 1e-3, 4008)
            out["d_gus"] = device_normal_bf16(torch, dev, (T, 2 * I), 1e-3, 4009)
    return out


# --------------------------------------------------------------------------
# Workload 5: heavy-tailed 8192x8192 stress case
# --------------------------------------------------------------------------

def student_t_with_injections(workload: int, tensor: int, n=8192):
    """Student-t(3) (n, n) with seeded injections (positions reported):
      * one all-zero 32x32 tile;
      * one 32x32 tile whose every row and column maximum is exactly 448
        (448 on a permutation pattern, |noise| < 448 elsewhere);
      * one 16-run along a row of 6 * 2^j times E2M1 grid values;
      * one 32x32 tile of BF16 subnormals (random multiples of 2^-133).
    """
    g = rng(workload, tensor)
    x = g.standard_t(3.0, size=(n, n))
    tiles = n // 32
    picks = g.choice(tiles * tiles, size=4, replace=False)
    pos = [(int(p // tiles) * 32, int(p % tiles) * 32) for p in picks]
    r, c = pos[0]
    x[r:r + 32, c:c + 32] = 0.0
    r, c = pos[1]
    blk = g.uniform(-400.0, 400.0, size=(32, 32))
    perm = g.permutation(32)
    blk[np.arange(32), perm] = 448.0 * g.choice([-1.0, 1.0], size=32)
    x[r:r + 32, c:c + 32] = blk
    r, c = pos[2]
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    j = int(g.integers(-4, 5))
    run = grid[g.integers(0, 8, size=16)] * 6.0 * 2.0 ** j * g.choice([-1.0, 1.0], size=16)
    run[int(g.integers(0, 16))] = 6.0 * 6.0 * 2.0 ** j
    x[r, c:c + 16] = run
    r, c = pos[3]
    x[r:r + 32, c:c + 32] = g.integers(-127, 128, size=(32, 32)) * 2.0 ** -133
    return to_bf16_bits(x), {"zero": pos[0], "max448": pos[1], "e2m1_run": pos[2],
                             "subnormal": pos[3]}


def workload_stress(n=8192):
    a, pa = student_t_with_injections(5, 0, n)
    b, pb = student_t_with_injections(5, 1, n)
    signs = rng(5, 2).choice(np.array([-1, 1], dtype=np.int8), size=16)
    return {"a": a, "b": b, "signs": signs, "inject_a": pa, "inject_b": pb}
