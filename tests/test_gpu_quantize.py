"""GPU parity: MXFP8 / NVFP4 quantizers and dequantize through the C ABI against
the CPU oracle, byte for byte (quantized codes, scales and FP32 scales)."""

import numpy as np
import pytest
import torch

import microscaling_precision_quantization_amd as mxq
from microscaling_precision_quantization_amd import inputs
from oracle import formats as F
from oracle import mxfp8 as omx
from oracle import nvfp4 as onv
from tests.gpu_util import assert_bytes_equal, dev_bf16, host

pytestmark = pytest.mark.gpu


def bf16(v):
    return inputs.to_bf16_bits(np.asarray(v, dtype=np.float64))


def check_mxfp8(xb, rowwise=True, colwise=True, what="", x_dev=None):
    x = dev_bf16(xb) if x_dev is None else x_dev
    qr, sr, qc, sc = mxq.quantize_mxfp8(x, rowwise, colwise)
    if rowwise:
        eq, es = omx.quantize_rowwise(xb)
        assert_bytes_equal(host(qr), eq, f"{what} q_row")
        assert_bytes_equal(host(sr), es, f"{what} s_row")
    if colwise:
        eq, es = omx.quantize_colwise(xb)
        assert_bytes_equal(host(qc), eq, f"{what} q_colT")
        assert_bytes_equal(host(sc), es, f"{what} s_colT")
    return qr, sr, qc, sc


def edge_case_tensor(rows=64, cols=256, seed=0):
    """Blocks of zeros, -0, the largest BF16, exact 448 grids, BF16 subnormals,
    mixed-sign tiny values and random data."""
    g = np.random.default_rng(seed)
    x = g.standard_normal((rows, cols)) * 3
    x[0:32, 0:32] = 0.0
    xb = bf16(x)
    xb[0:32, 0:32][::3, ::5] = 0x8000                       # -0 inside a zero block
    xb[32, 32:64] = 0x7F7F                                   # largest BF16
    xb[33, 32:64] = 0xFF7F
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    xb[34, 64:96] = bf16(448 * g.choice([-1, 1], 32) * (g.random(32) < 0.5))
    xb[35, 96:128] = bf16(grid[g.integers(0, 8, 32)] * 6 * 2.0 ** -3)
    xb[36:68 if rows >= 68 else rows, 128:160] = bf16(g.integers(-127, 128, (min(32, rows - 36), 32)) * 2.0 ** -133)
    xb[37, 160:192] = bf16(g.standard_normal(32) * 1e-30)
    return xb


def test_mxfp8_small_workload():
    w = inputs.workload_small_mxfp8()
    check_mxfp8(w["x"], what="X 256x512")
    check_mxfp8(w["w2"], what="W2 512x256")


@pytest.mark.parametrize("shape", [(32, 32), (96, 160), (160, 96), (4128, 96), (64, 416)])
def test_mxfp8_ragged_tiles(shape):
    g = inputs.rng(90, shape[0] * 7 + shape[1])
    xb = inputs.normal_bf16(g, shape, 2.0)
    check_mxfp8(xb, what=str(shape))


@pytest.mark.parametrize("shape", [(37, 64), (1, 32), (129, 160)])
def test_mxfp8_rowwise_only_any_rows(shape):
    xb = inputs.normal_bf16(inputs.rng(91, shape[0]), shape, 1.0)
    check_mxfp8(xb, rowwise=True, colwise=False, what=f"rowwise {shape}")


def test_mxfp8_colwise_only_and_strided_input():
    xb = inputs.normal_bf16(inputs.rng(92, 0), (64, 320), 1.0)
    wide = dev_bf16(xb)
    sub = wide[:, :256]                                         # ld_x = 320 > cols
    check_mxfp8(np.ascontiguousarray(xb[:, :256]), rowwise=True, colwise=True, what="strided", x_dev=sub)
    check_mxfp8(xb, rowwise=False, colwise=True, what="colwise only")


def test_mxfp8_edge_blocks():
    check_mxfp8(edge_case_tensor(), what="edge cases")


def test_mxfp8_linear_layer_full_size_and_deterministic():
    w = inputs.workload_linear_mxfp8()
    for name in ("x", "w", "dy"):
        first = check_mxfp8(w[name], what=name)
        again = mxq.quantize_mxfp8(dev_bf16(w[name]))
        for a, b in zip(first, again):
            assert_bytes_equal(host(a), host(b), f"{name} rerun")


def test_mxfp8_stress_full_size_sampled():
    n = 8192
    xb, inj = inputs.student_t_with_injections(5, 0, n)
    qr, sr, qc, sc = mxq.quantize_mxfp8(dev_bf16(xb))
    qr, sr, qc, sc = host(qr), host(sr), host(qc), host(sc)
    g = np.random.default_rng(1)
    bands = set(g.choice(n // 32, size=12, replace=False).tolist())
    bands |= {r // 32 for r, _ in inj.values()}
    for b in sorted(bands):
        r0 = b * 32
        eq, es = omx.quantize_rowwise(xb[r0:r0 + 32])
        assert_bytes_equal(qr[r0:r0 + 32], eq, f"band {b} rowwise")
        assert_bytes_equal(sr[r0:r0 + 32], es, f"band {b} rowwise scales")
        eq, es = omx.quantize_colwise(xb[r0:r0 + 32])
        assert_bytes_equal(qc[:, r0:r0 + 32], eq, f"band {b} colwise")
        assert_bytes_equal(sc[:, b:b + 1], es, f"band {b} colwise scales")


def test_mxfp8_multi_matches_single_calls():
    """One launch over several tensors writes exactly the bytes of one call per tensor."""
    g = inputs.rng(95, 0)
    shapes = [(4128, 96), (32, 32), (0, 64), (256, 544), (96, 160)]
    xs = [inputs.to_bf16_bits(g.standard_normal(sh) * g.lognormal(0, 2, (sh[0], 1))) for sh in shapes]
    dx = [dev_bf16(x) for x in xs]
    outs = [tuple(torch.empty(s, dtype=torch.uint8, device="cuda") for s in ((r, c), (r, c // 32), (c, r), (c, r // 32)))
            for r, c in shapes]
    mxq.quantize_mxfp8_multi(dx, outs)
    for x, o, sh in zip(dx, outs, shapes):
        if sh[0] == 0:
            continue
        ref = mxq.quantize_mxfp8(x)
        for a, b, nm in zip(o, ref, ("q_row", "s_row", "q_colT", "s_colT")):
            assert_bytes_equal(host(a), host(b), f"multi {sh} {nm}")
    # rowwise only, rows not a multiple of 32
    xs2 = [dev_bf16(inputs.normal_bf16(g, (37, 64), 1.0)), dev_bf16(inputs.normal_bf16(g, (1, 128), 1.0))]
    outs2 = [(torch.empty((37, 64), dtype=torch.uint8, device="cuda"), torch.empty((37, 2), dtype=torch.uint8, device="cuda"),
              None, None),
             (torch.empty((1, 128), dtype=torch.uint8, device="cuda"), torch.empty((1, 4), dtype=torch.uint8, device="cuda"),
              None, None)]
    mxq.quantize_mxfp8_multi(xs2, outs2)
    for x, o in zip(xs2, outs2):
        ref = mxq.quantize_mxfp8(x, colwise=False)
        assert_bytes_equal(host(o[0]), host(ref[0]), "multi rowwise q")
        assert_bytes_equal(host(o[1]), host(ref[1]), "multi rowwise s")


# ------------------------------- NVFP4 -------------------------------------

def check_token(xb, what=""):
    q, s, t = mxq.quantize_nvfp4_per_token(dev_bf16(xb))
    eq, es, et = onv.quantize_per_token(xb)
    assert_bytes_equal(host(q), eq, f"{what} packed")
    assert_bytes_equal(host(s), es, f"{what} block scales")
    assert_bytes_equal(host(t).view(np.uint32), et.view(np.uint32), f"{what} token scales")
    return q, s, t


@pytest.mark.parametrize("hidden", [16, 48, 512, 2048, 7168, 8208, 16384])
def test_nvfp4_per_token_row_lengths(hidden):
    g = inputs.rng(93, hidden)
    xb = inputs.to_bf16_bits(g.standard_normal((9, hidden)) * g.lognormal(0, 2, (9, 1)))
    check_token(xb, what=f"H={hidden}")


def test_nvfp4_per_token_moe_activations():
    w = inputs.workload_moe_qwen3(with_weights=False)
    check_token(w["x"], what="4096x2048")


def test_nvfp4_per_token_edge_cases():
    xb = edge_case_tensor(rows=48, cols=256, seed=4)
    xb[40] = 0                                                 # all-zero token
    xb[41] = 0x7F7F                                            # all largest BF16
    xb[42, :16] = bf16(np.full(16, 2688.0))
    check_token(xb, what="edge")


def test_nvfp4_per_token_batch_invariance_on_device():
    g = inputs.rng(94, 0)
    xb = inputs.to_bf16_bits(g.standard_normal((64, 1024)) * g.lognormal(0, 1, (64, 1)))
    q, s, t = mxq.quantize_nvfp4_per_token(dev_bf16(xb))
    q, s, t = host(q), host(s), host(t)
    perm = g.permutation(64)
    q2, s2, t2 = (host(a) for a in mxq.quantize_nvfp4_per_token(dev_bf16(xb[perm])))
    assert_bytes_equal(q2, q[perm], "permuted batch")
    assert_bytes_equal(s2, s[perm], "permuted batch scales")
    for r in (0, 31, 63):
        q1, s1, t1 = (host(a) for a in mxq.quantize_nvfp4_per_token(dev_bf16(xb[r:r + 1])))
        assert_bytes_equal(q1[0], q[r], f"token {r} alone")
        assert t1[0] == t[r]


def test_nvfp4_per_token_deepseek_activations_sampled():
    g = inputs.rng(4, 0)
    T, H = 16384, 7168
    xb = inputs.normal_bf16(g, (T, H), 1.0)
    q, s, t = (host(a) for a in mxq.quantize_nvfp4_per_token(dev_bf16(xb)))
    rows = np.random.default_rng(2).choice(T, 256, replace=False)
    eq, es, et = onv.quantize_per_token(xb[rows])
    assert_bytes_equal(q[rows], eq, "sampled packed")
    assert_bytes_equal(s[rows], es, "sampled scales")
    assert_bytes_equal(t[rows].view(np.uint32), et.view(np.uint32), "sampled token scales")


def test_nvfp4_strided_input_all_scopes():
    """A row stride above the column count (rows not stored back to back): the scope
    maxima take the per-row pass instead of the flat reduction; bytes against the oracle
    on the contiguous copy for token, tensor and group scopes."""
    g = inputs.rng(95, 2)
    G, N, K = 3, 64, 512
    xb = inputs.to_bf16_bits(g.standard_normal((G * N, K + 96)) * np.exp2(g.integers(-8, 8, (G * N, 1))))
    wide = dev_bf16(xb)
    sub = wide[:, :K]                                           # ld_x = K + 96
    x = np.ascontiguousarray(xb[:, :K])
    q, s, t = mxq.quantize_nvfp4_per_token(sub)
    eq, es, et = onv.quantize_per_token(x)
    assert_bytes_equal(host(q), eq, "strided token packed")
    assert_bytes_equal(host(t).view(np.uint32), et.view(np.uint32), "strided token t")
    q, s, t = mxq.quantize_nvfp4(sub, scope="tensor")
    eq, es, et = onv.quantize_per_tensor(x)
    assert_bytes_equal(host(q), eq, "strided tensor packed")
    assert_bytes_equal(host(s), es, "strided tensor scales")
    assert_bytes_equal(host(t).view(np.uint32), et.view(np.uint32), "strided tensor t")
    q, s, t = mxq.quantize_nvfp4(sub, scope="group", group_rows=N)
    eq, es, et = onv.quantize_per_group(x, np.arange(G + 1) * N)
    assert_bytes_equal(host(q), eq, "strided group packed")
    assert_bytes_equal(host(t).view(np.uint32), et.view(np.uint32), "strided group t")


def test_nvfp4_group_amax_at_group_edges():
    """Contiguous groups large enough that each group's maximum is reduced in 64 parts:
    every group's maximum sits on its last element, next to a larger first element of
    the following group; all-zero group included. Bytes and t against the oracle."""
    g = inputs.rng(95, 1)
    G, N, K = 5, 256, 4096
    x = g.standard_normal((G * N, K)) * 0.02
    for e in range(G):
        x[e * N + N - 1, K - 1] = 3.0 * (e + 1)          # group maximum, last element
        if e + 1 < G:
            x[(e + 1) * N, 0] = -50.0 * (e + 2)          # the next group's first element, larger
    x[2 * N:3 * N] = 0.0
    wb = inputs.to_bf16_bits(x)
    q, s, t = mxq.quantize_nvfp4(dev_bf16(wb), scope="group", group_rows=N)
    eq, es, et = onv.quantize_per_group(wb, np.arange(G + 1) * N)
    assert_bytes_equal(host(t).view(np.uint32), et.view(np.uint32), "group t")
    assert_bytes_equal(host(q), eq, "group packed")
    assert_bytes_equal(host(s), es, "group scales")


def test_nvfp4_per_tensor_and_group_weights():
    g = inputs.rng(95, 0)
    G, N, K = 5, 96, 256
    wb = inputs.normal_bf16(g, (G * N, K), 0.02)
    q, s, t = mxq.quantize_nvfp4(dev_bf16(wb), scope="group", group_rows=N)
    eq, es, et = onv.quantize_per_group(wb, np.arange(G + 1) * N)
    assert_bytes_equal(host(q), eq, "group packed")
    assert_bytes_equal(host(s), es, "group scales")
    assert_bytes_equal(host(t).view(np.uint32), et.view(np.uint32), "group t")
    q, s, t = mxq.quantize_nvfp4(dev_bf16(wb), scope="tensor")
    eq, es, et = onv.quantize_per_tensor(wb)
    assert_bytes_equal(host(q), eq, "tensor packed")
    assert_bytes_equal(host(s), es, "tensor scales")
    assert_bytes_equal(host(t).view(np.uint32), et.view(np.uint32), "tensor t")


@pytest.mark.parametrize("rht", [False, True])
@pytest.mark.parametrize("shape", [(64, 48), (256, 520), (48, 1040)])
def test_nvfp4_transposed_per_tensor(rht, shape):
    g = inputs.rng(96, shape[0] + shape[1] + rht)
    xb = inputs.to_bf16_bits(g.standard_t(3.0, size=shape))
    signs = np.where(g.random(16) < 0.5, -1, 1).astype(np.int8)
    q, s, t = mxq.quantize_nvfp4(dev_bf16(xb), scope="tensor", transpose=True, rht_signs=signs if rht else None)
    if rht:
        eq, es, et = onv.rht_quantize_colwise_per_tensor(xb, signs)
    else:
        eq, es, et = onv.quantize_per_tensor(np.ascontiguousarray(inputs.bf16_bits_to_float(xb).T))
    assert_bytes_equal(host(q), eq, "transposed packed")
    assert_bytes_equal(host(s), es, "transposed scales")
    assert_bytes_equal(host(t).view(np.uint32), et.view(np.uint32), "transposed t")


def test_nvfp4_rowwise_rht_per_tensor():
    g = inputs.rng(97, 0)
    xb = inputs.to_bf16_bits(g.standard_t(3.0, size=(40, 1024)))
    signs = np.where(g.random(16) < 0.5, -1, 1).astype(np.int8)
    q, s, t = mxq.quantize_nvfp4(dev_bf16(xb), scope="tensor", rht_signs=signs)
    u = onv.rht16_rows(inputs.bf16_bits_to_float(xb), signs)
    eq, es, et = onv.quantize_per_tensor(u)
    assert_bytes_equal(host(q), eq, "row rht packed")
    assert_bytes_equal(host(s), es, "row rht scales")


def test_nvfp4_transposed_group_scope():
    g = inputs.rng(98, 0)
    xb = inputs.normal_bf16(g, (64, 96), 1.0)
    q, s, t = mxq.quantize_nvfp4(dev_bf16(xb), scope="group", group_rows=32, transpose=True)
    xt = np.ascontiguousarray(inputs.bf16_bits_to_float(xb).T)
    eq, es, et = onv.quantize_per_group(xt, [0, 32, 64, 96])
    assert_bytes_equal(host(q), eq, "transposed group packed")
    assert_bytes_equal(host(t).view(np.uint32), et.view(np.uint32), "transposed group t")


def test_nvfp4_stress_rht_full_size_sampled():
    n = 8192
    xb, _ = inputs.student_t_with_injections(5, 0, n)
    signs = inputs.rng(5, 2).choice(np.array([-1, 1], dtype=np.int8), size=16)
    q, s, t = (host(a) for a in mxq.quantize_nvfp4(dev_bf16(xb), scope="tensor", transpose=True, rht_signs=signs))
    t_dev = t
    # the tensor amax is global: take it from the oracle on the full transform, check sampled rows bit-exactly
    x = inputs.bf16_bits_to_float(xb)
    cols = np.random.default_rng(3).choice(n, 64, replace=False)
    u_all_amax = np.float32(0)
    for c0 in range(0, n, 1024):
        u = onv.rht16_rows(np.ascontiguousarray(x[:, c0:c0 + 1024].T), signs)
        u_all_amax = max(u_all_amax, np.float32(np.max(np.abs(u))))
    _, et = onv.scope_scales(np.array([u_all_amax], dtype=np.float32))
    assert t_dev.view(np.uint32)[0] == et.view(np.uint32)[0]
    u = onv.rht16_rows(np.ascontiguousarray(x[:, cols].T), signs)
    eq, es, _ = onv.quantize_with_scope_amax(u, np.full(len(cols), u_all_amax, dtype=np.float32))
    assert_bytes_equal(q[cols], eq, "sampled RHT packed")
    assert_bytes_equal(s[cols], es, "sampled RHT scales")


@pytest.mark.parametrize("shape,group", [((96, 160), None), ((256, 512), 64), ((272, 48), None), ((512, 2048), 256),
                                         ((1024, 7168), 512), ((144, 64), 48), ((64, 96), 16), ((768, 256), 256)])
def test_nvfp4_2d_weights(shape, group):
    g = inputs.rng(96, shape[0] + shape[1])
    wb = inputs.to_bf16_bits(g.standard_normal(shape) * 0.02 * g.lognormal(0, 1, (shape[0], 1)))
    scope = "tensor" if group is None else "group"
    q, s, qt, st, t = mxq.quantize_nvfp4_2d(dev_bf16(wb), scope=scope, group_rows=group or 0)
    eq, es, eqt, est, et = onv.quantize_2d(wb, scope_rows=group)
    assert_bytes_equal(host(q), eq, "2d packed")
    assert_bytes_equal(host(s), es, "2d scales")
    assert_bytes_equal(host(qt), eqt, "2d transposed packed")
    assert_bytes_equal(host(st), est, "2d transposed scales")
    assert_bytes_equal(host(t).view(np.uint32), et.view(np.uint32), "2d t")
    # one copy at a time writes the same bytes
    q1, s1, _, _, _ = mxq.quantize_nvfp4_2d(dev_bf16(wb), scope=scope, group_rows=group or 0, colwise=False)
    _, _, qt1, st1, _ = mxq.quantize_nvfp4_2d(dev_bf16(wb), scope=scope, group_rows=group or 0, rowwise=False)
    assert_bytes_equal(host(q1), eq, "2d row only")
    assert_bytes_equal(host(qt1), eqt, "2d col only")
    assert_bytes_equal(host(st1), est, "2d col only scales")


@pytest.mark.parametrize("shape,seed", [((64, 2048), 1), ((33, 7168), 0xDEADBEEF12345678), ((128, 48), 7)])
def test_nvfp4_stochastic_per_token(shape, seed):
    g = inputs.rng(98, shape[1])
    xb = inputs.to_bf16_bits(g.standard_normal(shape) * 1e-3 * g.lognormal(0, 1, (shape[0], 1)))
    q, s, t = mxq.quantize_nvfp4(dev_bf16(xb), scope="row", sr_seed=seed)
    eq, es, et = onv.quantize_per_token(xb, sr_seed=seed)
    assert_bytes_equal(host(q), eq, "sr packed")
    assert_bytes_equal(host(s), es, "sr scales")
    assert_bytes_equal(host(t).view(np.uint32), et.view(np.uint32), "sr t")


def test_nvfp4_stochastic_tensor_and_group():
    g = inputs.rng(98, 1)
    xb = inputs.normal_bf16(g, (96, 256), 1e-3)
    q, s, t = mxq.quantize_nvfp4(dev_bf16(xb), scope="tensor", sr_seed=42)
    eq, es, et = onv.quantize_per_tensor(xb, sr_seed=42)
    assert_bytes_equal(host(q), eq, "sr tensor packed")
    assert_bytes_equal(host(t).view(np.uint32), et.view(np.uint32), "sr tensor t")
    q, s, t = mxq.quantize_nvfp4(dev_bf16(xb), scope="group", group_rows=32, sr_seed=43)
    x = inputs.bf16_bits_to_float(xb)
    amax = np.repeat(np.max(np.abs(x.reshape(3, 32, 256)), axis=(1, 2)).astype(np.float32), 32)
    eq, es, _ = onv.quantize_with_scope_amax(x, amax, sr_seed=43)
    assert_bytes_equal(host(q), eq, "sr group packed")
    assert_bytes_equal(host(s), es, "sr group scales")


@pytest.mark.parametrize("shape", [(256, 520), (64, 48), (528, 256)])
def test_nvfp4_stochastic_rht_transposed(shape):
    g = inputs.rng(98, shape[0] * 3 + shape[1])
    xb = inputs.to_bf16_bits(g.standard_t(3.0, size=shape) * 1e-3)
    signs = np.where(g.random(16) < 0.5, -1, 1).astype(np.int8)
    q, s, t = mxq.quantize_nvfp4(dev_bf16(xb), scope="tensor", transpose=True, rht_signs=signs, sr_seed=99)
    eq, es, et = onv.rht_quantize_colwise_per_tensor(xb, signs, sr_seed=99)
    assert_bytes_equal(host(q), eq, "sr rht packed")
    assert_bytes_equal(host(s), es, "sr rht scales")
    assert_bytes_equal(host(t).view(np.uint32), et.view(np.uint32), "sr rht t")


# ------------------------------ dequantize ---------------------------------

def test_dequantize_mxfp8_and_nvfp4():
    xb = edge_case_tensor(rows=64, cols=256, seed=5)
    qr, sr, _, _ = mxq.quantize_mxfp8(dev_bf16(xb), True, False)
    qh, sh = host(qr), host(sr)
    f32 = host(mxq.dequantize(mxq.MXFP8, qr, sr, out_dtype=torch.float32))
    assert_bytes_equal(f32.view(np.uint32), omx.dequantize_f32(qh, sh).view(np.uint32), "mxfp8 -> f32")
    b16 = host(mxq.dequantize(mxq.MXFP8, qr, sr))
    assert_bytes_equal(b16, F.f32_to_bf16_bits(omx.dequantize_f32(qh, sh)), "mxfp8 -> bf16")
    q, s, t = mxq.quantize_nvfp4_per_token(dev_bf16(xb))
    qh, sh, th = host(q), host(s), host(t)
    f32 = host(mxq.dequantize(mxq.NVFP4, q, s, t, t_scope="row", out_dtype=torch.float32))
    assert_bytes_equal(f32.view(np.uint32), onv.dequantize_f32(qh, sh, th).view(np.uint32), "nvfp4 -> f32")
    b16 = host(mxq.dequantize(mxq.NVFP4, q, s, t, t_scope="row"))
    assert_bytes_equal(b16, onv.dequantize_bf16_bits(qh, sh, th), "nvfp4 -> bf16")
    wb = inputs.normal_bf16(inputs.rng(99, 0), (4 * 32, 64), 0.02)
    q, s, t = mxq.quantize_nvfp4(dev_bf16(wb), scope="group", group_rows=32)
    b16 = host(mxq.dequantize(mxq.NVFP4, q, s, t, t_scope="group", group_rows=32))
    t_rows = np.repeat(host(t), 32)
    assert_bytes_equal(b16, onv.dequantize_bf16_bits(host(q), host(s), t_rows), "nvfp4 group -> bf16")


# -------------------- scope-scale overflow (FLT_MAX) branches --------------------

def subnormal_scope_rows(g, rows=32, cols=256):
    """Rows whose every value is a BF16 subnormal (|x| <= 127 * 2^-133), so every scope
    amax A is below 2688 / FLT_MAX: s_enc overflows to FLT_MAX and r_b clamps to FLT_MAX.
    Row 0 is the hand-worked token [2^-127, -2^-128, 3 * 2^-129, 0 ...]."""
    v = g.integers(-127, 128, (rows, cols))                  # value v * 2^-133: BF16 bits |v| (+ sign)
    xb = (np.abs(v) | np.where(v < 0, 0x8000, 0)).astype(np.uint16)
    xb[0] = 0
    xb[0, :3] = [0x0040, 0x8020, 0x0030]
    xb[1, :] = 0x0001                                        # the smallest subnormal everywhere
    xb[2, 16:] = 0                                           # one subnormal block, zeros after
    return xb


def test_nvfp4_scope_overflow_branch_per_token():
    xb = subnormal_scope_rows(inputs.rng(96, 0))
    q, s, t = check_token(xb, what="subnormal tokens")
    # the hand-worked values of the oracle pin, on the device
    assert host(t).view(np.uint32)[0] == 0x00200000
    assert list(host(s)[0, :2]) == [0x2B, 0x00] and list(host(q)[0, :2]) == [0xA4, 0x03]


def test_nvfp4_scope_overflow_branch_tensor_group_and_2d():
    xb = subnormal_scope_rows(inputs.rng(96, 1), rows=64, cols=512)
    q, s, t = mxq.quantize_nvfp4(dev_bf16(xb), scope="tensor")
    eq, es, et = onv.quantize_per_tensor(xb)
    assert host(t).view(np.uint32)[0] == 0x00200000 == et.view(np.uint32)[0]
    assert_bytes_equal(host(q), eq, "subnormal tensor packed")
    assert_bytes_equal(host(s), es, "subnormal tensor scales")
    # group scope: one group of subnormals beside a group of ordinary values
    wb = np.concatenate([xb[:32], inputs.normal_bf16(inputs.rng(96, 2), (32, 512), 0.02)])
    q, s, t = mxq.quantize_nvfp4(dev_bf16(wb), scope="group", group_rows=32)
    eq, es, et = onv.quantize_per_group(wb, [0, 32, 64])
    assert_bytes_equal(host(t).view(np.uint32), et.view(np.uint32), "subnormal group t")
    assert_bytes_equal(host(q), eq, "subnormal group packed")
    assert_bytes_equal(host(s), es, "subnormal group scales")
    # transposed (columnwise) blocking of the same subnormal tensor
    q, s, t = mxq.quantize_nvfp4(dev_bf16(xb), scope="tensor", transpose=True)
    eq, es, et = onv.quantize_per_tensor(np.ascontiguousarray(xb.T))
    assert_bytes_equal(host(q), eq, "subnormal colwise packed")
    assert_bytes_equal(host(t).view(np.uint32), et.view(np.uint32), "subnormal colwise t")
    # 2D 16x16 blocks
    qr, sr, qc, sc, t2 = mxq.quantize_nvfp4_2d(dev_bf16(xb), scope="tensor")
    eq, es, eqT, esT, et2 = onv.quantize_2d(xb)
    assert_bytes_equal(host(qr), eq, "subnormal 2d packed")
    assert_bytes_equal(host(qc), eqT, "subnormal 2d transposed")
    assert_bytes_equal(host(t2).view(np.uint32), et2.view(np.uint32), "subnormal 2d t")


# --------------------- run-twice determinism of the atomics ---------------------

def test_nvfp4_scope_maxima_are_deterministic_across_runs():
    """The tensor / group / 2D quantizers reduce their scope maxima with device atomics;
    a max is order-independent, so two runs (and a run on a freshly allocated
    workspace) must give the same bytes."""
    g = inputs.rng(97, 0)
    G, N, K = 4, 256, 2048
    wb = inputs.to_bf16_bits(g.standard_normal((G * N, K)) * np.exp2(g.integers(-6, 6, (G * N, 1))))
    x = dev_bf16(wb)
    runs = []
    for _ in range(3):
        runs.append([host(a) for a in mxq.quantize_nvfp4(x, scope="tensor")]
                    + [host(a) for a in mxq.quantize_nvfp4(x, scope="group", group_rows=N)]
                    + [host(a) for a in mxq.quantize_nvfp4_2d(x, scope="group", group_rows=N)]
                    + [host(a) for a in mxq.quantize_nvfp4(x, scope="tensor", transpose=True,
                                                           rht_signs=[1, -1] * 8)])
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    eq, es, et = onv.quantize_per_group(wb, np.arange(G + 1) * N)
    assert_bytes_equal(runs[0][3], eq, "group packed")
    assert_bytes_equal(runs[0][5].view(np.uint32), et.view(np.uint32), "group t")
