"""GPU parity: block-scaled GEMMs (MXFP8, NVFP4, BF16; dense and grouped) through
the C ABI against the FP64 product of the oracle's exact dequantized operands,
normwise relative error <= 2e-5 (exact zero when the reference is zero)."""

import numpy as np
import pytest
import torch

import microscaling_precision_quantization_amd as mxq
from microscaling_precision_quantization_amd import inputs
from oracle import formats as F
from oracle import gemm as og
from oracle import moe as omoe
from oracle import mxfp4 as om4
from oracle import mxfp8 as omx
from oracle import nvfp4 as onv
from tests.gpu_util import assert_bytes_equal, assert_gemm_close, dev, dev_bf16, host

pytestmark = pytest.mark.gpu


def mx_operands(xb, col=False):
    """Device rowwise or columnwise-transposed MXFP8 copy + the oracle's dequantized operand."""
    qr, sr, qc, sc = mxq.quantize_mxfp8(dev_bf16(xb), rowwise=not col, colwise=col)
    q, s = (qc, sc) if col else (qr, sr)
    return q, s, omx.dequantize_exact(host(q), host(s))


def test_mxfp8_gemm_small_workload():
    w = inputs.workload_small_mxfp8()
    qa, sa, ah = mx_operands(w["x"])               # X (256, 512) rowwise
    qb, sb, bh = mx_operands(w["w2"], col=True)    # W2 (512, 256): columnwise copy (256, 512)
    c = mxq.gemm_block_scaled(mxq.MXFP8, qa, sa, qb, sb)
    assert_gemm_close(host(c), og.gemm_tn_fp64(ah, bh), "X W2")


@pytest.mark.parametrize("mnk", [(300, 200, 96), (32, 32, 32), (257, 513, 160), (64, 1000, 1024)])
def test_mxfp8_gemm_ragged(mnk):
    M, N, K = mnk
    g = inputs.rng(80, M + N + K)
    a = inputs.to_bf16_bits(g.standard_normal((M, K)) * g.lognormal(0, 1, (M, 1)))
    b = inputs.normal_bf16(g, (N, K), 0.5)
    qa, sa, ah = mx_operands(a)
    qb, sb, bh = mx_operands(b)
    c = mxq.gemm_block_scaled(mxq.MXFP8, qa, sa, qb, sb)
    assert_gemm_close(host(c), og.gemm_tn_fp64(ah, bh), f"ragged {mnk}")


def test_mxfp8_gemm_strided_output_and_zero():
    g = inputs.rng(81, 0)
    a = inputs.normal_bf16(g, (64, 128), 1.0)
    b = np.zeros((96, 128), dtype=np.uint16)
    qa, sa, _ = mx_operands(a)
    qb, sb, _ = mx_operands(b)
    out = torch.full((64, 100), 7.0, device="cuda")
    mxq.gemm_block_scaled(mxq.MXFP8, qa, sa, qb, sb, out=out[:, :96])
    o = host(out)
    assert np.all(o[:, :96] == 0.0) and np.all(o[:, 96:] == 7.0)


def test_mxfp8_linear_layer_fprop_dgrad_wgrad():
    w = inputs.workload_linear_mxfp8()
    xq = mxq.quantize_mxfp8(dev_bf16(w["x"]))
    wq = mxq.quantize_mxfp8(dev_bf16(w["w"]))
    dq = mxq.quantize_mxfp8(dev_bf16(w["dy"]))
    deq = lambda q, s: omx.dequantize_exact(host(q), host(s))
    # fprop Y = X W^T: X rowwise (2048, 2048), W rowwise (8192, 2048)
    y = mxq.gemm_block_scaled(mxq.MXFP8, xq[0], xq[1], wq[0], wq[1])
    assert_gemm_close(host(y), og.gemm_tn_fp64(deq(xq[0], xq[1]), deq(wq[0], wq[1])), "fprop")
    # dgrad dX = dY W: dY rowwise (2048, 8192), W columnwise copy (2048, 8192)
    dx = mxq.gemm_block_scaled(mxq.MXFP8, dq[0], dq[1], wq[2], wq[3])
    assert_gemm_close(host(dx), og.gemm_tn_fp64(deq(dq[0], dq[1]), deq(wq[2], wq[3])), "dgrad")
    # wgrad dW = dY^T X: dY columnwise (8192, 2048), X columnwise (2048, 2048)
    dw = mxq.gemm_block_scaled(mxq.MXFP8, dq[2], dq[3], xq[2], xq[3])
    assert_gemm_close(host(dw), og.gemm_tn_fp64(deq(dq[2], dq[3]), deq(xq[2], xq[3])), "wgrad")


def test_mxfp8_stress_gemms_sampled_rows():
    n = 8192
    a, _ = inputs.student_t_with_injections(5, 0, n)
    b, _ = inputs.student_t_with_injections(5, 1, n)
    aq = mxq.quantize_mxfp8(dev_bf16(a))
    bq = mxq.quantize_mxfp8(dev_bf16(b))
    rows = np.sort(np.random.default_rng(4).choice(n, 48, replace=False))
    for name, (qa, sa, qb, sb) in {"fprop": (aq[0], aq[1], bq[0], bq[1]),
                                   "dgrad": (aq[0], aq[1], bq[2], bq[3]),
                                   "wgrad": (aq[2], aq[3], bq[2], bq[3])}.items():
        c = host(mxq.gemm_block_scaled(mxq.MXFP8, qa, sa, qb, sb))
        ah = omx.dequantize_exact(host(qa)[rows], host(sa)[rows])
        bh = omx.dequantize_exact(host(qb), host(sb))
        assert_gemm_close(c[rows], og.gemm_tn_fp64(ah, bh), f"8192^3 {name} (sampled rows)")
        del c


def nv_token(xb):
    q, s, t = mxq.quantize_nvfp4_per_token(dev_bf16(xb))
    return q, s, t, onv.dequantize_exact(host(q), host(s), host(t))


@pytest.mark.parametrize("mnk", [(300, 200, 256), (64, 64, 32), (256, 512, 2048)])
def test_nvfp4_gemm_dense(mnk):
    M, N, K = mnk
    g = inputs.rng(82, M + N + K)
    a = inputs.to_bf16_bits(g.standard_normal((M, K)) * g.lognormal(0, 1, (M, 1)))
    b = inputs.normal_bf16(g, (N, K), 0.02)
    qa, sa, ta, ah = nv_token(a)
    qb, sb, tb = mxq.quantize_nvfp4(dev_bf16(b), scope="tensor")
    bh = onv.dequantize_exact(host(qb), host(sb), np.repeat(host(tb), N))
    c = mxq.gemm_block_scaled(mxq.NVFP4, qa, sa, qb, sb, tA=ta, tB=tb, tA_scope="row", tB_scope="tensor")
    assert_gemm_close(host(c), og.gemm_tn_fp64(ah, bh), f"nvfp4 {mnk}")
    # per-row scales on both sides
    qb2, sb2, tb2, bh2 = nv_token(b)
    c = mxq.gemm_block_scaled(mxq.NVFP4, qa, sa, qb2, sb2, tA=ta, tB=tb2, tA_scope="row", tB_scope="row")
    assert_gemm_close(host(c), og.gemm_tn_fp64(ah, bh2), f"nvfp4 row/row {mnk}")


def test_nvfp4_wgrad_with_rht_small():
    g = inputs.rng(83, 0)
    T, Mo, Ni = 512, 192, 160
    dy = inputs.to_bf16_bits(g.standard_t(3.0, size=(T, Mo)))
    x = inputs.to_bf16_bits(g.standard_t(3.0, size=(T, Ni)))
    signs = np.where(g.random(16) < 0.5, -1, 1).astype(np.int8)
    qa, sa, ta = mxq.quantize_nvfp4(dev_bf16(dy), scope="tensor", transpose=True, rht_signs=signs)
    qb, sb, tb = mxq.quantize_nvfp4(dev_bf16(x), scope="tensor", transpose=True, rht_signs=signs)
    c = mxq.gemm_block_scaled(mxq.NVFP4, qa, sa, qb, sb, tA=ta, tB=tb, tA_scope="tensor", tB_scope="tensor")
    ah = onv.dequantize_exact(host(qa), host(sa), np.repeat(host(ta), Mo))
    bh = onv.dequantize_exact(host(qb), host(sb), np.repeat(host(tb), Ni))
    assert_gemm_close(host(c), og.gemm_tn_fp64(ah, bh), "rht wgrad")


def test_nvfp4_2d_weight_fprop_and_dgrad():
    """The one 2D-quantized weight serves fprop (row form) and dgrad (transposed form)."""
    g = inputs.rng(97, 0)
    T, N, K = 320, 384, 512
    x = inputs.to_bf16_bits(g.standard_normal((T, K)) * g.lognormal(0, 1, (T, 1)))
    dy = inputs.normal_bf16(g, (T, N), 1e-3)
    w = inputs.normal_bf16(g, (N, K), 0.02)
    qw, sw, qwt, swt, tw = mxq.quantize_nvfp4_2d(dev_bf16(w))
    qx, sx, tx, xh = nv_token(x)
    y = mxq.gemm_block_scaled(mxq.NVFP4, qx, sx, qw, sw, tA=tx, tB=tw, tA_scope="row", tB_scope="tensor")
    wh = onv.dequantize_exact(host(qw), host(sw), np.repeat(host(tw), N))
    assert_gemm_close(host(y), og.gemm_tn_fp64(xh, wh), "2d fprop")
    qd, sd, td, dh = nv_token(dy)
    dx = mxq.gemm_block_scaled(mxq.NVFP4, qd, sd, qwt, swt, tA=td, tB=tw, tA_scope="row", tB_scope="tensor")
    wth = onv.dequantize_exact(host(qwt), host(swt), np.repeat(host(tw), K))
    assert np.array_equal(wth, wh.T)                      # the same weight values in both passes
    assert_gemm_close(host(dx), og.gemm_tn_fp64(dh, wth), "2d dgrad")


@pytest.mark.parametrize("mnk", [(300, 200, 96), (128, 256, 1024)])
def test_bf16_gemm_dense(mnk):
    M, N, K = mnk
    g = inputs.rng(84, M + N + K)
    a = inputs.normal_bf16(g, (M, K), 1.0)
    b = inputs.normal_bf16(g, (N, K), 1.0)
    c = mxq.gemm_block_scaled(mxq.BF16, dev_bf16(a), None, dev_bf16(b), None)
    ref = og.gemm_tn_fp64(F.bf16_bits_to_f32(a), F.bf16_bits_to_f32(b))
    assert_gemm_close(host(c), ref, f"bf16 {mnk}")


@pytest.mark.parametrize("K", [512, 544, 576])
@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4", "bf16"])
def test_dense_256_tiles_ragged(fmt, K):
    """M, N large enough for the 256 x 256 tile kernel, ragged in M and N. K = 512:
    16-byte scale chunks; K = 576: per-stage scale loads; K = 544: a half K stage
    (per-lane tail handling and 1-block scale loads)."""
    M, N = 4196, 3112
    g = inputs.rng(86, K + len(fmt))
    a = inputs.to_bf16_bits(g.standard_normal((M, K)) * g.lognormal(0, 1, (M, 1)))
    b = inputs.normal_bf16(g, (N, K), 0.05)
    if fmt == "mxfp8":
        qa, sa, ah = mx_operands(a)
        qb, sb, bh = mx_operands(b)
        c = mxq.gemm_block_scaled(mxq.MXFP8, qa, sa, qb, sb)
    elif fmt == "nvfp4":
        qa, sa, ta, ah = nv_token(a)
        qb, sb, tb = mxq.quantize_nvfp4(dev_bf16(b), scope="tensor")
        bh = onv.dequantize_exact(host(qb), host(sb), np.repeat(host(tb), N))
        c = mxq.gemm_block_scaled(mxq.NVFP4, qa, sa, qb, sb, tA=ta, tB=tb, tA_scope="row", tB_scope="tensor")
    else:
        c = mxq.gemm_block_scaled(mxq.BF16, dev_bf16(a), None, dev_bf16(b), None)
        ah, bh = F.bf16_bits_to_f32(a), F.bf16_bits_to_f32(b)
    assert_gemm_close(host(c), og.gemm_tn_fp64(ah, bh), f"{fmt} 256-tile {M}x{N}x{K}")


# ------------------------------- grouped -----------------------------------

def small_moe(T=96, H=256, G=8, k=2, N=192, seed=0):
    g = inputs.rng(85, seed)
    x = inputs.to_bf16_bits(g.standard_normal((T, H)) * g.lognormal(0, 1, (T, 1)))
    logits = g.standard_normal((T, G)).astype(np.float32)
    logits[:, 3] = -50.0                                   # expert 3 receives no tokens
    r = inputs.route_topk(logits, k)
    w = inputs.normal_bf16(g, (G * N, H), 0.02)
    return x, r, w


def test_grouped_nvfp4_gather_vary_m():
    x, r, w = small_moe()
    G, N = 8, 192
    qx, sx, tx = mxq.quantize_nvfp4_per_token(dev_bf16(x))
    qw, sw, tw = mxq.quantize_nvfp4(dev_bf16(w), scope="group", group_rows=N)
    off = dev(r.offsets.astype(np.int64))
    idx = dev(r.row_index.astype(np.int32))
    c = mxq.grouped_gemm_block_scaled(mxq.NVFP4, off, qx, qw, N=N, K=x.shape[1], sA=sx, sB=sw, tA=tx, tB=tw,
                                      tA_scope="row", tB_scope="group", a_row_index=idx)
    xh = onv.dequantize_exact(host(qx), host(sx), host(tx))[r.row_index]
    wh = onv.dequantize_exact(host(qw), host(sw), np.repeat(host(tw), N)).reshape(G, N, -1)
    ref = omoe.grouped_gemm_ref(xh, r.offsets, wh)
    ch = host(c)
    for e in range(G):
        lo, hi = r.offsets[e], r.offsets[e + 1]
        if hi > lo:
            assert_gemm_close(ch[lo:hi], ref[lo:hi], f"expert {e}")


def test_grouped_nvfp4_gather_128x256_tiles():
    """Row-grouped NVFP4 with K % 256 == 0 runs on 128 x 256 tiles: groups from empty to
    three row tiles, N = 300 (a ragged second column tile), gathered A rows."""
    x, r, w = small_moe(T=600, H=512, G=5, k=2, N=300, seed=4)
    G, N = 5, 300
    qx, sx, tx = mxq.quantize_nvfp4_per_token(dev_bf16(x))
    qw, sw, tw = mxq.quantize_nvfp4(dev_bf16(w), scope="group", group_rows=N)
    c = mxq.grouped_gemm_block_scaled(mxq.NVFP4, dev(r.offsets.astype(np.int64)), qx, qw, N=N, K=x.shape[1], sA=sx,
                                      sB=sw, tA=tx, tB=tw, tA_scope="row", tB_scope="group",
                                      a_row_index=dev(r.row_index.astype(np.int32)))
    xh = onv.dequantize_exact(host(qx), host(sx), host(tx))[r.row_index]
    wh = onv.dequantize_exact(host(qw), host(sw), np.repeat(host(tw), N)).reshape(G, N, -1)
    ref = omoe.grouped_gemm_ref(xh, r.offsets, wh)
    ch = host(c)
    sizes = np.diff(r.offsets)
    assert sizes[3] == 0 and sizes.max() > 256
    for e in range(G):
        lo, hi = r.offsets[e], r.offsets[e + 1]
        if hi > lo:
            assert_gemm_close(ch[lo:hi], ref[lo:hi], f"expert {e}")


def test_grouped_nvfp4_dgrad_on_2d_expert_weights():
    """2D-scaled expert weights give an NVFP4 dgrad: per expert dX_g = dGU_g W_g with the
    per-expert transposed copy (G, K, N) as the stacked B operand."""
    x, r, _ = small_moe(seed=3)
    G, N, K = 8, 192, 256
    g = inputs.rng(85, 30)
    w = inputs.normal_bf16(g, (G * N, K), 0.02)
    S = int(r.offsets[-1])
    dgu = inputs.to_bf16_bits(g.standard_normal((S, N)) * 1e-3 * g.lognormal(0, 1, (S, 1)))
    qw, sw, qwt, swt, tw = mxq.quantize_nvfp4_2d(dev_bf16(w), scope="group", group_rows=N)
    qd, sd, td = mxq.quantize_nvfp4_per_token(dev_bf16(dgu))
    dx = mxq.grouped_gemm_block_scaled(mxq.NVFP4, dev(r.offsets.astype(np.int64)), qd, qwt, N=K, K=N, sA=sd, sB=swt,
                                       tA=td, tB=tw, tA_scope="row", tB_scope="group")
    ah = onv.dequantize_exact(host(qd), host(sd), host(td))
    wt = onv.dequantize_exact(host(qwt), host(swt), np.repeat(host(tw), K)).reshape(G, K, N)
    wr = onv.dequantize_exact(host(qw), host(sw), np.repeat(host(tw), N)).reshape(G, N, K)
    assert np.array_equal(wt, wr.transpose(0, 2, 1))          # fprop and dgrad read one weight
    ref = omoe.grouped_gemm_ref(ah, r.offsets, wt)
    ch = host(dx)
    for e in range(G):
        lo, hi = r.offsets[e], r.offsets[e + 1]
        if hi > lo:
            assert_gemm_close(ch[lo:hi], ref[lo:hi], f"2d dgrad expert {e}")


def test_grouped_mxfp8_vary_m_contiguous():
    x, r, w = small_moe(seed=1)
    G, N = 8, 192
    xs = x[r.row_index]                                       # already in expert order
    qx, sx, _, _ = mxq.quantize_mxfp8(dev_bf16(xs), True, False)
    qw, sw, _, _ = mxq.quantize_mxfp8(dev_bf16(w), True, False)
    c = mxq.grouped_gemm_block_scaled(mxq.MXFP8, dev(r.offsets.astype(np.int64)), qx, qw, N=N, K=x.shape[1],
                                      sA=sx, sB=sw)
    ref = omoe.grouped_gemm_ref(omx.dequantize_exact(host(qx), host(sx)), r.offsets,
                                omx.dequantize_exact(host(qw), host(sw)).reshape(G, N, -1))
    assert_gemm_close(host(c), ref, "mxfp8 grouped")


@pytest.mark.parametrize("fmt", ["mxfp8", "bf16"])
def test_grouped_vary_k_wgrad(fmt):
    g = inputs.rng(86, 0)
    G, M, N = 5, 96, 160
    sizes = np.array([64, 0, 160, 32, 256]) if fmt == "mxfp8" else np.array([40, 0, 168, 8, 256])
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    S = int(off[-1])
    a = inputs.normal_bf16(g, (M, S), 1.0)
    b = inputs.normal_bf16(g, (N, S), 1.0)
    if fmt == "mxfp8":
        qa, sa, _, _ = mxq.quantize_mxfp8(dev_bf16(a), True, False)
        qb, sb, _, _ = mxq.quantize_mxfp8(dev_bf16(b), True, False)
        c = mxq.grouped_gemm_block_scaled(mxq.MXFP8, dev(off), qa, qb, N=N, K=0, sA=sa, sB=sb, vary_k=True, M=M)
        ah, bh = omx.dequantize_exact(host(qa), host(sa)), omx.dequantize_exact(host(qb), host(sb))
    else:
        c = mxq.grouped_gemm_block_scaled(mxq.BF16, dev(off), dev_bf16(a), dev_bf16(b), N=N, K=0, vary_k=True, M=M)
        ah, bh = F.bf16_bits_to_f32(a).astype(np.float64), F.bf16_bits_to_f32(b).astype(np.float64)
    ch = host(c)
    for e in range(G):
        ref = ah[:, off[e]:off[e + 1]] @ bh[:, off[e]:off[e + 1]].T
        if sizes[e] == 0:
            assert np.all(ch[e] == 0.0)
        else:
            assert_gemm_close(ch[e], ref, f"{fmt} group {e}")


def test_grouped_bf16_vary_k_wide_output():
    """BF16 weight gradients with outputs of 64+ 256-tiles run on 128 x 256 tiles: per-group
    K of 40, 0 and 168 (K tails inside a stage), N = 2100 (a ragged column tile)."""
    g = inputs.rng(91, 0)
    M, N = 2048, 2100
    sizes = np.array([40, 0, 168])
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    S = int(off[-1])
    a = inputs.normal_bf16(g, (M, S), 1.0)
    b = inputs.normal_bf16(g, (N, S), 1.0)
    c = host(mxq.grouped_gemm_block_scaled(mxq.BF16, dev(off), dev_bf16(a), dev_bf16(b), N=N, K=0, vary_k=True, M=M))
    ah, bh = F.bf16_bits_to_f32(a).astype(np.float64), F.bf16_bits_to_f32(b).astype(np.float64)
    for e in range(len(sizes)):
        if sizes[e] == 0:
            assert np.all(c[e] == 0.0)
        else:
            assert_gemm_close(c[e], ah[:, off[e]:off[e + 1]] @ bh[:, off[e]:off[e + 1]].T, f"wide wgrad group {e}")



def test_grouped_bf16_vary_k_wide_output_many_tiles():
    """A wide BF16 weight gradient with more output tiles than CUs: ragged M (2100) and
    N (2050), per-group K of 600 (ten 64-K stages), 0, 520 and 64 (one stage), an empty
    group in between. The output is prefilled with NaN, so an element that no tile
    writes fails the check."""
    g = inputs.rng(92, 0)
    M, N = 2100, 2050
    sizes = np.array([600, 0, 520, 64])
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    S = int(off[-1])
    a = inputs.normal_bf16(g, (M, S), 1.0)
    b = inputs.normal_bf16(g, (N, S), 1.0)
    out = torch.full((len(sizes), M, N), float("nan"), device="cuda")
    mxq.grouped_gemm_block_scaled(mxq.BF16, dev(off), dev_bf16(a), dev_bf16(b), N=N, K=0, vary_k=True, M=M, out=out)
    c = host(out)
    assert not np.isnan(c).any()
    ah, bh = F.bf16_bits_to_f32(a).astype(np.float64), F.bf16_bits_to_f32(b).astype(np.float64)
    for e in range(len(sizes)):
        if sizes[e] == 0:
            assert np.all(c[e] == 0.0)
        else:
            assert_gemm_close(c[e], ah[:, off[e]:off[e + 1]] @ bh[:, off[e]:off[e + 1]].T, f"wide wgrad group {e}")

def test_grouped_bf16_vary_m():
    x, r, w = small_moe(seed=2)
    G, N = 8, 192
    xs = x[r.row_index]
    c = mxq.grouped_gemm_block_scaled(mxq.BF16, dev(r.offsets.astype(np.int64)), dev_bf16(xs), dev_bf16(w), N=N,
                                      K=x.shape[1])
    ref = omoe.grouped_gemm_ref(F.bf16_bits_to_f32(xs).astype(np.float64), r.offsets,
                                F.bf16_bits_to_f32(w).astype(np.float64).reshape(G, N, -1))
    assert_gemm_close(host(c), ref, "bf16 grouped")


def test_grouped_bf16_vary_m_large_groups():
    """Groups averaging >= 384 rows (here 430) run on 256 x 256 tiles: ragged group sizes
    (one empty, one of four row tiles with a 132-row tail), N not a multiple of the tile."""
    g = inputs.rng(90, 0)
    sizes = np.array([520, 0, 300, 900])
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    S, G, N, K = int(off[-1]), len(sizes), 300, 192
    a = inputs.normal_bf16(g, (S, K), 1.0)
    w = inputs.normal_bf16(g, (G * N, K), 0.05)
    c = mxq.grouped_gemm_block_scaled(mxq.BF16, dev(off), dev_bf16(a), dev_bf16(w), N=N, K=K)
    ref = omoe.grouped_gemm_ref(F.bf16_bits_to_f32(a).astype(np.float64), off,
                                F.bf16_bits_to_f32(w).astype(np.float64).reshape(G, N, -1))
    assert_gemm_close(host(c), ref, "bf16 grouped, large groups")



@pytest.mark.parametrize("fmt,sizes,N,K", [
    ("bf16", [2304], 128, 64),           # one group of nine 256-row tiles, one column tile
    ("bf16", [2304, 0, 256], 100, 64),
    ("nvfp4", [1152], 256, 256),         # nine 128-row tiles on the 128 x 256 NVFP4 tiles
    ("mxfp8", [1152], 128, 64),          # nine 128 x 128 tiles
    ("mxfp8", [640, 128, 384], 64, 96),
])
def test_grouped_row_groups_with_few_column_tiles(fmt, sizes, N, K):
    """Row groups whose tile count is not a multiple of 8 with one column tile: the
    XCD-contiguous tile order has to reach every tile (a grid too small for it left row
    tiles unwritten). Every output row is checked against the oracle."""
    g = inputs.rng(152, sum(sizes) + N + K)
    sizes = np.array(sizes)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    S, G = int(off[-1]), len(sizes)
    a = inputs.to_bf16_bits(g.standard_normal((S, K)) * g.lognormal(0, 1, (S, 1)))
    w = inputs.normal_bf16(g, (G * N, K), 0.05)
    c = torch.full((S, N), float("nan"), device="cuda")  # an unwritten tile stays NaN
    if fmt == "bf16":
        mxq.grouped_gemm_block_scaled(mxq.BF16, dev(off), dev_bf16(a), dev_bf16(w), N=N, K=K, out=c)
        ah, wh = F.bf16_bits_to_f32(a).astype(np.float64), F.bf16_bits_to_f32(w).astype(np.float64)
    elif fmt == "mxfp8":
        qa, sa, ah = mx_operands(a)
        qw, sw, wh = mx_operands(w)
        mxq.grouped_gemm_block_scaled(mxq.MXFP8, dev(off), qa, qw, N=N, K=K, sA=sa, sB=sw, out=c)
    else:
        qa, sa, ta = mxq.quantize_nvfp4_per_token(dev_bf16(a))
        qw, sw, tw = mxq.quantize_nvfp4(dev_bf16(w), scope="group", group_rows=N)
        mxq.grouped_gemm_block_scaled(mxq.NVFP4, dev(off), qa, qw, N=N, K=K, sA=sa, sB=sw, tA=ta, tB=tw,
                                      tA_scope="row", tB_scope="group", out=c)
        ah = onv.dequantize_exact(host(qa), host(sa), host(ta))
        wh = onv.dequantize_exact(host(qw), host(sw), np.repeat(host(tw), N))
    ref = omoe.grouped_gemm_ref(ah, off, wh.reshape(G, N, -1))
    ch = host(c)
    assert not np.isnan(ch).any(), f"{np.isnan(ch).any(axis=1).sum()} output rows never written"
    for e in range(G):
        lo, hi = off[e], off[e + 1]
        for r0 in range(lo, hi, 128):                     # every 128-row band on its own
            r1 = min(r0 + 128, hi)
            assert_gemm_close(ch[r0:r1], ref[r0:r1], f"{fmt} group {e} rows {r0}:{r1}")


# --------------------------------- MoE glue ---------------------------------

def test_swiglu_extreme_gates():
    """Gates across every range of the exponential (|g| up to 1e30, through the binary32
    and binary64 overflow points), signed zeros, results in the BF16 subnormal range and
    past its maximum, and products g u on BF16 midpoints: h is the correctly rounded
    BF16 value, bit for bit, and the per-row NVFP4 of it matches the oracle's run from
    the same FP32 gate/up values."""
    g = inputs.rng(87, 1)
    rows, inter = 64, 512
    gate = np.concatenate([np.linspace(-120, 120, 241),
                           [0.0, -0.0, 1e-30, -1e-30, 87.3, -87.3, 88.8, -88.8, 89.5, -89.5, 700.0, -700.0, 709.5,
                            -709.5, 710.0, -710.0, 745.5, -745.5, 1e4, -1e4, 1e30, -1e30],
                           -g.uniform(80, 100, 100), g.uniform(30, 40, 50).round()])
    gate = np.resize(gate, rows * inter).reshape(rows, inter)
    up = g.standard_normal((rows, inter)) * np.exp2(g.integers(-20, 20, (rows, 1)))
    up[0, :64] = 0.0
    up[1, :64] = -0.0
    up[2, :] = 3e38                                           # g u past the BF16 maximum
    up[3, :] = (2 * g.integers(128, 256, inter) + 1) * 2.0 ** -6 / 32.0
    gate[3, :] = 32.0                                         # g u = odd / 2: BF16 midpoints
    up[4, :] = np.exp2(g.integers(20, 60, inter).astype(float))   # h reaches BF16 subnormals
    gu = np.concatenate([gate, up], axis=1).astype(np.float32)
    h, q, s, t = mxq.moe_swiglu_quantize_nvfp4(dev(gu))
    h_ref = omoe.swiglu_bf16_ref(gu)
    assert_bytes_equal(host(h), h_ref, "h")
    finite = np.all(np.isfinite(F.bf16_bits_to_f32(h_ref)), axis=1)   # rows the quantizer accepts
    eq, es, et = onv.quantize_per_token(h_ref[finite])
    assert_bytes_equal(host(q)[finite], eq, "h packed")
    assert_bytes_equal(host(s)[finite], es, "h block scales")
    assert_bytes_equal(host(t)[finite].view(np.uint32), et.view(np.uint32), "h scales")


@pytest.mark.parametrize("inter", [16, 528, 2064, 4112, 8208, 16384])
def test_swiglu_requant_every_row_width(inter):
    """SwiGLU + per-row NVFP4 for row widths that reach every register-blocked instance of
    the kernel (1 to 32 chunks of 512), ragged last chunks and the 16384 maximum: h, the
    packed codes, the block scales and t bit for bit against the oracle from the FP32
    gate/up values."""
    g = inputs.rng(89, inter)
    rows = 24
    gu = (g.standard_normal((rows, 2 * inter)) * 4 * np.exp2(g.integers(-8, 8, (rows, 1)))).astype(np.float32)
    h, q, s, t = mxq.moe_swiglu_quantize_nvfp4(dev(gu))
    hh = omoe.swiglu_bf16_ref(gu)
    assert_bytes_equal(host(h), hh, f"h (inter {inter})")
    eq, es, et = onv.quantize_per_token(hh)
    assert_bytes_equal(host(q), eq, f"packed (inter {inter})")
    assert_bytes_equal(host(s), es, f"block scales (inter {inter})")
    assert np.array_equal(host(t).view(np.uint32), et.view(np.uint32))


def test_swiglu_requant_and_combine():
    g = inputs.rng(87, 0)
    rows, inter = 300, 768
    gu = (g.standard_normal((rows, 2 * inter)) * 3).astype(np.float32)
    h, q, s, t = mxq.moe_swiglu_quantize_nvfp4(dev(gu))
    hh = omoe.swiglu_bf16_ref(gu)                              # end to end from the FP32 gate/up
    assert_bytes_equal(host(h), hh, "h")
    eq, es, et = onv.quantize_per_token(hh)
    assert np.array_equal(host(q), eq) and np.array_equal(host(s), es)
    assert np.array_equal(host(t).view(np.uint32), et.view(np.uint32))
    T, k, H = 50, 4, 256
    o = g.standard_normal((T * k, H)).astype(np.float32)
    slot_of = g.permutation(T * k).reshape(T, k).astype(np.int64)
    wts = g.random((T, k)).astype(np.float32)
    y = mxq.moe_combine(dev(o), dev(slot_of), dev(wts))
    assert_gemm_close(host(y), omoe.combine_ref(o, slot_of, wts), "combine")


@pytest.mark.parametrize("k", [1, 2, 3, 4, 6, 8, 9])
def test_combine_every_topk_with_skipped_slots(k):
    """Combine for each top-k the launcher distinguishes (compile-time k or the generic
    loop), with slot indices below zero and past the end (they contribute nothing) and a
    hidden size that leaves a partial last pass: within 2e-5 of the oracle, and bit-equal
    to the FP32 sum in ascending j with a separate multiply and add per term."""
    g = inputs.rng(88, k)
    T, H = 70, 1028
    S = T * k + 5
    o = g.standard_normal((S, H)).astype(np.float32)
    slot_of = g.permutation(S)[:T * k].reshape(T, k).astype(np.int64)
    slot_of[g.random((T, k)) < 0.1] = -1
    slot_of[g.random((T, k)) < 0.05] = S + 3
    wts = g.random((T, k)).astype(np.float32)
    y = host(mxq.moe_combine(dev(o), dev(slot_of), dev(wts)))
    valid = (slot_of >= 0) & (slot_of < S)
    ref = omoe.combine_ref(o, np.where(valid, slot_of, 0), np.where(valid, wts, 0.0).astype(np.float32))
    assert_gemm_close(y, ref, f"combine k={k}")
    acc = np.zeros((T, H), dtype=np.float32)
    for j in range(k):
        m = valid[:, j]
        acc[m] = acc[m] + wts[m, j:j + 1] * o[slot_of[m, j]]
    assert np.array_equal(y.view(np.uint32), acc.view(np.uint32)), f"combine k={k} differs from the FP32 ascending sum"


# --------------------- native scaled-FP8 matrix-core path ---------------------

def matrix_core_bound(ah, bh, c_ref):
    """Elementwise error model of the scaled FP8 MFMA (measured): products of each
    aligned group of 8 consecutive K are summed in a window 13 bits below the group's
    largest product, so each group errs by < 8 * 2^-13 of that product; group sums
    and the accumulator are FP32 (a few ulps of the running magnitude)."""
    M, K = ah.shape
    N = bh.shape[0]
    bound = np.zeros((M, N))
    absum = np.zeros((M, N))
    for g0 in range(0, K, 8):
        p = np.abs(ah[:, None, g0:g0 + 8] * bh[None, :, g0:g0 + 8])
        bound += 8 * 2.0 ** -13 * p.max(axis=2)
        absum += p.sum(axis=2)
    return bound + (K // 8 + 2) * 2.0 ** -24 * absum   # FP32 accumulation of K/8 group sums


def test_matrix_core_linear_layer_meets_bound():
    w = inputs.workload_linear_mxfp8()
    xq = mxq.quantize_mxfp8(dev_bf16(w["x"]))
    wq = mxq.quantize_mxfp8(dev_bf16(w["w"]))
    dq = mxq.quantize_mxfp8(dev_bf16(w["dy"]))
    deq = lambda q, s: omx.dequantize_exact(host(q), host(s))
    for name, (qa, sa, qb, sb) in {"fprop": (xq[0], xq[1], wq[0], wq[1]), "dgrad": (dq[0], dq[1], wq[2], wq[3]),
                                   "wgrad": (dq[2], dq[3], xq[2], xq[3])}.items():
        c = mxq.gemm_mxfp8_matrix_core(qa, sa, qb, sb)
        assert_gemm_close(host(c), og.gemm_tn_fp64(deq(qa, sa), deq(qb, sb)), f"matrix core {name}")


@pytest.mark.parametrize("case", ["outliers", "student_t"])
def test_matrix_core_error_model(case):
    if case == "outliers":
        w = inputs.workload_small_mxfp8()
        a, b = w["x"], np.ascontiguousarray(w["w2"].T)
    else:
        g = inputs.rng(88, 0)
        a = inputs.to_bf16_bits(g.standard_t(3.0, size=(128, 1024)))
        b = inputs.to_bf16_bits(g.standard_t(3.0, size=(96, 1024)))
    qa, sa, ah = mx_operands(a)
    qb, sb, bh = mx_operands(b)
    c = host(mxq.gemm_mxfp8_matrix_core(qa, sa, qb, sb)).astype(np.float64)
    ref = og.gemm_tn_fp64(ah, bh)
    bound = matrix_core_bound(ah, bh, ref)
    assert np.all(np.abs(c - ref) <= bound), f"{case}: max excess {np.max(np.abs(c - ref) - bound):.3e}"
    # and the exact path meets the 2e-5 contract on the same data
    ce = mxq.gemm_block_scaled(mxq.MXFP8, qa, sa, qb, sb)
    assert_gemm_close(host(ce), ref, f"{case} exact path")


def test_mxfp8_exact_path_integer_operands_exact():
    g = inputs.rng(89, 0)
    a = g.integers(-15, 16, size=(64, 256)).astype(np.float64)
    b = g.integers(-15, 16, size=(48, 256)).astype(np.float64)
    a[:, ::32] = 448.0
    b[:, ::32] = 448.0
    qa, sa, _ = mx_operands(inputs.to_bf16_bits(a))
    qb, sb, _ = mx_operands(inputs.to_bf16_bits(b))
    c = host(mxq.gemm_block_scaled(mxq.MXFP8, qa, sa, qb, sb))
    assert np.array_equal(c, (a @ b.T).astype(np.float32))


def test_mxfp8_exact_path_lowest_scales_with_subnormal_codes():
    """Hand-made operands at the bottom of the MXFP8 range: A's blocks carry E8M0 codes
    0, 1, 2 with E4M3 subnormal codes whose values times 2^(s-127) are multiples of
    2^-133 (the documented exact range), B's blocks scales near 2^118 so the products land
    in the normal FP32 range. The result must meet the 2e-5 bound like any other."""
    g = inputs.rng(89, 1)
    M, N, K = 64, 96, 256
    qa = np.zeros((M, K), dtype=np.uint8)
    sa = g.integers(0, 3, (M, K // 32)).astype(np.uint8)
    # the E4M3 codes whose value times 2^(s-127) is a multiple of 2^-133, per scale code s;
    # half of each block is drawn from the subnormal ones among them
    ok = {s_: [c for c in range(0x7F) if (F.e4m3_value(c) * 2.0 ** (s_ - 127 + 133)) % 1 == 0] for s_ in range(3)}
    for m in range(M):
        for kb in range(K // 32):
            valid = np.array(ok[int(sa[m, kb])])
            sub = valid[valid < 0x08]
            codes = np.where(g.random(32) < 0.5, g.choice(sub, 32), g.choice(valid, 32))
            qa[m, kb * 32:(kb + 1) * 32] = codes | (g.integers(0, 2, 32) << 7)
    qb = g.integers(0, 0x7F, (N, K)).astype(np.uint8) | (g.integers(0, 2, (N, K)) << 7).astype(np.uint8)
    sb = g.integers(240, 246, (N, K // 32)).astype(np.uint8)
    c = mxq.gemm_block_scaled(mxq.MXFP8, dev(qa), dev(sa), dev(qb), dev(sb))
    ref = og.gemm_tn_fp64(omx.dequantize_exact(qa, sa), omx.dequantize_exact(qb, sb))
    assert np.max(np.abs(omx.dequantize_exact(qa, sa))) < 2.0 ** -116            # really at the bottom
    assert_gemm_close(host(c), ref, "lowest scales, subnormal codes")


# ------------------------------ batched -------------------------------------

def _batch_case(fmt, shapes, seed):
    g = inputs.rng(150, seed)
    probs = []
    for M, N, K in shapes:
        if M == 0:                                     # an empty problem: skipped by the batch
            u8 = lambda *sh: torch.empty(sh, dtype=torch.uint8, device="cuda")
            probs.append(dict(A=u8(0, K), sA=u8(0, K // 32), B=u8(N, K), sB=u8(N, K // 32),
                              out=torch.empty((0, N), device="cuda")))
            continue
        a = inputs.to_bf16_bits(g.standard_normal((M, K)) * g.lognormal(0, 1, (M, 1)))
        b = inputs.normal_bf16(g, (N, K), 0.05)
        if fmt == mxq.MXFP8:
            qa, sa, _, _ = mxq.quantize_mxfp8(dev_bf16(a), True, False)
            qb, sb, _, _ = mxq.quantize_mxfp8(dev_bf16(b), True, False)
            d = dict(A=qa, sA=sa, B=qb, sB=sb)
        elif fmt == mxq.MXFP4:
            qa, sa, _, _ = mxq.quantize_mxfp4(dev_bf16(a), True, False)
            qb, sb, _, _ = mxq.quantize_mxfp4(dev_bf16(b), True, False)
            d = dict(A=qa, sA=sa, B=qb, sB=sb)
        elif fmt == mxq.NVFP4:
            qa, sa, ta = mxq.quantize_nvfp4_per_token(dev_bf16(a))
            qb, sb, tb = mxq.quantize_nvfp4(dev_bf16(b), scope="tensor")
            d = dict(A=qa, sA=sa, B=qb, sB=sb, tA=ta, tB=tb, tA_scope="row", tB_scope="tensor")
        else:
            d = dict(A=dev_bf16(a), sA=None, B=dev_bf16(b), sB=None)
        d["out"] = torch.full((M, N + 3), 5.0, device="cuda")[:, :N]
        probs.append(d)
    return probs


@pytest.mark.parametrize("fmt,shapes", [
    ("mxfp8", [(2048, 8192, 2048), (2048, 2048, 8192), (8192, 2048, 2048)]),     # the linear layer's three GEMMs
    ("mxfp8", [(300, 200, 96), (64, 1000, 1024), (257, 513, 160), (0, 64, 64)]),  # ragged, K % 64 != 0, empty
    ("mxfp8", [(2100, 3000, 1024), (1500, 2300, 512), (0, 64, 512), (3000, 700, 512)]),   # 128x256 tiles, ragged
    ("nvfp4", [(300, 200, 256), (256, 512, 2048)]),
    ("mxfp4", [(4196, 3112, 512), (64, 1000, 1024), (32, 32, 32)]),
    ("bf16", [(300, 200, 96), (128, 256, 1024)]),
    ("mxfp8", [(300, 200, 4096), (64, 1000, 1024), (2048, 2048, 8192)]),         # long-K, few-tile members
    ("bf16", [(384, 640, 8192), (130, 70, 4224), (300, 200, 96)]),
])
def test_gemm_batch_matches_single_calls(fmt, shapes):
    f = {"mxfp8": mxq.MXFP8, "nvfp4": mxq.NVFP4, "mxfp4": mxq.MXFP4, "bf16": mxq.BF16}[fmt]
    probs = _batch_case(f, shapes, len(shapes) + f)
    mxq.gemm_block_scaled_batch(f, probs)
    for q, (M, N, K) in zip(probs, shapes):
        if M == 0:
            continue
        ref = mxq.gemm_block_scaled(f, q["A"], q["sA"], q["B"], q["sB"], tA=q.get("tA"), tB=q.get("tB"),
                                    tA_scope=q.get("tA_scope", "row"), tB_scope=q.get("tB_scope", "tensor"))
        got = host(q["out"].contiguous())
        assert np.array_equal(got.view(np.uint32), host(ref).view(np.uint32)), (fmt, M, N, K)
        assert np.all(host(q["out"].as_strided((M, 3), (N + 3, 1), N)) == 5.0)     # padding columns untouched
        # and against the oracle at the batch's own shape (not only through the single call)
        assert_gemm_close(got, og.gemm_tn_fp64(_oracle_operand(f, q, "A"), _oracle_operand(f, q, "B")),
                          f"batched {fmt} {(M, N, K)}")


def _oracle_operand(f, q, side):
    """The oracle's exact dequantization of one batch operand (from the device's bytes)."""
    x, sx = host(q[side]), None if q["s" + side] is None else host(q["s" + side])
    if f == mxq.MXFP8:
        return omx.dequantize_exact(x, sx)
    if f == mxq.MXFP4:
        return om4.dequantize_exact(x, sx)
    if f == mxq.NVFP4:
        t = host(q["t" + side])
        return onv.dequantize_exact(x, sx, t if len(t) == x.shape[0] else np.repeat(t, x.shape[0]))
    return F.bf16_bits_to_f32(x).astype(np.float64)


# ------------- dequantized-backward dgrad straight from NVFP4 weights -------------

def _nvfp4t_case(seed, G, K, N, rows, zero_group=None):
    g = inputs.rng(170, seed)
    w = inputs.to_bf16_bits(g.standard_normal((G * K, N)) * 0.02 * np.exp2(g.integers(-3, 3, (G * K, 1))))
    if zero_group is not None:                              # an all-zero expert with -0 entries
        w[zero_group * K:(zero_group + 1) * K] = 0
        w[zero_group * K, ::7] = 0x8000
    offsets = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    S = int(offsets[-1])
    a = inputs.to_bf16_bits(g.standard_normal((S, K)) * 1e-3)
    qw, sw, tw = mxq.quantize_nvfp4(dev_bf16(w), scope="group", group_rows=K)
    wb = onv.dequantize_bf16_bits(host(qw), host(sw), np.repeat(host(tw), K))      # (G K, N) BF16 bits
    b_hat = F.bf16_bits_to_f32(wb).astype(np.float64).reshape(G, K, N).transpose(0, 2, 1)
    ref = omoe.grouped_gemm_ref(F.bf16_bits_to_f32(a).astype(np.float64), offsets, b_hat)
    return dict(a=a, qw=qw, sw=sw, tw=tw, off=offsets, ref=ref, S=S)


@pytest.mark.parametrize("G,K,N,rows,zg", [
    (6, 512, 768, [0, 400, 513, 256, 390, 1000], None),     # 256-row tiles on both paths: bit-identical
    (4, 200, 400, [37, 0, 300, 129], 1),                     # K tail (200 % 64), N tail (400 % 256), zero expert
    (3, 1024, 2048, [700, 64, 900], 2),
    (3, 328, 528, [700, 512, 400], None),                    # K tail 8, last column tile 16 wide (N % 32 = 16)
    (3, 24, 272, [1, 300, 0], None),                         # K below one stage, a one-row expert
])
def test_bf16_nvfp4t_dgrad_from_quantized_weights(G, K, N, rows, zg):
    """The BF16 x NVFP4-weights-transposed grouped GEMM (the weight dequantization done in
    the GEMM loader) against the oracle's FP64 product of the BF16 dequantized weights,
    per expert, and bit for bit against the two-step path (dequantize_transposed, then the
    BF16 grouped GEMM) where both run the same tiles."""
    c = _nvfp4t_case(G + K + N, G, K, N, rows, zg)
    off = dev(c["off"])
    got = host(mxq.grouped_gemm_block_scaled(mxq.BF16_NVFP4T, off, dev_bf16(c["a"]), c["qw"], N=N, K=K, sB=c["sw"],
                                             tB=c["tw"], tB_scope="group", total=c["S"]))
    for e in range(G):
        lo, hi = c["off"][e], c["off"][e + 1]
        if hi > lo:
            assert_gemm_close(got[lo:hi], c["ref"][lo:hi], f"expert {e}")
    wT = mxq.dequantize_transposed(mxq.NVFP4, c["qw"], c["sw"], c["tw"], t_scope="group", groups=G, group_rows=K,
                                   cols=N)
    two_step = host(mxq.grouped_gemm_block_scaled(mxq.BF16, off, dev_bf16(c["a"]), wT, N=N, K=K, total=c["S"]))
    if c["S"] / G >= 384:
        assert np.array_equal(got.view(np.uint32), two_step.view(np.uint32))
    else:
        assert_gemm_close(got, two_step.astype(np.float64), "against the two-step path")


@pytest.mark.parametrize("fmt,mnk", [("mxfp8", (300, 200, 4096)), ("mxfp8", (64, 64, 8192)),
                                     ("bf16", (384, 640, 8192)), ("bf16", (130, 70, 4224))])
def test_long_k_few_tiles_gemm_oracle_and_deterministic(fmt, mnk):
    """Long-K problems with few output tiles (ragged ones included): within the bound of
    the oracle, the same bits on a second run, and the columns past N of a strided output
    untouched."""
    M, N, K = mnk
    g = inputs.rng(151, M + N + K)
    a = inputs.to_bf16_bits(g.standard_normal((M, K)) * g.lognormal(0, 1, (M, 1)))
    b = inputs.normal_bf16(g, (N, K), 0.05)
    if fmt == "mxfp8":
        qa, sa, ah = mx_operands(a)
        qb, sb, bh = mx_operands(b)
        f = mxq.MXFP8
    else:
        qa, sa, ah = dev_bf16(a), None, F.bf16_bits_to_f32(a)
        qb, sb, bh = dev_bf16(b), None, F.bf16_bits_to_f32(b)
        f = mxq.BF16
    outs = []
    for _ in range(2):
        out = torch.full((M, N + 5), 3.0, device="cuda")
        mxq.gemm_block_scaled(f, qa, sa, qb, sb, out=out[:, :N])
        o = host(out)
        assert np.all(o[:, N:] == 3.0)
        outs.append(o[:, :N].copy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert_gemm_close(outs[0], og.gemm_tn_fp64(ah, bh), f"long K {fmt} {mnk}")


# ------------- the documented K limit (2^22): 32-bit operand offsets -------------

def _small_int_operand(g, shape):
    """Integers in [-2, 2]: exact in BF16, and after the block scaling exact in E4M3 and
    E2M1 too (a block maximum of 1 or 2 scales to a power of two of the element format)."""
    v = g.integers(-2, 3, shape).astype(np.float32)
    return v, inputs.to_bf16_bits(v)


@pytest.mark.parametrize("fmt", ["bf16", "mxfp8", "mxfp4", "nvfp4"])
def test_dense_gemm_at_the_k_limit_is_exact(fmt):
    """K = 2^22, the largest K the GEMM entry points accept. Small integer operands make
    every product exact and keep every partial sum an integer far below 2^24, so the FP32
    result must equal the exact product bit for bit: a K chunk dropped, repeated or read
    from the wrong place by the 32-bit offset arithmetic would change it. M and N leave
    ragged tiles. NVFP4 (both operands per-tensor, quantized from their transposes with
    16-blocks along K, the only NVFP4 quantizer without a row-length limit): A and B have
    amax 2, so s_enc = 1344 and every q S = 1344 x (S = 448, q = 3x in blocks of amax 2;
    S = 224, q = 6x in blocks of amax 1); the accumulator holds 1344^2 = 2^12 441 times an
    integer sum, exact in FP32, and the epilogue's two FP32 products by tA and tB follow."""
    g = inputs.rng(175, ["bf16", "mxfp8", "mxfp4", "nvfp4"].index(fmt))
    M, N, K = 40, (48 if fmt == "nvfp4" else 36), 1 << 22
    a, ab = _small_int_operand(g, (M, K))
    b, bb = _small_int_operand(g, (N, K))
    exact = a.astype(np.float64) @ b.astype(np.float64).T                # integers
    if fmt == "nvfp4":
        qa, sa, ta = mxq.quantize_nvfp4(dev_bf16(np.ascontiguousarray(ab.T)), scope="tensor", transpose=True)
        qb, sb, tb = mxq.quantize_nvfp4(dev_bf16(np.ascontiguousarray(bb.T)), scope="tensor", transpose=True)
        c = mxq.gemm_block_scaled(mxq.NVFP4, qa, sa, qb, sb, tA=ta, tB=tb, tA_scope="tensor", tB_scope="tensor")
        ta, tb = host(ta), host(tb)
        assert ta[0].view(np.uint32) == np.float32(1.0 / 1344.0).view(np.uint32) and tb[0] == ta[0]
        acc = (exact * 1344.0 * 1344.0).astype(np.float32)                 # exact: 441 |sum| < 2^24
        ref = (acc * ta[0]) * tb[0]
        assert np.array_equal(host(c), ref), "nvfp4 at K = 2^22"
        return
    if fmt == "bf16":
        c = mxq.gemm_block_scaled(mxq.BF16, dev_bf16(ab), None, dev_bf16(bb), None)
    else:
        quant, f = (mxq.quantize_mxfp8, mxq.MXFP8) if fmt == "mxfp8" else (mxq.quantize_mxfp4, mxq.MXFP4)
        qa, sa, _, _ = quant(dev_bf16(ab), True, False)
        qb, sb, _, _ = quant(dev_bf16(bb), True, False)
        c = mxq.gemm_block_scaled(f, qa, sa, qb, sb)
    assert np.array_equal(host(c), exact.astype(np.float32)), f"{fmt} at K = 2^22"


def test_grouped_weight_gradient_at_the_k_limit_is_exact():
    """The BF16 weight-gradient grouped GEMM with the reduction total at its limit, 2^22,
    over three groups (one empty, boundaries multiples of 8): exact per group as above."""
    g = inputs.rng(176, 0)
    M, N, total = 48, 40, 1 << 22
    offsets = np.array([0, 1_500_000, 1_500_000, total], dtype=np.int64)
    a, ab = _small_int_operand(g, (M, total))
    b, bb = _small_int_operand(g, (N, total))
    c = host(mxq.grouped_gemm_block_scaled(mxq.BF16, dev(offsets), dev_bf16(ab), dev_bf16(bb), N=N, K=0,
                                           vary_k=True, M=M, total=total))
    for e in range(3):
        lo, hi = offsets[e], offsets[e + 1]
        ref = (a[:, lo:hi].astype(np.float64) @ b[:, lo:hi].astype(np.float64).T).astype(np.float32)
        assert np.array_equal(c[e], ref), f"group {e}"


# ------------- more groups than two rounds of the 64-ary group search reach -------------

@pytest.mark.parametrize("G", [4097, 5000])
def test_grouped_rows_with_more_than_4096_groups(G):
    """Row-grouped BF16 GEMM over more groups than two rounds of the tile->group search
    cover (64^2 = 4096): most groups empty or a few rows long, every group's rows within
    2e-5 of the oracle, the padding rows of each group's last tile never written."""
    g = inputs.rng(177, G)
    N, K = 40, 64
    sizes = g.geometric(0.25, G) - 1                          # many zeros, a few rows each
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    S = int(off[-1])
    a = inputs.normal_bf16(g, (S, K))
    w = inputs.normal_bf16(g, (G * N, K), 0.05)
    out = torch.full((S, N), float("nan"), device="cuda")
    mxq.grouped_gemm_block_scaled(mxq.BF16, dev(off), dev_bf16(a), dev_bf16(w), N=N, K=K, total=S, out=out)
    got = host(out)
    ref = omoe.grouped_gemm_ref(F.bf16_bits_to_f32(a).astype(np.float64), off,
                                F.bf16_bits_to_f32(w).astype(np.float64).reshape(G, N, K))
    assert_gemm_close(got, ref, f"{G} groups")


def test_grouped_weight_gradient_with_more_than_4096_groups():
    """Weight-gradient (vary-K) grouped BF16 GEMM over 5000 groups, group boundaries
    multiples of 8 and many empty groups (their outputs are zero)."""
    g = inputs.rng(178, 0)
    G, M, N = 5000, 32, 40
    sizes = 8 * (g.geometric(0.3, G) - 1)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    total = int(off[-1])
    a = inputs.normal_bf16(g, (M, total))
    b = inputs.normal_bf16(g, (N, total))
    got = host(mxq.grouped_gemm_block_scaled(mxq.BF16, dev(off), dev_bf16(a), dev_bf16(b), N=N, K=0, vary_k=True,
                                             M=M, total=total))
    af, bf = F.bf16_bits_to_f32(a).astype(np.float64), F.bf16_bits_to_f32(b).astype(np.float64)
    for e in range(G):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            assert np.all(got[e] == 0.0), f"empty group {e}"
        else:
            assert_gemm_close(got[e], af[:, lo:hi] @ bf[:, lo:hi].T, f"group {e}")


# ------------- weight gradients from the K-major (slot-major) gradient -------------

@pytest.mark.parametrize("M,N,sizes", [
    (296, 260, [96, 0, 40, 416, 8]),                    # 128x128 tiles, ragged M and N, K tails of 8
    (2048, 2048, [520, 0, 64, 1000]),                   # 256x256 tiles (64 per group)
    (776, 1032, [0, 0, 136]),                           # empty leading groups, one group
    (8, 136, [8, 24, 0]),                               # the narrowest A (one 16-byte chunk per row)
])
def test_weight_gradient_from_k_major_a(M, N, sizes):
    """vary_k = 2 reads A as the (total, M) slot-major tensor through LDS transpose reads:
    bit-identical to vary_k = 1 on the transposed copy (same operand values, same K order)
    and within 2e-5 of the oracle per group; empty groups give zeros."""
    g = inputs.rng(181, M)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    total = int(off[-1])
    a_km = inputs.normal_bf16(g, (total, M))                 # slot-major: row k holds the M values
    b = inputs.normal_bf16(g, (N, total), 0.05)
    got2 = host(mxq.grouped_gemm_block_scaled(mxq.BF16, dev(off), dev_bf16(a_km), dev_bf16(b), N=N, K=0, vary_k=2,
                                              M=M, total=total))
    got1 = host(mxq.grouped_gemm_block_scaled(mxq.BF16, dev(off), dev_bf16(np.ascontiguousarray(a_km.T)), dev_bf16(b),
                                              N=N, K=0, vary_k=True, M=M, total=total))
    assert np.array_equal(got2.view(np.uint32), got1.view(np.uint32)), "vary_k 2 differs from vary_k 1"
    af, bf = F.bf16_bits_to_f32(a_km).astype(np.float64), F.bf16_bits_to_f32(b).astype(np.float64)
    for e in range(len(sizes)):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            assert np.all(got2[e] == 0.0)
        else:
            assert_gemm_close(got2[e], af[lo:hi].T @ bf[:, lo:hi].T, f"group {e}")
