"""GPU parity of the composed workloads: the transposed dequantization that feeds
the dequantized-backward GEMMs (bit-exact against the oracle's BF16 dequantization),
and the routed-expert MoE layer with padded expert segments, forward and
dequantized backward, checked stage by stage (each stage's reference consumes the
device's actual input to that stage)."""

import numpy as np
import pytest
import torch

import microscaling_precision_quantization_amd as mxq
from microscaling_precision_quantization_amd import inputs, pipeline
from oracle import formats as F
from oracle import moe as omoe
from oracle import mxfp4 as om4
from oracle import mxfp8 as omx
from oracle import nvfp4 as onv
from tests.gpu_util import assert_bytes_equal, assert_gemm_close, dev, dev_bf16, host

pytestmark = pytest.mark.gpu


def test_dequantize_transposed_nvfp4_groups():
    G, N, K = 3, 96, 160
    wb = inputs.normal_bf16(inputs.rng(120, 0), (G * N, K), 0.02)
    q, s, t = mxq.quantize_nvfp4(dev_bf16(wb), scope="group", group_rows=N)
    out = host(mxq.binding.dequantize_transposed(mxq.NVFP4, q, s, t, t_scope="group", groups=G, group_rows=N))
    ref = onv.dequantize_bf16_bits(host(q), host(s), np.repeat(host(t), N)).reshape(G, N, K).transpose(0, 2, 1)
    assert_bytes_equal(out, np.ascontiguousarray(ref), "nvfp4 per-expert transpose")


@pytest.mark.parametrize("scope", ["row", "tensor", "group"])
def test_dequantize_transposed_nvfp4_ragged_tiles(scope):
    """Without a gather: columns % 32 == 16 (a half 32-element unit at the tile edge),
    200 output columns per group (a ragged second 128-column tile), two groups."""
    G, N, K = 2, 200, 176
    xb = inputs.to_bf16_bits(inputs.rng(120, 5).standard_normal((G * N, K)) * np.exp2(inputs.rng(120, 6).integers(-6, 6, (G * N, 1))))
    if scope == "row":
        q, s, t = mxq.quantize_nvfp4_per_token(dev_bf16(xb))
        t_rows = host(t)
    elif scope == "tensor":
        q, s, t = mxq.quantize_nvfp4(dev_bf16(xb), scope="tensor")
        t_rows = np.repeat(host(t), G * N)
    else:
        q, s, t = mxq.quantize_nvfp4(dev_bf16(xb), scope="group", group_rows=N)
        t_rows = np.repeat(host(t), N)
    out = host(mxq.binding.dequantize_transposed(mxq.NVFP4, q, s, t, t_scope=scope, groups=G, group_rows=N))
    ref = onv.dequantize_bf16_bits(host(q), host(s), t_rows).reshape(G, N, K).transpose(0, 2, 1)
    assert_bytes_equal(out, np.ascontiguousarray(ref), f"nvfp4 transpose, {scope} scale")


def test_dequantize_transposed_gather_and_padding():
    T, H = 77, 272
    xb = inputs.to_bf16_bits(inputs.rng(120, 1).standard_normal((T, H)) * 3)
    q, s, t = mxq.quantize_nvfp4_per_token(dev_bf16(xb))
    src = inputs.rng(120, 2).integers(-1, T, size=200).astype(np.int32)    # -1 = padding (zero column)
    src[5] = T + 3                                                          # out of range: zero column too
    out = host(mxq.binding.dequantize_transposed(mxq.NVFP4, q, s, t, t_scope="row", groups=1, group_rows=T,
                                                 src_row=dev(src)))[0]
    deq = onv.dequantize_bf16_bits(host(q), host(s), host(t))
    ref = np.zeros((H, len(src)), dtype=np.uint16)
    ok = (src >= 0) & (src < T)
    ref[:, ok] = deq[src[ok]].T
    assert_bytes_equal(out, ref, "nvfp4 gathered transpose")


def test_dequantize_transposed_mxfp8_and_bf16():
    xb = inputs.normal_bf16(inputs.rng(120, 3), (136, 96), 1.0)
    qr, sr, _, _ = mxq.quantize_mxfp8(dev_bf16(xb), True, False)
    out = host(mxq.binding.dequantize_transposed(mxq.MXFP8, qr, sr))[0]
    ref = F.f32_to_bf16_bits(omx.dequantize_f32(host(qr), host(sr))).T
    assert_bytes_equal(out, np.ascontiguousarray(ref), "mxfp8 transpose")
    yb = inputs.normal_bf16(inputs.rng(120, 4), (2 * 40, 48), 1.0)
    out = host(mxq.binding.dequantize_transposed(mxq.BF16, dev_bf16(yb), groups=2, group_rows=40, cols=48))
    assert_bytes_equal(out, np.ascontiguousarray(yb.reshape(2, 40, 48).transpose(0, 2, 1)), "bf16 transpose")


def small_moe_case(pad):
    T, H, G, I, k = 200, 256, 8, 128, 2
    g = inputs.rng(121, pad)
    x = inputs.to_bf16_bits(g.standard_normal((T, H)) * g.lognormal(0, 1, (T, 1)))
    logits = g.standard_normal((T, G)).astype(np.float32)
    logits[:, 5] = -60.0                                   # expert 5 receives no token
    r = inputs.route_topk(logits, k, pad=pad)
    w_gu = inputs.normal_bf16(g, (G * 2 * I, H), 0.02)
    w_d = inputs.normal_bf16(g, (G * H, I), 0.02)
    return T, H, G, I, k, x, r, w_gu, w_d


@pytest.mark.parametrize("pad", [1, 32])
def test_moe_layer_forward_and_dequantized_backward(pad):
    T, H, G, I, k, x, r, w_gu, w_d = small_moe_case(pad)
    rd = pipeline.MoeRoutingDevice(r, torch.device("cuda"))
    m = pipeline.MoeNvfp4(T, H, G, I, rd, torch.device("cuda"), keep_h=True)
    m.quantize_weights(dev_bf16(w_gu), dev_bf16(w_d))
    y = m.forward(dev_bf16(x))
    torch.cuda.synchronize()
    S = rd.slots
    live = r.row_index >= 0
    # A3: per-token quantize
    eq, es, et = onv.quantize_per_token(x)
    assert_bytes_equal(host(m.qx), eq, "tokens packed")
    assert_bytes_equal(host(m.tx).view(np.uint32), et.view(np.uint32), "token scales")
    # A4: per-expert weights
    qg, sg, tg = (host(a) for a in m.wq["gu"])
    eq, es, et = onv.quantize_per_group(w_gu, np.arange(G + 1) * 2 * I)
    assert_bytes_equal(qg, eq, "w_gu packed")
    assert_bytes_equal(tg.view(np.uint32), et.view(np.uint32), "w_gu scales")
    # A9 + A10 gate_up (gather inside the GEMM; padding slots are zero rows)
    xh = onv.dequantize_exact(host(m.qx), host(m.sx), host(m.tx))
    a_slots = np.zeros((S, H))
    a_slots[live] = xh[r.row_index[live]]
    wgh = onv.dequantize_exact(qg, sg, np.repeat(tg, 2 * I)).reshape(G, 2 * I, H)
    gu = host(m.gu)
    ref = omoe.grouped_gemm_ref(a_slots, r.offsets, wgh)
    for e in range(G):
        lo, hi = r.offsets[e], r.offsets[e + 1]
        if hi > lo:
            assert_gemm_close(gu[lo:hi], ref[lo:hi], f"gate_up expert {e}")
    assert np.all(gu[~live] == 0.0)
    # A11: SwiGLU (correctly rounded BF16) + per-row requant, from the device's FP32 gate/up
    h = omoe.swiglu_bf16_ref(gu)
    assert_bytes_equal(host(m.h), h, "h")
    eq, es, et = onv.quantize_per_token(h)
    assert_bytes_equal(host(m.qh), eq, "h packed")
    assert_bytes_equal(host(m.th).view(np.uint32), et.view(np.uint32), "h scales")
    # A10 down
    qd, sd, td = (host(a) for a in m.wq["d"])
    wdh = onv.dequantize_exact(qd, sd, np.repeat(td, H)).reshape(G, H, I)
    hh = onv.dequantize_exact(host(m.qh), host(m.sh), host(m.th))
    o = host(m.o)
    ref = omoe.grouped_gemm_ref(hh, r.offsets, wdh)
    for e in range(G):
        lo, hi = r.offsets[e], r.offsets[e + 1]
        if hi > lo:
            assert_gemm_close(o[lo:hi], ref[lo:hi], f"down expert {e}")
    # A12 combine
    assert_gemm_close(host(y), omoe.combine_ref(o, r.slot_of, r.topk_w), "combine")

    if pad == 1:
        return
    # A6 + A13: dequantized backward on synthetic upstream gradients (padding slots zero)
    gg = inputs.rng(122, 0)
    d_o = inputs.normal_bf16(gg, (S, H), 1e-3)
    d_gu = inputs.normal_bf16(gg, (S, 2 * I), 1e-3)
    d_o[~live] = 0
    d_gu[~live] = 0
    b = pipeline.MoeDequantBackward(m)                         # dgrads straight from the NVFP4 weights
    b.dequantize_weights()
    b.backward(dev_bf16(d_o), dev_bf16(d_gu))
    b2 = pipeline.MoeDequantBackward(m, fused_weights=False)    # BF16 weight transposes first
    b2.dequantize_weights()
    b2.backward(dev_bf16(d_o), dev_bf16(d_gu))
    torch.cuda.synchronize()
    wd_b = onv.dequantize_bf16_bits(qd, sd, np.repeat(td, H)).reshape(G, H, I)
    assert_bytes_equal(host(b2.w_dT), np.ascontiguousarray(wd_b.transpose(0, 2, 1)), "W_d^T")
    wgu_b = onv.dequantize_bf16_bits(qg, sg, np.repeat(tg, 2 * I)).reshape(G, 2 * I, H)
    assert_bytes_equal(host(b2.w_guT), np.ascontiguousarray(wgu_b.transpose(0, 2, 1)), "W_gu^T")
    h_b = onv.dequantize_bf16_bits(host(m.qh), host(m.sh), host(m.th))
    assert_bytes_equal(host(b.hT)[0], np.ascontiguousarray(h_b.T), "h_hat^T")
    x_b = onv.dequantize_bf16_bits(host(m.qx), host(m.sx), host(m.tx))
    xs = np.zeros((S, H), dtype=np.uint16)
    xs[live] = x_b[r.row_index[live]]
    assert_bytes_equal(host(b.xT)[0], np.ascontiguousarray(xs.T), "X_hat gathered^T")
    f64 = lambda bits: F.bf16_bits_to_f32(bits).astype(np.float64)
    dh, dx, dw_d, dw_gu = host(b.dh), host(b.dx), host(b.dw_d), host(b.dw_gu)
    for e in range(G):
        lo, hi = r.offsets[e], r.offsets[e + 1]
        if hi == lo:
            assert np.all(dw_d[e] == 0) and np.all(dw_gu[e] == 0)
            continue
        assert_gemm_close(dh[lo:hi], f64(d_o[lo:hi]) @ f64(wd_b[e]), f"down dgrad {e}")
        assert_gemm_close(host(b2.dh[lo:hi]), f64(d_o[lo:hi]) @ f64(wd_b[e]), f"down dgrad {e} (two-step)")
        assert_gemm_close(dw_d[e], f64(d_o[lo:hi]).T @ f64(h_b[lo:hi]), f"down wgrad {e}")
        assert_gemm_close(dx[lo:hi], f64(d_gu[lo:hi]) @ f64(wgu_b[e]), f"gate_up dgrad {e}")
        assert_gemm_close(host(b2.dx[lo:hi]), f64(d_gu[lo:hi]) @ f64(wgu_b[e]), f"gate_up dgrad {e} (two-step)")
        assert_gemm_close(dw_gu[e], f64(d_gu[lo:hi]).T @ f64(xs[lo:hi]), f"gate_up wgrad {e}")


def test_shared_expert_bf16_forward_backward():
    T, H, I = 160, 256, 96
    g = inputs.rng(123, 0)
    x = inputs.normal_bf16(g, (T, H), 1.0)
    w_sgu = inputs.normal_bf16(g, (2 * I, H), 0.02)
    w_sd = inputs.normal_bf16(g, (H, I), 0.02)
    d_o = inputs.normal_bf16(g, (T, H), 1e-3)
    d_gu = inputs.normal_bf16(g, (T, 2 * I), 1e-3)
    sh = pipeline.SharedExpertBf16(T, H, I, torch.device("cuda"))
    args = [dev_bf16(a) for a in (x, w_sgu, w_sd)]
    sh.forward(*args)
    sh.backward(*args, dev_bf16(d_o), dev_bf16(d_gu))
    torch.cuda.synchronize()
    f64 = lambda bits: F.bf16_bits_to_f32(bits).astype(np.float64)
    gu = host(sh.gu)
    assert_gemm_close(gu, f64(x) @ f64(w_sgu).T, "shared gate_up")
    h = host(sh.h)
    assert_bytes_equal(h, omoe.swiglu_bf16_ref(gu), "shared h")
    assert_gemm_close(host(sh.o), f64(h) @ f64(w_sd).T, "shared down")
    assert_gemm_close(host(sh.dh), f64(d_o) @ f64(w_sd), "shared down dgrad")
    assert_gemm_close(host(sh.dw_sd), f64(d_o).T @ f64(h), "shared down wgrad")
    assert_gemm_close(host(sh.dx), f64(d_gu) @ f64(w_sgu), "shared gate_up dgrad")
    assert_gemm_close(host(sh.dw_sgu), f64(d_gu).T @ f64(x), "shared gate_up wgrad")


# ------------------------- full-size workloads (sampled) -------------------------

def check_moe_sampled(m, r, x_bits, w_gu_bits_of, w_d_bits_of, experts, tokens, what):
    """Stage-wise parity of a full-size MoE forward on sampled experts and tokens.
    w_*_bits_of(e) returns expert e's BF16 weight bits."""
    T, H, G, I = m.T, m.H, m.G, m.I
    live = r.row_index >= 0
    eq, es, et = onv.quantize_per_token(x_bits)
    assert_bytes_equal(host(m.qx), eq, f"{what} tokens packed")
    assert_bytes_equal(host(m.sx), es, f"{what} tokens scales")
    assert_bytes_equal(host(m.tx).view(np.uint32), et.view(np.uint32), f"{what} token scales")
    xh = onv.dequantize_exact(eq, es, et)
    qg, sg, tg = m.wq["gu"]
    qd, sd, td = m.wq["d"]
    tg, td = host(tg), host(td)
    for e in experts:
        lo, hi = int(r.offsets[e]), int(r.offsets[e + 1])
        # A4 for this expert
        gq, gs, gt = onv.quantize_per_group(w_gu_bits_of(e), [0, 2 * I])
        assert_bytes_equal(host(qg[e * 2 * I:(e + 1) * 2 * I]), gq, f"{what} w_gu[{e}] packed")
        assert_bytes_equal(host(sg[e * 2 * I:(e + 1) * 2 * I]), gs, f"{what} w_gu[{e}] scales")
        assert tg.view(np.uint32)[e] == gt.view(np.uint32)[0]
        dq, ds, dt = onv.quantize_per_group(w_d_bits_of(e), [0, H])
        assert_bytes_equal(host(qd[e * H:(e + 1) * H]), dq, f"{what} w_d[{e}] packed")
        assert td.view(np.uint32)[e] == dt.view(np.uint32)[0]
        if hi == lo:
            continue
        rows = r.row_index[lo:hi]
        a = np.zeros((hi - lo, H))
        a[rows >= 0] = xh[rows[rows >= 0]]
        gu = host(m.gu[lo:hi])
        assert_gemm_close(gu, a @ onv.dequantize_exact(gq, gs, np.repeat(gt, 2 * I)).T, f"{what} gate_up[{e}]")
        h_ref = omoe.swiglu_bf16_ref(gu)                       # from the device's FP32 gate/up
        if m.h is not None:
            assert_bytes_equal(host(m.h[lo:hi]), h_ref, f"{what} h[{e}]")
        hq, hs, ht = host(m.qh[lo:hi]), host(m.sh[lo:hi]), host(m.th[lo:hi])
        eq, es, et = onv.quantize_per_token(h_ref)
        assert_bytes_equal(hq, eq, f"{what} h[{e}] packed")
        assert_bytes_equal(hs, es, f"{what} h[{e}] block scales")
        assert_bytes_equal(ht.view(np.uint32), et.view(np.uint32), f"{what} h[{e}] scales")
        o = host(m.o[lo:hi])
        assert_gemm_close(o, onv.dequantize_exact(hq, hs, ht) @ onv.dequantize_exact(dq, ds, np.repeat(dt, H)).T,
                          f"{what} down[{e}]")
    # combine on sampled tokens, from the device's slot outputs
    so = r.slot_of[tokens]
    o_rows = host(m.o[torch.from_numpy(so.reshape(-1)).cuda()]).reshape(len(tokens), so.shape[1], H)
    ref = np.einsum("tj,tjh->th", r.topk_w[tokens].astype(np.float64), o_rows.astype(np.float64))
    assert_gemm_close(host(m.y[torch.from_numpy(tokens).cuda()]), ref, f"{what} combine (sampled tokens)")
    assert not np.any(live[r.slot_of.reshape(-1)] == 0)


def test_moe_qwen3_full_size_sampled():
    w = inputs.workload_moe_qwen3()
    T, H, G, I = w["x"].shape[0], w["hidden"], w["experts"], w["inter"]
    d = torch.device("cuda")
    rd = pipeline.MoeRoutingDevice(w["routing"], d)
    m = pipeline.MoeNvfp4(T, H, G, I, rd, d, keep_h=True)
    m.quantize_weights(dev_bf16(w["w_gu"].reshape(G * 2 * I, H)), dev_bf16(w["w_d"].reshape(G * H, I)))
    m.forward(dev_bf16(w["x"]))
    torch.cuda.synchronize()
    experts = [0, 37, 64, 127]
    tokens = np.sort(np.random.default_rng(7).choice(T, 64, replace=False))
    check_moe_sampled(m, w["routing"], w["x"], lambda e: w["w_gu"][e], lambda e: w["w_d"][e], experts, tokens,
                      "qwen3")


def test_moe_deepseek_full_size_sampled():
    w = inputs.workload_moe_deepseek()
    T, H, G, I = w["x"].shape[0], w["hidden"], w["experts"], w["inter"]
    d = torch.device("cuda")
    t = inputs.deepseek_device_tensors(torch, d, w)
    r = w["routing"]
    rd = pipeline.MoeRoutingDevice(r, d)
    m = pipeline.MoeNvfp4(T, H, G, I, rd, d, keep_h=True)
    m.quantize_weights(t["w_gu"], t["w_d"])
    x = dev_bf16(w["x"])
    m.forward(x)
    b = pipeline.MoeDequantBackward(m)
    b.dequantize_weights()
    b.backward(t["d_o"], t["d_gu"])
    sh = pipeline.SharedExpertBf16(T, H, I, d)
    sh.forward(x, t["w_sgu"], t["w_sd"])
    sh.backward(x, t["w_sgu"], t["w_sd"], t["d_os"], t["d_gus"])
    torch.cuda.synchronize()
    bits = lambda ten: host(ten)
    experts = [3, 200]
    tokens = np.sort(np.random.default_rng(8).choice(T, 32, replace=False))
    check_moe_sampled(m, r, w["x"], lambda e: bits(t["w_gu"][e * 2 * I:(e + 1) * 2 * I]),
                      lambda e: bits(t["w_d"][e * H:(e + 1) * H]), experts, tokens, "deepseek")
    # dequantized backward on the sampled experts
    f64 = lambda b16: F.bf16_bits_to_f32(b16).astype(np.float64)
    qg, sg, tg = (host(a) for a in m.wq["gu"])
    xq = onv.dequantize_bf16_bits(host(m.qx), host(m.sx), host(m.tx))
    for e in experts:
        lo, hi = int(r.offsets[e]), int(r.offsets[e + 1])
        wgu_b = onv.dequantize_bf16_bits(qg[e * 2 * I:(e + 1) * 2 * I], sg[e * 2 * I:(e + 1) * 2 * I],
                                         np.repeat(tg[e:e + 1], 2 * I))
        wguT = mxq.dequantize_transposed(mxq.NVFP4, m.wq["gu"][0][e * 2 * I:(e + 1) * 2 * I],
                                         m.wq["gu"][1][e * 2 * I:(e + 1) * 2 * I], m.wq["gu"][2][e:e + 1],
                                         t_scope="group", groups=1, group_rows=2 * I, cols=H)
        assert_bytes_equal(host(wguT[0]), np.ascontiguousarray(wgu_b.T), f"W_gu^T[{e}]")
        qd, sd, td = (host(a[e * H:(e + 1) * H]) if a.dim() == 2 else host(a) for a in m.wq["d"])
        wd_b = onv.dequantize_bf16_bits(qd, sd, np.repeat(td[e:e + 1], H))
        d_o, d_gu = host(t["d_o"][lo:hi]), host(t["d_gu"][lo:hi])
        h_b = onv.dequantize_bf16_bits(host(m.qh[lo:hi]), host(m.sh[lo:hi]), host(m.th[lo:hi]))
        rows = r.row_index[lo:hi]
        xs = np.zeros((hi - lo, H), dtype=np.uint16)
        xs[rows >= 0] = xq[rows[rows >= 0]]
        assert_gemm_close(host(b.dh[lo:hi]), f64(d_o) @ f64(wd_b), f"down dgrad[{e}]")
        assert_gemm_close(host(b.dw_d[e]), f64(d_o).T @ f64(h_b), f"down wgrad[{e}]")
        assert_gemm_close(host(b.dx[lo:hi]), f64(d_gu) @ f64(wgu_b), f"gate_up dgrad[{e}]")
        assert_gemm_close(host(b.dw_gu[e]), f64(d_gu).T @ f64(xs), f"gate_up wgrad[{e}]")
    # shared expert on sampled token rows (its weight gradients in full)
    xb, wsgu, wsd = w["x"], host(t["w_sgu"]), host(t["w_sd"])
    gu = host(sh.gu[torch.from_numpy(tokens).cuda()])
    assert_gemm_close(gu, f64(xb[tokens]) @ f64(wsgu).T, "shared gate_up (sampled rows)")
    h = host(sh.h)
    assert_bytes_equal(h[tokens], omoe.swiglu_bf16_ref(gu), "shared h (sampled rows)")
    assert_gemm_close(host(sh.o[torch.from_numpy(tokens).cuda()]), f64(h[tokens]) @ f64(wsd).T, "shared down")
    d_os, d_gus = host(t["d_os"]), host(t["d_gus"])
    assert_gemm_close(host(sh.dw_sd), f64(d_os).T @ f64(h), "shared down wgrad")
    assert_gemm_close(host(sh.dx[torch.from_numpy(tokens).cuda()]), f64(d_gus[tokens]) @ f64(wsgu),
                      "shared gate_up dgrad (sampled rows)")


def test_stress_nvfp4_rht_wgrad_full_size_sampled():
    n = 8192
    w = inputs.workload_stress(n)
    st = pipeline.StressStep(n, w["signs"], torch.device("cuda"))
    a, b = dev_bf16(w["a"]), dev_bf16(w["b"])
    st.quantize_rht(a, b)
    st.nvfp4_wgrad()
    torch.cuda.synchronize()
    qa, sa, ta = (host(v) for v in st.nv["a"])
    qb, sb, tb = (host(v) for v in st.nv["b"])
    rows = np.sort(np.random.default_rng(9).choice(n, 32, replace=False))
    ah = onv.dequantize_exact(qa[rows], sa[rows], np.repeat(ta, len(rows)))
    bh = onv.dequantize_exact(qb, sb, np.repeat(tb, n))
    c = host(st.c["wgrad_nvfp4"][torch.from_numpy(rows).cuda()])
    assert_gemm_close(c, ah @ bh.T, "8192^3 NVFP4 RHT wgrad (sampled rows)")
    # RHT keeps the product: the FP64 product of the unquantized transformed operands
    # equals A^T B up to FP32 rounding of the transform (orthogonality of H16 diag(s) / 4)
    x = inputs.bf16_bits_to_float(w["a"])
    y = inputs.bf16_bits_to_float(w["b"])
    cols = rows[:8]
    ua = onv.rht16_rows(np.ascontiguousarray(x[:, cols].T), w["signs"]).astype(np.float64)
    ub = onv.rht16_rows(np.ascontiguousarray(y.T[:256]), w["signs"]).astype(np.float64)
    direct = x[:, cols].T.astype(np.float64) @ y[:, :256].astype(np.float64)
    assert np.linalg.norm(ua @ ub.T - direct) <= 1e-6 * np.linalg.norm(direct)


def test_linear_mxfp4_layer_matches_direct_calls():
    """The MXFP4 linear layer (one multi-tensor quantize launch, three native FP4 GEMMs)
    writes exactly what the single calls write."""
    g = inputs.rng(122, 0)
    T, Di, Do = 256, 384, 320
    x = dev_bf16(inputs.normal_bf16(g, (T, Di), 1.0))
    w = dev_bf16(inputs.normal_bf16(g, (Do, Di), 0.02))
    dy = dev_bf16(inputs.normal_bf16(g, (T, Do), 1e-3))
    L = pipeline.LinearMxfp4(T, Di, Do, torch.device("cuda:0"))
    L.step(x, w, dy)
    for name, t in (("x", x), ("w", w), ("dy", dy)):
        ref = mxq.quantize_mxfp4(t)
        for a, b, nm in zip(L.q[name], ref, ("q_row", "s_row", "q_colT", "s_colT")):
            assert_bytes_equal(host(a), host(b), f"{name} {nm}")
    xq, wq, dq = L.q["x"], L.q["w"], L.q["dy"]
    for got, (A, sA, Bq, sB) in ((L.y, (xq[0], xq[1], wq[0], wq[1])), (L.dx, (dq[0], dq[1], wq[2], wq[3])),
                                 (L.dw, (dq[2], dq[3], xq[2], xq[3]))):
        ref = mxq.gemm_block_scaled(mxq.MXFP4, A, sA, Bq, sB)
        assert_bytes_equal(host(got).view(np.uint32), host(ref).view(np.uint32), "gemm")
        ah = om4.dequantize_exact(host(A), host(sA))
        bh = om4.dequantize_exact(host(Bq), host(sB))
        assert_gemm_close(host(got), ah @ bh.T, "linear mxfp4")


def test_linear_fp8_block_layer_matches_direct_calls():
    g = inputs.rng(123, 0)
    T, Di, Do = 256, 384, 640
    x = dev_bf16(inputs.normal_bf16(g, (T, Di), 1.0))
    w = dev_bf16(inputs.normal_bf16(g, (Do, Di), 0.02))
    dy = dev_bf16(inputs.normal_bf16(g, (T, Do), 1e-3))
    L = pipeline.LinearFp8Block(T, Di, Do, torch.device("cuda:0"))
    L.step(x, w, dy)
    for got, ref in ((L.qx, mxq.quantize_fp8_block_act(x, True, True)), (L.qw, mxq.quantize_fp8_block_weight(w)),
                     (L.qdy, mxq.quantize_fp8_block_act(dy, True, True))):
        for a, b in zip(got, ref):
            assert_bytes_equal(host(a).view(np.uint8), host(b).view(np.uint8), "fp8 block copy")
    for got, args, blocks in ((L.y, (L.qx[0], L.qx[1], L.qw[0], L.qw[1]), True),
                              (L.dx, (L.qdy[0], L.qdy[1], L.qw[2], L.qw[3]), True),
                              (L.dw, (L.qdy[2], L.qdy[3], L.qx[2], L.qx[3]), False)):
        ref = mxq.gemm_fp8_blockwise(*args, b_blocks=blocks)
        assert_bytes_equal(host(got).view(np.uint32), host(ref).view(np.uint32), "fp8 block gemm")
