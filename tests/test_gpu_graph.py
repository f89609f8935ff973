"""Whole steps captured in one HIP graph (torch.cuda.graph over the C-ABI calls on the
capture stream) and replayed: every replay, with new data copied into the step's
inputs and eager work and synchronizations between replays, gives the same bits as
the same step run eagerly. The library's launches record only kernels (zero fills are
kernels too), so a graph replays them as issued."""

import numpy as np
import pytest
import torch

from microscaling_precision_quantization_amd import inputs, pipeline
from tests.gpu_util import dev_bf16

pytestmark = pytest.mark.gpu


def _bits(ts):
    return [t.detach().clone().view(torch.uint8) if t.dtype != torch.uint8 else t.detach().clone() for t in ts]


def _check_graph(step, outputs, feeds, what):
    """step(): the eager step; outputs(): tensors to compare; feeds: callables that each
    write a new input set into the step's input buffers."""
    feeds[0]()
    step()                                               # warm (first-use set-up outside the capture)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for n, feed in enumerate(feeds):
        feed()
        g.replay()
        torch.cuda.synchronize()
        got = _bits(outputs())
        torch.randn(1 << 20, device="cuda").sum().item()  # unrelated eager work between replays
        feed()
        step()
        torch.cuda.synchronize()
        exp = _bits(outputs())
        for i, (a, b) in enumerate(zip(got, exp)):
            assert torch.equal(a, b), f"{what}: replay {n}, output {i} differs from the eager step"


def test_graph_replay_linear_mxfp8_step():
    T, Di, Do = 256, 512, 1024
    L = pipeline.LinearMxfp8(T, Di, Do, torch.device("cuda"))
    x = torch.empty((T, Di), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((Do, Di), dtype=torch.bfloat16, device="cuda")
    dy = torch.empty((T, Do), dtype=torch.bfloat16, device="cuda")

    def feed(seed):
        def f():
            g = inputs.rng(160, seed)
            x.copy_(dev_bf16(inputs.to_bf16_bits(g.standard_normal((T, Di)) * g.lognormal(0, 1, (T, 1)))))
            w.copy_(dev_bf16(inputs.normal_bf16(g, (Do, Di), 0.02)))
            dy.copy_(dev_bf16(inputs.normal_bf16(g, (T, Do), 1e-3)))
        return f

    def step():
        L.quantize(x, w, dy)
        L.gemm_all()

    outputs = lambda: [*L.q["x"], *L.q["w"], *L.q["dy"], L.y, L.dx, L.dw]
    _check_graph(step, outputs, [feed(s) for s in range(3)], "linear MXFP8 step")


def test_graph_replay_moe_forward_and_dequantized_backward():
    T, H, G, I, k = 192, 512, 8, 256, 2
    r = inputs.route_topk(inputs.rng(161, 0).standard_normal((T, G)).astype(np.float32), k, pad=32)
    d = torch.device("cuda")
    rd = pipeline.MoeRoutingDevice(r, d)
    moe = pipeline.MoeNvfp4(T, H, G, I, rd, d)
    bwd = pipeline.MoeDequantBackward(moe)
    S = rd.slots
    x = torch.empty((T, H), dtype=torch.bfloat16, device=d)
    w_gu = torch.empty((G * 2 * I, H), dtype=torch.bfloat16, device=d)
    w_d = torch.empty((G * H, I), dtype=torch.bfloat16, device=d)
    d_o = torch.empty((S, H), dtype=torch.bfloat16, device=d)
    d_gu = torch.empty((S, 2 * I), dtype=torch.bfloat16, device=d)
    live = torch.from_numpy(r.row_index >= 0).to(d)[:, None]

    def feed(seed):
        def f():
            g = inputs.rng(162, seed)
            x.copy_(dev_bf16(inputs.to_bf16_bits(g.standard_normal((T, H)) * g.lognormal(0, 1, (T, 1)))))
            w_gu.copy_(dev_bf16(inputs.normal_bf16(g, (G * 2 * I, H), 0.02)))
            w_d.copy_(dev_bf16(inputs.normal_bf16(g, (G * H, I), 0.02)))
            d_o.copy_(dev_bf16(inputs.normal_bf16(g, (S, H), 1e-3)) * live)
            d_gu.copy_(dev_bf16(inputs.normal_bf16(g, (S, 2 * I), 1e-3)) * live)
        return f

    def step():
        moe.quantize_weights(w_gu, w_d)
        moe.quantize_tokens(x)
        moe.gate_up()
        moe.swiglu()
        moe.down()
        moe.combine()
        bwd.backward(d_o, d_gu)

    outputs = lambda: [moe.qx, moe.gu, moe.qh, moe.o, moe.y, *moe.wq["gu"], *moe.wq["d"],
                       bwd.hT, bwd.xT, bwd.dh, bwd.dx, bwd.dw_d, bwd.dw_gu]
    _check_graph(step, outputs, [feed(s) for s in range(3)], "MoE forward + dequantized backward")
