"""GPU check of grouped_gemm_block_scaled_noalloc, the grouped GEMM entry point whose
scheduler scratch lives in the library's static device array (for callers that cannot
allocate): called through the C ABI, its output must equal grouped_gemm_block_scaled's
bit for bit (the same kernels run) and meet the 2e-5 bound against the oracle, on two
calls in a row, the second smaller, so stale scratch from the first would show; and
captured in a HIP graph, each replay with new data equal to the workspace entry point."""

import ctypes

import numpy as np
import pytest
import torch

import microscaling_precision_quantization_amd as mxq
from microscaling_precision_quantization_amd import binding as B
from microscaling_precision_quantization_amd import inputs
from oracle import moe as omoe
from oracle import nvfp4 as onv
from tests.gpu_util import assert_gemm_close, dev, dev_bf16, host

pytestmark = pytest.mark.gpu


def _moe_case(seed, tokens, groups, N, K, topk=2):
    """Per-token NVFP4 tokens, per-expert NVFP4 weights, a random routing with some
    empty experts; returns device operands, offsets, gather index and the oracle."""
    g = inputs.rng(160, seed)
    x = inputs.to_bf16_bits(g.standard_normal((tokens, K)) * g.lognormal(0, 1, (tokens, 1)))
    w = inputs.normal_bf16(g, (groups * N, K), 0.02)
    choice = np.stack([g.choice(groups, topk, replace=False) for _ in range(tokens)])
    choice[choice % 7 == 3] = 0                                  # leaves a few experts empty
    order = np.argsort(choice.ravel(), kind="stable")
    row_index = (order // topk).astype(np.int32)
    counts = np.bincount(choice.ravel(), minlength=groups)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    qx, sx, tx = mxq.quantize_nvfp4_per_token(dev_bf16(x))
    qw, sw, tw = mxq.quantize_nvfp4(dev_bf16(w), scope="group", group_rows=N)
    xh = onv.dequantize_exact(host(qx), host(sx), host(tx))
    wh = onv.dequantize_exact(host(qw), host(sw), np.repeat(host(tw), N)).reshape(groups, N, K)
    ref = omoe.grouped_gemm_ref(xh[row_index], offsets, wh)
    return dict(qx=qx, sx=sx, tx=tx, qw=qw, sw=sw, tw=tw, off=dev(offsets), idx=dev(row_index), total=len(row_index),
                groups=groups, N=N, K=K, tokens=tokens, ref=ref, offsets=offsets)


def _call_noalloc(c, out, groups=None):
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    return B.lib().grouped_gemm_block_scaled_noalloc(
        B.NVFP4, c["groups"] if groups is None else groups, p(c["off"]), 0, c["total"], 0, c["N"], c["K"], p(c["idx"]),
        c["tokens"], p(c["qx"]), p(c["sx"]), p(c["tx"]), B.SCOPE["row"], p(c["qw"]), p(c["sw"]), p(c["tw"]),
        B.SCOPE["group"], p(out), B._stream(out.device))


def _call_workspace(c):
    return mxq.grouped_gemm_block_scaled(mxq.NVFP4, c["off"], c["qx"], c["qw"], N=c["N"], K=c["K"], sA=c["sx"],
                                         sB=c["sw"], tA=c["tx"], tB=c["tw"], tA_scope="row", tB_scope="group",
                                         a_row_index=c["idx"], total=c["total"], a_rows=c["tokens"])


def test_noalloc_grouped_gemm_matches_the_workspace_entry_point_twice():
    big = _moe_case(0, tokens=700, groups=96, N=256, K=512)
    small = _moe_case(1, tokens=90, groups=12, N=128, K=256)
    outs = []
    for c in (big, small):                                        # second call: fewer groups, smaller problem
        out = torch.full((c["total"], c["N"]), 9.0, device="cuda")
        assert _call_noalloc(c, out) == 0
        outs.append(out)
    torch.cuda.synchronize()
    for c, out in zip((big, small), outs):
        got = host(out)
        ref_ws = host(_call_workspace(c))
        assert np.array_equal(got.view(np.uint32), ref_ws.view(np.uint32)), "differs from grouped_gemm_block_scaled"
        for e in range(c["groups"]):
            lo, hi = c["offsets"][e], c["offsets"][e + 1]
            if hi > lo:
                assert_gemm_close(got[lo:hi], c["ref"][lo:hi], f"expert {e}")


def test_noalloc_rejects_more_groups_than_its_scratch_holds():
    c = _moe_case(2, tokens=64, groups=8, N=128, K=256)
    out = torch.full((c["total"], c["N"]), 9.0, device="cuda")
    assert _call_noalloc(c, out, groups=8192) == 5                # MXQ_ERR_WORKSPACE: nothing launched
    torch.cuda.synchronize()
    assert np.all(host(out) == 9.0)


def test_noalloc_grouped_gemm_in_a_captured_hip_graph():
    """The use the entry point exists for: captured in a HIP graph (no allocation, no
    workspace argument) and replayed with new token data copied into its operands, with
    eager work and synchronizations between replays; every replay equals the workspace
    entry point on the same data, bit for bit."""
    c = _moe_case(3, tokens=300, groups=24, N=256, K=512)
    out = torch.full((c["total"], c["N"]), 9.0, device="cuda")
    assert _call_noalloc(c, out) == 0                             # first use outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        assert _call_noalloc(c, out) == 0
    torch.cuda.synchronize()
    for trial in range(3):
        g = inputs.rng(161, trial)
        x = inputs.to_bf16_bits(g.standard_normal((c["tokens"], c["K"])) * g.lognormal(0, 1, (c["tokens"], 1)))
        qx, sx, tx = mxq.quantize_nvfp4_per_token(dev_bf16(x))
        c["qx"].copy_(qx)
        c["sx"].copy_(sx)
        c["tx"].copy_(tx)
        out.fill_(7.0)
        graph.replay()
        torch.cuda.synchronize()
        got = host(out)
        ref_ws = host(_call_workspace(c))                         # eager call between replays
        torch.cuda.synchronize()
        assert np.array_equal(got.view(np.uint32), ref_ws.view(np.uint32)), f"replay {trial}"


def test_noalloc_at_its_group_limit():
    """MXQ_NOALLOC_MAX_GROUPS groups (8191), the most the static scratch holds: mostly
    empty experts, bit-identical to the workspace entry point and within 2e-5 per expert."""
    g = inputs.rng(162, 0)
    groups, N, K, tokens = 8191, 64, 256, 600
    x = inputs.to_bf16_bits(g.standard_normal((tokens, K)))
    w = inputs.normal_bf16(g, (groups * N, K), 0.02)
    choice = g.integers(0, groups, (tokens, 2))
    choice[:, 1] = (choice[:, 0] + 1 + g.integers(0, groups - 1, tokens)) % groups     # two distinct experts
    order = np.argsort(choice.ravel(), kind="stable")
    row_index = (order // 2).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(np.bincount(choice.ravel(), minlength=groups))]).astype(np.int64)
    qx, sx, tx = mxq.quantize_nvfp4_per_token(dev_bf16(x))
    qw, sw, tw = mxq.quantize_nvfp4(dev_bf16(w), scope="group", group_rows=N)
    c = dict(qx=qx, sx=sx, tx=tx, qw=qw, sw=sw, tw=tw, off=dev(offsets), idx=dev(row_index), total=len(row_index),
             groups=groups, N=N, K=K, tokens=tokens)
    out = torch.full((c["total"], N), 9.0, device="cuda")
    assert _call_noalloc(c, out) == 0
    torch.cuda.synchronize()
    got = host(out)
    assert np.array_equal(got.view(np.uint32), host(_call_workspace(c)).view(np.uint32))
    xh = onv.dequantize_exact(host(qx), host(sx), host(tx))[row_index]
    qwh, swh, twh = host(qw), host(sw), host(tw)
    for e in np.nonzero(np.diff(offsets))[0]:                    # the experts that got tokens
        lo, hi = offsets[e], offsets[e + 1]
        we = onv.dequantize_exact(qwh[e * N:(e + 1) * N], swh[e * N:(e + 1) * N], np.repeat(twh[e], N))
        assert_gemm_close(got[lo:hi], xh[lo:hi] @ we.T, f"expert {e}")
