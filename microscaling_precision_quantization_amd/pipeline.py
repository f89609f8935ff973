"""The hot path's workloads as sequences of libmxq calls.

Orchestration only: every function below issues C-ABI calls through the binding
on torch's current stream, into buffers allocated once up front; no step of the
method runs in Python. Shapes and roles follow the pages' workloads: the MXFP8
linear layer (fprop, dgrad, wgrad), the per-token NVFP4 routed-expert MoE layer
(forward, and the dequantized backward of "Miles Blackwell RL", remio.ai,
section "La Compatibilidad de Miles Blackwell Ahora Abarca Todo el Ciclo de
RL"), the BF16 shared expert, and the heavy-tailed stress case with the NVFP4
random-Hadamard weight gradient (7minutos.es NVFP4 page, section "La
metodologia de formacion de cuatro partes").

All GEMMs are "TN": C[m, n] = sum_k A[m, k] B[n, k], both operands K-contiguous.
"""

from __future__ import annotations

import torch

from . import binding as B


def _u8(shape, dev):
    return torch.empty(shape, dtype=torch.uint8, device=dev)


def _f32(shape, dev):
    return torch.empty(shape, dtype=torch.float32, device=dev)


def _bf16(shape, dev):
    return torch.empty(shape, dtype=torch.bfloat16, device=dev)


# ---------------------------------------------------------------------------
# MXFP8 linear layer
# ---------------------------------------------------------------------------

class LinearMxfp8:
    """Y = X W^T, dX = dY W, dW = dY^T X with X (T, Din), W (Dout, Din), dY (T, Dout).

    Every tensor is quantized once into a rowwise and a columnwise-transposed copy;
    fprop uses X and W rowwise, dgrad dY rowwise and W columnwise, wgrad dY and X
    columnwise (blocks along each GEMM's reduction axis)."""

    def __init__(self, tokens: int, d_in: int, d_out: int, dev):
        T, Di, Do = tokens, d_in, d_out
        self.q = {n: (_u8((r, c), dev), _u8((r, c // 32), dev), _u8((c, r), dev), _u8((c, r // 32), dev))
                  for n, (r, c) in {"x": (T, Di), "w": (Do, Di), "dy": (T, Do)}.items()}
        self.y, self.dx, self.dw = _f32((T, Do), dev), _f32((T, Di), dev), _f32((Do, Di), dev)

    def quantize(self, x, w, dy):
        """All six copies (rowwise + columnwise of X, W, dY) in one launch."""
        B.quantize_mxfp8_multi([x, w, dy], [self.q["x"], self.q["w"], self.q["dy"]])

    def gemm_args(self):
        xr, xrs, xc, xcs = self.q["x"]
        wr, wrs, wc, wcs = self.q["w"]
        dr, drs, dc, dcs = self.q["dy"]
        return {"fprop": (xr, xrs, wr, wrs, self.y), "dgrad": (dr, drs, wc, wcs, self.dx),
                "wgrad": (dc, dcs, xc, xcs, self.dw)}

    FMT = B.MXFP8

    def gemm(self, name: str):
        A, sA, Bq, sB, out = self.gemm_args()[name]
        B.gemm_block_scaled(self.FMT, A, sA, Bq, sB, out=out)

    def gemm_all(self):
        """fprop, dgrad and wgrad in one batched launch (bit-identical to three calls)."""
        B.gemm_block_scaled_batch(self.FMT, [dict(A=A, sA=sA, B=Bq, sB=sB, out=out)
                                             for A, sA, Bq, sB, out in self.gemm_args().values()])

    def step(self, x, w, dy):
        self.quantize(x, w, dy)
        self.gemm_all()


class LinearMxfp4(LinearMxfp8):
    """The same three GEMMs with MXFP4 operands (E2M1 + E8M0 per 32), on the native
    FP4 scaled MFMA."""

    def __init__(self, tokens: int, d_in: int, d_out: int, dev):
        T, Di, Do = tokens, d_in, d_out
        self.q = {n: (_u8((r, c // 2), dev), _u8((r, c // 32), dev), _u8((c, r // 2), dev), _u8((c, r // 32), dev))
                  for n, (r, c) in {"x": (T, Di), "w": (Do, Di), "dy": (T, Do)}.items()}
        self.y, self.dx, self.dw = _f32((T, Do), dev), _f32((T, Di), dev), _f32((Do, Di), dev)

    FMT = B.MXFP4

    def quantize(self, x, w, dy):
        B.quantize_mxfp4_multi([x, w, dy], [self.q["x"], self.q["w"], self.q["dy"]])


class LinearFp8Block:
    """The linear layer in DeepSeek-V3-style blockwise FP8: X and dY in 1 x 128 tiles (row
    copy for fprop / dgrad, 128 x 1 transposed copy for wgrad, both from one read), W in
    128 x 128 blocks (row copy for fprop, transposed copy for dgrad); FP32 scales applied
    around the matrix product."""

    def __init__(self, tokens: int, d_in: int, d_out: int, dev):
        T, Di, Do = tokens, d_in, d_out
        f32 = lambda *sh: torch.empty(sh, dtype=torch.float32, device=dev)
        act = lambda r, c: (_u8((r, c), dev), f32(r, c // 128), _u8((c, r), dev), f32(c, r // 128))
        self.qx, self.qdy = act(T, Di), act(T, Do)
        self.qw = (_u8((Do, Di), dev), f32(Do // 128, Di // 128), _u8((Di, Do), dev), f32(Di // 128, Do // 128))
        self.y, self.dx, self.dw = _f32((T, Do), dev), _f32((T, Di), dev), _f32((Do, Di), dev)

    def quantize(self, x, w, dy):
        B.quantize_fp8_block_act(x, True, True, out=self.qx)
        B.quantize_fp8_block_weight(w, out=self.qw)
        B.quantize_fp8_block_act(dy, True, True, out=self.qdy)

    def gemm(self, name: str):
        xr, xs, xc, xcs = self.qx
        wr, ws, wc, wcs = self.qw
        dr, ds, dc, dcs = self.qdy
        if name == "fprop":
            B.gemm_fp8_blockwise(xr, xs, wr, ws, b_blocks=True, out=self.y)
        elif name == "dgrad":
            B.gemm_fp8_blockwise(dr, ds, wc, wcs, b_blocks=True, out=self.dx)
        else:
            B.gemm_fp8_blockwise(dc, dcs, xc, xcs, b_blocks=False, out=self.dw)

    def gemm_all(self):
        """fprop, dgrad and wgrad in one batched launch (bit-identical to the single calls)."""
        xr, xs, xc, xcs = self.qx
        wr, ws, wc, wcs = self.qw
        dr, ds, dc, dcs = self.qdy
        B.gemm_fp8_blockwise_batch([dict(A=xr, sA=xs, B=wr, sB=ws, b_blocks=True, out=self.y),
                                    dict(A=dr, sA=ds, B=wc, sB=wcs, b_blocks=True, out=self.dx),
                                    dict(A=dc, sA=dcs, B=xc, sB=xcs, b_blocks=False, out=self.dw)])

    def step(self, x, w, dy):
        self.quantize(x, w, dy)
        self.gemm_all()


# ---------------------------------------------------------------------------
# Routed-expert MoE layer with per-token NVFP4 activations and NVFP4 expert weights
# ---------------------------------------------------------------------------

class MoeRoutingDevice:
    """Device copies of a host routing (offsets may be padded per expert)."""

    def __init__(self, r, dev):
        self.offsets = torch.from_numpy(r.offsets.astype("int64")).to(dev)
        self.row_index = torch.from_numpy(r.row_index.astype("int32")).to(dev)
        self.slot_of = torch.from_numpy(r.slot_of.astype("int64")).to(dev)
        self.weights = torch.from_numpy(r.topk_w).to(dev)
        self.slots = int(r.offsets[-1])
        self.groups = len(r.offsets) - 1


class MoeNvfp4:
    """SwiGLU routed experts: per expert g, GU = X_g W_gu,g^T (gate rows, then up rows),
    h = silu(gate) * up, O = h W_d,g^T; tokens combine their top-k outputs by weight.

    X is quantized per token once, before the gather (a token's bits do not depend on
    the batch); the SwiGLU output is requantized per slot row; the expert weights carry
    one FP32 scale per expert matrix (gate and up share one)."""

    def __init__(self, tokens: int, hidden: int, experts: int, inter: int, routing: MoeRoutingDevice, dev,
                 keep_h: bool = False):
        T, H, G, I, S = tokens, hidden, experts, inter, routing.slots
        self.T, self.H, self.G, self.I, self.S, self.dev, self.r = T, H, G, I, S, dev, routing
        self.qx, self.sx, self.tx = _u8((T, H // 2), dev), _u8((T, H // 16), dev), _f32((T,), dev)
        self.gu = _f32((S, 2 * I), dev)
        self.h = _bf16((S, I), dev) if keep_h else None
        self.qh, self.sh, self.th = _u8((S, I // 2), dev), _u8((S, I // 16), dev), _f32((S,), dev)
        self.o = _f32((S, H), dev)
        self.y = _f32((T, H), dev)
        ws = B.lib().mxq_workspace_bytes(B.OP_GROUPED_GEMM, G, 0, 0)
        self.ws = _u8((ws,), dev)
        self.wq = None

    # A4: expert weights, one FP32 scale per expert matrix (two passes: amax, quantize)
    def quantize_weights(self, w_gu, w_d):
        G, H, I, dev = self.G, self.H, self.I, self.dev
        if self.wq is None:
            self.wq = {"gu": (_u8((G * 2 * I, H // 2), dev), _u8((G * 2 * I, H // 16), dev), _f32((G,), dev)),
                       "d": (_u8((G * H, I // 2), dev), _u8((G * H, I // 16), dev), _f32((G,), dev))}
            self.wq_ws = _u8((B.lib().mxq_workspace_bytes(B.OP_QUANTIZE_NVFP4, 0, 0, G),), dev)
        for key, w, gr in (("gu", w_gu, 2 * I), ("d", w_d, H)):
            q, s, t = self.wq[key]
            B._check("quantize_nvfp4", B.lib().quantize_nvfp4(
                B._ptr(w), w.shape[0], w.shape[1], w.stride(0), B.SCOPE["group"], gr, 0, None, B._ptr(q),
                B._ptr(s), B._ptr(t), B._ptr(self.wq_ws), self.wq_ws.numel(), B._stream(dev)))
        return self.wq

    def quantize_weights_2d(self, w_gu, w_d):
        """Expert weights with 16x16 block scales (row and transposed copies hold the same
        codes: the forward and the dgrad of one quantized weight)."""
        G, H, I, dev = self.G, self.H, self.I, self.dev
        if getattr(self, "wq2d", None) is None:
            # row copies (G*N, K) and per-expert transposed copies (G*K, N) of W_gu and W_d
            self.wq2d = {"gu": (_u8((G * 2 * I, H // 2), dev), _u8((G * 2 * I, H // 16), dev),
                                _u8((G * H, 2 * I // 2), dev), _u8((G * H, 2 * I // 16), dev), _f32((G,), dev)),
                         "d": (_u8((G * H, I // 2), dev), _u8((G * H, I // 16), dev),
                               _u8((G * I, H // 2), dev), _u8((G * I, H // 16), dev), _f32((G,), dev))}
            self.wq2d_ws = _u8((B.lib().mxq_workspace_bytes(B.OP_QUANTIZE_NVFP4, 0, 0, G),), dev)
        for key, w, gr in (("gu", w_gu, 2 * I), ("d", w_d, H)):
            B.quantize_nvfp4_2d(w, scope="group", group_rows=gr, out=self.wq2d[key], workspace=self.wq2d_ws)
        return self.wq2d

    def quantize_tokens(self, x):                                  # A3
        B._check("quantize_nvfp4_per_token", B.lib().quantize_nvfp4_per_token(
            B._ptr(x), self.T, self.H, x.stride(0), B._ptr(self.qx), B._ptr(self.sx), B._ptr(self.tx),
            B._stream(x.device)))

    def gate_up(self):                                             # A9 + A10 (gather inside the GEMM)
        qw, sw, tw = self.wq["gu"]
        B.grouped_gemm_block_scaled(B.NVFP4, self.r.offsets, self.qx, qw, N=2 * self.I, K=self.H, sA=self.sx,
                                    sB=sw, tA=self.tx, tB=tw, tA_scope="row", tB_scope="group",
                                    a_row_index=self.r.row_index, total=self.S, a_rows=self.T, out=self.gu,
                                    workspace=self.ws)

    def swiglu(self):                                              # A11
        B._check("moe_swiglu_quantize_nvfp4", B.lib().moe_swiglu_quantize_nvfp4(
            B._ptr(self.gu), self.S, self.I, B._ptr(self.h), B._ptr(self.qh), B._ptr(self.sh), B._ptr(self.th),
            B._stream(self.dev)))

    def down(self):                                                # A10
        qw, sw, tw = self.wq["d"]
        B.grouped_gemm_block_scaled(B.NVFP4, self.r.offsets, self.qh, qw, N=self.H, K=self.I, sA=self.sh,
                                    sB=sw, tA=self.th, tB=tw, tA_scope="row", tB_scope="group", total=self.S,
                                    out=self.o, workspace=self.ws)

    def combine(self):                                             # A12
        B.moe_combine(self.o, self.r.slot_of, self.r.weights, out=self.y)

    def forward(self, x):
        self.quantize_tokens(x)
        self.gate_up()
        self.swiglu()
        self.down()
        self.combine()
        return self.y

    def gemm_flops(self) -> dict:
        """Useful work of the two forward GEMMs: 2 * routed slots * N * K (padding excluded)."""
        live = self.T * (self.r.slot_of.shape[1])
        return {"gate_up": 2 * live * 2 * self.I * self.H, "down": 2 * live * self.H * self.I}


class MoeDequantBackward:
    """Dequantized backward of the routed experts (BF16 GEMMs on BF16 dequantizations
    of the exact forward operands), given upstream gradients dO (S, H) of the down
    outputs and dGU (S, 2I) of the gate_up outputs (padding slots zero):
        down:    dh = dO W_d,g          dW_d,g = dO_g^T h_hat_g
        gate_up: dX = dGU W_gu,g        dW_gu,g = dGU_g^T X_hat_g
    dgrad GEMMs vary M per expert; wgrad GEMMs vary K (the slots). The dgrads read the
    forward's NVFP4 expert weights directly (fused_weights: the GEMM loader builds the
    transposed BF16 dequantization, the BF16_NVFP4T format); with fused_weights=False
    they read BF16 transposes written by dequantize_transposed first. The wgrads read dO and
    dGU as they are (slot-major, K-major A, vary_k=2); their other operands, the NVFP4
    activations, are dequantized into K-contiguous BF16 transposes by dequantize_transposed."""

    def __init__(self, fwd: MoeNvfp4, fused_weights: bool = True):
        f = fwd
        dev, G, H, I, S = f.dev, f.G, f.H, f.I, f.S
        self.f = f
        self.fused = fused_weights
        if not fused_weights:
            self.w_dT = _bf16((G, I, H), dev)      # W_hat_d,g^T
            self.w_guT = _bf16((G, H, 2 * I), dev) # W_hat_gu,g^T
        self.hT = _bf16((1, I, S), dev)            # h_hat^T (slots along K)
        self.xT = _bf16((1, H, S), dev)            # X_hat gathered into slots, transposed
        self.dh = _f32((S, I), dev)
        self.dx = _f32((S, H), dev)
        self.dw_d = _f32((G, H, I), dev)
        self.dw_gu = _f32((G, 2 * I, H), dev)

    def dequantize_weights(self):                                  # A6 (static per step)
        """BF16 transposed weights for the two-step dgrads (nothing to do when fused)."""
        if self.fused:
            return
        f = self.f
        qw, sw, tw = f.wq["d"]
        B.dequantize_transposed(B.NVFP4, qw, sw, tw, t_scope="group", groups=f.G, group_rows=f.H, cols=f.I,
                                out=self.w_dT)
        qw, sw, tw = f.wq["gu"]
        B.dequantize_transposed(B.NVFP4, qw, sw, tw, t_scope="group", groups=f.G, group_rows=2 * f.I, cols=f.H,
                                out=self.w_guT)

    def dequantize_activations(self, d_o, d_gu):                   # A6 + layout for wgrad
        f = self.f
        B.dequantize_transposed(B.NVFP4, f.qh, f.sh, f.th, t_scope="row", groups=1, group_rows=f.S, cols=f.I,
                                out=self.hT)
        B.dequantize_transposed(B.NVFP4, f.qx, f.sx, f.tx, t_scope="row", groups=1, group_rows=f.T, cols=f.H,
                                src_row=f.r.row_index, out_cols=f.S, out=self.xT)

    def gemms(self, d_o, d_gu):                                    # A13
        f = self.f
        off = f.r.offsets
        if self.fused:
            qw, sw, tw = f.wq["d"]
            B.grouped_gemm_block_scaled(B.BF16_NVFP4T, off, d_o, qw, N=f.I, K=f.H, sB=sw, tB=tw, tB_scope="group",
                                        total=f.S, out=self.dh, workspace=f.ws)
        else:
            B.grouped_gemm_block_scaled(B.BF16, off, d_o, self.w_dT, N=f.I, K=f.H, total=f.S, out=self.dh,
                                        workspace=f.ws)
        B.grouped_gemm_block_scaled(B.BF16, off, d_o, self.hT[0], N=f.I, K=0, vary_k=2, M=f.H,
                                    total=f.S, out=self.dw_d, workspace=f.ws)
        if self.fused:
            qw, sw, tw = f.wq["gu"]
            B.grouped_gemm_block_scaled(B.BF16_NVFP4T, off, d_gu, qw, N=f.H, K=2 * f.I, sB=sw, tB=tw,
                                        tB_scope="group", total=f.S, out=self.dx, workspace=f.ws)
        else:
            B.grouped_gemm_block_scaled(B.BF16, off, d_gu, self.w_guT, N=f.H, K=2 * f.I, total=f.S, out=self.dx,
                                        workspace=f.ws)
        B.grouped_gemm_block_scaled(B.BF16, off, d_gu, self.xT[0], N=f.H, K=0, vary_k=2, M=2 * f.I,
                                    total=f.S, out=self.dw_gu, workspace=f.ws)

    def backward(self, d_o, d_gu):
        self.dequantize_activations(d_o, d_gu)
        self.gemms(d_o, d_gu)

    def gemm_flops(self) -> dict:
        f = self.f
        live = f.T * f.r.slot_of.shape[1]
        return {"down_dgrad": 2 * live * f.H * f.I, "down_wgrad": 2 * live * f.H * f.I,
                "gate_up_dgrad": 2 * live * 2 * f.I * f.H, "gate_up_wgrad": 2 * live * 2 * f.I * f.H}


class SharedExpertBf16:
    """The shared expert in BF16 (it sees every token; kept in higher precision):
    GU = X W_sgu^T, h = silu(gate) * up (BF16), O = h W_sd^T; backward with upstream
    dO (T, H) and dGU (T, 2I): dh = dO W_sd, dW_sd = dO^T h, dX = dGU W_sgu,
    dW_sgu = dGU^T X."""

    def __init__(self, tokens: int, hidden: int, inter: int, dev):
        T, H, I = tokens, hidden, inter
        self.T, self.H, self.I, self.dev = T, H, I, dev
        self.gu = _f32((T, 2 * I), dev)
        self.h = _bf16((T, I), dev)
        self.qh, self.sh, self.th = _u8((T, I // 2), dev), _u8((T, I // 16), dev), _f32((T,), dev)
        self.o = _f32((T, H), dev)
        self.w_sdT = _bf16((1, I, H), dev)
        self.w_sguT = _bf16((1, H, 2 * I), dev)
        self.hT = _bf16((1, I, T), dev)
        self.xT = _bf16((1, H, T), dev)
        self.d_oT = _bf16((1, H, T), dev)
        self.d_guT = _bf16((1, 2 * I, T), dev)
        self.dh = _f32((T, I), dev)
        self.dw_sd = _f32((H, I), dev)
        self.dx = _f32((T, H), dev)
        self.dw_sgu = _f32((2 * I, H), dev)

    def forward(self, x, w_sgu, w_sd):
        B.gemm_block_scaled(B.BF16, x, None, w_sgu, None, out=self.gu)
        # SwiGLU to BF16 (the NVFP4 copy the same call emits is not used by this expert)
        B._check("moe_swiglu_quantize_nvfp4", B.lib().moe_swiglu_quantize_nvfp4(
            B._ptr(self.gu), self.T, self.I, B._ptr(self.h), B._ptr(self.qh), B._ptr(self.sh), B._ptr(self.th),
            B._stream(self.dev)))
        B.gemm_block_scaled(B.BF16, self.h, None, w_sd, None, out=self.o)

    def transposes(self, x, w_sgu, w_sd, d_o, d_gu):
        T, H, I = self.T, self.H, self.I
        B.dequantize_transposed(B.BF16, w_sd, groups=1, group_rows=H, cols=I, out=self.w_sdT)
        B.dequantize_transposed(B.BF16, w_sgu, groups=1, group_rows=2 * I, cols=H, out=self.w_sguT)
        B.dequantize_transposed(B.BF16, self.h, groups=1, group_rows=T, cols=I, out=self.hT)
        B.dequantize_transposed(B.BF16, x, groups=1, group_rows=T, cols=H, out=self.xT)
        B.dequantize_transposed(B.BF16, d_o, groups=1, group_rows=T, cols=H, out=self.d_oT)
        B.dequantize_transposed(B.BF16, d_gu, groups=1, group_rows=T, cols=2 * I, out=self.d_guT)

    def backward(self, x, w_sgu, w_sd, d_o, d_gu):
        self.transposes(x, w_sgu, w_sd, d_o, d_gu)
        # the four backward GEMMs are independent: one batched launch (longest K first)
        B.gemm_block_scaled_batch(B.BF16, [
            dict(A=d_o, sA=None, B=self.w_sdT[0], sB=None, out=self.dh),
            dict(A=self.d_oT[0], sA=None, B=self.hT[0], sB=None, out=self.dw_sd),
            dict(A=d_gu, sA=None, B=self.w_sguT[0], sB=None, out=self.dx),
            dict(A=self.d_guT[0], sA=None, B=self.xT[0], sB=None, out=self.dw_sgu)])

    def gemm_flops(self) -> dict:
        T, H, I = self.T, self.H, self.I
        return {"fwd": 2 * T * H * 2 * I + 2 * T * I * H, "bwd": 2 * (2 * T * H * I + 2 * T * H * 2 * I)}


# ---------------------------------------------------------------------------
# Heavy-tailed stress case: MXFP8 fprop/dgrad/wgrad at n^3 + NVFP4 RHT wgrad
# ---------------------------------------------------------------------------

class StressStep:
    """A, B (n, n) BF16. MXFP8 rowwise + columnwise of both; fprop C = A B^T (A row,
    B row), dgrad C = A B (A row, B col), wgrad C = A^T B (A col, B col); then the
    NVFP4 wgrad C = A^T B on 16-point random-Hadamard-transformed operands: each
    column of A and B (the reduction axis of this GEMM runs down the columns) is
    transformed in 16-chunks and quantized 1x16 along it with one FP32 scale per
    tensor (amax after the transform), stored transposed."""

    def __init__(self, n: int, signs, dev):
        self.n, self.dev = n, dev
        self.signs = [int(v) for v in signs]
        self.qa = (_u8((n, n), dev), _u8((n, n // 32), dev), _u8((n, n), dev), _u8((n, n // 32), dev))
        self.qb = (_u8((n, n), dev), _u8((n, n // 32), dev), _u8((n, n), dev), _u8((n, n // 32), dev))
        self.c = {k: _f32((n, n), dev) for k in ("fprop", "dgrad", "wgrad", "wgrad_nvfp4", "fprop_mxfp4")}
        self.nv = {k: (_u8((n, n // 2), dev), _u8((n, n // 16), dev), _f32((1,), dev)) for k in ("a", "b")}
        ws = B.lib().mxq_workspace_bytes(B.OP_QUANTIZE_NVFP4, n, n, 1)
        self.ws = _u8((ws,), dev)
        self._signs_c = (B.ctypes.c_int8 * 16)(*self.signs)

    def quantize_mxfp8(self, a, b):
        B.quantize_mxfp8_multi([a, b], [self.qa, self.qb])

    def mxfp8_gemm_args(self):
        ar, ars, ac, acs = self.qa
        br, brs, bc, bcs = self.qb
        return {"fprop": (ar, ars, br, brs), "dgrad": (ar, ars, bc, bcs), "wgrad": (ac, acs, bc, bcs)}

    def mxfp8_gemm(self, name):
        A, sA, Bq, sB = self.mxfp8_gemm_args()[name]
        B.gemm_block_scaled(B.MXFP8, A, sA, Bq, sB, out=self.c[name])

    def mxfp8_gemm_all(self):
        """fprop, dgrad and wgrad in one batched launch (bit-identical to three calls)."""
        B.gemm_block_scaled_batch(B.MXFP8, [dict(A=A, sA=sA, B=Bq, sB=sB, out=self.c[k])
                                            for k, (A, sA, Bq, sB) in self.mxfp8_gemm_args().items()])

    def quantize_rht(self, a, b):
        for k, x in (("a", a), ("b", b)):
            q, s, t = self.nv[k]
            B._check("quantize_nvfp4", B.lib().quantize_nvfp4(
                B._ptr(x), self.n, self.n, x.stride(0), B.SCOPE["tensor"], 0, 1, self._signs_c, B._ptr(q),
                B._ptr(s), B._ptr(t), B._ptr(self.ws), self.ws.numel(), B._stream(self.dev)))

    def quantize_rht_sr(self, a, seed: int):
        """The gradient operand A with stochastically rounded elements (gradients only)."""
        q, s, t = self.nv["a"]
        B._check("quantize_nvfp4_stochastic", B.lib().quantize_nvfp4_stochastic(
            B._ptr(a), self.n, self.n, a.stride(0), B.SCOPE["tensor"], 0, 1, self._signs_c, seed, B._ptr(q),
            B._ptr(s), B._ptr(t), B._ptr(self.ws), self.ws.numel(), B._stream(self.dev)))

    def quantize_mxfp4(self, a, b):
        """MXFP4 rowwise + columnwise copies of A and B (one launch)."""
        if not hasattr(self, "q4"):
            n, dev = self.n, self.dev
            mk = lambda: (_u8((n, n // 2), dev), _u8((n, n // 32), dev), _u8((n, n // 2), dev), _u8((n, n // 32), dev))
            self.q4 = {"a": mk(), "b": mk()}
        B.quantize_mxfp4_multi([a, b], [self.q4["a"], self.q4["b"]])

    def mxfp4_gemm(self):
        """C = A B^T on the MXFP4 rowwise copies (native FP4 scaled MFMA)."""
        ar, ars, _, _ = self.q4["a"]
        br, brs, _, _ = self.q4["b"]
        B.gemm_block_scaled(B.MXFP4, ar, ars, br, brs, out=self.c["fprop_mxfp4"])

    def nvfp4_wgrad(self):
        qa, sa, ta = self.nv["a"]
        qb, sb, tb = self.nv["b"]
        B.gemm_block_scaled(B.NVFP4, qa, sa, qb, sb, tA=ta, tB=tb, tA_scope="tensor", tB_scope="tensor",
                            out=self.c["wgrad_nvfp4"])

    def step(self, a, b):
        self.quantize_mxfp8(a, b)
        self.mxfp8_gemm_all()
        self.quantize_rht(a, b)
        self.nvfp4_wgrad()
