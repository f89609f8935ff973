"""Thin Python binding of libmxq (ctypes).

Argument marshalling only: every function here allocates its outputs with torch
on the input's device, passes raw device pointers and torch's current HIP stream
to the C ABI in include/mxq.h, and raises MxqError on a non-zero status. No
step of the quantize / GEMM path runs in Python, and there is no fallback: if
libmxq.so is missing the first call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxq.so")

MXFP8, NVFP4, BF16, MXFP4 = 1, 2, 3, 4
_PACKED4 = (NVFP4, MXFP4)          # formats with two elements per byte
OUT_BF16, OUT_F32 = 0, 1
SCOPE = {"row": 0, "token": 0, "tensor": 1, "group": 2}
OP_QUANTIZE_NVFP4, OP_GROUPED_GEMM = 1, 2

_c_void_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_size = ctypes.c_size_t

_SIGS = {
    "quantize_mxfp8": [_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p],
    "quantize_mxfp8_multi": [_c_void_p, _int, _c_void_p],
    "quantize_mxfp4": [_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p],
    "quantize_mxfp4_multi": [_c_void_p, _int, _c_void_p],
    "quantize_fp8_block_act": [_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p],
    "quantize_fp8_block_weight": [_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p],
    "gemm_block_scaled_batch": [_int, _c_void_p, _int, _c_void_p],
    "gemm_fp8_blockwise": [_i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _int, _c_void_p, _i64,
                           _c_void_p],
    "gemm_fp8_blockwise_batch": [_c_void_p, _int, _c_void_p],
    "quantize_nvfp4_per_token": [_c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p],
    "quantize_nvfp4": [_c_void_p, _i64, _i64, _i64, _int, _i64, _int, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                       _c_void_p, _size, _c_void_p],
    "quantize_nvfp4_stochastic": [_c_void_p, _i64, _i64, _i64, _int, _i64, _int, _c_void_p, ctypes.c_uint64,
                                  _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p],
    "quantize_nvfp4_2d": [_c_void_p, _i64, _i64, _i64, _int, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                          _c_void_p, _c_void_p, _size, _c_void_p],
    "dequantize": [_int, _c_void_p, _c_void_p, _c_void_p, _int, _i64, _i64, _i64, _c_void_p, _int, _c_void_p],
    "dequantize_transposed": [_int, _c_void_p, _c_void_p, _c_void_p, _int, _i64, _i64, _i64, _c_void_p, _i64,
                              _c_void_p, _i64, _c_void_p],
    "gemm_block_scaled": [_int, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p, _int, _c_void_p, _c_void_p,
                          _c_void_p, _int, _c_void_p, _i64, _c_void_p],
    "gemm_mxfp8_matrix_core": [_i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64,
                               _c_void_p],
    "grouped_gemm_block_scaled": [_int, _i64, _c_void_p, _int, _i64, _i64, _i64, _i64, _c_void_p, _i64, _c_void_p,
                                  _c_void_p, _c_void_p, _int, _c_void_p, _c_void_p, _c_void_p, _int, _c_void_p,
                                  _c_void_p, _size, _c_void_p],
    "moe_swiglu_quantize_nvfp4": [_c_void_p, _i64, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p],
    "moe_combine": [_c_void_p, _i64, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p],
    "mxq_scale_bytes": [_int, _i64, _i64],
    "mxq_workspace_bytes": [_int, _i64, _i64, _i64],
    "mxq_status_string": [_int],
    "mxq_abi_version": [],
}
_RESTYPES = {"mxq_scale_bytes": _size, "mxq_workspace_bytes": _size, "mxq_status_string": ctypes.c_char_p}

_lib = None


class MxqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed with status {status}: {status_string(status)}")


def lib() -> ctypes.CDLL:
    """Load libmxq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m microscaling_precision_quantization_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = _RESTYPES.get(name, _int)
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().mxq_status_string(status).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise MxqError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _bf16(x):
    if x.dtype != torch.bfloat16:
        raise TypeError("expected a bfloat16 tensor")
    if not x.is_cuda:
        raise TypeError("expected a device tensor")
    return x


def _u8(shape, dev):
    return torch.empty(shape, dtype=torch.uint8, device=dev)


# ---------------------------------------------------------------------------
# Quantizers
# ---------------------------------------------------------------------------

def quantize_mxfp8(x: torch.Tensor, rowwise: bool = True, colwise: bool = True, out=None):
    """MXFP8 rowwise (R, C) + columnwise-transposed (C, R) copies of BF16 x.

    Returns (q_row, s_row, q_colT, s_colT); skipped copies are None. `out` may
    supply preallocated (q_row, s_row, q_colT, s_colT) buffers.
    """
    _bf16(x)
    R, C = x.shape
    dev = x.device
    if out is not None:
        q_row, s_row, q_col, s_col = out
    else:
        q_row = _u8((R, C), dev) if rowwise else None
        s_row = _u8((R, C // 32), dev) if rowwise else None
        q_col = _u8((C, R), dev) if colwise else None
        s_col = _u8((C, R // 32), dev) if colwise else None
    _check("quantize_mxfp8", lib().quantize_mxfp8(_ptr(x), R, C, x.stride(0), _ptr(q_row), _ptr(s_row),
                                                  _ptr(q_col), _ptr(s_col), _stream(dev)))
    return q_row, s_row, q_col, s_col


def quantize_mxfp4(x: torch.Tensor, rowwise: bool = True, colwise: bool = True, out=None):
    """MXFP4 rowwise (R, C/2) + columnwise-transposed (C, R/2) packed copies of BF16 x.

    Returns (q_row, s_row, q_colT, s_colT); skipped copies are None.
    """
    _bf16(x)
    R, C = x.shape
    dev = x.device
    if out is not None:
        q_row, s_row, q_col, s_col = out
    else:
        q_row = _u8((R, C // 2), dev) if rowwise else None
        s_row = _u8((R, C // 32), dev) if rowwise else None
        q_col = _u8((C, R // 2), dev) if colwise else None
        s_col = _u8((C, R // 32), dev) if colwise else None
    _check("quantize_mxfp4", lib().quantize_mxfp4(_ptr(x), R, C, x.stride(0), _ptr(q_row), _ptr(s_row),
                                                  _ptr(q_col), _ptr(s_col), _stream(dev)))
    return q_row, s_row, q_col, s_col


def quantize_fp8_block_act(x: torch.Tensor, rowwise: bool = True, colwise: bool = False, out=None):
    """Blockwise FP8 of an activation / gradient: (q_row (R, C), s_row (R, C/128)) with 1 x 128
    tiles along rows and (q_colT (C, R), s_colT (C, R/128)) with tiles of 128 down columns,
    stored transposed; skipped copies are None."""
    _bf16(x)
    R, C = x.shape
    dev = x.device
    f32 = lambda *sh: torch.empty(sh, dtype=torch.float32, device=dev)
    if out is not None:
        q_row, s_row, q_col, s_col = out
    else:
        q_row, s_row = (_u8((R, C), dev), f32(R, C // 128)) if rowwise else (None, None)
        q_col, s_col = (_u8((C, R), dev), f32(C, R // 128)) if colwise else (None, None)
    _check("quantize_fp8_block_act", lib().quantize_fp8_block_act(
        _ptr(x), R, C, x.stride(0), _ptr(q_row), _ptr(s_row), _ptr(q_col), _ptr(s_col), _stream(dev)))
    return q_row, s_row, q_col, s_col


def quantize_fp8_block_weight(x: torch.Tensor, rowwise: bool = True, colwise: bool = True, out=None):
    """Blockwise FP8 of a weight (128 x 128 blocks): (q_row (R, C), s_row (R/128, C/128),
    q_colT (C, R), s_colT (C/128, R/128)); skipped copies are None."""
    _bf16(x)
    R, C = x.shape
    dev = x.device
    f32 = lambda *sh: torch.empty(sh, dtype=torch.float32, device=dev)
    if out is not None:
        q_row, s_row, q_col, s_col = out
    else:
        q_row = _u8((R, C), dev) if rowwise else None
        s_row = f32(R // 128, C // 128) if rowwise else None
        q_col = _u8((C, R), dev) if colwise else None
        s_col = f32(C // 128, R // 128) if colwise else None
    _check("quantize_fp8_block_weight", lib().quantize_fp8_block_weight(
        _ptr(x), R, C, x.stride(0), _ptr(q_row), _ptr(s_row), _ptr(q_col), _ptr(s_col), _stream(dev)))
    return q_row, s_row, q_col, s_col


class _Mxfp8Tensor(ctypes.Structure):
    _fields_ = [("x", _c_void_p), ("rows", _i64), ("cols", _i64), ("ld_x", _i64), ("q_row", _c_void_p),
                ("s_row", _c_void_p), ("q_colT", _c_void_p), ("s_colT", _c_void_p)]


def _mx_multi(fn: str, xs, outs):
    n = len(xs)
    arr = (_Mxfp8Tensor * n)()
    for i, (x, o) in enumerate(zip(xs, outs)):
        _bf16(x)
        q_row, s_row, q_col, s_col = o
        arr[i] = _Mxfp8Tensor(x.data_ptr(), x.shape[0], x.shape[1], x.stride(0),
                              *(None if t is None else t.data_ptr() for t in (q_row, s_row, q_col, s_col)))
    _check(fn, getattr(lib(), fn)(ctypes.cast(arr, _c_void_p), n, _stream(xs[0].device)))
    return outs


def quantize_mxfp8_multi(xs, outs):
    """quantize_mxfp8 of several BF16 tensors in one launch; outs[i] = (q_row, s_row,
    q_colT, s_colT) preallocated (a skipped copy is (None, None) in its slots)."""
    return _mx_multi("quantize_mxfp8_multi", xs, outs)


def quantize_mxfp4_multi(xs, outs):
    """quantize_mxfp4 of several BF16 tensors in one launch; outs as quantize_mxfp8_multi
    with packed (R, C/2) / (C, R/2) element buffers."""
    return _mx_multi("quantize_mxfp4_multi", xs, outs)


def quantize_nvfp4_per_token(x: torch.Tensor):
    """Per-token NVFP4 of BF16 x (T, H): (packed (T, H/2), E4M3 scales (T, H/16), t (T,))."""
    _bf16(x)
    T, H = x.shape
    dev = x.device
    q, s = _u8((T, H // 2), dev), _u8((T, H // 16), dev)
    t = torch.empty(T, dtype=torch.float32, device=dev)
    _check("quantize_nvfp4_per_token", lib().quantize_nvfp4_per_token(_ptr(x), T, H, x.stride(0), _ptr(q), _ptr(s),
                                                                      _ptr(t), _stream(dev)))
    return q, s, t


def quantize_nvfp4(x: torch.Tensor, scope: str = "tensor", group_rows: int = 0, transpose: bool = False,
                   rht_signs=None, workspace: torch.Tensor | None = None, sr_seed: int | None = None):
    """General NVFP4 quantizer (see include/mxq.h). rht_signs: 16 ints in {-1, +1} or None.
    sr_seed: None = round-to-nearest-even; an int = stochastic rounding of the elements
    (quantize_nvfp4_stochastic) with that seed."""
    _bf16(x)
    R, C = x.shape
    dev = x.device
    out_rows, out_cols = (C, R) if transpose else (R, C)
    sc = SCOPE[scope]
    n_scopes = out_rows if sc == 0 else 1 if sc == 1 else (out_rows // group_rows if group_rows else 0)
    q, s = _u8((out_rows, out_cols // 2), dev), _u8((out_rows, out_cols // 16), dev)
    t = torch.empty(max(n_scopes, 1), dtype=torch.float32, device=dev)
    signs = None
    if rht_signs is not None:
        signs = (ctypes.c_int8 * 16)(*[int(v) for v in rht_signs])
    ws_bytes = lib().mxq_workspace_bytes(OP_QUANTIZE_NVFP4, out_rows, out_cols, n_scopes) if sc != 0 else 0
    if workspace is None and ws_bytes:
        workspace = _u8((ws_bytes,), dev)
    wsn = workspace.numel() if workspace is not None else 0
    if sr_seed is None:
        _check("quantize_nvfp4", lib().quantize_nvfp4(_ptr(x), R, C, x.stride(0), sc, group_rows, int(transpose),
                                                      signs, _ptr(q), _ptr(s), _ptr(t), _ptr(workspace), wsn,
                                                      _stream(dev)))
    else:
        _check("quantize_nvfp4_stochastic", lib().quantize_nvfp4_stochastic(
            _ptr(x), R, C, x.stride(0), sc, group_rows, int(transpose), signs, int(sr_seed), _ptr(q), _ptr(s), _ptr(t),
            _ptr(workspace), wsn, _stream(dev)))
    return q, s, t


def quantize_nvfp4_2d(x: torch.Tensor, scope: str = "tensor", group_rows: int = 0, rowwise: bool = True,
                      colwise: bool = True, out=None, workspace: torch.Tensor | None = None):
    """NVFP4 with 16x16 block scales: (q_row, s_row, q_colT, s_colT, t); skipped copies are None.
    The transposed copy is per scope group: (groups * cols, group_rows / 2)."""
    _bf16(x)
    R, C = x.shape
    dev = x.device
    n_scopes = 1 if scope == "tensor" else (R // group_rows if group_rows else 0)
    if out is not None:
        q_row, s_row, q_col, s_col, t = out
    else:
        q_row = _u8((R, C // 2), dev) if rowwise else None
        s_row = _u8((R, C // 16), dev) if rowwise else None
        gr = R if scope == "tensor" else group_rows
        q_col = _u8((max(n_scopes, 1) * C, gr // 2), dev) if colwise else None
        s_col = _u8((max(n_scopes, 1) * C, gr // 16), dev) if colwise else None
        t = torch.empty(max(n_scopes, 1), dtype=torch.float32, device=dev)
    ws_bytes = lib().mxq_workspace_bytes(OP_QUANTIZE_NVFP4, R, C, n_scopes)
    if workspace is None:
        workspace = _u8((max(ws_bytes, 4),), dev)
    _check("quantize_nvfp4_2d", lib().quantize_nvfp4_2d(_ptr(x), R, C, x.stride(0), SCOPE[scope], group_rows,
                                                        _ptr(q_row), _ptr(s_row), _ptr(q_col), _ptr(s_col),
                                                        _ptr(t), _ptr(workspace), workspace.numel(), _stream(dev)))
    return q_row, s_row, q_col, s_col, t


def dequantize(fmt: int, q: torch.Tensor, s: torch.Tensor, t: torch.Tensor | None = None, t_scope: str = "row",
               group_rows: int = 0, out_dtype: torch.dtype = torch.bfloat16):
    rows = q.shape[0]
    cols = q.shape[1] * (2 if fmt in _PACKED4 else 1)
    out = torch.empty((rows, cols), dtype=out_dtype, device=q.device)
    od = OUT_F32 if out_dtype == torch.float32 else OUT_BF16
    _check("dequantize", lib().dequantize(fmt, _ptr(q), _ptr(s), _ptr(t), SCOPE[t_scope], group_rows, rows, cols,
                                          _ptr(out), od, _stream(q.device)))
    return out


def dequantize_transposed(fmt: int, q: torch.Tensor, s=None, t=None, t_scope: str = "row", groups: int = 1,
                          group_rows: int | None = None, cols: int | None = None, src_row=None,
                          out_cols: int | None = None, out=None):
    """BF16 (groups, cols, out_cols): out[g, c, j] = dequantized input (g * group_rows + src(j), c)."""
    rows = q.shape[0]
    if cols is None:
        cols = q.shape[1] * (2 if fmt == NVFP4 else 1)
    if group_rows is None:
        group_rows = rows // max(groups, 1)
    if out_cols is None:
        out_cols = src_row.numel() if src_row is not None else group_rows
    if out is None:
        out = torch.empty((groups, cols, out_cols), dtype=torch.bfloat16, device=q.device)
    _check("dequantize_transposed", lib().dequantize_transposed(
        fmt, _ptr(q), _ptr(s), _ptr(t), SCOPE[t_scope], groups, group_rows, cols, _ptr(src_row), out_cols,
        _ptr(out), out.stride(-2), _stream(q.device)))
    return out


# ---------------------------------------------------------------------------
# GEMMs
# ---------------------------------------------------------------------------

def gemm_block_scaled(fmt: int, A, sA, B, sB, tA=None, tB=None, tA_scope="row", tB_scope="tensor", out=None):
    """C = A_hat B_hat^T in FP32; A (M, K-bytes) and B (N, K-bytes) K-contiguous."""
    M = A.shape[0]
    N = B.shape[0]
    K = A.shape[1] * (2 if fmt in _PACKED4 else 1)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    _check("gemm_block_scaled", lib().gemm_block_scaled(fmt, M, N, K, _ptr(A), _ptr(sA), _ptr(tA), SCOPE[tA_scope],
                                                        _ptr(B), _ptr(sB), _ptr(tB), SCOPE[tB_scope], _ptr(out),
                                                        out.stride(0), _stream(A.device)))
    return out


class _GemmProblem(ctypes.Structure):
    _fields_ = [("M", _i64), ("N", _i64), ("K", _i64), ("A", _c_void_p), ("sA", _c_void_p), ("tA", _c_void_p),
                ("tA_scope", _int), ("B", _c_void_p), ("sB", _c_void_p), ("tB", _c_void_p), ("tB_scope", _int),
                ("C", _c_void_p), ("ldc", _i64)]


def gemm_block_scaled_batch(fmt: int, problems):
    """Several gemm_block_scaled problems of one format in one launch. problems: list of
    dicts with A, sA, B, sB, out and optionally tA, tB, tA_scope, tB_scope."""
    n = len(problems)
    arr = (_GemmProblem * n)()
    dev = problems[0]["A"].device
    for i, q in enumerate(problems):
        A, B_, out = q["A"], q["B"], q["out"]
        K = A.shape[1] * (2 if fmt in _PACKED4 else 1)
        ptr = lambda t: None if t is None else t.data_ptr()
        arr[i] = _GemmProblem(A.shape[0], B_.shape[0], K, A.data_ptr(), ptr(q.get("sA")), ptr(q.get("tA")),
                              SCOPE[q.get("tA_scope", "row")], B_.data_ptr(), ptr(q.get("sB")), ptr(q.get("tB")),
                              SCOPE[q.get("tB_scope", "tensor")], out.data_ptr(), out.stride(0))
    _check("gemm_block_scaled_batch", lib().gemm_block_scaled_batch(fmt, ctypes.cast(arr, _c_void_p), n, _stream(dev)))
    return [q["out"] for q in problems]


def gemm_fp8_blockwise(A, sA, B, sB, b_blocks: bool = True, out=None):
    """Blockwise FP8 GEMM C = A_hat B_hat^T (FP32); sB per 128 x 128 block (b_blocks) or per row."""
    M, K = A.shape
    N = B.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    _check("gemm_fp8_blockwise", lib().gemm_fp8_blockwise(M, N, K, _ptr(A), _ptr(sA), _ptr(B), _ptr(sB), int(b_blocks),
                                                          _ptr(out), out.stride(0), _stream(A.device)))
    return out


class _Fp8BlockProblem(ctypes.Structure):
    _fields_ = [("M", _i64), ("N", _i64), ("K", _i64), ("A", _c_void_p), ("sA", _c_void_p), ("B", _c_void_p),
                ("sB", _c_void_p), ("b_blocks", _int), ("C", _c_void_p), ("ldc", _i64)]


def gemm_fp8_blockwise_batch(problems):
    """Several gemm_fp8_blockwise problems in one launch. problems: list of dicts with A, sA,
    B, sB, b_blocks and out."""
    n = len(problems)
    arr = (_Fp8BlockProblem * n)()
    dev = problems[0]["A"].device
    for i, q in enumerate(problems):
        A, B_, out = q["A"], q["B"], q["out"]
        arr[i] = _Fp8BlockProblem(A.shape[0], B_.shape[0], A.shape[1], A.data_ptr(), q["sA"].data_ptr(), B_.data_ptr(),
                                  q["sB"].data_ptr(), int(q["b_blocks"]), out.data_ptr(), out.stride(0))
    _check("gemm_fp8_blockwise_batch", lib().gemm_fp8_blockwise_batch(ctypes.cast(arr, _c_void_p), n, _stream(dev)))
    return [q["out"] for q in problems]


def gemm_mxfp8_matrix_core(A, sA, B, sB, out=None):
    """MXFP8 GEMM on the native scaled-FP8 matrix core (see include/mxq.h for its accumulation)."""
    M, K = A.shape
    N = B.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    _check("gemm_mxfp8_matrix_core", lib().gemm_mxfp8_matrix_core(M, N, K, _ptr(A), _ptr(sA), _ptr(B), _ptr(sB),
                                                                  _ptr(out), out.stride(0), _stream(A.device)))
    return out


def grouped_gemm_block_scaled(fmt: int, offsets, A, B, N: int, K: int, sA=None, sB=None, tA=None, tB=None,
                              tA_scope="row", tB_scope="group", a_row_index=None, vary_k=False, M: int = 0,
                              total: int | None = None, a_rows: int | None = None, out=None, workspace=None):
    """One GEMM per group; see include/mxq.h for the two modes.

    vary_k=False: out (total_slots, N); vary_k=True: out (groups, M, N).
    """
    groups = offsets.numel() - 1
    dev = A.device
    if total is None:
        total = int(offsets[-1].item())
    if out is None:
        shape = (groups, M, N) if vary_k else (total, N)
        out = torch.empty(shape, dtype=torch.float32, device=dev)
    ws_bytes = lib().mxq_workspace_bytes(OP_GROUPED_GEMM, groups, 0, 0)
    if workspace is None:
        workspace = _u8((max(ws_bytes, 1),), dev)
    _check("grouped_gemm_block_scaled", lib().grouped_gemm_block_scaled(
        fmt, groups, _ptr(offsets), int(vary_k), total, M, N, K, _ptr(a_row_index), a_rows if a_rows is not None
        else (A.shape[0] if a_row_index is not None else 0), _ptr(A), _ptr(sA), _ptr(tA),
        SCOPE[tA_scope], _ptr(B), _ptr(sB), _ptr(tB), SCOPE[tB_scope], _ptr(out), _ptr(workspace),
        workspace.numel(), _stream(dev)))
    return out


# ---------------------------------------------------------------------------
# MoE glue
# ---------------------------------------------------------------------------

def moe_swiglu_quantize_nvfp4(gate_up: torch.Tensor, keep_h: bool = True):
    """SwiGLU of (rows, 2*inter) FP32 gate_up, then per-row NVFP4: (h_bf16 | None, q, s, t)."""
    rows, two_i = gate_up.shape
    inter = two_i // 2
    dev = gate_up.device
    h = torch.empty((rows, inter), dtype=torch.bfloat16, device=dev) if keep_h else None
    q, s = _u8((rows, inter // 2), dev), _u8((rows, inter // 16), dev)
    t = torch.empty(rows, dtype=torch.float32, device=dev)
    _check("moe_swiglu_quantize_nvfp4", lib().moe_swiglu_quantize_nvfp4(_ptr(gate_up), rows, inter, _ptr(h), _ptr(q),
                                                                        _ptr(s), _ptr(t), _stream(dev)))
    return h, q, s, t


def moe_combine(o_slots: torch.Tensor, slot_of: torch.Tensor, weights: torch.Tensor, out=None):
    T, k = slot_of.shape
    H = o_slots.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=o_slots.device)
    _check("moe_combine", lib().moe_combine(_ptr(o_slots), o_slots.shape[0], T, k, H, _ptr(slot_of), _ptr(weights),
                                            _ptr(out),
                                            _stream(o_slots.device)))
    return out


def scale_bytes(fmt: int, rows: int, cols: int) -> int:
    return lib().mxq_scale_bytes(fmt, rows, cols)


def abi_version() -> int:
    return lib().mxq_abi_version()
