"""Thin Python binding of libmxq (ctypes).

Argument marshalling only: every function here allocates its outputs with torch
on the input's device, passes raw device pointers and torch's current HIP stream
to the C ABI in include/mxq.h, and raises MxqError on a non-zero status. No
step of the quantize / GEMM path runs in Python, and there is no fallback: if
libmxq.so is missing the first call raises. MXQ_LIBRARY, when set, names another
build of the same library to load instead (the host-sanitizer build that the ABI
tests run under).
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MXQ_LIBRARY") or os.path.join(_HERE, "libmxq.so")

MXFP8, NVFP4, BF16, MXFP4 = 1, 2, 3, 4
BF16_NVFP4T = 5                    # grouped only: BF16 A x stacked NVFP4 weights (K, N) read transposed
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
    "grouped_gemm_block_scaled_noalloc": [_int, _i64, _c_void_p, _int, _i64, _i64, _i64, _i64, _c_void_p, _i64,
                                          _c_void_p, _c_void_p, _c_void_p, _int, _c_void_p, _c_void_p, _c_void_p,
                                          _int, _c_void_p, _c_void_p],
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


class _Checks:
    """Host-side checks of the tensors handed to one C-ABI call: dtype, exact shape, unit
    inner stride and a dense layout (ld=True: rows may be padded, row stride >= the row
    length) for each tensor as it is named, then, in done(), that all of them live on the
    one GPU the call runs on. Every mismatch raises ValueError before anything reaches
    the library, so a wrong buffer can never be read or written past its end."""

    def __init__(self, dev):
        self.dev = dev
        self.seen = []

    def need(self, t, name: str, dtype, shape, ld: bool = False):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name}: expected a tensor, got {type(t).__name__}")
        if t.dtype != dtype:
            raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
        shape = tuple(int(v) for v in shape)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {shape}")
        if t.numel():
            if t.dim() and t.stride(-1) != 1:
                raise ValueError(f"{name}: the innermost dimension must be contiguous")
            if ld:
                if t.dim() != 2 or t.stride(0) < t.shape[1]:
                    raise ValueError(f"{name}: expected a 2-D tensor with row stride >= {t.shape[1]}")
            elif not t.is_contiguous():
                raise ValueError(f"{name}: expected a contiguous tensor")
        self.seen.append((name, t))
        return t

    def opt(self, t, *a, **kw):
        return None if t is None else self.need(t, *a, **kw)

    def operand(self, fmt: int, name: str, t, rows: int, K: int, s=None):
        """A K-contiguous GEMM operand of `rows` rows and K elements (+ its block scales)."""
        width = K if fmt == BF16 else K // _elems_per_byte(fmt)
        self.need(t, name, _operand_dtype(fmt), (rows, width))
        if fmt != BF16:
            if s is None:
                raise ValueError(f"s{name}: block scales are required for this format")
            self.need(s, "s" + name, torch.uint8, (rows, K // _scale_block(fmt)))

    def outer_scale(self, name: str, t, scope: str, rows: int):
        if t is None:
            raise ValueError(f"{name}: NVFP4 needs its FP32 scale")
        self.need(t, name, torch.float32, (rows if SCOPE[scope] == 0 else 1,))

    def done(self):
        for name, t in self.seen:
            if not t.is_cuda:
                raise ValueError(f"{name}: expected a GPU tensor, got one on {t.device}")
            if t.device != self.dev:
                raise ValueError(f"{name}: on {t.device}, expected {self.dev}")


def _elems_per_byte(fmt: int) -> int:
    return 2 if fmt in _PACKED4 else 1


def _operand_dtype(fmt: int):
    return torch.bfloat16 if fmt == BF16 else torch.uint8


def _scale_block(fmt: int) -> int:
    return 16 if fmt == NVFP4 else 32


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
        _mx_check_out("quantize_mxfp8", x, out, 1)
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
        _mx_check_out("quantize_mxfp4", x, out, 2)
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


def _mx_check_out(fn: str, x, out, per_byte: int):
    """Output buffers of an MXFP8 / MXFP4 quantize: (R, C/per_byte) + (R, C/32) rowwise,
    (C, R/per_byte) + (C, R/32) columnwise; a skipped copy is (None, None)."""
    R, C = x.shape
    q_row, s_row, q_col, s_col = out
    if (q_row is None) != (s_row is None) or (q_col is None) != (s_col is None):
        raise ValueError(f"{fn}: a copy needs both its element and its scale buffer")
    c = _Checks(x.device)
    c.opt(q_row, "q_row", torch.uint8, (R, C // per_byte))
    c.opt(s_row, "s_row", torch.uint8, (R, C // 32))
    c.opt(q_col, "q_colT", torch.uint8, (C, R // per_byte))
    c.opt(s_col, "s_colT", torch.uint8, (C, R // 32))
    c.done()


def _mx_multi(fn: str, xs, outs):
    n = len(xs)
    if len(outs) != n:
        raise ValueError(f"{fn}: {n} inputs but {len(outs)} output tuples")
    arr = (_Mxfp8Tensor * n)()
    for i, (x, o) in enumerate(zip(xs, outs)):
        _mx_check_out(fn, x, o, 2 if fn.startswith("quantize_mxfp4") else 1)
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
    elif (out.dtype != torch.bfloat16 or out.dim() != 3 or tuple(out.shape[:2]) != (groups, cols)
          or out.shape[2] < out_cols or out.stride(-1) != 1 or out.stride(0) != cols * out.stride(1)
          or out.device != q.device):
        raise ValueError(f"out: expected BF16 (groups={groups}, cols={cols}, >= {out_cols}) rows on {q.device}")
    _check("dequantize_transposed", lib().dequantize_transposed(
        fmt, _ptr(q), _ptr(s), _ptr(t), SCOPE[t_scope], groups, group_rows, cols, _ptr(src_row), out_cols,
        _ptr(out), out.stride(-2), _stream(q.device)))
    return out


# ---------------------------------------------------------------------------
# GEMMs
# ---------------------------------------------------------------------------

def _gemm_args(fmt: int, A, sA, B, sB, tA, tB, tA_scope, tB_scope, out):
    """Validate one TN GEMM's operands and output; returns (M, N, K)."""
    if fmt not in (MXFP8, NVFP4, BF16, MXFP4):
        raise ValueError(f"unknown format {fmt}")
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D (rows, K-contiguous bytes or elements)")
    M, N = A.shape[0], B.shape[0]
    K = A.shape[1] * _elems_per_byte(fmt)
    c = _Checks(A.device)
    c.operand(fmt, "A", A, M, K, sA)
    c.operand(fmt, "B", B, N, K, sB)
    if fmt == NVFP4:
        c.outer_scale("tA", tA, tA_scope, M)
        c.outer_scale("tB", tB, tB_scope, N)
    if out is not None:
        c.need(out, "out", torch.float32, (M, N), ld=True)
    c.done()
    return M, N, K


def gemm_block_scaled(fmt: int, A, sA, B, sB, tA=None, tB=None, tA_scope="row", tB_scope="tensor", out=None):
    """C = A_hat B_hat^T in FP32; A (M, K-bytes) and B (N, K-bytes) K-contiguous."""
    M, N, K = _gemm_args(fmt, A, sA, B, sB, tA, tB, tA_scope, tB_scope, out)
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
        if A.device != dev:
            raise ValueError(f"problem {i}: operands on {A.device}, the batch runs on {dev}")
        _, _, K = _gemm_args(fmt, A, q.get("sA"), B_, q.get("sB"), q.get("tA"), q.get("tB"),
                             q.get("tA_scope", "row"), q.get("tB_scope", "tensor"), out)
        ptr = lambda t: None if t is None else t.data_ptr()
        arr[i] = _GemmProblem(A.shape[0], B_.shape[0], K, A.data_ptr(), ptr(q.get("sA")), ptr(q.get("tA")),
                              SCOPE[q.get("tA_scope", "row")], B_.data_ptr(), ptr(q.get("sB")), ptr(q.get("tB")),
                              SCOPE[q.get("tB_scope", "tensor")], out.data_ptr(), out.stride(0))
    _check("gemm_block_scaled_batch", lib().gemm_block_scaled_batch(fmt, ctypes.cast(arr, _c_void_p), n, _stream(dev)))
    return [q["out"] for q in problems]


def _fp8_block_args(A, sA, B, sB, b_blocks: bool, out):
    """Validate a blockwise-FP8 GEMM; returns (M, N, K)."""
    M, K = A.shape
    N = B.shape[0]
    c = _Checks(A.device)
    c.need(A, "A", torch.uint8, (M, K))
    c.need(sA, "sA", torch.float32, (M, K // 128))
    c.need(B, "B", torch.uint8, (N, K))
    c.need(sB, "sB", torch.float32, ((N + 127) // 128, K // 128) if b_blocks else (N, K // 128))
    if out is not None:
        c.need(out, "out", torch.float32, (M, N), ld=True)
    c.done()
    return M, N, K


def gemm_fp8_blockwise(A, sA, B, sB, b_blocks: bool = True, out=None):
    """Blockwise FP8 GEMM C = A_hat B_hat^T (FP32); sB per 128 x 128 block (b_blocks) or per row."""
    M, N, K = _fp8_block_args(A, sA, B, sB, b_blocks, out)
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
        if A.device != dev:
            raise ValueError(f"problem {i}: operands on {A.device}, the batch runs on {dev}")
        _fp8_block_args(A, q["sA"], B_, q["sB"], q["b_blocks"], out)
        arr[i] = _Fp8BlockProblem(A.shape[0], B_.shape[0], A.shape[1], A.data_ptr(), q["sA"].data_ptr(), B_.data_ptr(),
                                  q["sB"].data_ptr(), int(q["b_blocks"]), out.data_ptr(), out.stride(0))
    _check("gemm_fp8_blockwise_batch", lib().gemm_fp8_blockwise_batch(ctypes.cast(arr, _c_void_p), n, _stream(dev)))
    return [q["out"] for q in problems]


def gemm_mxfp8_matrix_core(A, sA, B, sB, out=None):
    """MXFP8 GEMM on the native scaled-FP8 matrix core (see include/mxq.h for its accumulation)."""
    M, N, K = _gemm_args(MXFP8, A, sA, B, sB, None, None, "row", "tensor", out)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    _check("gemm_mxfp8_matrix_core", lib().gemm_mxfp8_matrix_core(M, N, K, _ptr(A), _ptr(sA), _ptr(B), _ptr(sB),
                                                                  _ptr(out), out.stride(0), _stream(A.device)))
    return out


def _grouped_args(fmt, offsets, A, B, N, K, sA, sB, tA, tB, tA_scope, tB_scope, a_row_index, vary_k, M, total,
                  a_rows, out):
    """Validate a grouped GEMM's host-visible shapes (the offsets' values are checked on
    the device)."""
    c = _Checks(A.device)
    c.need(offsets, "offsets", torch.int64, (offsets.numel(),))
    G = offsets.numel() - 1
    if G < 0:
        raise ValueError("offsets: needs groups + 1 entries")
    if fmt == BF16_NVFP4T:
        if vary_k or a_row_index is not None:
            raise ValueError("BF16_NVFP4T: row-grouped only, no gather")
        c.need(A, "A", torch.bfloat16, (total, K))
        c.need(B.reshape(-1, B.shape[-1]) if B.dim() == 3 else B, "B", torch.uint8, (G * K, N // 2))
        if sB is None or tB is None:
            raise ValueError("BF16_NVFP4T: sB and tB (one FP32 scale per group) are required")
        c.need(sB.reshape(-1, sB.shape[-1]) if sB.dim() == 3 else sB, "sB", torch.uint8, (G * K, N // 16))
        c.need(tB, "tB", torch.float32, (G,))
        if out is not None:
            c.need(out, "out", torch.float32, (total, N))
        c.done()
        return
    if vary_k:
        if a_row_index is not None:
            raise ValueError("a_row_index is not supported with vary_k")
        if vary_k == 2:                                     # K-major A: (total, M), BF16 only
            if fmt != BF16:
                raise ValueError("vary_k=2 (K-major A) is BF16 only")
            c.operand(fmt, "A", A, total, M, None)
        else:
            c.operand(fmt, "A", A, M, total, sA)
        c.operand(fmt, "B", B, N, total, sB)
        if out is not None:
            c.need(out, "out", torch.float32, (G, M, N))
        c.done()
        return
    rows = A.shape[0]
    if a_row_index is not None:
        c.need(a_row_index, "a_row_index", torch.int32, (total,))
        if a_rows is not None and a_rows != rows:
            raise ValueError(f"a_rows = {a_rows} but A has {rows} rows")
    elif rows != total:
        raise ValueError(f"A: {rows} rows, expected total = {total} (no gather)")
    c.operand(fmt, "A", A, rows, K, sA)
    width = K if fmt == BF16 else K // _elems_per_byte(fmt)
    if B.shape[-1] != width or B.numel() != G * N * width:
        raise ValueError(f"B: shape {tuple(B.shape)}, expected {G} stacked ({N}, {width}) operands")
    if not B.is_contiguous():
        raise ValueError("B: expected a contiguous tensor")
    c.operand(fmt, "B", B.reshape(G * N, width), G * N, K, None if sB is None else sB.reshape(-1, sB.shape[-1]))
    if fmt == NVFP4:
        c.outer_scale("tA", tA, tA_scope, rows)
        if tB is None:
            raise ValueError("tB: NVFP4 needs its FP32 scale")
        c.need(tB, "tB", torch.float32, (G if SCOPE[tB_scope] == 2 else G * N if SCOPE[tB_scope] == 0 else 1,))
    if out is not None:
        c.need(out, "out", torch.float32, (total, N))
    c.done()


def grouped_gemm_block_scaled(fmt: int, offsets, A, B, N: int, K: int, sA=None, sB=None, tA=None, tB=None,
                              tA_scope="row", tB_scope="group", a_row_index=None, vary_k=False, M: int = 0,
                              total: int | None = None, a_rows: int | None = None, out=None, workspace=None):
    """One GEMM per group; see include/mxq.h for the two modes.

    vary_k=False: out (total_slots, N); vary_k=True: out (groups, M, N); vary_k=2: as True
    with A given K-major, (total, M).
    """
    groups = offsets.numel() - 1
    dev = A.device
    if total is None:
        total = int(offsets[-1].item())
    _grouped_args(fmt, offsets, A, B, N, K, sA, sB, tA, tB, tA_scope, tB_scope, a_row_index, vary_k, M, total,
                  a_rows, out)
    if out is None:
        shape = (groups, M, N) if vary_k else (total, N)
        out = torch.empty(shape, dtype=torch.float32, device=dev)
    ws_bytes = lib().mxq_workspace_bytes(OP_GROUPED_GEMM, groups, 0, 0)
    if workspace is None:
        workspace = _u8((max(ws_bytes, 1),), dev)
    elif workspace.numel() < ws_bytes:
        raise ValueError(f"workspace: {workspace.numel()} bytes, the call needs {ws_bytes}")
    _check("grouped_gemm_block_scaled", lib().grouped_gemm_block_scaled(
        fmt, groups, _ptr(offsets), int(vary_k), total, M, N, K, _ptr(a_row_index), a_rows if a_rows is not None
        else (A.shape[0] if a_row_index is not None else 0), _ptr(A), _ptr(sA), _ptr(tA),
        SCOPE[tA_scope], _ptr(B), _ptr(sB), _ptr(tB), SCOPE[tB_scope], _ptr(out), _ptr(workspace),
        workspace.numel(), _stream(dev)))
    return out


def grouped_gemm_block_scaled_noalloc(fmt: int, offsets, A, B, N: int, K: int, sA=None, sB=None, tA=None, tB=None,
                                      tA_scope="row", tB_scope="group", a_row_index=None, vary_k=False, M: int = 0,
                                      total: int | None = None, a_rows: int | None = None, out=None):
    """grouped_gemm_block_scaled with the scheduler scratch in the library's static device
    array (no workspace): for callers that cannot allocate. `out` must be given (this
    call allocates nothing)."""
    if out is None:
        raise ValueError("out: the no-allocation call needs a preallocated output")
    if total is None:
        raise ValueError("total: pass it explicitly (reading it from the device offsets would synchronize)")
    _grouped_args(fmt, offsets, A, B, N, K, sA, sB, tA, tB, tA_scope, tB_scope, a_row_index, vary_k, M, total,
                  a_rows, out)
    _check("grouped_gemm_block_scaled_noalloc", lib().grouped_gemm_block_scaled_noalloc(
        fmt, offsets.numel() - 1, _ptr(offsets), int(vary_k), total, M, N, K, _ptr(a_row_index),
        a_rows if a_rows is not None else (A.shape[0] if a_row_index is not None else 0), _ptr(A), _ptr(sA), _ptr(tA),
        SCOPE[tA_scope], _ptr(B), _ptr(sB), _ptr(tB), SCOPE[tB_scope], _ptr(out), _stream(A.device)))
    return out


# ---------------------------------------------------------------------------
# MoE glue
# ---------------------------------------------------------------------------

def moe_swiglu_quantize_nvfp4(gate_up: torch.Tensor, keep_h: bool = True):
    """SwiGLU of (rows, 2*inter) FP32 gate_up, then per-row NVFP4: (h_bf16 | None, q, s, t)."""
    rows, two_i = gate_up.shape
    inter = two_i // 2
    dev = gate_up.device
    c = _Checks(dev)
    c.need(gate_up, "gate_up", torch.float32, (rows, 2 * inter))
    c.done()
    h = torch.empty((rows, inter), dtype=torch.bfloat16, device=dev) if keep_h else None
    q, s = _u8((rows, inter // 2), dev), _u8((rows, inter // 16), dev)
    t = torch.empty(rows, dtype=torch.float32, device=dev)
    _check("moe_swiglu_quantize_nvfp4", lib().moe_swiglu_quantize_nvfp4(_ptr(gate_up), rows, inter, _ptr(h), _ptr(q),
                                                                        _ptr(s), _ptr(t), _stream(dev)))
    return h, q, s, t


def moe_combine(o_slots: torch.Tensor, slot_of: torch.Tensor, weights: torch.Tensor, out=None):
    T, k = slot_of.shape
    H = o_slots.shape[1]
    c = _Checks(o_slots.device)
    c.need(o_slots, "o_slots", torch.float32, tuple(o_slots.shape))
    c.need(slot_of, "slot_of", torch.int64, (T, k))
    c.need(weights, "weights", torch.float32, (T, k))
    c.opt(out, "out", torch.float32, (T, H))
    c.done()
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
