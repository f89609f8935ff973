"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any launch."""

import ctypes
import os
import re

import pytest

from microscaling_precision_quantization_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mxq.h")
P = 0x10000          # a 16-byte aligned fake device address: validation never dereferences it
MIS = 0x10004        # misaligned


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:mxq_status|size_t|const char\*|int)\s+(\w+)\s*\(", src, flags=re.M)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) >= 12
    L = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(L, n), f"libmxq.so does not export {n}"


def test_abi_version_and_status_strings():
    assert B.abi_version() == 1
    for s in range(7):
        assert B.status_string(s)


def q8(*a):
    return B.lib().quantize_mxfp8(*a)


def test_quantize_mxfp8_validation():
    assert q8(None, 32, 32, 32, P, P, None, None, None) == 1           # x NULL
    assert q8(P, 32, 32, 32, None, None, None, None, None) == 1        # no output
    assert q8(P, 32, 32, 32, P, None, None, None, None) == 1           # half a pair
    assert q8(P, 32, 48, 48, P, P, None, None, None) == 2              # cols % 32
    assert q8(P, 40, 32, 32, None, None, P, P, None) == 2              # rows % 32 with colwise
    assert q8(P, 32, 64, 32, P, P, None, None, None) == 2              # ld_x < cols
    assert q8(MIS, 32, 32, 32, P, P, None, None, None) == 3            # misaligned x
    assert q8(P, 32, 32, 36, P, P, None, None, None) == 3              # ld_x % 8
    assert q8(P, -1, 32, 32, P, P, None, None, None) == 2
    assert q8(P, 0, 32, 32, P, P, P, P, None) == 0                     # empty: no-op


def test_quantize_mxfp4_validation():
    q4 = B.lib().quantize_mxfp4
    assert q4(None, 32, 32, 32, P, P, None, None, None) == 1           # x NULL
    assert q4(P, 32, 32, 32, None, None, None, None, None) == 1        # no output
    assert q4(P, 32, 32, 32, None, None, P, None, None) == 1           # half a pair
    assert q4(P, 32, 48, 48, P, P, None, None, None) == 2              # cols % 32
    assert q4(P, 48, 32, 32, None, None, P, P, None) == 2              # rows % 32 with colwise
    assert q4(P, 32, 64, 32, P, P, None, None, None) == 2              # ld_x < cols
    assert q4(P, 32, 32, 32, MIS, P, None, None, None) == 3            # misaligned q_row
    assert q4(P, 32, 32, 36, P, P, None, None, None) == 3              # ld_x % 8
    assert q4(P, 0, 32, 32, P, P, P, P, None) == 0                     # empty: no-op


def test_fp8_block_validation():
    L = B.lib()
    qa = L.quantize_fp8_block_act
    assert qa(P, 4, 96, 96, P, P, None, None, None) == 2        # row copy: cols % 128
    assert qa(P, 96, 128, 128, None, None, P, P, None) == 2     # transposed copy: rows % 128
    assert qa(P, 128, 12, 12, None, None, P, P, None) == 2      # cols % 8
    assert qa(P, 4, 128, 128, P, MIS + 1, None, None, None) == 3   # misaligned scales
    assert qa(P, 4, 128, 128, None, None, None, None, None) == 1
    assert qa(P, 4, 128, 128, P, None, None, None, None) == 1
    assert qa(P, 0, 128, 128, P, P, None, None, None) == 0
    qw = L.quantize_fp8_block_weight
    assert qw(P, 128, 96, 96, P, P, None, None, None) == 2   # cols % 128
    assert qw(P, 64, 128, 128, P, P, None, None, None) == 2  # rows % 128
    assert qw(P, 128, 128, 128, None, None, None, None, None) == 1
    assert qw(P, 128, 128, 128, P, None, None, None, None) == 1
    assert qw(P, 128, 128, 128, P, P, MIS, P, None) == 3
    g = L.gemm_fp8_blockwise
    assert g(32, 32, 96, P, P, P, P, 1, P, 32, None) == 2    # K % 128
    assert g(32, 32, 128, P, P, P, P, 2, P, 32, None) == 4
    assert g(32, 32, 128, P, None, P, P, 1, P, 32, None) == 1
    assert g(32, 32, 128, P, P, P, P, 1, P, 16, None) == 2   # ldc < N
    assert g(0, 32, 128, P, P, P, P, 1, P, 32, None) == 0


def test_gemm_batch_validation():
    L = B.lib()
    mk = lambda *d: (B._GemmProblem * len(d))(*[B._GemmProblem(*x) for x in d])
    ok = (32, 32, 64, P, P, None, 0, P, P, None, 0, P, 32)
    call = lambda fmt, arr, n: L.gemm_block_scaled_batch(fmt, ctypes.cast(arr, ctypes.c_void_p), n, None)
    assert call(1, mk(ok), 0) == 2
    assert call(1, mk(*[ok] * 9), 9) == 2
    assert call(9, mk(ok), 1) == 4
    assert call(1, mk(ok, (32, 32, 48, P, P, None, 0, P, P, None, 0, P, 32)), 2) == 2     # K % 32
    assert call(1, mk(ok, (32, 32, 64, P, None, None, 0, P, P, None, 0, P, 32)), 2) == 1  # scales missing
    assert call(2, mk((32, 32, 64, P, P, None, 0, P, P, P, 1, P, 32)), 1) == 1             # NVFP4 without tA
    assert call(1, mk(ok, (32, 32, 64, MIS, P, None, 0, P, P, None, 0, P, 32)), 2) == 3
    assert call(1, mk((0, 32, 64, None, None, None, 0, None, None, None, 0, None, 32)), 1) == 0   # empty: no-op
    assert L.gemm_block_scaled_batch(1, None, 1, None) == 1


def multi(descs):
    arr = (B._Mxfp8Tensor * max(len(descs), 1))(*[B._Mxfp8Tensor(*d) for d in descs])
    return B.lib().quantize_mxfp8_multi(ctypes.cast(arr, ctypes.c_void_p), len(descs), None)


def test_quantize_mxfp8_multi_validation():
    ok = (P, 64, 64, 64, P, P, P, P)
    assert multi([]) == 2                                               # count 0
    assert multi([ok] * 9) == 2                                         # beyond the maximum
    assert multi([ok, (P, 64, 64, 64, P, P, None, None)]) == 4          # mixed copies
    assert multi([ok, (P, 64, 48, 48, P, P, P, P)]) == 2                # cols % 32 in the 2nd tensor
    assert multi([ok, (MIS, 64, 64, 64, P, P, P, P)]) == 3
    assert multi([ok, (None, 64, 64, 64, P, P, P, P)]) == 1
    assert multi([(P, 0, 64, 64, P, P, P, P)]) == 0                     # all empty: no-op
    assert B.lib().quantize_mxfp8_multi(None, 1, None) == 1
    arr = (B._Mxfp8Tensor * 2)(B._Mxfp8Tensor(*ok), B._Mxfp8Tensor(P, 64, 48, 48, P, P, P, P))
    assert B.lib().quantize_mxfp4_multi(ctypes.cast(arr, ctypes.c_void_p), 2, None) == 2       # MXFP4: cols % 32
    assert B.lib().quantize_mxfp4_multi(ctypes.cast(arr, ctypes.c_void_p), 0, None) == 2


def test_nvfp4_validation():
    L = B.lib()
    assert L.quantize_nvfp4_per_token(P, 4, 40, 40, P, P, P, None) == 2       # hidden % 16
    assert L.quantize_nvfp4_per_token(P, 4, 32768, 32768, P, P, P, None) == 2  # beyond the row limit
    assert L.quantize_nvfp4_per_token(P, 0, 32, 32, P, P, P, None) == 0
    bad = (ctypes.c_int8 * 16)(*([1] * 15 + [0]))
    assert L.quantize_nvfp4(P, 32, 32, 32, 1, 0, 0, bad, P, P, P, P, 256, None) == 4   # sign not +-1
    assert L.quantize_nvfp4(P, 32, 32, 32, 0, 0, 1, None, P, P, P, None, 0, None) == 4  # ROW + transpose
    assert L.quantize_nvfp4(P, 32, 32, 32, 1, 0, 0, None, P, P, P, None, 0, None) == 5  # no workspace
    assert L.quantize_nvfp4(P, 32, 32, 32, 2, 5, 0, None, P, P, P, P, 256, None) == 2   # group rows
    assert L.quantize_nvfp4(P, 32, 32, 32, 9, 0, 0, None, P, P, P, P, 256, None) == 4   # bad scope


def test_quantize_nvfp4_2d_validation():
    q2 = B.lib().quantize_nvfp4_2d
    assert q2(P, 32, 40, 40, 1, 0, P, P, None, None, P, P, 256, None) == 2     # cols % 16
    assert q2(P, 24, 32, 32, 1, 0, P, P, None, None, P, P, 256, None) == 2     # rows % 16
    assert q2(P, 32, 32, 32, 0, 0, P, P, None, None, P, P, 256, None) == 4     # ROW scope
    assert q2(P, 64, 32, 32, 2, 24, P, P, None, None, P, P, 256, None) == 2    # group rows % 16
    assert q2(P, 32, 32, 32, 1, 0, None, None, None, None, P, P, 256, None) == 1
    assert q2(P, 32, 32, 32, 1, 0, P, None, None, None, P, P, 256, None) == 1  # half a pair
    assert q2(P, 32, 32, 32, 1, 0, P, P, None, None, P, None, 0, None) == 5    # no workspace
    assert q2(P, 32, 32, 32, 1, 0, P, P, MIS, P, P, P, 256, None) == 3
    assert q2(P, 0, 32, 32, 1, 0, P, P, None, None, P, None, 0, None) == 0     # empty


def test_gemm_validation():
    L = B.lib()
    g = L.gemm_block_scaled
    assert g(1, 32, 32, 48, P, P, None, 0, P, P, None, 0, P, 32, None) == 2      # K % 32
    assert g(1, 32, 32, 64, P, None, None, 0, P, P, None, 0, P, 32, None) == 1   # scales missing
    assert g(2, 32, 32, 64, P, P, None, 0, P, P, P, 1, P, 32, None) == 1         # NVFP4 needs t's
    assert g(2, 32, 32, 64, P, P, P, 2, P, P, P, 1, P, 32, None) == 4            # GROUP tA scope
    assert g(9, 32, 32, 64, P, P, None, 0, P, P, None, 0, P, 32, None) == 4
    assert g(1, 32, 32, 64, P, P, None, 0, P, P, None, 0, P, 16, None) == 2      # ldc < N
    assert g(1, 32, 32, 64, MIS, P, None, 0, P, P, None, 0, P, 32, None) == 3
    assert g(1, 0, 32, 64, P, P, None, 0, P, P, None, 0, P, 32, None) == 0       # empty
    assert g(4, 32, 32, 48, P, P, None, 0, P, P, None, 0, P, 32, None) == 2      # MXFP4 K % 32
    assert g(4, 32, 32, 64, P, P, None, 0, P, None, None, 0, P, 32, None) == 1   # MXFP4 scales missing
    assert g(4, 32, 32, 64, P, P, None, 0, MIS, P, None, 0, P, 32, None) == 3
    gg = L.grouped_gemm_block_scaled
    assert gg(1, 4, P, 0, 64, 0, 32, 64, None, 0, P, P, None, 0, P, P, None, 0, P, None, 0, None) == 5
    assert gg(2, 4, P, 1, 64, 32, 32, 64, None, 0, P, P, P, 0, P, P, P, 2, P, P, 4096, None) == 4   # NVFP4 vary_k
    assert gg(1, 4, None, 0, 64, 0, 32, 64, None, 0, P, P, None, 0, P, P, None, 0, P, P, 4096, None) == 1
    assert gg(1, 0, P, 0, 0, 0, 32, 64, None, 0, P, P, None, 0, P, P, None, 0, P, None, 0, None) == 0
    assert gg(4, 4, P, 1, 48, 32, 32, 0, None, 0, P, P, None, 0, P, P, None, 0, P, P, 4096, None) == 2   # MXFP4 total % 32
    # vary_k = 2 (K-major A): BF16 only, M % 8 == 0; other mode values are unknown
    assert gg(1, 4, P, 2, 64, 32, 32, 0, None, 0, P, P, None, 0, P, P, None, 0, P, P, 4096, None) == 4
    assert gg(3, 4, P, 2, 64, 36, 32, 0, None, 0, P, None, None, 0, P, None, None, 0, P, P, 4096, None) == 2
    assert gg(3, 4, P, 3, 64, 40, 32, 0, None, 0, P, None, None, 0, P, None, None, 0, P, P, 4096, None) == 4
    assert gg(3, 0, P, 2, 0, 40, 32, 0, None, 0, P, None, None, 0, P, None, None, 0, P, P, 4096, None) == 0


def test_dequant_and_moe_validation():
    L = B.lib()
    assert L.dequantize(2, P, P, None, 0, 0, 4, 32, P, 0, None) == 1      # NVFP4 without t
    assert L.dequantize(1, P, P, None, 0, 0, 4, 48, P, 0, None) == 2
    assert L.dequantize(3, P, P, None, 0, 0, 4, 32, P, 0, None) == 4
    assert L.dequantize(4, P, P, None, 0, 0, 4, 48, P, 0, None) == 2      # MXFP4 cols % 32
    assert L.dequantize(4, P, None, None, 0, 0, 4, 32, P, 0, None) == 1
    dt = L.dequantize_transposed
    assert dt(2, P, P, None, 0, 1, 64, 32, None, 64, P, 64, None) == 1       # NVFP4 without t
    assert dt(1, P, P, None, 0, 1, 64, 48, None, 64, P, 64, None) == 2       # cols % 32 (MXFP8)
    assert dt(3, P, None, None, 0, 1, 64, 32, None, 12, P, 16, None) == 2    # out_cols % 8
    assert dt(3, P, None, None, 0, 1, 64, 32, None, 72, P, 72, None) == 2    # no gather: out_cols > group_rows
    assert dt(3, P, None, None, 0, 1, 64, 32, None, 64, P, 56, None) == 2    # ld_out < out_cols
    assert dt(3, P, None, None, 0, 70000, 64, 32, None, 64, P, 64, None) == 2  # too many groups
    assert dt(3, MIS, None, None, 0, 1, 64, 32, None, 64, P, 64, None) == 3
    assert dt(2, P, P, P, 7, 1, 64, 32, None, 64, P, 64, None) == 4          # bad scope
    assert dt(3, P, None, None, 0, 0, 64, 32, None, 64, P, 64, None) == 0    # empty
    assert L.moe_swiglu_quantize_nvfp4(P, 4, 24, None, P, P, P, None) == 2
    assert L.moe_combine(P, 8, 4, 2, 6, P, P, P, None) == 2
    assert L.moe_combine(P, 8, 0, 2, 8, P, P, P, None) == 0


def test_scale_and_workspace_sizes():
    assert B.scale_bytes(B.MXFP8, 256, 512) == 256 * 16
    assert B.scale_bytes(B.NVFP4, 4096, 2048) == 4096 * 128
    assert B.scale_bytes(B.MXFP8, 4, 48) == 0
    assert B.scale_bytes(B.MXFP4, 128, 1024) == 128 * 32
    L = B.lib()
    assert L.mxq_workspace_bytes(B.OP_QUANTIZE_NVFP4, 0, 0, 3) >= 12
    assert L.mxq_workspace_bytes(B.OP_GROUPED_GEMM, 128, 0, 0) >= 129 * 8


def test_fp8_block_batch_validation():
    """Every descriptor is checked on the host before anything is launched (fake device
    addresses: no case here reaches a launch)."""
    f = B.lib().gemm_fp8_blockwise_batch

    def prob(**kw):
        d = dict(M=128, N=128, K=256, A=P, sA=P, B=P, sB=P, b_blocks=1, C=P, ldc=128)
        d.update(kw)
        return B._Fp8BlockProblem(**d)

    def call(*probs, count=None):
        arr = (B._Fp8BlockProblem * len(probs))(*probs)
        return f(ctypes.cast(arr, ctypes.c_void_p), len(probs) if count is None else count, None)

    assert call(prob(), count=0) == 2                                   # count < 1
    assert call(*[prob(M=0) for _ in range(9)]) == 2                    # count > MXQ_GEMM_BATCH_MAX
    assert f(None, 1, None) == 1                                        # NULL array
    assert call(prob(), prob(K=200)) == 2                               # K % 128 in a later descriptor
    assert call(prob(), prob(sB=None)) == 1
    assert call(prob(b_blocks=2)) == 4
    assert call(prob(A=MIS)) == 3
    assert call(prob(sA=P + 2)) == 3                                    # scales 4-byte aligned
    assert call(prob(ldc=64)) == 2                                      # ldc < N
    assert call(prob(M=-1)) == 2
    assert call(prob(M=0), prob(N=0, A=None)) == 0                      # only empty problems: no-op


def test_matrix_core_rejects_k_beyond_32bit_offsets():
    f = B.lib().gemm_mxfp8_matrix_core
    assert f(32, 32, (1 << 22) + 32, P, P, P, P, P, 32, None) == 2      # K > 2^22
    assert f(32, 32, 48, P, P, P, P, P, 32, None) == 2                  # K % 32


def test_binding_rejects_mismatched_buffers_before_any_call():
    """The Python binding checks every operand, scale and output shape, dtype and layout on
    the host (CPU tensors here: the shape checks run before the device check, and no
    library call is reached)."""
    import torch
    u8 = lambda *s: torch.zeros(s, dtype=torch.uint8)
    f32 = lambda *s: torch.zeros(s, dtype=torch.float32)
    A, sA, Bq, sB = u8(64, 128), u8(64, 4), u8(32, 128), u8(32, 4)
    with pytest.raises(ValueError, match="out: shape"):
        B.gemm_block_scaled(B.MXFP8, A, sA, Bq, sB, out=f32(64, 16))          # undersized output
    with pytest.raises(ValueError, match="B: shape"):
        B.gemm_block_scaled(B.MXFP8, A, sA, u8(32, 96), u8(32, 3))            # B narrower than A's K
    with pytest.raises(ValueError, match="sB: shape"):
        B.gemm_block_scaled(B.MXFP8, A, sA, Bq, u8(32, 2))                    # short scale matrix
    with pytest.raises(ValueError, match="contiguous"):
        B.gemm_block_scaled(B.MXFP8, u8(128, 64).t(), sA, Bq, sB)             # strided operand
    with pytest.raises(ValueError, match="dtype"):
        B.gemm_block_scaled(B.BF16, A, None, Bq, None)                        # BF16 format, uint8 data
    with pytest.raises(ValueError, match="tA"):
        B.gemm_block_scaled(B.NVFP4, u8(64, 64), u8(64, 8), u8(32, 64), u8(32, 8), tA=f32(63), tB=f32(1))
    with pytest.raises(ValueError, match="GPU tensor"):
        B.gemm_block_scaled(B.MXFP8, A, sA, Bq, sB, out=f32(64, 32))          # right shapes, host memory
    with pytest.raises(ValueError, match="out: shape"):
        B.gemm_block_scaled_batch(B.MXFP8, [dict(A=A, sA=sA, B=Bq, sB=sB, out=f32(32, 32)),
                                            dict(A=A, sA=sA, B=Bq, sB=sB, out=f32(64, 32))])
    with pytest.raises(ValueError, match="sB: shape"):
        B.gemm_fp8_blockwise(u8(64, 256), f32(64, 2), u8(256, 256), f32(256, 2), b_blocks=True)
    with pytest.raises(ValueError, match="out: shape"):
        B.gemm_mxfp8_matrix_core(A, sA, Bq, sB, out=f32(64, 31))
    off = torch.tensor([0, 32, 64], dtype=torch.int64)
    with pytest.raises(ValueError, match="B: shape"):
        B.grouped_gemm_block_scaled(B.BF16, off, torch.zeros(64, 128, dtype=torch.bfloat16),
                                    torch.zeros(1, 16, 128, dtype=torch.bfloat16), N=16, K=128, total=64)
    with pytest.raises(ValueError, match="out: shape"):
        B.grouped_gemm_block_scaled(B.BF16, off, torch.zeros(64, 128, dtype=torch.bfloat16),
                                    torch.zeros(2, 16, 128, dtype=torch.bfloat16), N=16, K=128, total=64,
                                    out=f32(64, 8))
    with pytest.raises(ValueError, match="q_colT: shape"):
        B.quantize_mxfp8_multi([torch.zeros(64, 64, dtype=torch.bfloat16)], [(u8(64, 64), u8(64, 2), u8(32, 64),
                                                                             u8(64, 2))])
