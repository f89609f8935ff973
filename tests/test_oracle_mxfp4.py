"""Pins for the oracle's MXFP4 quantizer (CPU only): block size 32 and the E2M1
value set printed on the pages (7minutos.es, "Que es realmente NVFP4"), power-of-two
E8M0 scales, the closed form of the round-up exponent rule, where the block amax
lands (the lost +-4 / +-6 samples of "NVFP4 frente a MXFP4"), an elementwise error
bound, and the transposed columnwise copy."""

import numpy as np

from microscaling_precision_quantization_amd import inputs
from oracle import formats as F
from oracle import mxfp4
from tests.conftest import read_golden


def data(r=64, c=256, seed=0):
    g = np.random.default_rng(seed)
    return inputs.to_bf16_bits(g.standard_normal((r, c)) * g.lognormal(0, 3, (r, 1)))


def test_block_size_and_value_set_are_the_printed_ones():
    sizes = dict(line.split() for line in read_golden("block_sizes.txt"))
    assert int(sizes["mxfp4"]) == mxfp4.BLOCK == 32
    printed = {float(v) for v in read_golden("e2m1_values.txt")}
    p, s = mxfp4.quantize_rowwise(data())
    assert set(np.unique(np.abs(mxfp4.dequantize_exact(p, np.full_like(s, 127)))).tolist()) <= printed


def test_scale_closed_form():
    x = data(128, 512, seed=1)
    p, s = mxfp4.quantize_rowwise(x)
    a = np.max(np.abs(inputs.bf16_bits_to_float(x)).reshape(128, 16, 32), axis=2).astype(np.float64)
    X = F.decode_e8m0(s)
    assert np.all((X == 2.0 ** np.round(np.log2(X))))                       # powers of two
    assert np.all(a <= 6 * X)
    assert np.all((s == 0) | (a > 6 * X / 2))                                # smallest such power
    # boundary: amax exactly 6 * 2^k -> s = 127 + k; the next BF16 above -> s = 128 + k
    for k in (-3, 0, 5):
        blk = np.zeros((1, 32))
        blk[0, 0] = 6.0 * 2.0 ** k
        _, sb = mxfp4.quantize_rowwise(inputs.to_bf16_bits(blk))
        assert sb[0, 0] == 127 + k
        blk[0, 0] = np.nextafter(np.float32(6.0 * 2.0 ** k), np.float32(np.inf))
        blk = inputs.bf16_bits_to_float(inputs.to_bf16_bits(blk) + np.uint16(1)).reshape(1, 32)
        _, sb = mxfp4.quantize_rowwise(inputs.to_bf16_bits(blk))
        assert sb[0, 0] == 128 + k


def test_block_amax_lands_on_3_4_or_6():
    # with the rounded-up power-of-two scale the block amax maps into (3, 6]: codes 3, 4 or 6,
    # i.e. the top samples +-4 / +-6 can be lost (the page's worst case), never exceeded
    x = data(64, 512, seed=2)
    p, s = mxfp4.quantize_rowwise(x)
    xv = np.abs(inputs.bf16_bits_to_float(x)).reshape(64, 16, 32)
    codes = mxfp4.unpack_codes(p).reshape(64, 16, 32) & 7
    j = np.argmax(xv, axis=2)
    amax_code = np.take_along_axis(codes, j[:, :, None], axis=2)[:, :, 0]
    assert set(np.unique(amax_code[s > 0]).tolist()) <= {5, 6, 7}
    assert {5, 6, 7} <= set(np.unique(amax_code[s > 0]).tolist())          # all three occur


def test_error_bound_and_zero_block():
    x = data(64, 256, seed=3)
    x[5, 32:64] = 0
    p, s = mxfp4.quantize_rowwise(x)
    xv = inputs.bf16_bits_to_float(x).astype(np.float64)
    xh = mxfp4.dequantize_exact(p, s)
    X = np.repeat(F.decode_e8m0(s), 32, axis=1)
    v = np.abs(xv) / X
    half_spacing = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    assert np.all(np.abs(xh - xv) <= half_spacing * X)
    assert s[5, 1] == 0 and np.all(xh[5, 32:64] == 0)


def test_columnwise_copy_is_rowwise_copy_of_the_transpose():
    x = data(96, 64, seed=4)
    pc, sc = mxfp4.quantize_colwise(x)
    pr, sr = mxfp4.quantize_rowwise(np.ascontiguousarray(x.T))
    assert np.array_equal(pc, pr) and np.array_equal(sc, sr)
