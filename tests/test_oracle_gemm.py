"""Pins for the GEMM pass criterion (CPU only).

The criterion is the normwise relative error ||C - C_ref||_F / ||C_ref||_F of the
output against the FP64 reference, with an all-zero reference demanding an
exactly zero output. Pinned by hand-computed Frobenius norms (so a swapped
denominator, a missing square root or a wrong zero-reference branch fails).
"""

import math

import numpy as np

from oracle import gemm


def test_normwise_error_hand_worked():
    # C = [[1, 0], [0, 0]] against C_ref = I2: ||C - C_ref|| = 1, ||C_ref|| = sqrt(2)
    assert gemm.normwise_rel_err(np.array([[1.0, 0.0], [0.0, 0.0]]), np.eye(2)) == 1.0 / math.sqrt(2.0)
    # the denominator is the reference's norm, not the output's: swapped it is 1 / 1
    assert gemm.normwise_rel_err(np.eye(2), np.array([[1.0, 0.0], [0.0, 0.0]])) == 1.0
    # a 3-4-5 triangle: ||[0, 0.5]|| / ||[3, 4]|| = 0.5 / 5
    assert gemm.normwise_rel_err(np.array([[3.0, 4.5]]), np.array([[3.0, 4.0]])) == 0.1
    # Frobenius, not a max or an L1 norm: error [1, 1, 1, 1] over [2, 0, 0, 0] is 2 / 2
    assert gemm.normwise_rel_err(np.array([[3.0, 1.0], [1.0, 1.0]]), np.array([[2.0, 0.0], [0.0, 0.0]])) == 1.0


def test_zero_reference_needs_an_exactly_zero_output():
    z = np.zeros((3, 2))
    assert gemm.normwise_rel_err(z, z) == 0.0
    assert gemm.normwise_rel_err(-z, z) == 0.0                  # -0 is zero
    c = z.copy()
    c[1, 1] = 1e-300
    assert gemm.normwise_rel_err(c, z) == math.inf
    assert not gemm.normwise_rel_err(c, z) <= gemm.GEMM_RTOL


def test_float32_inputs_are_compared_in_fp64():
    # 1 + 2^-24 is not an FP32 value, but the FP64 difference of FP32 inputs is exact
    c = np.array([1.0 + 2.0 ** -23], dtype=np.float32)
    r = np.array([1.0], dtype=np.float32)
    assert gemm.normwise_rel_err(c, r) == 2.0 ** -23


def test_tiny_and_huge_entries_do_not_underflow_the_norms():
    # squares of 1e-200 underflow FP64; the ratio must still be the scale-free one
    r = np.array([[3.0, 4.0]]) * 1e-200
    c = np.array([[3.0, 4.5]]) * 1e-200
    assert abs(gemm.normwise_rel_err(c, r) - 0.1) < 1e-15
    big = 1e300                                   # squares of 3e300 overflow FP64
    assert abs(gemm.normwise_rel_err(c * 1e200 * big, r * 1e200 * big) - 0.1) < 1e-15
