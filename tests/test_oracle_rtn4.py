"""Pins of the oracle's INT4 weight-only round-to-nearest (the AdaLN
modulation projections: paper.gecl.asia notes, Method item 5).

Closed-form properties rather than a retyped formula: the error bound of
round-to-nearest (half a step), the row maximum landing exactly on +-7,
exact reconstruction of rows that lie on the grid, ties going to the even
level, zero rows, and the projection of a one-hot activation being the
dequantized weight column.
"""
import numpy as np
import pytest

import oracle
import workloads as wl


def _rows(seed, n, d, scale=0.02):
    return (np.random.default_rng(seed).standard_normal((n, d)) * scale).astype(np.float32)


def test_error_bound_and_range():
    W = _rows(1, 64, 384)
    W[3, 7] = 0.9  # an outlier row
    q, s = oracle.rtn4_quantize(W, wl.F32, 384)
    assert q.min() >= -7 and q.max() <= 7
    err = np.abs(W.astype(np.float64) - q * s[:, None].astype(np.float64))
    assert np.all(err <= 0.5 * s[:, None] * (1 + 1e-6) + 1e-12)
    # the largest |w| of every row maps to +-7
    idx = np.argmax(np.abs(W), axis=1)
    assert np.all(np.abs(q[np.arange(64), idx]) == 7)


def test_rows_on_the_grid_reconstruct_exactly():
    ks = np.array([-7, -3, 0, 1, 5, 7] * 32, np.float32)
    W = np.stack([ks * c for c in (0.25, 0.5, 2.0, 0.125)]).astype(np.float32)
    q, s = oracle.rtn4_quantize(W, wl.F32, W.shape[1])
    np.testing.assert_array_equal(q, np.broadcast_to(ks.astype(np.int8), q.shape))
    np.testing.assert_array_equal(q * s[:, None], W)


def test_ties_go_to_even():
    # amax = 7 makes the step 1: w = k + 0.5 is an exact tie in fp32
    row = np.array([7.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 6.5] + [0.0] * 120, np.float32)
    q, s = oracle.rtn4_quantize(row[None, :], wl.F32, row.size)
    assert s[0] == 1.0
    np.testing.assert_array_equal(q[0, :8], [7, 0, 2, 2, 0, -2, -2, 6])


def test_zero_rows():
    W = np.zeros((2, 128), np.float32)
    q, s = oracle.rtn4_quantize(W, wl.F32, 128)
    assert np.all(q == 0) and np.all(s == 0)


def test_linear_of_one_hot_is_the_dequantized_column():
    W = wl.f32_to_bf16_bits(_rows(5, 40, 256))
    q, s = oracle.rtn4_quantize(W, wl.BF16, 256)
    x = np.zeros((3, 256), np.float32)
    x[0, 0] = 1.0
    x[1, 17] = -2.0
    x[2, 255] = 0.5
    y = oracle.rtn4_linear(x, wl.F32, q, s)
    np.testing.assert_array_equal(y[0], q[:, 0] * s.astype(np.float64))
    np.testing.assert_array_equal(y[1], -2.0 * q[:, 17] * s.astype(np.float64))
    np.testing.assert_array_equal(y[2], 0.5 * q[:, 255] * s.astype(np.float64))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_linear_against_dequantized_gemm(dt):
    """Brute force on small shapes (numpy's GEMM as the primitive)."""
    W = _rows(7, 48, 512)
    x = np.random.default_rng(8).standard_normal((5, 512)).astype(np.float32)
    if dt == "bf16":
        W, x = wl.f32_to_bf16_bits(W), wl.f32_to_bf16_bits(x)
        Wf, xf, code = wl.bf16_bits_to_f32(W), wl.bf16_bits_to_f32(x), wl.BF16
    else:
        Wf, xf, code = W, x, wl.F32
    q, s = oracle.rtn4_quantize(W, code, 512)
    y = oracle.rtn4_linear(x, code, q, s)
    ref = xf.astype(np.float64) @ (q * s[:, None].astype(np.float64)).T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    # quantization error against the unquantized product stays small
    exact = xf.astype(np.float64) @ Wf.astype(np.float64).T
    assert np.linalg.norm(y - exact) / np.linalg.norm(exact) < 0.15
