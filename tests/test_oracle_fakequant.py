"""Pins of the oracle's fake quantization (dequantized rotated tokens, the
pages' evaluation path: paper.gecl.asia notes, Dataset/Evaluation).

* distortion: for Gaussian tokens the rotated coordinates are (up to the
  sphere's finite-d correction) N(0, 1/d), so the mean squared
  reconstruction error per unit norm is Max's tabulated MSE of the
  Lloyd-Max quantizer (tests/golden/lloyd_max_gaussian.txt);
* centroid condition: an MSE-optimal quantizer's error is orthogonal to its
  output on average, so E||x_hat||^2 / s^2 = 1 - MSE;
* the values agree with the packed codes of the same tokens, level by
  level, through the storage order;
* a GEMM of fake-quantized activations and weights is the oracle's low-bit
  linear;
* zero tokens reconstruct to zero.
"""
import os

import numpy as np
import pytest

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lloyd_max_gaussian.txt")


def _max_mse():
    out = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        parts = [p.strip() for p in line.split("|")]
        out[int(parts[0])] = float(parts[3])
    return out


def _gauss(rows, d, seed):
    return np.random.default_rng(seed).standard_normal((rows, d)).astype(np.float32)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_distortion_matches_max_table(bits):
    d, rows = 1024, 384
    x = _gauss(rows, d, 100 + bits)
    xh, s = oracle.fake_quantize(x, wl.F32, d, 5, bits)
    _, _, z = oracle.rotate_quantize(x, wl.F32, d, 5, bits, want_codes=False, want_z=True)
    err = np.sum((s[:, None] * z - xh) ** 2, axis=1) / s ** 2
    mse = _max_mse()[bits]
    assert abs(err.mean() / mse - 1) < 0.02, (err.mean(), mse)


@pytest.mark.parametrize("bits", [2, 4])
def test_centroid_condition(bits):
    d, rows = 1024, 384
    x = _gauss(rows, d, 200 + bits)
    xh, s = oracle.fake_quantize(x, wl.F32, d, 9, bits)
    energy = np.sum(xh ** 2, axis=1) / s ** 2
    assert abs(energy.mean() - (1 - _max_mse()[bits])) < 0.02 * _max_mse()[bits] + 2e-3


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_values_follow_the_codes(bits):
    d = 384
    x = wl.custom_activations(40, d, wl.BF16, 3, n_out=4, out_factor=30.0, sigma_s=1.0)
    xh, s = oracle.fake_quantize(x, wl.BF16, d, 17, bits)
    codes, s2, _ = oracle.rotate_quantize(x, wl.BF16, d, 17, bits)
    lv, _ = oracle.codebook(d, bits)
    for r in range(x.shape[0]):
        natural = oracle.unpack_row(codes[r], d, bits)
        np.testing.assert_array_equal(xh[r], s[r] * lv[natural])
    np.testing.assert_array_equal(s, s2)


def test_gemm_of_fake_quantized_operands_is_the_linear():
    K = 256
    x = wl.activations("tiny", "tiny")
    W = wl.weights("tiny", "tiny")
    seed = wl.get_linear("tiny", "tiny").seed
    xh, _ = oracle.fake_quantize(x, wl.F32, K, seed, 4)
    wh, _ = oracle.fake_quantize(W, wl.F32, K, seed, 3)
    ac, an, _ = oracle.rotate_quantize(x, wl.F32, K, seed, 4)
    wc, wn, _ = oracle.rotate_quantize(W, wl.F32, K, seed, 3)
    y = oracle.linear(ac, an, 4, wc, wn, 3, K)
    np.testing.assert_allclose(xh @ wh.T, y, rtol=1e-12, atol=1e-12 * np.abs(y).max())


def test_zero_tokens():
    x = np.zeros((3, 256), np.float32)
    xh, s = oracle.fake_quantize(x, wl.F32, 256, 1, 4)
    assert np.all(s == 0) and np.all(xh == 0)
