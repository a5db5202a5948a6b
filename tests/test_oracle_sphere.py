"""Pins of the oracle's exact-sphere-marginal codebook (the closed-form
marginal of one coordinate of a uniform point on S^{d-1}, which the
pith.science referee asks for; its Gaussian limit N(0, 1/d) is the one the
pages use).

* d = 3: the marginal is uniform on [-1, 1] (Archimedes), so the Lloyd-Max
  quantizer is the uniform one with levels -1 + (2k+1)/L;
* large d: the codebook tends to Max's Gaussian one scaled by 1/sqrt(d),
  monotonically, with the relative gaps 0.8% (d=256), 0.07% (d=3072) and
  0.015% (d=13824) at 4 bits;
* cell masses of the oracle's incomplete beta against SciPy's numerical
  integration of the density c_d (1 - t^2)^((d-3)/2);
* the centroid condition for every cell, by SciPy quadrature;
* antisymmetry;
* 8 bits (where Lloyd's alternation is followed by Newton's method): the
  d = 3 uniform quantizer, every centroid condition, antisymmetry, and a
  gap to the Gaussian codebook that shrinks like 1/d (the marginal's
  first-order correction to N(0, 1/d) is O(1/d)).
"""
import math

import numpy as np
import pytest
from scipy import integrate

import oracle


def _density(d):
    lc = math.lgamma(d / 2) - 0.5 * math.log(math.pi) - math.lgamma((d - 1) / 2)
    c = math.exp(lc)
    return lambda t: c * (1.0 - t * t) ** ((d - 3) / 2)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_d3_is_the_uniform_quantizer(bits):
    L = 1 << bits
    lv, th, _ = oracle.codebook_sphere(3, bits)
    np.testing.assert_allclose(lv, -1 + (2 * np.arange(L) + 1) / L, atol=1e-12)
    np.testing.assert_allclose(th, -1 + 2 * np.arange(1, L) / L, atol=1e-12)


def test_gaussian_limit():
    ul, _, _ = oracle.codebook_unit(4)
    gaps = []
    for d in (256, 3072, 13824):
        lv, _, _ = oracle.codebook_sphere(d, 4)
        gaps.append(np.max(np.abs(lv * math.sqrt(d) - ul) / np.abs(ul)))
    assert gaps[0] > gaps[1] > gaps[2]
    np.testing.assert_allclose(gaps, [0.0081, 0.00068, 0.00015], rtol=0.1)


@pytest.mark.parametrize("d", [5, 256, 3072])
def test_cell_masses_against_quadrature(d):
    f = _density(d)
    s = 1 / math.sqrt(d)
    for a, b in [(-1.0, 1.0), (0.0, 0.5 * s), (0.3 * s, 2.1 * s), (-3 * s, -1 * s),
                 (2.5 * s, 1.0)]:
        a, b = max(a, -1.0), min(b, 1.0)  # the support is [-1, 1]
        if a >= b:
            assert oracle.sphere_mass(a, b, d) == 0.0
            continue
        pts = [p for p in (0.0,) if a < p < b]
        ref, _ = integrate.quad(f, a, b, epsabs=1e-14, epsrel=1e-12, limit=200, points=pts or None)
        assert abs(oracle.sphere_mass(a, b, d) - ref) <= 1e-11 * max(ref, 1e-3), (a, b)


@pytest.mark.parametrize("d,bits", [(5, 3), (256, 4), (3072, 2), (256, 8), (3072, 8)])
def test_centroid_condition(d, bits):
    f = _density(d)
    lv, th, _ = oracle.codebook_sphere(d, bits)
    edges = np.concatenate([[-1.0], th, [1.0]])
    for k in range(lv.size):
        a, b = edges[k], edges[k + 1]
        m, _ = integrate.quad(f, a, b, epsabs=1e-15, epsrel=1e-12, limit=200)
        mu, _ = integrate.quad(lambda t: t * f(t), a, b, epsabs=1e-15, epsrel=1e-12, limit=200)
        assert abs(mu / m - lv[k]) <= 1e-9 / math.sqrt(d), (k, mu / m, lv[k])
    np.testing.assert_allclose(th, 0.5 * (lv[1:] + lv[:-1]), rtol=0, atol=1e-15)


def test_antisymmetric():
    lv, th, _ = oracle.codebook_sphere(384, 4)
    np.testing.assert_allclose(lv, -lv[::-1], atol=1e-15)
    np.testing.assert_allclose(th, -th[::-1], atol=1e-15)
    # 8 bits: Newton stops at the incomplete beta's rounding noise
    for d in (384, 13824):
        lv, th, _ = oracle.codebook_sphere(d, 8)
        np.testing.assert_allclose(lv, -lv[::-1], atol=1e-11)
        np.testing.assert_allclose(th, -th[::-1], atol=1e-11)
        assert np.all(np.diff(lv) > 0)


def test_gaussian_limit_8bit_scales_like_one_over_d():
    ul, _, _ = oracle.codebook_unit(8)
    ds = (256, 3072, 13824)
    gaps = []
    for d in ds:
        lv, _, _ = oracle.codebook_sphere(d, 8)
        gaps.append(np.max(np.abs(lv * math.sqrt(d) - ul) / np.abs(ul)))
    assert gaps[0] > gaps[1] > gaps[2]
    for i in range(2):
        ratio = gaps[i] / gaps[i + 1]
        assert abs(ratio / (ds[i + 1] / ds[i]) - 1) < 0.15, (gaps, ratio)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
def test_codebooks_are_exactly_symmetric(bits):
    """Both densities are even, so their Lloyd-Max quantizers are symmetric:
    c_{L-1-k} = -c_k exactly and the middle threshold is 0, so a zero token
    takes code 2^(b-1) at every bit width (the Newton refinement above 4
    bits must not leave a rounding asymmetry behind)."""
    r = oracle.codebook_unit(bits)
    lv, th = np.asarray(r[0]), np.asarray(r[1])
    assert np.array_equal(lv, -lv[::-1]) and th[len(th) // 2] == 0.0
    for d in (3, 96, 3072):
        lvs, ths, _ = oracle.codebook_sphere(d, bits)
        lvs, ths = np.asarray(lvs), np.asarray(ths)
        assert np.array_equal(lvs, -lvs[::-1]) and ths[len(ths) // 2] == 0.0
    x = np.zeros((2, 224), np.float32)
    for sphere in (False, True):
        codes, norms, _ = oracle.rotate_quantize(x, oracle.F32, 224, 5, bits, sphere=sphere)
        assert (oracle.unpack_row(codes[0], 224, bits) == 1 << (bits - 1)).all()
