"""Pins for the oracle's Lloyd-Max codebook C_{d,b}.

Pages: paper.gecl.asia notes, Core Idea and Method item 3 (Lloyd-Max
codebook on f_d ~ N(0,1/d), depends only on d and b); pith.science
Figure 2 caption (C_{d,b} per dimension); references Lloyd 1982 and Max 1960.
Pinned against: Max's published table (tests/golden), the 1-bit closed form
sqrt(2/pi), the centroid and midpoint conditions evaluated by SciPy
quadrature (an independent numerical route), symmetry and local optimality.
"""
import os

import numpy as np
import pytest
from scipy import integrate, stats

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _max_table():
    rows = {}
    with open(os.path.join(GOLD, "lloyd_max_gaussian.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            b, lv, th, mse = [s.strip() for s in line.split("|")]
            rows[int(b)] = ([float(v) for v in lv.split()], [float(v) for v in th.split()],
                            float(mse))
    return rows


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_matches_max_1960_table(bits):
    lv, th, _ = oracle.codebook_unit(bits)
    tl, tt, tmse = _max_table()[bits]
    L = 1 << bits
    assert np.allclose(lv[L // 2:], tl, atol=1.5e-3, rtol=0)
    assert np.allclose(th[L // 2 - 1:], tt, atol=1.5e-3, rtol=0)
    assert abs(oracle.codebook_mse(bits, lv, th) - tmse) < 2e-3 * tmse


def test_one_bit_closed_form():
    lv, th, _ = oracle.codebook_unit(1)
    assert abs(lv[1] - np.sqrt(2 / np.pi)) < 1e-14
    assert abs(lv[0] + np.sqrt(2 / np.pi)) < 1e-14
    assert th[0] == 0.0


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_symmetry_and_midpoints(bits):
    lv, th, _ = oracle.codebook_unit(bits)
    L = 1 << bits
    assert np.all(np.diff(lv) > 0)
    for k in range(L):
        assert abs(lv[k] + lv[L - 1 - k]) < 1e-13
    assert np.allclose(th, 0.5 * (lv[:-1] + lv[1:]), atol=0, rtol=1e-15)
    assert th[L // 2 - 1] == pytest.approx(0.0, abs=1e-14)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_levels_are_cell_centroids_by_quadrature(bits):
    lv, th, _ = oracle.codebook_unit(bits)
    L = 1 << bits
    edges = np.concatenate([[-np.inf], th, [np.inf]])
    for k in range(L):
        a, b = edges[k], edges[k + 1]
        m, _ = integrate.quad(stats.norm.pdf, a, b, epsabs=1e-14, epsrel=1e-13)
        mu, _ = integrate.quad(lambda t: t * stats.norm.pdf(t), a, b, epsabs=1e-14, epsrel=1e-13)
        assert abs(mu / m - lv[k]) < 1e-9


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_mse_closed_form_agrees_with_quadrature_and_is_locally_optimal(bits):
    lv, th, _ = oracle.codebook_unit(bits)

    def mse_q(levels):
        t = 0.5 * (levels[:-1] + levels[1:])
        edges = np.concatenate([[-np.inf], t, [np.inf]])
        tot = 0.0
        for k in range(len(levels)):
            v, _ = integrate.quad(lambda x: (x - levels[k]) ** 2 * stats.norm.pdf(x),
                                  edges[k], edges[k + 1], epsabs=1e-14, epsrel=1e-12)
            tot += v
        return tot

    base = mse_q(lv)
    assert abs(oracle.codebook_mse(bits, lv, th) - base) < 1e-10
    for k in range(len(lv)):
        for eps in (1e-3, -1e-3):
            p = lv.copy()
            p[k] += eps
            p = np.sort(p)
            assert mse_q(p) > base


@pytest.mark.parametrize("d", [256, 3072, 13824])
def test_dimension_scaling(d):
    for bits in (2, 4):
        lu, tu, _ = oracle.codebook_unit(bits)
        ld, td = oracle.codebook(d, bits)
        assert np.allclose(ld, lu / np.sqrt(d), rtol=1e-15, atol=0)
        assert np.allclose(td, tu / np.sqrt(d), rtol=1e-15, atol=0)


# ---- 5 to 8 bits (W8A8 is the top of the pages' bit range: llmdb.app
# summary).  No page prints these codebooks; they are pinned by the two
# Lloyd-Max conditions evaluated by quadrature (a log-concave density has
# exactly one quantizer meeting both, Fleischer 1964), by symmetry, and by
# the Panter-Dite high-resolution distortion (sqrt(3) pi / 2) 4^-b.


@pytest.mark.parametrize("bits", [5, 8])
def test_high_rate_levels_are_cell_centroids_by_quadrature(bits):
    lv, th, _ = oracle.codebook_unit(bits)
    L = 1 << bits
    assert np.all(np.diff(lv) > 0)
    assert np.max(np.abs(lv + lv[::-1])) < 1e-12
    assert np.allclose(th, 0.5 * (lv[:-1] + lv[1:]), atol=0, rtol=1e-15)
    edges = np.concatenate([[-np.inf], th, [np.inf]])
    worst = 0.0
    for k in range(L):
        a, b = edges[k], edges[k + 1]
        m, _ = integrate.quad(stats.norm.pdf, a, b, epsabs=1e-16, epsrel=1e-13)
        mu, _ = integrate.quad(lambda t: t * stats.norm.pdf(t), a, b, epsabs=1e-16,
                               epsrel=1e-13)
        worst = max(worst, abs(mu / m - lv[k]))
    assert worst < 1e-8


def test_eight_bit_distortion_against_panter_dite():
    pd = np.sqrt(3.0) * np.pi / 2.0
    ratios = []
    for bits in (5, 6, 7, 8):
        lv, th, _ = oracle.codebook_unit(bits)
        ratios.append(oracle.codebook_mse(bits, lv, th) * 4.0 ** bits / pd)
    # below the asymptote and approaching it monotonically from below
    assert all(0.9 < r < 1.0 for r in ratios)
    assert all(a < b for a, b in zip(ratios, ratios[1:]))
    assert ratios[-1] > 0.985


def test_eight_bit_codebook_is_a_local_minimum():
    """Moving any one of a few levels (inner, middle, outer) raises the
    distortion, by quadrature over the affected cells only."""
    lv, th, _ = oracle.codebook_unit(8)

    def local_mse(levels, lo, hi):
        t = 0.5 * (levels[:-1] + levels[1:])
        edges = np.concatenate([[-np.inf], t, [np.inf]])
        return sum(integrate.quad(lambda x: (x - levels[k]) ** 2 * stats.norm.pdf(x),
                                  edges[k], edges[k + 1], epsabs=1e-18, epsrel=1e-12)[0]
                   for k in range(lo, hi))

    for k in (0, 64, 127, 128, 200, 255):
        lo, hi = max(k - 1, 0), min(k + 2, 256)
        base = local_mse(lv, lo, hi)
        for eps in (1e-3, -1e-3):
            p = lv.copy()
            p[k] += eps
            assert local_mse(p, lo, hi) > base
