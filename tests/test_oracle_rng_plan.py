"""Pins for the oracle's rotation plan: SplitMix64 stream, permutation Pi,
Rademacher signs D, block size h.

Pages: pith.science, Supplementary A setup (y = P_pi x, D_j Rademacher,
d = k h); paper.gecl.asia notes, Key Insight (h is the largest power-of-two
block).  The pages give no RNG, so Pi is pinned through the generator's
published outputs, the bijection property and the uniformity of the shuffle.
"""
import itertools
import os

import numpy as np
import pytest
from scipy import stats

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden_sm64():
    vals = []
    with open(os.path.join(GOLD, "splitmix64_seed0.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                vals.append(int(line, 16))
    return vals


def test_splitmix64_published_outputs():
    assert oracle.splitmix64(0, 4) == _golden_sm64()


@pytest.mark.parametrize("d,h", [(256, 256), (3072, 1024), (5120, 1024), (12288, 4096),
                                 (13824, 512), (384, 128), (160, 32), (65536, 65536)])
def test_block_size_is_largest_power_of_two(d, h):
    got = oracle.block_size(d)
    assert got == h
    assert d % got == 0 and (d // got) % 2 == 1


@pytest.mark.parametrize("d", [128, 256, 3072, 13824])
def test_plan_is_bijection_with_pm1_signs(d):
    perm, sign = oracle.plan(d, 1234)
    assert sorted(perm.tolist()) == list(range(d))
    assert set(np.unique(sign).tolist()) <= {-1, 1}
    # roughly half the signs are negative (binomial, 6 sigma)
    n_neg = int((sign < 0).sum())
    assert abs(n_neg - d / 2) < 6 * np.sqrt(d / 4) + 1


def test_plan_reproducible_and_seed_dependent():
    p1, s1 = oracle.plan(3072, 21)
    p2, s2 = oracle.plan(3072, 21)
    p3, s3 = oracle.plan(3072, 22)
    assert np.array_equal(p1, p2) and np.array_equal(s1, s2)
    assert not np.array_equal(p1, p3)


def test_shuffle_is_uniform_over_all_permutations():
    """Durstenfeld with j uniform on [0, i] reaches all d! orders with equal
    probability; an off-by-one (Sattolo, j in [0, i)) only reaches the
    (d-1)! cyclic ones.  Chi-square over 24000 seeds at d = 4."""
    d = 4
    perms = list(itertools.permutations(range(d)))
    index = {p: i for i, p in enumerate(perms)}
    counts = np.zeros(len(perms))
    n = 24000
    for seed in range(n):
        p, _ = oracle.plan(d, seed)
        counts[index[tuple(p.tolist())]] += 1
    assert (counts > 0).all()
    chi2 = ((counts - n / 24) ** 2 / (n / 24)).sum()
    assert stats.chi2.sf(chi2, df=23) > 1e-4


def test_signs_follow_the_permutation_draws():
    """The sign of coordinate i is the top bit of SplitMix64 draw (d-1)+i:
    the shuffle consumes the first d-1 draws."""
    d = 128
    draws = oracle.splitmix64(77, (d - 1) + d)
    _, sign = oracle.plan(d, 77)
    expect = np.array([-1 if (r >> 63) else 1 for r in draws[d - 1:]], dtype=np.int8)
    assert np.array_equal(sign, expect)
