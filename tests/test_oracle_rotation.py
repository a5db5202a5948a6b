"""Pins for the oracle's RPBH rotation: normalise, permute, sign, block
Walsh-Hadamard.

Pages: pith.science Supplementary A setup (d = k h, y = P_pi x,
z^(j) = H_h D_j y^(j), (H_h)_li = +-1/sqrt(h)); paper.gecl.asia notes,
Method items 1, 2, 4 (norm kept apart; W Pi^T and Pi x cancel); pith.science
Figure 2 / Figure 3 captions (rotated coordinates follow f_d ~ N(0,1/d)).
Pinned against: SciPy's Sylvester Hadamard matrix, H H^T = h I, norm
preservation, R^T R = I, the exact fold cancellation (W R^T)(R x) = W x,
basis-vector structure, the exact sphere marginal for Gaussian inputs, and
a Kolmogorov-Smirnov gate on workload-shaped inputs.
"""
import numpy as np
import pytest
from scipy import linalg, stats

import oracle
import workloads as wl


@pytest.mark.parametrize("h", [2, 4, 32, 256, 1024])
def test_fwht_matches_scipy_sylvester_hadamard(h):
    rng = np.random.default_rng(h)
    v = rng.standard_normal(h)
    H = linalg.hadamard(h).astype(np.float64)
    assert np.allclose(oracle.fwht(v), H @ v, rtol=0, atol=1e-10 * np.sqrt(h))


@pytest.mark.parametrize("h", [1, 2, 8, 64, 256])
def test_hadamard_entries_are_orthogonal(h):
    H = np.array([[oracle.hadamard_entry(a, b) for b in range(h)] for a in range(h)], np.float64)
    assert np.array_equal(H @ H.T, h * np.eye(h))
    assert np.array_equal(H, linalg.hadamard(h))


def _rot_matrix(d, seed, use_signs=True):
    perm, sign = oracle.plan(d, seed)
    R = np.empty((d, d))
    for j in range(d):
        e = np.zeros(d)
        e[j] = 1.0
        R[:, j], nrm = oracle.rotate_token(e, perm, sign, use_signs)
        assert nrm == 1.0
    return R


@pytest.mark.parametrize("d,use_signs", [(384, True), (384, False), (256, True), (640, True),
                                          (96, True), (160, False), (224, True)])
def test_rotation_is_orthogonal(d, use_signs):
    R = _rot_matrix(d, 5, use_signs)
    assert np.allclose(R.T @ R, np.eye(d), rtol=0, atol=1e-13)


@pytest.mark.parametrize("d,seed", [(3072, 21), (160, 4), (4160, 8)])
def test_basis_vector_spreads_over_one_block(d, seed):
    h = oracle.block_size(d)
    perm, sign = oracle.plan(d, seed)
    inv = np.argsort(perm)
    for m in (0, 17, d - 1):
        e = np.zeros(d)
        e[m] = 1.0
        z, _ = oracle.rotate_token(e, perm, sign)
        nz = np.nonzero(z)[0]
        blk = inv[m] // h
        assert nz.min() == blk * h and nz.max() == blk * h + h - 1 and nz.size == h
        assert np.allclose(np.abs(z[nz]), 1 / np.sqrt(h), rtol=1e-15)


@pytest.mark.parametrize("d", [256, 3072, 13824, 96, 4160])
def test_norm_preserved_and_zero_token(d):
    perm, sign = oracle.plan(d, 3)
    rng = np.random.default_rng(d)
    x = rng.standard_normal(d) * 7.0
    z, nrm = oracle.rotate_token(x, perm, sign)
    assert abs(nrm - np.linalg.norm(x)) < 1e-12 * nrm
    assert abs(np.linalg.norm(z) - 1.0) < 1e-13
    assert abs(np.mean(z * z) - 1.0 / d) < 1e-15
    z0, n0 = oracle.rotate_token(np.zeros(d), perm, sign)
    assert n0 == 0.0 and not z0.any()


@pytest.mark.parametrize("d,use_signs", [(384, True), (3072, True), (3072, False), (224, True),
                                         (4160, False)])
def test_weight_fold_cancels_exactly(d, use_signs):
    """Unquantised, rows of W Pi^T times Pi x give W x: here each weight row
    and the token go through the oracle's own rotation (norm kept apart)."""
    perm, sign = oracle.plan(d, 9)
    rng = np.random.default_rng(1)
    W = rng.standard_normal((16, d)) * 0.02
    x = rng.standard_normal(d)
    zx, sx = oracle.rotate_token(x, perm, sign, use_signs)
    y = np.empty(16)
    for i in range(16):
        zw, rw = oracle.rotate_token(W[i], perm, sign, use_signs)
        y[i] = rw * sx * np.dot(zw, zx)
    ref = W @ x
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-13 * np.abs(ref).max())


def test_gaussian_token_has_exact_sphere_marginal():
    """A standard Gaussian vector is rotation invariant, so after
    normalisation every coordinate is that of a uniform unit vector:
    z_i^2 ~ Beta(1/2, (d-1)/2) exactly."""
    d, n = 3072, 64
    perm, sign = oracle.plan(d, 21)
    rng = np.random.default_rng(2)
    zs = [oracle.rotate_token(rng.standard_normal(d), perm, sign)[0] for _ in range(n)]
    z2 = np.concatenate(zs) ** 2
    res = stats.kstest(z2, stats.beta(0.5, (d - 1) / 2).cdf)
    assert res.statistic < 0.01


GATED = [("image_qkv", "qkv"), ("image_mlp", "up"), ("image_mlp", "down"),
         ("video_block", "qkv"), ("video_block", "down")]


@pytest.mark.parametrize("cfg,name", GATED)
def test_marginal_gate_on_workload_inputs(cfg, name):
    """Outlier-laden workload inputs, after rotation, follow N(0, 1/d):
    KS(sqrt(d) z, N(0,1)) <= 0.02 pooled over 64 tokens."""
    lin = wl.get_linear(cfg, name)
    d = lin.act.d
    rows = wl.sample_rows(lin.act.M, 64, 3)
    x = wl.activations(cfg, name, rows)
    _, _, z = oracle.rotate_quantize(x, lin.act.dtype, d, lin.seed, 4, want_codes=False,
                                     want_z=True)
    z = z[np.linalg.norm(z, axis=1) > 0]
    ks = stats.kstest((np.sqrt(d) * z).ravel(), "norm").statistic
    assert ks <= 0.02


@pytest.mark.parametrize("cfg,name", [("tiny", "tiny"), ("stress", "proj")])
def test_marginal_reported_for_extreme_inputs(cfg, name):
    """Inputs with extreme single-coordinate energy (the pages' stated
    limitation) are reported, not gated: the statistic is only bounded."""
    lin = wl.get_linear(cfg, name)
    d = lin.act.d
    rows = wl.sample_rows(lin.act.M, 64, 3)
    x = wl.activations(cfg, name, rows)
    _, _, z = oracle.rotate_quantize(x, lin.act.dtype, d, lin.seed, 4, want_codes=False,
                                     want_z=True)
    z = z[np.linalg.norm(z, axis=1) > 0]
    ks = stats.kstest((np.sqrt(d) * z).ravel(), "norm").statistic
    print(f"{cfg}/{name}: KS = {ks:.4f}")
    assert ks < 0.1


def test_signs_flag_changes_only_signs_before_hadamard():
    d = 384
    perm, sign = oracle.plan(d, 4)
    rng = np.random.default_rng(5)
    x = rng.standard_normal(d)
    z_on, _ = oracle.rotate_token(x, perm, sign, True)
    flipped = x.copy()
    # applying D to the gathered vector equals flipping x at the source index
    flipped[perm] = flipped[perm] * sign
    z_off, _ = oracle.rotate_token(flipped, perm, sign, False)
    assert np.allclose(z_on, z_off, rtol=0, atol=1e-15)
