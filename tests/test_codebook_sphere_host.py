"""The library's exact-sphere codebook (oq_codebook_ex with
OQ_CODEBOOK_SPHERE: Gauss-Legendre masses and Max's shooting method on the
host) against the oracle's (incomplete beta and Lloyd's iteration); both
are fp64 and independent, the library rounds to fp32.  CPU only."""
import numpy as np
import pytest

import oracle


@pytest.fixture(scope="module")
def q():
    import quantization_dit_linear_amd as q
    q.lib()
    return q


@pytest.mark.parametrize("d", [128, 256, 3072, 5120, 12288, 13824, 16384])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_library_sphere_codebook_matches_oracle(q, d, bits):
    lv, th = q.codebook(d, bits, sphere=True)
    rl, rt, _ = oracle.codebook_sphere(d, bits)
    np.testing.assert_allclose(lv, rl, rtol=2e-7, atol=1e-9 / np.sqrt(d))
    np.testing.assert_allclose(th, rt, rtol=2e-7, atol=1e-9 / np.sqrt(d))


@pytest.mark.parametrize("d", [128, 256, 3072, 5120, 12288, 13824, 16384])
def test_library_sphere_codebook_8bit(q, d):
    """8 bits: the library runs Newton from the Gaussian codebook, the
    oracle Lloyd then Newton from it; at 8 bits the Lloyd-Max conditions
    pin the levels only to about 1e-7 sigma in double precision (one nearly
    flat direction), so the two agree to that, which stays well inside the
    1e-6 window around each threshold that the code parity exempts."""
    lv, th = q.codebook(d, 8, sphere=True)
    rl, rt, _ = oracle.codebook_sphere(d, 8)
    s = np.sqrt(d)
    window = 1e-6 * np.maximum(np.abs(rt * s), 1.0)
    assert np.max(np.abs(th.astype(np.float64) * s - rt * s) / window) <= 0.8
    np.testing.assert_allclose(lv * s, rl * s, rtol=0, atol=1e-6)
    assert np.all(np.diff(lv) > 0)


def test_family_flag_validation(q):
    import ctypes
    lv = np.zeros(16, np.float32)
    th = np.zeros(16, np.float32)
    L = q.lib()
    assert L.oq_codebook_ex(3072, 4, 1 << 7, lv.ctypes.data, th.ctypes.data) == q.OQ_EINVAL
    assert L.oq_codebook_ex(3000, 4, q.OQ_CODEBOOK_SPHERE, lv.ctypes.data,
                            th.ctypes.data) == q.OQ_EUNSUPPORTED
    # the Gaussian family stays defined for any d
    assert L.oq_codebook_ex(3000, 4, 0, lv.ctypes.data, th.ctypes.data) == q.OQ_OK
