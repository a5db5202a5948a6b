"""The library's 8-bit codebook (host side of oq_codebook: Max's shooting
method) against the oracle's (Lloyd's alternation, then Newton on the
Lloyd-Max conditions); both fp64 and independent, the library rounds to
fp32.  Plus the host validation of 8-bit calls.  CPU only: none of these
calls reaches the GPU."""
import numpy as np
import pytest

import oracle


@pytest.fixture(scope="module")
def q():
    import quantization_dit_linear_amd as q
    q.lib()
    return q


@pytest.mark.parametrize("bits", [5, 6, 7, 8])
@pytest.mark.parametrize("d", [128, 3072, 13824])
def test_library_codebook_matches_oracle(q, d, bits):
    lv, th = q.codebook(d, bits)
    rl, rt = oracle.codebook(d, bits)
    # fp32 rounding plus the shooting method's ~1e-9 (unit scale) drift
    np.testing.assert_allclose(lv, rl, rtol=1.2e-7, atol=4e-9 / np.sqrt(d))
    np.testing.assert_allclose(th, rt, rtol=1.2e-7, atol=4e-9 / np.sqrt(d))


def test_eight_bit_thresholds_rounded_like_the_oracle(q):
    """The fp32 thresholds the kernels compare against are the oracle's
    rounded to fp32, except where the two fp64 values straddle a rounding
    boundary (at most a couple of the 255)."""
    _, th = q.codebook(1, 8)
    _, rt = oracle.codebook(1, 8)
    assert np.sum(th != rt.astype(np.float32)) <= 2


def test_eight_bit_validation(q):
    L = q.lib()
    lv = np.zeros(256, np.float32)
    th = np.zeros(256, np.float32)
    # the sphere family: 1-4 and 8 bits
    assert L.oq_codebook_ex(3072, 8, q.OQ_CODEBOOK_SPHERE, lv.ctypes.data,
                            th.ctypes.data) == q.OQ_OK
    assert L.oq_codebook_ex(3072, 6, q.OQ_CODEBOOK_SPHERE, lv.ctypes.data,
                            th.ctypes.data) == q.OQ_EUNSUPPORTED
    assert L.oq_codebook_ex(3072, 9, 0, lv.ctypes.data, th.ctypes.data) == q.OQ_EUNSUPPORTED
    assert L.oq_codes_bytes(10, 3072, 8) == 10 * 3072
    # W8A8 only: mixed pairs are rejected before any device work
    assert L.oq_linear(None, None, 8, None, None, 4, 0, 0, 3072, None, None) == q.OQ_EUNSUPPORTED
    assert L.oq_linear(None, None, 4, None, None, 8, 0, 0, 3072, None, None) == q.OQ_EUNSUPPORTED
    assert L.oq_linear(None, None, 8, None, None, 8, 0, 5, 3072, None, None) == q.OQ_OK
    assert L.oq_linear(None, None, 5, None, None, 5, 0, 5, 3072, None, None) == q.OQ_EUNSUPPORTED
    assert L.oq_linear_ex(None, None, 8, None, None, 8, 0, 5, 3072, q.OQ_CODEBOOK_SPHERE, None,
                          None) == q.OQ_OK
    # rotate: 8 bits accepted in both families (empty input is a no-op)
    assert L.oq_rotate_quantize(None, q.OQ_BF16, 0, 3072, 1, 0, 8, None, None, None) == q.OQ_OK
    assert L.oq_rotate_quantize(None, q.OQ_BF16, 0, 3072, 1, q.OQ_CODEBOOK_SPHERE, 8, None, None,
                                None) == q.OQ_OK
    assert L.oq_rotate_quantize(None, q.OQ_BF16, 0, 3072, 1, 0, 6, None, None,
                                None) == q.OQ_EUNSUPPORTED
