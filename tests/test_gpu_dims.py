"""GPU parity for token lengths that are not multiples of 128 (d % 32 == 0):
the whole 128-coordinate groups keep the group slot order and the last 32,
64 or 96 coordinates are stored in coordinate order.  These lengths run on
the general kernel; the linear takes them when K % 64 == 0 (whole 64-slot K
steps).  Same acceptance rules as the other parity tests: codes bit-exact
outside the 1e-6 boundary window, norms and rotated values within 1e-5,
linear outputs within 2e-3 relative Frobenius of the fp64 oracle.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests import parity
from tests.gpu_util import bf16_to_np, host, say, to_device

pytestmark = pytest.mark.gpu

# (d, h = d & -d): partial last groups of 32, 64 and 96 coordinates, h from
# 32 to 64, one to 127 whole groups
DIMS = [32, 64, 96, 160, 192, 224, 320, 1088, 4160, 16352]


@pytest.fixture(scope="module")
def q():
    import torch
    import quantization_dit_linear_amd as q
    assert torch.cuda.is_available()
    q.lib()
    return q


def _sync():
    import torch
    torch.cuda.synchronize()


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_rotate_quantize_other_lengths(q, d, bits):
    """Codes, norms and rotated values of 37 tokens (one of them zero),
    bf16 input, signs on."""
    x = wl.custom_activations(37, d, wl.BF16, d + bits, n_out=max(1, d // 100),
                              out_factor=50.0, sigma_s=1.5, zero_rows=(5,))
    say("dims rotate", d, bits)
    xd = to_device(x)
    codes, norms = q.rotate_quantize(xd, 17, bits)
    z, n2 = q.rotate(xd, 17)
    _sync()
    rc, rn, rz = oracle.rotate_quantize(x, wl.BF16, d, 17, bits, want_z=True)
    thr = oracle.codebook_unit(bits)[1]
    parity.assert_codes_match(host(codes), rc, rz, d, bits, thr, f"d={d} b={bits}")
    parity.assert_norms_match(host(norms), rn, f"d={d}")
    parity.assert_norms_match(host(n2), rn, f"d={d}")
    parity.assert_rotated_match(host(z), rz, f"d={d}")
    allc = parity.unpack_codes(host(codes), d, bits)
    assert (allc[5] == 1 << (bits - 1)).all() and host(norms)[5] == 0


@pytest.mark.parametrize("d", [96, 224, 1088])
@pytest.mark.parametrize("signs", [True, False])
def test_fp32_input_and_sign_modes(q, d, signs):
    x = wl.custom_activations(21, d, wl.F32, 3 * d, n_out=2, out_factor=20.0, sigma_s=1.0)
    say("dims fp32", d, signs)
    codes, norms = q.rotate_quantize(to_device(x), 5, 4, signs=signs)
    _sync()
    rc, rn, rz = oracle.rotate_quantize(x, wl.F32, d, 5, 4, use_signs=signs, want_z=True)
    parity.assert_codes_match(host(codes), rc, rz, d, 4, oracle.codebook_unit(4)[1], f"d={d}")
    parity.assert_norms_match(host(norms), rn, f"d={d}")


@pytest.mark.parametrize("d", [96, 160, 4160])
def test_fake_quantize_other_lengths(q, d):
    """Fake quantization writes every coordinate in coordinate order, the
    partial group's included."""
    x = wl.custom_activations(30, d, wl.BF16, d + 11, n_out=2, out_factor=30.0, sigma_s=1.0,
                              zero_rows=(3,))
    say("dims fake quant", d)
    xh, norms = q.fake_quantize(to_device(x), 7, 3)
    _sync()
    ref, rn = oracle.fake_quantize(x, wl.BF16, d, 7, 3)
    _, _, z = oracle.rotate_quantize(x, wl.BF16, d, 7, 3, want_codes=False, want_z=True)
    parity.assert_norms_match(host(norms), rn, f"d={d}")
    parity.assert_dequant_match(bf16_to_np(xh), ref, z, d, oracle.codebook_unit(3)[1], f"d={d}")


@pytest.mark.parametrize("d", [96, 1088])
def test_permuted_input_other_lengths(q, d):
    """Rows permuted by oq_permute_rows (a producer's output rows) then
    rotated with OQ_ROT_INPUT_PERMUTED give the oracle's codes."""
    import torch
    x = wl.custom_activations(19, d, wl.BF16, d + 2, n_out=2, out_factor=20.0, sigma_s=1.0)
    perm, _ = oracle.plan(d, 9)
    say("dims permute rows", d)
    # the permutation acts on the coordinates: permute the rows of x^T
    xt = to_device(np.ascontiguousarray(x.T))
    xpt = q.permute_rows(xt, 9)
    _sync()
    got_t = host(xpt.view(torch.int16)).view(np.uint16)
    np.testing.assert_array_equal(got_t, x.T[perm])
    xp = np.ascontiguousarray(got_t.T)
    c, n = q.rotate_quantize(to_device(xp), 9, 4, permuted=True)
    _sync()
    rc, rn, rz = oracle.rotate_quantize(x, wl.BF16, d, 9, 4, want_z=True)
    parity.assert_codes_match(host(c), rc, rz, d, 4, oracle.codebook_unit(4)[1], "permuted")
    parity.assert_norms_match(host(n), rn, "permuted")


@pytest.mark.parametrize("K", [64, 192, 320, 1088])
@pytest.mark.parametrize("ba,bw", [(4, 4), (4, 3), (3, 2), (2, 4), (8, 8)])
def test_linear_whole_k_steps(q, K, ba, bw):
    """K % 128 == 64: the last K step holds a partial group's 64 slots in
    coordinate order; ragged M and N, every kind of decode."""
    M, N = 300, 136
    ac, an = wl.random_codes(M, K, ba, K + ba)
    wc, wn = wl.random_codes(N, K, bw, K + 10 * bw)
    say("dims linear", M, N, K, ba, bw)
    import torch
    y = q.linear(to_device(ac), to_device(an), ba, to_device(wc), to_device(wn), bw, K)
    torch.cuda.synchronize()
    got = bf16_to_np(y)
    ref = oracle.linear(ac, an, ba, wc, wn, bw, K)
    assert parity.rel_fro(got, ref) <= parity.LINEAR_FRO
    assert np.all(np.abs(got - ref) <= 1e-2 * np.abs(ref).max() + 1e-30)


@pytest.mark.parametrize("K", [192, 4160])
def test_end_to_end_other_lengths(q, K):
    """Weights prepared and tokens rotated by the library, then its linear,
    against the oracle's own pipeline on the same inputs."""
    import torch
    M, N, seed = 77, 200, 31
    x = wl.custom_activations(M, K, wl.BF16, K + 1, n_out=2, out_factor=30.0, sigma_s=1.0)
    rng = np.random.default_rng(K)
    W = wl.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    say("dims end to end", M, N, K)
    wc, wn = q.prepare_weights(to_device(W), seed, 4)
    ac, an = q.rotate_quantize(to_device(x), seed, 4)
    y = q.linear(ac, an, 4, wc, wn, 4, K)
    torch.cuda.synchronize()
    rwc, rwn, rwz = oracle.rotate_quantize(W, wl.BF16, K, seed, 4, want_z=True)
    rac, ran, raz = oracle.rotate_quantize(x, wl.BF16, K, seed, 4, want_z=True)
    thr = oracle.codebook_unit(4)[1]
    parity.assert_codes_match(host(wc), rwc, rwz, K, 4, thr, "weights")
    parity.assert_norms_match(host(wn), rwn, "weight norms")
    parity.assert_codes_match(host(ac), rac, raz, K, 4, thr, "activations")
    # the linear against the oracle's linear of the library's own codes
    ref = oracle.linear(host(ac), host(an).astype(np.float64), 4, host(wc),
                        host(wn).astype(np.float64), 4, K)
    assert parity.rel_fro(bf16_to_np(y), ref) <= parity.LINEAR_FRO


@pytest.mark.parametrize("d", [384, 3072, 4096, 5120, 13824])
def test_non_finite_tokens_leave_the_others_alone(q, d):
    """Non-finite tokens give unspecified codes and no error; every other
    token of the same call (same workgroup batches included) still matches
    the oracle.  Rows 3, 7 and 11 carry a NaN, a +Inf, and a -Inf with a
    NaN; row 15 is finite but its sum of squares overflows fp32."""
    import torch
    x = wl.custom_activations(20, d, wl.BF16, d + 7, n_out=2, out_factor=20.0, sigma_s=1.0)
    x = x.copy()
    x[3, 5] = 0x7FC0          # NaN
    x[7, d - 1] = 0x7F80      # +Inf
    x[11, 0] = 0xFF80         # -Inf
    x[11, d // 2] = 0x7FC0
    x[15, :] = wl.f32_to_bf16_bits(np.full(d, 1e30, np.float32))
    bad = [3, 7, 11, 15]
    good = np.array([r for r in range(20) if r not in bad])
    say("non-finite tokens", d)
    xd = to_device(x)
    codes, norms = q.rotate_quantize(xd, 13, 4)
    z, _ = q.rotate(xd, 13)
    _sync()
    rc, rn, rz = oracle.rotate_quantize(x[good], wl.BF16, d, 13, 4, want_z=True)
    thr = oracle.codebook_unit(4)[1]
    parity.assert_codes_match(host(codes)[good], rc, rz, d, 4, thr, f"d={d}")
    parity.assert_norms_match(host(norms)[good], rn, f"d={d}")
    parity.assert_rotated_match(host(z)[good], rz, f"d={d}")
    # the linear: a non-finite norm spoils its own output row only -- the
    # other rows are bit-identical to the same call with a finite norm,
    # which itself matches the oracle
    ac, an = wl.random_codes(6, d, 4, 3)
    wc, wn = wl.random_codes(512, d, 4, 4)
    an_nan = an.copy()
    an_nan[2] = np.nan
    y = bf16_to_np(q.linear(to_device(ac), to_device(an), 4, to_device(wc), to_device(wn), 4, d))
    y_nan = bf16_to_np(q.linear(to_device(ac), to_device(an_nan), 4, to_device(wc),
                                to_device(wn), 4, d))
    torch.cuda.synchronize()
    keep = np.array([0, 1, 3, 4, 5])
    assert np.array_equal(y_nan[keep], y[keep])
    assert not np.isfinite(y_nan[2]).any()
    ref = oracle.linear(ac, an, 4, wc, wn, 4, d)
    assert parity.rel_fro(y, ref) <= parity.LINEAR_FRO


@pytest.mark.parametrize("d,bits", [(96, 4), (160, 2), (224, 8), (4160, 3)])
def test_sphere_family_other_lengths(q, d, bits):
    """The exact-sphere codebook family at lengths with a partial last group
    (its thresholds depend on d), codes and norms against the oracle."""
    x = wl.custom_activations(23, d, wl.BF16, d + 5 * bits, n_out=2, out_factor=30.0,
                              sigma_s=1.0, zero_rows=(4,))
    say("dims sphere", d, bits)
    c, n = q.rotate_quantize(to_device(x), 29, bits, sphere=True)
    _sync()
    rc, rn, rz = oracle.rotate_quantize(x, wl.BF16, d, 29, bits, want_z=True, sphere=True)
    _, th, _ = oracle.codebook_sphere(d, bits)
    parity.assert_codes_match(host(c), rc, rz, d, bits, np.asarray(th) * np.sqrt(d), f"d={d}")
    parity.assert_norms_match(host(n), rn, f"d={d}")


@pytest.mark.parametrize("K,bw,ba", [(192, 4, 4), (1088, 2, 4), (320, 8, 8)])
def test_sphere_linear_whole_k_steps(q, K, bw, ba):
    """The sphere family through the linear at K % 128 == 64, end to end:
    the library's weight and activation codes against the oracle's linear
    of the same codes."""
    import torch
    M, N, seed = 70, 150, 37
    x = wl.custom_activations(M, K, wl.BF16, K + 3, n_out=2, out_factor=20.0, sigma_s=1.0)
    rng = np.random.default_rng(K + bw)
    W = wl.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    say("dims sphere linear", K, bw, ba)
    wc, wn = q.prepare_weights(to_device(W), seed, bw, sphere=True)
    ac, an = q.rotate_quantize(to_device(x), seed, ba, sphere=True)
    y = bf16_to_np(q.linear(ac, an, ba, wc, wn, bw, K, sphere=True))
    torch.cuda.synchronize()
    ref = oracle.linear(host(ac), host(an).astype(np.float64), ba, host(wc),
                        host(wn).astype(np.float64), bw, K, sphere=True)
    assert parity.rel_fro(y, ref) <= parity.LINEAR_FRO
