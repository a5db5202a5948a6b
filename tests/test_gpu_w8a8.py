"""GPU parity of the 8-bit path (W8A8, the top of the bit range in the
llmdb.app summary) against the oracle: rotate-quantize to byte codes on the
bf16 fast path and the general kernel, weight preparation, fake
quantization, permuted input, and the W8A8 linear (LDS level-table decode)
on every tile path, at full size on sampled rows and end to end.
Tolerances are the ones of the lower bit widths: codes bit-exact outside a
1e-6 window around each of the 255 thresholds (at most 1e-4 of the
coordinates), norms 1e-5, linear 2e-3 relative Frobenius."""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests import parity
from tests.gpu_util import bf16_to_np, host, say, to_device

pytestmark = pytest.mark.gpu

THR8 = None


@pytest.fixture(scope="module")
def q():
    import torch
    import quantization_dit_linear_amd as q
    assert torch.cuda.is_available()
    q.lib()
    return q


def _thr():
    global THR8
    if THR8 is None:
        THR8 = oracle.codebook_unit(8)[1]
    return THR8


def _check_rows(q, x, dtype, d, seed, signs, what):
    import torch
    say("rotate_quantize 8 bits", what, x.shape, "signs", signs)
    codes, norms = q.rotate_quantize(to_device(x), seed, 8, signs=signs)
    torch.cuda.synchronize()
    assert codes.shape == (x.shape[0], d)
    rc, rn, rz = oracle.rotate_quantize(x, dtype, d, seed, 8, use_signs=signs, want_z=True)
    parity.assert_codes_match(host(codes), rc, rz, d, 8, _thr(), what)
    parity.assert_norms_match(host(norms), rn, what)


@pytest.mark.parametrize("signs", [True, False])
def test_tiny_fp32_general_kernel(q, signs):
    lin = wl.get_linear("tiny", "tiny")
    _check_rows(q, wl.activations("tiny", "tiny"), wl.F32, 256, lin.seed, signs, "tiny")


@pytest.mark.parametrize("cfg,name", [("image_qkv", "qkv"), ("image_mlp", "down"),
                                      ("video_block", "qkv"), ("video_block", "down"),
                                      ("stress", "proj")])
def test_workload_rows_fast_path(q, cfg, name):
    lin = wl.get_linear(cfg, name)
    x = wl.activations(cfg, name, np.arange(0, 300))
    _check_rows(q, x, lin.act.dtype, lin.act.d, lin.seed, True, f"{cfg}/{name}")


@pytest.mark.parametrize("d", [384, 1024, 2048, 4096, 8192, 16384])
def test_other_dimensions(q, d):
    """Fast path (1024, 2048, 4096) and the general kernel (384, 8192, 16384)."""
    x = wl.custom_activations(50, d, wl.BF16, d + 8, n_out=3, out_factor=30.0, sigma_s=1.0,
                              zero_rows=(4,))
    _check_rows(q, x, wl.BF16, d, 11, True, f"d={d}")


def test_zero_token_codes(q):
    import torch
    d = 3072
    x = wl.custom_activations(9, d, wl.BF16, 1, n_out=1, out_factor=10.0, sigma_s=1.0,
                              zero_rows=(2,))
    codes, norms = q.rotate_quantize(to_device(x), 5, 8)
    torch.cuda.synchronize()
    assert (host(codes)[2] == 128).all() and host(norms)[2] == 0


@pytest.mark.parametrize("cfg,name", [("image_qkv", "qkv"), ("video_block", "down")])
def test_weight_prep_rows(q, cfg, name):
    import torch
    lin = wl.get_linear(cfg, name)
    W = wl.weights(cfg, name)[:160]
    K = lin.weight.K
    say("prepare_weights 8 bits", cfg, name)
    codes, rn = q.prepare_weights(to_device(W), lin.seed, 8)
    torch.cuda.synchronize()
    rc, rr, rz = oracle.rotate_quantize(W, lin.weight.dtype, K, lin.seed, 8, want_z=True)
    parity.assert_codes_match(host(codes), rc, rz, K, 8, _thr(), f"W8 {cfg}/{name}")
    parity.assert_norms_match(host(rn), rr, f"W8 {cfg}/{name}")


@pytest.mark.parametrize("d,dtype", [(3072, wl.BF16), (8192, wl.BF16), (256, wl.F32)])
def test_fake_quantize(q, d, dtype):
    import torch
    x = wl.custom_activations(40, d, dtype, d + 2, n_out=2, out_factor=20.0, sigma_s=1.0)
    say("fake_quantize 8 bits", d)
    xh, norms = q.fake_quantize(to_device(x), 21, 8)
    torch.cuda.synchronize()
    ref, rn = oracle.fake_quantize(x, dtype, d, 21, 8)
    _, _, z = oracle.rotate_quantize(x, dtype, d, 21, 8, want_codes=False, want_z=True)
    parity.assert_norms_match(host(norms), rn, "fq8")
    parity.assert_dequant_match(bf16_to_np(xh), ref, z, d, _thr(), "fq8")


def test_permuted_input(q):
    import torch
    lin = wl.get_linear("image_qkv", "qkv")
    d = lin.act.d
    x = wl.activations("image_qkv", "qkv", np.arange(0, 130))
    perm, _ = oracle.plan(d, lin.seed)
    xp = np.ascontiguousarray(x[:, perm])
    say("permuted input 8 bits")
    c1, n1 = q.rotate_quantize(to_device(xp), lin.seed, 8, permuted=True)
    torch.cuda.synchronize()
    rc, rn, rz = oracle.rotate_quantize(x, lin.act.dtype, d, lin.seed, 8, want_z=True)
    parity.assert_codes_match(host(c1), rc, rz, d, 8, _thr(), "permuted 8")
    parity.assert_norms_match(host(n1), rn, "permuted 8")


def _linear(q, ac, an, wc, wn, K):
    import torch
    y = q.linear(to_device(ac), to_device(an), 8, to_device(wc), to_device(wn), 8, K)
    torch.cuda.synchronize()
    return bf16_to_np(y)


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (3, 5, 128), (200, 136, 384), (257, 129, 1152),
                                   (1000, 700, 256), (2600, 2344, 384), (7387, 2204, 512)])
def test_linear_shapes(q, M, N, K):
    """Both tile sizes (128 x 128 for the small problems, 256 x 256 from
    110 tiles on), ragged edges and a sparse last round."""
    ac, an = wl.random_codes(M, K, 8, M + 40)
    wc, wn = wl.random_codes(N, K, 8, N + 41)
    say("linear W8A8", M, N, K)
    y = _linear(q, ac, an, wc, wn, K)
    if M <= 1000:
        rows = np.arange(M)
    else:
        rows = np.unique(np.concatenate([wl.sample_rows(M, 16, 9),
                                         np.linspace(min(6144, M - 1), M - 1, 24).astype(np.int64),
                                         [0, M - 1]]))
    ref = oracle.linear(ac, an, 8, wc, wn, 8, K, rows=rows)
    assert parity.rel_fro(y[rows], ref) <= parity.LINEAR_FRO
    assert np.all(np.abs(y[rows] - ref) <= 1e-2 * np.abs(ref).max() + 1e-30)


def test_linear_full_size_sampled_rows(q):
    lin = wl.get_linear("image_qkv", "qkv")
    M, N, K = lin.act.M, lin.weight.N, lin.act.d
    ac, an = wl.random_codes(M, K, 8, 51)
    wc, wn = wl.random_codes(N, K, 8, 52)
    say("linear W8A8 full", M, N, K)
    y = _linear(q, ac, an, wc, wn, K)
    rows = wl.sample_rows(M, 24, 3)
    ref = oracle.linear(ac, an, 8, wc, wn, 8, K, rows=rows)
    assert parity.rel_fro(y[rows], ref) <= parity.LINEAR_FRO


def test_end_to_end(q):
    """x, W -> prepare, rotate-quantize, linear at 8 bits on the GPU against
    the same steps in the oracle; the quantized product is within the
    8-bit distortion of W x (relative error ~ sqrt(2 * 4.1e-5))."""
    import torch
    lin = wl.get_linear("image_qkv", "qkv")
    K = lin.act.d
    x = wl.activations("image_qkv", "qkv", np.arange(0, 200))
    W = wl.weights("image_qkv", "qkv")[:300]
    say("end-to-end W8A8")
    wc, wn = q.prepare_weights(to_device(W), lin.seed, 8)
    ac, an = q.rotate_quantize(to_device(x), lin.seed, 8)
    y = q.linear(ac, an, 8, wc, wn, 8, K)
    torch.cuda.synchronize()
    y = bf16_to_np(y)
    oac, oan, _ = oracle.rotate_quantize(x, wl.BF16, K, lin.seed, 8)
    owc, own, _ = oracle.rotate_quantize(W, wl.BF16, K, lin.seed, 8)
    ref = oracle.linear(oac, oan, 8, owc, own, 8, K)
    assert parity.rel_fro(y, ref) <= parity.LINEAR_FRO
    exact = wl.bf16_bits_to_f32(x).astype(np.float64) @ wl.bf16_bits_to_f32(W).astype(np.float64).T
    assert parity.rel_fro(y, exact) < 0.03
