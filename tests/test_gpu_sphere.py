"""GPU parity with the exact-sphere-marginal codebook family
(OQ_CODEBOOK_SPHERE): rotate-quantize on the fast and general kernels,
weight preparation, the linear (oq_linear_ex) and fake quantization,
against the oracle run with the same family."""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests import parity
from tests.gpu_util import bf16_to_np, host, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch
    import quantization_dit_linear_amd as q
    assert torch.cuda.is_available()
    q.lib()
    return q


def _thr_unit(d, bits):
    _, th, _ = oracle.codebook_sphere(d, bits)
    return th * np.sqrt(d)


@pytest.mark.parametrize("cfg,name,bits", [("image_qkv", "qkv", 4), ("image_mlp", "down", 3),
                                           ("video_block", "down", 2), ("tiny", "tiny", 4),
                                           ("image_qkv", "qkv", 8), ("video_block", "down", 8),
                                           ("tiny", "tiny", 8)])
def test_rotate_quantize_sphere(q, cfg, name, bits):
    import torch
    lin = wl.get_linear(cfg, name)
    d = lin.act.d
    x = wl.activations(cfg, name, np.arange(0, min(lin.act.M, 120)))
    say("sphere rotate", cfg, name, bits)
    c, n = q.rotate_quantize(to_device(x), lin.seed, bits, sphere=True)
    torch.cuda.synchronize()
    rc, rn, rz = oracle.rotate_quantize(x, lin.act.dtype, d, lin.seed, bits, want_z=True,
                                        sphere=True)
    parity.assert_codes_match(host(c), rc, rz, d, bits, _thr_unit(d, bits), "sphere")
    parity.assert_norms_match(host(n), rn, "sphere")


def test_sphere_codes_differ_from_gaussian_where_expected(q):
    """The families differ only where a coordinate falls between the two
    codebooks' thresholds: a small, nonzero fraction at d = 256."""
    import torch
    x = wl.activations("tiny", "tiny")
    cs, _ = q.rotate_quantize(to_device(x), 11, 4, sphere=True)
    cg, _ = q.rotate_quantize(to_device(x), 11, 4)
    torch.cuda.synchronize()
    a, b = parity.unpack_codes(host(cs), 256, 4), parity.unpack_codes(host(cg), 256, 4)
    frac = float((a != b).mean())
    assert 0 < frac < 0.05
    assert np.abs(a.astype(int) - b.astype(int)).max() == 1


@pytest.mark.parametrize("bw,ba", [(4, 4), (2, 4), (8, 8)])
def test_linear_sphere(q, bw, ba):
    import torch
    lin = wl.get_linear("image_qkv", "qkv")
    K = lin.act.d
    x = wl.activations("image_qkv", "qkv", np.arange(96))
    W = wl.weights("image_qkv", "qkv")[:160]
    say("sphere linear", bw, ba)
    wc, wn = q.prepare_weights(to_device(W), lin.seed, bw, sphere=True)
    ac, an = q.rotate_quantize(to_device(x), lin.seed, ba, sphere=True)
    y = bf16_to_np(q.linear(ac, an, ba, wc, wn, bw, K, sphere=True))
    torch.cuda.synchronize()
    owc, own, _ = oracle.rotate_quantize(W, lin.weight.dtype, K, lin.seed, bw, sphere=True)
    oac, oan, _ = oracle.rotate_quantize(x, lin.act.dtype, K, lin.seed, ba, sphere=True)
    # the linear on the GPU's own codes against the oracle's linear on the same codes
    ref_same = oracle.linear(host(ac), host(an), ba, host(wc), host(wn), bw, K, sphere=True)
    assert parity.rel_fro(y, ref_same) <= parity.LINEAR_FRO
    ref = oracle.linear(oac, oan, ba, owc, own, bw, K, sphere=True)
    assert parity.rel_fro(y, ref) <= parity.LINEAR_FRO


def test_fake_quant_sphere(q):
    import torch
    lin = wl.get_linear("image_qkv", "qkv")
    d = lin.act.d
    x = wl.activations("image_qkv", "qkv", np.arange(48))
    say("sphere fake quant")
    xh, n = q.fake_quantize(to_device(x), lin.seed, 4, sphere=True)
    torch.cuda.synchronize()
    codes, rn, z = oracle.rotate_quantize(x, lin.act.dtype, d, lin.seed, 4, want_z=True,
                                          sphere=True)
    lv, _, _ = oracle.codebook_sphere(d, 4)
    ref = np.stack([rn[r] * lv[oracle.unpack_row(codes[r], d, 4)] for r in range(x.shape[0])])
    parity.assert_dequant_match(bf16_to_np(xh), ref, z, d, _thr_unit(d, 4), "sphere fq")
