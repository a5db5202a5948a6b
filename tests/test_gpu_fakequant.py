"""GPU parity of the fake-quantization output (OQ_OUT_BF16_DEQUANT: bf16
s * level[code] at every rotated coordinate) against the oracle, and the
quality of the quantized product it gives -- the pages' own evaluation
path (paper.gecl.asia notes, Dataset/Evaluation)."""
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


def _check(q, x, dtype, d, seed, bits, signs, what):
    import torch
    say("fake_quantize", what, x.shape, "bits", bits, "signs", signs)
    xh, norms = q.fake_quantize(to_device(x), seed, bits, signs=signs)
    torch.cuda.synchronize()
    ref, rn = oracle.fake_quantize(x, dtype, d, seed, bits, use_signs=signs)
    _, _, z = oracle.rotate_quantize(x, dtype, d, seed, bits, use_signs=signs, want_codes=False,
                                     want_z=True)
    parity.assert_norms_match(host(norms), rn, what)
    parity.assert_dequant_match(bf16_to_np(xh), ref, z, d, oracle.codebook_unit(bits)[1], what)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("signs", [True, False])
def test_tiny_fp32(q, bits, signs):
    lin = wl.get_linear("tiny", "tiny")
    _check(q, wl.activations("tiny", "tiny"), wl.F32, 256, lin.seed, bits, signs, "tiny")


@pytest.mark.parametrize("cfg,name,bits", [("image_qkv", "qkv", 4), ("image_mlp", "down", 4),
                                           ("video_block", "qkv", 4), ("video_block", "down", 3),
                                           ("stress", "proj", 2)])
def test_workload_rows(q, cfg, name, bits):
    lin = wl.get_linear(cfg, name)
    x = wl.activations(cfg, name, np.arange(0, 150))
    _check(q, x, lin.act.dtype, lin.act.d, lin.seed, bits, True, f"{cfg}/{name}")


@pytest.mark.parametrize("d", [384, 2048, 8192])
def test_other_dimensions(q, d):
    """Block sizes on the fast path (2048) and on the general kernel (384, 8192)."""
    x = wl.custom_activations(40, d, wl.BF16, d + 1, n_out=3, out_factor=30.0, sigma_s=1.0,
                              zero_rows=(7,))
    _check(q, x, wl.BF16, d, 3, 4, True, f"d={d}")


@pytest.mark.parametrize("bw,ba", [(4, 4), (2, 4)])
def test_quality_of_fake_quantized_product(q, bw, ba):
    """image_qkv rows: the fake-quantized product on the GPU has the same
    error against the exact product x W^T as the oracle's (fp64), and
    matches the native low-bit linear up to bf16 operand rounding."""
    import torch
    lin = wl.get_linear("image_qkv", "qkv")
    K = lin.act.d
    rows = wl.sample_rows(lin.act.M, 64, 11)
    x = wl.activations("image_qkv", "qkv", rows)
    W = wl.weights("image_qkv", "qkv")[:512]
    say("quality", bw, ba)
    xh, _ = q.fake_quantize(to_device(x), lin.seed, ba)
    wh, _ = q.fake_quantize(to_device(W), lin.seed, bw)
    y_fq = (xh.float() @ wh.float().t()).cpu().numpy().astype(np.float64)
    ac, an = q.rotate_quantize(to_device(x), lin.seed, ba)
    wc, wn = q.prepare_weights(to_device(W), lin.seed, bw)
    y_lin = bf16_to_np(q.linear(ac, an, ba, wc, wn, bw, K))
    torch.cuda.synchronize()
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    wf = wl.bf16_bits_to_f32(W).astype(np.float64)
    exact = xf @ wf.T
    oxh, _ = oracle.fake_quantize(x, lin.act.dtype, K, lin.seed, ba)
    owh, _ = oracle.fake_quantize(W, lin.weight.dtype, K, lin.seed, bw)
    err_ref = parity.rel_fro(oxh @ owh.T, exact)
    err_gpu = parity.rel_fro(y_fq, exact)
    say("rel error vs exact: gpu", err_gpu, "oracle", err_ref)
    assert abs(err_gpu - err_ref) <= 2e-3 * max(err_ref, 1e-3) + 1e-4
    # an MSE quantizer's product error stays near sqrt(D_a + D_w) (Max's MSE)
    mse = {2: 0.1175, 3: 0.03454, 4: 0.009497}
    assert err_ref < 1.5 * np.sqrt(mse[ba] + mse[bw])
    assert parity.rel_fro(y_fq, y_lin) <= 4e-3
