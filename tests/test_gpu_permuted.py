"""Folding the rotation permutation into the producer: oq_permute_rows and
rotate-quantize with OQ_ROT_INPUT_PERMUTED.  Rows permuted by the plan's
pi give, with the flag, exactly the outputs of the unpermuted rows without
it; the permutation is checked against the oracle's plan (paper.gecl.asia
notes, Limitations: the run-time cost of the rotation)."""
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


@pytest.mark.parametrize("d,cols,dtype", [(3072, 256, "bf16"), (12288, 96, "f32"),
                                          (384, 1, "bf16"), (256, 3, "u8")])
def test_permute_rows_matches_oracle_plan(q, d, cols, dtype):
    """dst row i = src row pi(i): weight rows, a bias vector (2-byte rows),
    odd row sizes (1-byte elements, 3 per row)."""
    import torch
    rng = np.random.default_rng(d + cols)
    if dtype == "bf16":
        src = wl.f32_to_bf16_bits(rng.standard_normal((d, cols)).astype(np.float32))
    elif dtype == "f32":
        src = rng.standard_normal((d, cols)).astype(np.float32)
    else:
        src = rng.integers(0, 256, (d, cols), dtype=np.uint8)
    perm, _ = oracle.plan(d, 99)
    say("permute_rows", d, cols, dtype)
    out = q.permute_rows(to_device(src), 99)
    torch.cuda.synchronize()
    if dtype == "bf16":
        got = host(out.view(torch.int16)).view(np.uint16)
    else:
        got = host(out)
    np.testing.assert_array_equal(got, src[perm])


def _codes(q, x, seed, bits, signs, permuted):
    import torch
    c, n = q.rotate_quantize(to_device(x), seed, bits, signs=signs, permuted=permuted)
    torch.cuda.synchronize()
    return host(c), host(n)


@pytest.mark.parametrize("cfg,name,bits", [("image_qkv", "qkv", 4), ("image_mlp", "down", 4),
                                           ("video_block", "down", 3), ("video_block", "qkv", 2)])
@pytest.mark.parametrize("signs", [True, False])
def test_permuted_input_same_codes(q, cfg, name, bits, signs):
    lin = wl.get_linear(cfg, name)
    d = lin.act.d
    x = wl.activations(cfg, name, np.arange(0, 130))
    perm, _ = oracle.plan(d, lin.seed)
    xp = np.ascontiguousarray(x[:, perm])
    say("permuted input", cfg, name, bits, signs)
    c0, n0 = _codes(q, x, lin.seed, bits, signs, False)
    c1, n1 = _codes(q, xp, lin.seed, bits, signs, True)
    rc, rn, rz = oracle.rotate_quantize(x, lin.act.dtype, d, lin.seed, bits, use_signs=signs,
                                        want_z=True)
    parity.assert_codes_match(c1, rc, rz, d, bits, oracle.codebook_unit(bits)[1], "permuted")
    parity.assert_norms_match(n1, rn, "permuted")
    # the same values reach the same positions; only the fp32 sum of squares
    # runs in another order, so the norms agree to rounding and a code can
    # differ only where it sits on a decision boundary (checked above)
    np.testing.assert_allclose(n1, n0, rtol=2e-6)
    assert (c1 != c0).sum() <= parity.CODE_MAX_FRAC * c0.size


@pytest.mark.parametrize("d,dtype", [(256, "f32"), (8192, "bf16")])
def test_permuted_input_general_kernel(q, d, dtype):
    """fp32 input and d = 8192 run on the general kernel."""
    if dtype == "f32":
        x = wl.custom_activations(24, d, wl.F32, 5, n_out=2, out_factor=20.0, sigma_s=1.0)
        dt = wl.F32
    else:
        x = wl.custom_activations(24, d, wl.BF16, 6, n_out=2, out_factor=20.0, sigma_s=1.0)
        dt = wl.BF16
    perm, _ = oracle.plan(d, 3)
    xp = np.ascontiguousarray(x[:, perm])
    say("permuted general", d, dtype)
    c1, n1 = _codes(q, xp, 3, 4, True, True)
    rc, rn, rz = oracle.rotate_quantize(x, dt, d, 3, 4, want_z=True)
    parity.assert_codes_match(c1, rc, rz, d, 4, oracle.codebook_unit(4)[1], "permuted general")
    parity.assert_norms_match(n1, rn, "permuted general")


def test_permuted_input_fake_quant(q):
    import torch
    lin = wl.get_linear("image_qkv", "qkv")
    d = lin.act.d
    x = wl.activations("image_qkv", "qkv", np.arange(40))
    perm, _ = oracle.plan(d, lin.seed)
    xp = np.ascontiguousarray(x[:, perm])
    say("permuted fake quant")
    a, _ = q.fake_quantize(to_device(x), lin.seed, 4)
    xd = to_device(xp)
    b = torch.empty_like(a)
    nb = torch.empty((xd.shape[0],), dtype=torch.float32, device=xd.device)
    rc = q.lib().oq_rotate_quantize(q._dev_ptr(xd, "x"), q.OQ_BF16, xd.shape[0], d, lin.seed,
                                    q.OQ_OUT_BF16_DEQUANT | q.OQ_ROT_INPUT_PERMUTED, 4,
                                    q._dev_ptr(b, "out"), q._dev_ptr(nb, "n"), q._stream(None))
    assert rc == 0
    torch.cuda.synchronize()
    ga, gb = bf16_to_np(a), bf16_to_np(b)
    assert (ga != gb).sum() <= parity.CODE_MAX_FRAC * ga.size
