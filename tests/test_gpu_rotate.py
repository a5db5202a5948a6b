"""GPU parity of oq_rotate_quantize / oq_prepare_weights against the oracle.

Codes bit-exact except within 1e-6 of a decision boundary (at most 1e-4 of
coordinates), norms and rotated values within 1e-5 relative -- on the same
seeded inputs, across the five workload shapes, all bit widths and both
sign modes, plus edge cases (zero tokens, one token, ragged counts, empty
input).
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests import parity
from tests.gpu_util import host, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch
    import quantization_dit_linear_amd as q
    assert torch.cuda.is_available()
    q.lib()
    return q


def _thr(bits):
    return oracle.codebook_unit(bits)[1]


def _check_rows(q, x, dtype, d, seed, bits, signs, what):
    say(what, x.shape, "bits", bits, "signs", signs)
    xd = to_device(x)
    codes, norms = q.rotate_quantize(xd, seed, bits, signs=signs)
    z_gpu, n2 = q.rotate(xd, seed, signs=signs)
    import torch
    torch.cuda.synchronize()
    rc, rn, rz = oracle.rotate_quantize(x, dtype, d, seed, bits, use_signs=signs, want_z=True)
    n_mis = parity.assert_codes_match(host(codes), rc, rz, d, bits, _thr(bits), what)
    parity.assert_norms_match(host(norms), rn, what)
    parity.assert_norms_match(host(n2), rn, what)
    parity.assert_rotated_match(host(z_gpu), rz, what)
    return n_mis


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("signs", [True, False])
def test_tiny_config_full(q, bits, signs):
    lin = wl.get_linear("tiny", "tiny")
    x = wl.activations("tiny", "tiny")
    _check_rows(q, x, wl.F32, 256, lin.seed, bits, signs, "tiny")


CASES = [("image_qkv", "qkv", 4), ("image_mlp", "up", 4), ("image_mlp", "down", 4),
         ("video_block", "qkv", 4), ("video_block", "down", 4),
         ("stress", "proj", 3), ("stress", "proj", 4), ("video_block", "up", 2)]


@pytest.mark.parametrize("cfg,name,bits", CASES)
@pytest.mark.parametrize("signs", [True, False])
def test_workload_rows(q, cfg, name, bits, signs):
    """A few hundred rows of every workload activation: several workgroup
    batches plus a ragged tail."""
    lin = wl.get_linear(cfg, name)
    rows = np.arange(0, 300, dtype=np.int64)
    x = wl.activations(cfg, name, rows)
    _check_rows(q, x, lin.act.dtype, lin.act.d, lin.seed, bits, signs, f"{cfg}/{name}")


def test_zero_tokens_and_single_token(q):
    import torch
    d = 3072
    x = wl.custom_activations(37, d, wl.BF16, 5, n_out=30, out_factor=50.0, sigma_s=1.0,
                              zero_rows=(0, 5, 36))
    _check_rows(q, x, wl.BF16, d, 99, 4, True, "zero-tokens")
    say("zero token codes")
    codes, norms = q.rotate_quantize(to_device(x), 99, 4)
    torch.cuda.synchronize()
    allc = parity.unpack_codes(host(codes), d, 4)
    assert (allc[[0, 5, 36]] == 8).all() and (host(norms)[[0, 5, 36]] == 0).all()
    _check_rows(q, x[3:4], wl.BF16, d, 99, 4, True, "single-token")


def test_empty_input_is_noop(q):
    import torch
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    say("empty")
    codes, norms = q.rotate_quantize(x, 1, 4)
    torch.cuda.synchronize()
    assert codes.shape == (0, 128) and norms.shape == (0,)


@pytest.mark.parametrize("d", [128, 384, 640, 1024, 1152, 2048, 4096, 8192, 16384])
def test_other_dimensions(q, d):
    """Block sizes 128..16384 and odd block counts."""
    x = wl.custom_activations(70, d, wl.BF16, d, n_out=3, out_factor=30.0, sigma_s=1.0)
    _check_rows(q, x, wl.BF16, d, 7, 4, True, f"d={d}")


@pytest.mark.parametrize("cfg,name,bits", [("tiny", "tiny", 4), ("image_qkv", "qkv", 4),
                                           ("image_mlp", "down", 2), ("video_block", "down", 3)])
def test_weight_prep_rows(q, cfg, name, bits):
    import torch
    lin = wl.get_linear(cfg, name)
    W = wl.weights(cfg, name)[:200]
    K = lin.weight.K
    say("prepare_weights", cfg, name, W.shape)
    codes, rn = q.prepare_weights(to_device(W), lin.seed, bits)
    torch.cuda.synchronize()
    rc, rr, rz = oracle.rotate_quantize(W, lin.weight.dtype, K, lin.seed, bits, want_z=True)
    parity.assert_codes_match(host(codes), rc, rz, K, bits, _thr(bits), f"W {cfg}/{name}")
    parity.assert_norms_match(host(rn), rr, f"W {cfg}/{name}")


# every activation (config, linear, A bits) the workloads name
FULL = sorted({(cfg, lin.name, ba) for cfg in wl.CONFIGS if cfg != "tiny"
               for lin in wl.CONFIGS[cfg]["linears"] for _, ba in lin.bit_pairs})


@pytest.mark.parametrize("cfg,name,bits", FULL)
def test_full_size_sampled_rows(q, cfg, name, bits):
    """The whole activation matrix at its real size, in the launch the
    benchmark times; the oracle checks a seeded sample of rows."""
    import torch
    lin = wl.get_linear(cfg, name)
    d = lin.act.d
    x = wl.activations(cfg, name)
    say("full", cfg, name, x.shape)
    xd = to_device(x)
    codes, norms = q.rotate_quantize(xd, lin.seed, bits)
    torch.cuda.synchronize()
    rows = wl.sample_rows(lin.act.M, 96, 1)
    rc, rn, rz = oracle.rotate_quantize(x[rows], lin.act.dtype, d, lin.seed, bits, want_z=True)
    parity.assert_codes_match(host(codes)[rows], rc, rz, d, bits, _thr(bits), f"{cfg}/{name}")
    parity.assert_norms_match(host(norms)[rows], rn, f"{cfg}/{name}")


def test_explicit_plan_handles(q):
    """oq_plan_create / oq_plan_destroy: results are the same with a pinned
    plan, after it is freed (rebuilt lazily), and with two handles."""
    import torch
    d = 3072
    x = wl.custom_activations(20, d, wl.BF16, 77, n_out=2, out_factor=20.0, sigma_s=1.0)
    xd = to_device(x)
    say("plan handles")
    with q.Plan(d, 1234):
        c1, n1 = q.rotate_quantize(xd, 1234, 4)
        torch.cuda.synchronize()
    c2, n2 = q.rotate_quantize(xd, 1234, 4)
    torch.cuda.synchronize()
    p1, p2 = q.Plan(d, 1234), q.Plan(d, 1234)
    p1.close()
    c3, _ = q.rotate_quantize(xd, 1234, 4)
    torch.cuda.synchronize()
    p2.close()
    assert torch.equal(c1, c2) and torch.equal(c1, c3) and torch.equal(n1, n2)
    rc, rn, rz = oracle.rotate_quantize(x, wl.BF16, d, 1234, 4, want_z=True)
    parity.assert_codes_match(host(c1), rc, rz, d, 4, _thr(4), "plan handles")


# every weight (config, linear, W bits) the workloads name
FULL_W = sorted({(cfg, lin.name, bw) for cfg in wl.CONFIGS if cfg != "tiny"
                 for lin in wl.CONFIGS[cfg]["linears"] for bw, _ in lin.bit_pairs})


@pytest.mark.parametrize("cfg,name,bits", FULL_W)
def test_weight_prep_full_size_sampled_rows(q, cfg, name, bits):
    """The whole weight matrix prepared at once; a seeded sample of rows
    checked against the oracle."""
    import torch
    lin = wl.get_linear(cfg, name)
    K, N = lin.weight.K, lin.weight.N
    W = wl.weights(cfg, name)
    say("prepare_weights full", cfg, name, W.shape, bits)
    codes, rn = q.prepare_weights(to_device(W), lin.seed, bits)
    torch.cuda.synchronize()
    rows = wl.sample_rows(N, 64, 4)
    rc, rr, rz = oracle.rotate_quantize(W[rows], lin.weight.dtype, K, lin.seed, bits, want_z=True)
    parity.assert_codes_match(host(codes)[rows], rc, rz, K, bits, _thr(bits), f"W {cfg}/{name}")
    parity.assert_norms_match(host(rn)[rows], rr, f"W {cfg}/{name}")


@pytest.mark.parametrize("cfg,name,bits", [("image_qkv", "qkv", 4), ("tiny", "tiny", 4),
                                           ("video_block", "down", 8)])
def test_rotate_quantize_in_a_hip_graph(q, cfg, name, bits):
    """rotate+quantize (the bf16 fast kernel, and the general kernel for the
    fp32 tiny workload) captured in a HIP graph: every replay, with eager
    work and synchronisations in between, gives the eager codes and norms
    bit for bit."""
    import torch
    lin = wl.get_linear(cfg, name)
    x = to_device(wl.activations(cfg, name, np.arange(0, min(lin.act.M, 256))))
    say("rotate graph", cfg, name, bits)
    c0, n0 = q.rotate_quantize(x, lin.seed, bits)
    torch.cuda.synchronize()
    rc, rn = c0.clone(), n0.clone()
    c, n = torch.empty_like(c0), torch.empty_like(n0)
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        q.rotate_quantize(x, lin.seed, bits, out=c, norms=n)
    for _ in range(3):
        c.fill_(0xAB)
        n.fill_(-1.0)
        q.rotate_quantize(x, lin.seed, bits, out=c0, norms=n0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(c, rc) and torch.equal(n, rn)
        assert torch.equal(c0, rc) and torch.equal(n0, rn)


def _rotated_basis_token(d, seed, ks, coefs):
    """A token whose rotation is sum_j coefs[j] e_{ks[j]} (before bf16
    rounding of x): in rotation order y = sum_j c_j H_h e_k / sqrt(h), and
    x_{pi(i)} = D_i y_i undoes the permutation and the signs."""
    perm, sign = oracle.plan(d, seed)
    h = oracle.block_size(d)
    i = np.arange(h)
    y = np.zeros(d)
    for k, c in zip(ks, coefs):
        b0, kk = (k // h) * h, k % h
        par = np.array([bin(v).count("1") & 1 for v in (i & kk)])
        y[b0:b0 + h] += c * (1.0 - 2.0 * par) / np.sqrt(h)
    x = np.zeros(d)
    x[perm] = sign * y
    return x


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("d", [1024, 2048, 3072, 4096, 5120, 12288, 13824])
def test_rotated_basis_tokens(q, d, bits):
    """Tokens whose energy lands on one or a few rotated coordinates, so
    sqrt(d) z reaches +-sqrt(d), far outside the central Lloyd-Max cells:
    the codes there must be the extreme ones, as the oracle says."""
    seed = 31
    h = oracle.block_size(d)
    other = h + 1 if d > h else 1
    rows = [([5], [1.0]), ([d - 1], [-3.0]), ([0, other], [0.8, 0.6]),
            ([7, 9, 11], [0.9, -0.3, 0.3]), ([d // 2], [1e-3]), ([d - 2, 3], [-0.6, 0.8])]
    x = np.stack([_rotated_basis_token(d, seed, ks, cs) for ks, cs in rows])
    rng = np.random.default_rng(d + bits)
    x = np.concatenate([x, rng.standard_normal((3, d))]).astype(np.float32)
    xb = wl.f32_to_bf16_bits(x)
    _check_rows(q, xb, wl.BF16, d, seed, bits, True, f"basis d={d} b={bits}")
    import torch
    codes, _ = q.rotate_quantize(to_device(xb), seed, bits)
    torch.cuda.synchronize()
    c = parity.unpack_codes(host(codes), d, bits)
    top = (1 << bits) - 1
    assert c[0, 5] == top and c[1, d - 1] == 0, "extreme coordinates take the extreme codes"
