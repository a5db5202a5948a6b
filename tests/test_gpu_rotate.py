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


@pytest.mark.parametrize("M", [1, 2, 7, 513])
@pytest.mark.parametrize("bits", [2, 4])
def test_partial_last_tile_token_counts(q, M, bits):
    """d = 13824 runs one token (27 slots) per batch in 7 wave tiles, the
    last holding 3 slots: every code, norm and rotated value of 1, 2, 7 and
    513 tokens (more batches than one per workgroup for 513) against the
    oracle, so the tile's missing fourth slot never shows up in an output."""
    d = 13824
    x = wl.custom_activations(M, d, wl.BF16, d + M, n_out=max(1, d // 100), out_factor=50.0,
                              sigma_s=1.5, zero_rows=(M - 1,) if M > 2 else ())
    _check_rows(q, x, wl.BF16, d, 123, bits, True, f"d=13824 M={M}")


@pytest.mark.parametrize("M", [1, 3, 5, 260])
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("d", [4096, 12288])
def test_split_tile_token_counts(q, d, M, bits):
    """h = 4096: each 4-slot wave tile is one Hadamard block, produced by two
    waves that each hold half of its groups.  Token counts that leave the
    last batch part-filled (1, 3, 5) and several batches per workgroup
    (260), checked code by code, with norms and rotated values, against the
    oracle, so a group handed to the wrong half or stored at the other
    half's place fails."""
    x = wl.custom_activations(M, d, wl.BF16, d + 3 * M + bits, n_out=max(1, d // 100),
                              out_factor=50.0, sigma_s=1.5, zero_rows=(M - 1,) if M > 2 else ())
    _check_rows(q, x, wl.BF16, d, 321, bits, True, f"split d={d} M={M} b={bits}")


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


# token sizes the bf16 fast kernel is built for, each at a full-size shape:
# the workload activations where one has that size, else a custom batch of
# outlier-laden tokens (token count not a multiple of the batch)
FAST_FULL = [(1024, None, None), (2048, None, None), (3072, "image_qkv", "qkv"),
             (4096, None, None), (5120, "video_block", "qkv"),
             (12288, "image_mlp", "down"), (13824, "video_block", "down")]


@pytest.mark.parametrize("d,cfg,name", FAST_FULL)
def test_rotated_values_fast_kernel_full_size(q, d, cfg, name):
    """The fp32 rotated unit vectors and norms of the bf16 fast kernel (the
    one that makes every workload's codes) at full size, checked on a seeded
    sample of rows against the oracle's fp64 z = H_h D Pi x / (s sqrt(h)):
    per token ||dz|| <= 1e-5, every |dz_i| <= 1e-5 max|z|, norms to 1e-5
    relative (pith.science, Supplementary A setup)."""
    import torch
    if cfg is None:
        M, seed = 12003, 57
        x = wl.custom_activations(M, d, wl.BF16, d + 5, n_out=max(1, d // 100),
                                  out_factor=50.0, sigma_s=1.5, zero_rows=(M - 2,))
    else:
        lin = wl.get_linear(cfg, name)
        assert lin.act.d == d
        M, seed = lin.act.M, lin.seed
        x = wl.activations(cfg, name)
    say("rotated full", d, cfg, name, x.shape)
    xd = to_device(x)
    z, n = q.rotate(xd, seed)
    torch.cuda.synchronize()
    rows = wl.sample_rows(M, 64, 3)
    if cfg is None:
        rows = np.unique(np.concatenate([rows, [M - 2]]))  # the zero token
    zs = host(z[torch.from_numpy(rows).cuda()])
    ns = host(n)[rows]
    del z
    rc, rn, rz = oracle.rotate_quantize(x[rows], wl.BF16, d, seed, 4, want_z=True)
    parity.assert_rotated_match(zs, rz, f"z d={d}")
    nz = rn > 0
    parity.assert_norms_match(ns[nz], rn[nz], f"norms d={d}")
    assert (ns[~nz] == 0).all() and (zs[~nz] == 0).all()


@pytest.mark.parametrize("d", [1024, 3072, 4096, 5120, 12288, 13824])
@pytest.mark.parametrize("signs", [True, False])
def test_rotated_values_fast_kernel_permuted_input(q, d, signs):
    """Rotated values of input already in rotation order (the fast kernel's
    scatter-free form): the same z as the unpermuted input, to fp32
    rounding, and within the tolerance of the oracle."""
    import torch
    M, seed = 203, 77
    x = wl.custom_activations(M, d, wl.BF16, d + 11, n_out=3, out_factor=40.0, sigma_s=1.0)
    perm, _ = oracle.plan(d, seed)
    say("rotated permuted", d, signs)
    z, n = q.rotate(to_device(np.ascontiguousarray(x[:, perm])), seed, signs=signs,
                    permuted=True)
    torch.cuda.synchronize()
    rc, rn, rz = oracle.rotate_quantize(x, wl.BF16, d, seed, 4, use_signs=signs, want_z=True)
    parity.assert_rotated_match(host(z), rz, f"z permuted d={d}")
    parity.assert_norms_match(host(n), rn, f"norms permuted d={d}")


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


@pytest.mark.parametrize("M", [1, 3])
@pytest.mark.parametrize("d", [13824, 12288, 4096])
def test_partial_last_tile_writes_nothing_past_the_outputs(q, d, M):
    """d = 13824: the fourth row of each token's last wave tile works on a
    copy and must store nothing; d = 12288 and 4096 (two waves per wave
    tile, several tokens per batch): a part-filled last batch must store
    nothing for its missing tokens.  Codes, fake-quantized values, rotated
    values and norms go into the front of buffers two rows longer, filled
    with a sentinel: the extra rows keep it, and the front matches a call
    into buffers of the exact size."""
    import ctypes
    import torch
    seed, bits = 123, 4
    x = to_device(wl.custom_activations(M, d, wl.BF16, d + 7, n_out=30, out_factor=50.0,
                                        sigma_s=1.0))
    say("guard rows", d, M)

    def guarded(shape, dtype):
        t = torch.empty((M + 2,) + shape, dtype=dtype, device="cuda")
        t.view(torch.uint8).fill_(0xAB)
        return t

    def untouched(t):
        return bool((t[M:].contiguous().view(torch.uint8) == 0xAB).all().item())

    codes, norms = guarded((d * bits // 8,), torch.uint8), guarded((), torch.float32)
    q.rotate_quantize(x, seed, bits, out=codes[:M], norms=norms[:M])
    c_ref, n_ref = q.rotate_quantize(x, seed, bits)
    dq, dn = guarded((d,), torch.bfloat16), guarded((), torch.float32)
    q.fake_quantize(x, seed, bits, out=dq[:M], norms=dn[:M])
    dq_ref, _ = q.fake_quantize(x, seed, bits)
    z, zn = guarded((d,), torch.float32), guarded((), torch.float32)
    rc = q.lib().oq_rotate_quantize(ctypes.c_void_p(x.data_ptr()), q.OQ_BF16, M, d, seed,
                                    q.OQ_OUT_F32_ROTATED, bits, ctypes.c_void_p(z.data_ptr()),
                                    ctypes.c_void_p(zn.data_ptr()),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    z_ref, _ = q.rotate(x, seed)
    torch.cuda.synchronize()
    for t in (codes, norms, dq, dn, z, zn):
        assert untouched(t), "a store landed past the last row"
    assert torch.equal(codes[:M], c_ref) and torch.equal(norms[:M], n_ref)
    assert torch.equal(dq[:M], dq_ref) and torch.equal(z[:M], z_ref)


@pytest.mark.parametrize("d", [1024, 3072, 5120, 12288, 13824])
def test_power_of_two_scaling_is_exact(q, d):
    """Scaling tokens by 2^k changes no code and no rotated value, and
    scales the norm by exactly 2^k (z = H D Pi x / (s sqrt(h)) is
    scale-free, and with power-of-two factors every product, sum, square
    root and reciprocal of the kernel scales exactly while nothing
    underflows).  k = -60 puts the sum of squares below 2^-64, where the
    square root runs on a rescaled sum; k = 40 keeps it below the fp32
    range limit even for the x50 outlier channels."""
    import torch
    M, seed, bits = 37, 91, 4
    x = wl.custom_activations(M, d, wl.BF16, d + 29, n_out=max(1, d // 100), out_factor=50.0,
                              sigma_s=1.0, zero_rows=(5,))
    xd = to_device(x)
    say("power-of-two scaling", d)
    c0, n0 = q.rotate_quantize(xd, seed, bits)
    z0, _ = q.rotate(xd, seed)
    for k in (-60, -40, -20, 20, 40):
        xk = (xd.float() * 2.0 ** k).to(torch.bfloat16)  # exact: bf16 keeps the mantissa
        assert torch.equal(xk.float(), xd.float() * 2.0 ** k)
        ck, nk = q.rotate_quantize(xk, seed, bits)
        zk, _ = q.rotate(xk, seed)
        torch.cuda.synchronize()
        assert torch.equal(ck, c0), f"codes change under 2^{k}"
        assert torch.equal(nk, n0 * 2.0 ** k), f"norms not scaled exactly by 2^{k}"
        assert torch.equal(zk, z0), f"rotated values change under 2^{k}"


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("d", [1024, 5120, 12288, 13824])
def test_negated_tokens_take_mirrored_codes(q, d, bits):
    """The Lloyd-Max codebook is symmetric (its thresholds come in +-
    pairs, zero the middle one at even level counts): -x must give the same
    norms, z -> -z up to the transform's rounding (the matrix cores' sums
    need not round negatives as mirror images), and code (2^b - 1) - c for
    every coordinate farther than the parity window from a threshold; an
    exact zero sits on the middle threshold and takes the upper middle code
    in both."""
    import torch
    M, seed = 29, 57
    x = wl.custom_activations(M, d, wl.BF16, d + bits, n_out=max(1, d // 100), out_factor=50.0,
                              sigma_s=1.0, zero_rows=(3,))
    xd = to_device(x)
    xd[7] = 0.5  # a constant token: exact zeros after the transform
    say("negated tokens", d, bits)
    c0, n0 = q.rotate_quantize(xd, seed, bits)
    c1, n1 = q.rotate_quantize(-xd, seed, bits)
    z0, _ = q.rotate(xd, seed)
    z1, _ = q.rotate(-xd, seed)
    torch.cuda.synchronize()
    assert torch.equal(n1, n0)
    za, zb = host(z0).astype(np.float64), host(z1).astype(np.float64)
    assert np.abs(za + zb).max() <= 1e-6 * np.abs(za).max()
    u0 = parity.unpack_codes(host(c0), d, bits).astype(np.int64)
    u1 = parity.unpack_codes(host(c1), d, bits).astype(np.int64)
    u = np.sqrt(d) * za  # unpacked codes and rotated values: coordinate order
    tau = np.asarray(oracle.codebook_unit(bits)[1], np.float64)
    near = (np.abs(u[..., None] - tau) <= parity.CODE_WINDOW * np.maximum(np.abs(tau), 1.0)).any(-1)
    top = (1 << bits) - 1
    zero = (za == 0) & (zb == 0)
    far = ~near & ~zero
    assert (u1[far] == top - u0[far]).all(), f"{int((u1[far] != top - u0[far]).sum())} unmirrored"
    assert zero.any(), "the constant token must give exact zeros"
    assert (u0[zero] == 1 << (bits - 1)).all() and (u1[zero] == 1 << (bits - 1)).all()
