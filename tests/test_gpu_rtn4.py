"""GPU parity of the AdaLN INT4 weight-only RTN path (oq_rtn4_prepare_weights,
oq_rtn4_linear) against the oracle: codes and scales bit-exact (the same
fp32 decisions), outputs within one bf16 rounding of the fp64 projection
plus the fp32 summation bound K u sum |x q| scale.
paper.gecl.asia notes, Method item 5."""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import bf16_to_np, host, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch
    import quantization_dit_linear_amd as q
    assert torch.cuda.is_available()
    q.lib()
    return q


def _pack(qv):
    """Oracle int8 codes [N, K] -> offset-binary nibbles, even k low."""
    u = (qv.astype(np.int16) + 8).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def _check_out(y, x, code, rq, rs):
    """One bf16 rounding of the result plus the fp32 summation bound
    K u sum_k |x_mk q_nk| scale_n (u = 2^-24)."""
    ref = oracle.rtn4_linear(x, code, rq, rs)
    xf = wl.bf16_bits_to_f32(x) if code == wl.BF16 else x
    mag = np.abs(xf.astype(np.float64)) @ np.abs(rq.astype(np.float64)).T * rs[None, :]
    K = x.shape[1]
    tol = 2.0 ** -8 * np.abs(ref) + 2.0 * K * 2.0 ** -24 * mag + 1e-30
    assert np.all(np.abs(y - ref) <= tol), float(np.max(np.abs(y - ref) / tol))


def _prep_check(q, W, code, K, what):
    import torch
    say("rtn4 prepare", what, W.shape)
    q4, sc = q.rtn4_prepare_weights(to_device(W))
    torch.cuda.synchronize()
    rq, rs = oracle.rtn4_quantize(W, code, K)
    np.testing.assert_array_equal(host(q4), _pack(rq))
    np.testing.assert_array_equal(host(sc), rs)
    return q4, sc, rq, rs


@pytest.mark.parametrize("name", ["image", "video"])
def test_adaln_shapes(q, name):
    import torch
    x, W = wl.adaln_inputs(name)
    M, K = x.shape
    q4, sc, rq, rs = _prep_check(q, W, wl.BF16, K, name)
    say("rtn4 linear", name)
    y = bf16_to_np(q.rtn4_linear(to_device(x), q4, sc))
    torch.cuda.synchronize()
    _check_out(y, x, wl.BF16, rq, rs)


def test_edge_rows_and_fp32(q):
    """Zero rows, an outlier row, exact ties, fp32 weights and activations,
    more activation rows than one block (8)."""
    import torch
    rng = np.random.default_rng(3)
    K = 256
    W = (rng.standard_normal((40, K)) * 0.02).astype(np.float32)
    W[1] = 0.0
    W[2, 5] = 3.0
    W[3, :8] = [7.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 6.5]
    W[3, 8:] = 0.0
    q4, sc, rq, rs = _prep_check(q, W, wl.F32, K, "edge fp32")
    x = rng.standard_normal((19, K)).astype(np.float32)
    say("rtn4 linear fp32", x.shape)
    y = bf16_to_np(q.rtn4_linear(to_device(x), q4, sc))
    torch.cuda.synchronize()
    _check_out(y, x, wl.F32, rq, rs)
    assert np.all(y[:, 1] == 0)


@pytest.mark.parametrize("M,K,N,dtype", [(1, 256, 1001, "bf16"), (3, 3072, 777, "bf16"),
                                         (4, 1088, 260, "f32"), (2, 16384, 67, "f32"),
                                         (1, 32, 9, "f32"), (4, 16384, 33, "bf16")])
def test_small_batches(q, M, K, N, dtype):
    """Up to 4 activation rows run on the register-resident kernel: one and
    four rows (4-row output blocks), fp32 and bf16 input, output counts that
    leave the last block partial, K from one chunk (32) to 512 chunks (8
    waves per workgroup)."""
    import torch
    rng = np.random.default_rng(M * 100 + K + N)
    Wf = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wf[N // 2] = 0.0
    xf = rng.standard_normal((M, K)).astype(np.float32)
    xf[0, K // 3] = 40.0
    if dtype == "bf16":
        W, x, code = wl.f32_to_bf16_bits(Wf), wl.f32_to_bf16_bits(xf), wl.BF16
    else:
        W, x, code = Wf, xf, wl.F32
    q4, sc, rq, rs = _prep_check(q, W, code, K, f"small {M}x{K}->{N}")
    say("rtn4 small batch", M, K, N, dtype)
    y = bf16_to_np(q.rtn4_linear(to_device(x), q4, sc))
    torch.cuda.synchronize()
    _check_out(y, x, code, rq, rs)
    assert np.all(y[:, N // 2] == 0)


@pytest.mark.parametrize("M", [1, 2, 4])
def test_bf16_range_fallback(q, M):
    """bf16 activations run on fp16 dot products after a per-chunk power-of-two
    scaling, exact while a 32-coordinate chunk spans at most 2^29; wider
    chunks, bf16 subnormals and zero chunks take the fp32 decode or scale
    trivially.  Chunk 0: magnitudes 2^20 and 2^-20 (fallback); chunk 1: a
    subnormal (fallback); chunk 2: all zero; chunk 3: exponents 15 and -14,
    the widest exact span; chunk 4: exponents 15 and -15 (fallback); the
    rest ordinary values."""
    import torch
    rng = np.random.default_rng(40 + M)
    K, N = 512, 203
    Wf = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    xf = rng.standard_normal((M, K)).astype(np.float32)
    for m in range(M):
        xf[m, 0], xf[m, 5] = 2.0 ** 20, -(2.0 ** -20)
        xf[m, 33] = np.float32(3.0 * 2.0 ** -133)
        xf[m, 64:96] = 0.0
        xf[m, 96], xf[m, 100] = 1.5 * 2.0 ** 15, 2.0 ** -14
        xf[m, 128], xf[m, 130] = -1.25 * 2.0 ** 15, 2.0 ** -15
    W, x = wl.f32_to_bf16_bits(Wf), wl.f32_to_bf16_bits(xf)
    q4, sc, rq, rs = _prep_check(q, W, wl.BF16, K, f"range {M}")
    say("rtn4 bf16 range fallback", M)
    y = bf16_to_np(q.rtn4_linear(to_device(x), q4, sc))
    torch.cuda.synchronize()
    _check_out(y, x, wl.BF16, rq, rs)
