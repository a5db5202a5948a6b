"""The C ABI without a GPU: the library loads, exports every function the
header declares, solves the codebook on the host, and rejects bad
arguments before making any HIP call.  Also checks the numpy unpacker the
parity tests use against the oracle's."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from tests import parity

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def q():
    import quantization_dit_linear_amd as q
    return q


def _declared():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if not h.endswith(".h"):
            continue
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(oq_[a-z_0-9]+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_symbol(q):
    names = _declared()
    assert "oq_linear" in names and "oq_rotate_quantize" in names and "oq_diag_mfma_f16" in names
    lib = ctypes.CDLL(q.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(q._SIGS), "binding and header disagree"


def test_version_and_strerror(q):
    assert q.lib().oq_version() >= 100
    for s in (0, -1, -2, -3, -4, -99):
        assert isinstance(q.strerror(s), str) and q.strerror(s)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_host_codebook_properties(q, bits):
    d = 3072
    lv, th = q.codebook(d, bits)
    L = 1 << bits
    assert lv.dtype == np.float32 and lv.shape == (L,) and th.shape == (L - 1,)
    assert np.all(np.diff(lv) > 0)
    assert np.array_equal(lv, -lv[::-1])
    assert th[L // 2 - 1] == 0.0
    ol, ot = oracle.codebook(d, bits)
    assert np.allclose(lv, ol, rtol=2e-7, atol=0)
    assert np.allclose(th, ot, rtol=2e-7, atol=1e-12)


def test_codebook_rejects(q):
    L = q.lib()
    buf = np.zeros(512, np.float32)
    assert L.oq_codebook(256, 9, buf.ctypes.data, buf.ctypes.data) == q.OQ_EUNSUPPORTED
    assert L.oq_codebook(256, 0, buf.ctypes.data, buf.ctypes.data) == q.OQ_EUNSUPPORTED
    assert L.oq_codebook(0, 4, buf.ctypes.data, buf.ctypes.data) == q.OQ_EINVAL
    assert L.oq_codebook(256, 4, None, buf.ctypes.data) == q.OQ_EINVAL


def test_codes_bytes(q):
    assert q.codes_bytes(10, 3072, 4) == 10 * 1536
    assert q.codes_bytes(3, 256, 3) == 3 * 96
    assert q.codes_bytes(-1, 256, 3) == -1


# Fake but aligned, non-null "device" addresses: every call below must be
# rejected by validation before the library touches the GPU.
A16, B16, C16, D16 = 0x100000, 0x200000, 0x300000, 0x10000000


@pytest.mark.parametrize("fn", ["oq_rotate_quantize", "oq_prepare_weights"])
def test_rotate_validation_rejects_before_hip(q, fn):
    f = getattr(q.lib(), fn)
    ok_args = dict(x=A16, dt=1, n=8, d=3072, seed=1, flags=0, bits=4, out=B16, nrm=C16)

    def call(**kw):
        a = dict(ok_args, **kw)
        return f(a["x"], a["dt"], a["n"], a["d"], a["seed"], a["flags"], a["bits"], a["out"],
                 a["nrm"], None)

    assert call(x=None) == q.OQ_EINVAL
    assert call(out=None) == q.OQ_EINVAL
    assert call(nrm=None) == q.OQ_EINVAL
    assert call(x=A16 + 2) == q.OQ_EINVAL
    assert call(out=B16 + 4) == q.OQ_EINVAL
    assert call(nrm=C16 + 1) == q.OQ_EINVAL
    assert call(dt=7) == q.OQ_EINVAL
    assert call(flags=1 << 5) == q.OQ_EINVAL
    assert call(n=-1) == q.OQ_EINVAL
    assert call(d=0) == q.OQ_EINVAL
    assert call(d=3000) == q.OQ_EUNSUPPORTED
    assert call(d=32768) == q.OQ_EUNSUPPORTED
    assert call(bits=1) == q.OQ_EUNSUPPORTED
    assert call(bits=5) == q.OQ_EUNSUPPORTED
    # empty input is a no-op that succeeds without any device work
    assert call(n=0) == q.OQ_OK
    assert call(n=0, x=None, out=None, nrm=None) == q.OQ_OK
    assert call(n=0, d=3000) == q.OQ_EUNSUPPORTED
    # token lengths: multiples of 32 up to 16384 (a partial last group of
    # 32, 64 or 96 coordinates is stored in coordinate order)
    assert call(n=0, d=96) == q.OQ_OK
    assert call(n=0, d=32) == q.OQ_OK
    assert call(n=0, d=16352) == q.OQ_OK
    assert call(n=0, d=16416) == q.OQ_EUNSUPPORTED
    assert call(d=48) == q.OQ_EUNSUPPORTED
    assert call(d=16) == q.OQ_EUNSUPPORTED
    # the two alternative outputs exclude each other
    assert call(flags=q.OQ_OUT_F32_ROTATED | q.OQ_OUT_BF16_DEQUANT) == q.OQ_EINVAL
    if fn == "oq_prepare_weights":
        assert call(flags=q.OQ_OUT_F32_ROTATED) == q.OQ_EINVAL
        assert call(flags=q.OQ_OUT_BF16_DEQUANT) == q.OQ_EINVAL


def test_linear_validation_rejects_before_hip(q):
    f = q.lib().oq_linear
    base = dict(a=A16, sa=C16, ba=4, w=B16, sw=C16 + 64, bw=4, M=16, N=16, K=3072, y=D16)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["a"], a["sa"], a["ba"], a["w"], a["sw"], a["bw"], a["M"], a["N"], a["K"],
                 a["y"], None)

    assert call(a=None) == q.OQ_EINVAL
    assert call(w=None) == q.OQ_EINVAL
    assert call(y=None) == q.OQ_EINVAL
    assert call(sa=None) == q.OQ_EINVAL
    assert call(a=A16 + 8) == q.OQ_EINVAL
    assert call(y=D16 + 1) == q.OQ_EINVAL
    assert call(M=1 << 31) == q.OQ_EUNSUPPORTED
    assert call(N=(1 << 30) + 1) == q.OQ_EUNSUPPORTED
    assert call(M=-1) == q.OQ_EINVAL
    assert call(K=100) == q.OQ_EUNSUPPORTED
    # the linear takes whole 64-slot K steps: K % 64 == 0
    assert call(K=96) == q.OQ_EUNSUPPORTED
    assert call(K=160) == q.OQ_EUNSUPPORTED
    assert call(K=192, M=0) == q.OQ_OK
    assert call(K=64, N=0) == q.OQ_OK
    assert call(ba=5) == q.OQ_EUNSUPPORTED
    assert call(bw=1) == q.OQ_EUNSUPPORTED
    assert call(M=0) == q.OQ_OK
    assert call(N=0) == q.OQ_OK
    assert call(M=0, a=None, y=None) == q.OQ_OK


def test_linear_rejects_an_output_overlapping_its_inputs(q):
    """y [M][N] bf16 may not share a byte with a_codes [M][K b_a/8],
    a_norms [M], w_codes [N][K b_w/8] or w_norms [N]: the call returns
    OQ_EINVAL before any device work."""
    f = q.lib().oq_linear
    M, N, K = 16, 32, 3072
    a_b, w_b, y_b = M * K // 2, N * K // 2, M * N * 2
    A, SA, W, SW, Y = 0x1000000, 0x2000000, 0x3000000, 0x4000000, 0x5000000

    def call(a=A, sa=SA, w=W, sw=SW, y=Y):
        return f(a, sa, 4, w, sw, 4, M, N, K, y, None)

    # y starting inside, ending inside, or covering each input range
    for base, nb in ((A, a_b), (SA, 4 * M), (W, w_b), (SW, 4 * N)):
        assert call(y=base) == q.OQ_EINVAL
        assert call(y=base + nb - 16) == q.OQ_EINVAL
        assert call(y=base - y_b + 16) == q.OQ_EINVAL
    assert call(a=Y + 16) == q.OQ_EINVAL
    assert call(sa=Y + y_b - 4) == q.OQ_EINVAL
    assert call(w=Y) == q.OQ_EINVAL
    assert call(sw=Y + 64) == q.OQ_EINVAL


def test_binding_fails_loudly_without_gpu_tensors(q):
    import torch
    x = torch.zeros(4, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        q.rotate_quantize(x, 1, 4)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_numpy_unpacker_agrees_with_oracle(bits):
    rng = np.random.default_rng(bits)
    d = 384
    codes = rng.integers(0, 1 << bits, (5, d)).astype(np.uint8)
    packed = np.stack([oracle.pack_row(c, bits) for c in codes])
    assert np.array_equal(parity.unpack_codes(packed, d, bits), codes)


def test_flag_and_status_constants_match_header(q):
    """The binding's constants are the header's #defines / enum values."""
    src = open(os.path.join(ROOT, "include", "orbitquant.h")).read()
    for name, val in re.findall(r"#define\s+(OQ_[A-Z0-9_]+)\s+\(1u\s*<<\s*(\d+)\)", src):
        assert getattr(q, name) == 1 << int(val), name
    for name in ("OQ_ROT_NO_SIGNS", "OQ_OUT_F32_ROTATED", "OQ_OUT_BF16_DEQUANT"):
        assert re.search(r"#define\s+" + name + r"\b", src), name


def test_plan_handles_validate_before_hip(q):
    import ctypes
    L = q.lib()
    h = ctypes.c_void_p(123)
    assert L.oq_plan_create(3072, 1, 0, None) == q.OQ_EINVAL
    assert L.oq_plan_create(3072, 1, 1 << 4, ctypes.byref(h)) == q.OQ_EINVAL
    assert h.value is None  # cleared on error
    assert L.oq_plan_create(0, 1, 0, ctypes.byref(h)) == q.OQ_EINVAL
    assert L.oq_plan_create(3000, 1, 0, ctypes.byref(h)) == q.OQ_EUNSUPPORTED
    assert L.oq_plan_create(32768, 1, 0, ctypes.byref(h)) == q.OQ_EUNSUPPORTED
    assert L.oq_plan_destroy(None) == q.OQ_EINVAL
    junk = (ctypes.c_uint32 * 8)()  # not a handle: wrong tag
    assert L.oq_plan_destroy(ctypes.cast(junk, ctypes.c_void_p)) == q.OQ_EINVAL


def test_permute_rows_validates_before_hip(q):
    L = q.lib()
    f = L.oq_permute_rows
    assert f(None, B16, 3072, 16, 1, None) == q.OQ_EINVAL
    assert f(A16, None, 3072, 16, 1, None) == q.OQ_EINVAL
    assert f(A16, A16, 3072, 16, 1, None) == q.OQ_EINVAL  # in place is not supported
    assert f(A16, B16, 3072, 0, 1, None) == q.OQ_EINVAL
    assert f(A16, B16, 0, 16, 1, None) == q.OQ_EINVAL
    assert f(A16, B16, 3000, 16, 1, None) == q.OQ_EUNSUPPORTED
    assert f(A16, B16, 48, 16, 1, None) == q.OQ_EUNSUPPORTED
    assert f(A16, B16, 32768, 16, 1, None) == q.OQ_EUNSUPPORTED


def test_rtn4_validates_before_hip(q):
    L = q.lib()
    p = L.oq_rtn4_prepare_weights
    assert p(None, 1, 8, 256, B16, C16, None) == q.OQ_EINVAL
    assert p(A16, 1, 8, 256, None, C16, None) == q.OQ_EINVAL
    assert p(A16, 1, 8, 256, B16 + 4, C16, None) == q.OQ_EINVAL
    assert p(A16, 5, 8, 256, B16, C16, None) == q.OQ_EINVAL
    assert p(A16, 1, 8, 100, B16, C16, None) == q.OQ_EUNSUPPORTED
    assert p(A16, 1, -1, 256, B16, C16, None) == q.OQ_EINVAL
    assert p(None, 1, 0, 256, None, None, None) == q.OQ_OK
    f = L.oq_rtn4_linear
    assert f(None, 1, 2, B16, C16, 8, 256, A16, None) == q.OQ_EINVAL
    assert f(A16, 1, 2, B16 + 8, C16, 8, 256, A16, None) == q.OQ_EINVAL
    assert f(A16 + 4, 1, 2, B16, C16, 8, 256, A16, None) == q.OQ_EINVAL
    assert f(A16, 1, 2, B16, C16, 8, 100, A16, None) == q.OQ_EUNSUPPORTED
    assert f(A16, 1, 2, B16, C16, 8, 32768, A16, None) == q.OQ_EUNSUPPORTED
    assert f(None, 1, 0, None, None, 8, 256, None, None) == q.OQ_OK
