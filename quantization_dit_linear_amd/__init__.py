"""OrbitQuant online quantized-linear path for MI355X (gfx950).

Thin Python binding over ``liborbitquant.so`` (C ABI in
``include/orbitquant.h``).  This module only marshals arguments: every step
of the path runs in the library's HIP kernels.  PyTorch supplies device
memory and the current stream, nothing else.  There is no CPU fallback: if
the library is missing or cannot run, the call raises.

Functions mirror the C entry points:

* :func:`codebook`        -> ``oq_codebook``
* :func:`rotate_quantize` -> ``oq_rotate_quantize``
* :func:`rotate`          -> ``oq_rotate_quantize`` with ``OQ_OUT_F32_ROTATED``
* :func:`fake_quantize`   -> ``oq_rotate_quantize`` with ``OQ_OUT_BF16_DEQUANT``
* :func:`prepare_weights` -> ``oq_prepare_weights``
* :func:`linear`          -> ``oq_linear``
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liborbitquant.so")

OQ_OK, OQ_EINVAL, OQ_EUNSUPPORTED, OQ_ENOMEM, OQ_EDEVICE = 0, -1, -2, -3, -4
OQ_F32, OQ_BF16 = 0, 1
OQ_ROT_NO_SIGNS, OQ_OUT_F32_ROTATED, OQ_OUT_BF16_DEQUANT, OQ_ROT_INPUT_PERMUTED = 1, 2, 4, 8
OQ_CODEBOOK_SPHERE = 16

# every symbol the header declares, with (restype, argtypes)
_P = ctypes.c_void_p
_SIGS = {
    "oq_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "oq_version": (ctypes.c_int, []),
    "oq_codebook": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _P, _P]),
    "oq_codes_bytes": (ctypes.c_int64, [ctypes.c_int64, ctypes.c_int, ctypes.c_int]),
    "oq_codebook_ex": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_uint32, _P, _P]),
    "oq_linear_ex": (ctypes.c_int, [_P, _P, ctypes.c_int, _P, _P, ctypes.c_int, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int, ctypes.c_uint32, _P, _P]),
    "oq_rotate_quantize": (ctypes.c_int, [_P, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                          ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int,
                                          _P, _P, _P]),
    "oq_prepare_weights": (ctypes.c_int, [_P, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                          ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int,
                                          _P, _P, _P]),
    "oq_linear": (ctypes.c_int, [_P, _P, ctypes.c_int, _P, _P, ctypes.c_int, ctypes.c_int64,
                                 ctypes.c_int64, ctypes.c_int, _P, _P]),
    "oq_release_plans": (ctypes.c_int, []),
    "oq_plan_create": (ctypes.c_int, [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint32,
                                      ctypes.POINTER(ctypes.c_void_p)]),
    "oq_plan_destroy": (ctypes.c_int, [ctypes.c_void_p]),
    "oq_permute_rows": (ctypes.c_int, [_P, _P, ctypes.c_int64, ctypes.c_int64, ctypes.c_uint64,
                                       _P]),
    "oq_rtn4_prepare_weights": (ctypes.c_int, [_P, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                               _P, _P, _P]),
    "oq_rtn4_linear": (ctypes.c_int, [_P, ctypes.c_int, ctypes.c_int64, _P, _P, ctypes.c_int64,
                                      ctypes.c_int, _P, _P]),
    "oq_diag_mfma_f16": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _P, _P]),
}

_lib = None


class OQError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


def lib():
    """The loaded ctypes library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (python -m "
                "quantization_dit_linear_amd.build or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def strerror(status):
    return lib().oq_strerror(status).decode()


def _check(status, where):
    if status != OQ_OK:
        raise OQError(status, where)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev_ptr(t, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if t.device.index is not None and t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} lives on {t.device}, not on the current device "
                         f"cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _expect(t, shape, dtype, name):
    """The shape and dtype a buffer must have for the call (the library
    trusts its sizes): checked before anything touches the device."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


# ------------------------------------------------------------------- API --

def codebook(d, bits, *, sphere=False):
    """(levels float32[2^bits], thresholds float32[2^bits-1]) of C_{d,bits}
    (sphere: the exact-sphere-marginal family)."""
    L = 1 << bits
    lv = np.zeros(256, np.float32)
    th = np.zeros(256, np.float32)
    flags = OQ_CODEBOOK_SPHERE if sphere else 0
    _check(lib().oq_codebook_ex(d, bits, flags, lv.ctypes.data, th.ctypes.data), "oq_codebook_ex")
    return lv[:L].copy(), th[:L - 1].copy()


def codes_bytes(rows, d, bits):
    return lib().oq_codes_bytes(rows, d, bits)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return OQ_BF16
    if t.dtype == torch.float32:
        return OQ_F32
    raise TypeError(f"unsupported input dtype {t.dtype} (bfloat16 or float32)")


def rotate_quantize(x, seed, bits, *, signs=True, permuted=False, sphere=False, out=None,
                    norms=None, stream=None):
    """Codes (uint8 [M, d*bits/8], storage order) and norms (float32 [M]).
    permuted=True: x's columns are already in rotation order (OQ_ROT_INPUT_PERMUTED);
    sphere=True: the exact-sphere-marginal codebook (OQ_CODEBOOK_SPHERE)."""
    import torch
    if x.dim() != 2:
        raise ValueError("x must be [tokens, d]")
    M, d = x.shape
    if out is None:
        out = torch.empty((M, d * bits // 8), dtype=torch.uint8, device=x.device)
    if norms is None:
        norms = torch.empty((M,), dtype=torch.float32, device=x.device)
    _expect(out, (M, d * bits // 8), torch.uint8, "out")
    _expect(norms, (M,), torch.float32, "norms")
    flags = ((0 if signs else OQ_ROT_NO_SIGNS) | (OQ_ROT_INPUT_PERMUTED if permuted else 0)
             | (OQ_CODEBOOK_SPHERE if sphere else 0))
    rc = lib().oq_rotate_quantize(_dev_ptr(x, "x"), _dtype_code(x), M, d, seed, flags, bits,
                                  _dev_ptr(out, "out"), _dev_ptr(norms, "norms"),
                                  _stream(stream))
    _check(rc, "oq_rotate_quantize")
    return out, norms


def rotate(x, seed, *, signs=True, permuted=False, stream=None):
    """Rotated unit vectors z (float32 [M, d], coordinate order) and norms.
    bf16 tokens of the fast-path sizes run through the same kernel as the
    codes; permuted=True: x's columns are already in rotation order."""
    import torch
    if x.dim() != 2:
        raise ValueError("x must be [tokens, d]")
    M, d = x.shape
    z = torch.empty((M, d), dtype=torch.float32, device=x.device)
    norms = torch.empty((M,), dtype=torch.float32, device=x.device)
    flags = (OQ_OUT_F32_ROTATED | (0 if signs else OQ_ROT_NO_SIGNS)
             | (OQ_ROT_INPUT_PERMUTED if permuted else 0))
    rc = lib().oq_rotate_quantize(_dev_ptr(x, "x"), _dtype_code(x), M, d, seed, flags, 4,
                                  _dev_ptr(z, "z"), _dev_ptr(norms, "norms"), _stream(stream))
    _check(rc, "oq_rotate_quantize")
    return z, norms


def fake_quantize(x, seed, bits, *, signs=True, sphere=False, out=None, norms=None,
                  stream=None):
    """Dequantized rotated rows (bfloat16 [M, d], coordinate order): row m,
    coordinate i holds s_m * C_{d,bits}[code_mi]; and the norms.  Works for
    activation tokens and weight rows alike (the same quantizer); a bf16 GEMM
    of two such matrices with the same seed is the fake-quantized product."""
    import torch
    if x.dim() != 2:
        raise ValueError("x must be [rows, d]")
    M, d = x.shape
    if out is None:
        out = torch.empty((M, d), dtype=torch.bfloat16, device=x.device)
    if norms is None:
        norms = torch.empty((M,), dtype=torch.float32, device=x.device)
    _expect(out, (M, d), torch.bfloat16, "out")
    _expect(norms, (M,), torch.float32, "norms")
    flags = (OQ_OUT_BF16_DEQUANT | (0 if signs else OQ_ROT_NO_SIGNS)
             | (OQ_CODEBOOK_SPHERE if sphere else 0))
    rc = lib().oq_rotate_quantize(_dev_ptr(x, "x"), _dtype_code(x), M, d, seed, flags, bits,
                                  _dev_ptr(out, "out"), _dev_ptr(norms, "norms"),
                                  _stream(stream))
    _check(rc, "oq_rotate_quantize")
    return out, norms


def prepare_weights(W, seed, bits, *, signs=True, sphere=False, out=None, norms=None,
                    stream=None):
    """Weight codes (uint8 [N, K*bits/8]) and row norms (float32 [N])."""
    import torch
    if W.dim() != 2:
        raise ValueError("W must be [d_out, d_in]")
    N, K = W.shape
    if out is None:
        out = torch.empty((N, K * bits // 8), dtype=torch.uint8, device=W.device)
    if norms is None:
        norms = torch.empty((N,), dtype=torch.float32, device=W.device)
    _expect(out, (N, K * bits // 8), torch.uint8, "out")
    _expect(norms, (N,), torch.float32, "norms")
    flags = (0 if signs else OQ_ROT_NO_SIGNS) | (OQ_CODEBOOK_SPHERE if sphere else 0)
    rc = lib().oq_prepare_weights(_dev_ptr(W, "W"), _dtype_code(W), N, K, seed, flags, bits,
                                  _dev_ptr(out, "w_codes"), _dev_ptr(norms, "row_norms"),
                                  _stream(stream))
    _check(rc, "oq_prepare_weights")
    return out, norms


def linear(a_codes, a_norms, a_bits, w_codes, w_norms, w_bits, K, *, sphere=False, out=None,
           stream=None):
    """bf16 y [M, N] = s_m r_n sum_k C_w[p_nk] C_a[q_mk] (sphere: the
    exact-sphere-marginal codebooks, oq_linear_ex)."""
    import torch
    if a_codes.dim() != 2 or w_codes.dim() != 2:
        raise ValueError("a_codes and w_codes must be [rows, K*bits/8]")
    M = a_codes.shape[0]
    N = w_codes.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a_codes.device)
    _expect(a_codes, (M, K * a_bits // 8), torch.uint8, "a_codes")
    _expect(w_codes, (N, K * w_bits // 8), torch.uint8, "w_codes")
    _expect(a_norms, (M,), torch.float32, "a_norms")
    _expect(w_norms, (N,), torch.float32, "w_norms")
    _expect(out, (M, N), torch.bfloat16, "out")
    if sphere:
        rc = lib().oq_linear_ex(_dev_ptr(a_codes, "a_codes"), _dev_ptr(a_norms, "a_norms"),
                                a_bits, _dev_ptr(w_codes, "w_codes"), _dev_ptr(w_norms, "w_norms"),
                                w_bits, M, N, K, OQ_CODEBOOK_SPHERE, _dev_ptr(out, "y"),
                                _stream(stream))
    else:
        rc = lib().oq_linear(_dev_ptr(a_codes, "a_codes"), _dev_ptr(a_norms, "a_norms"), a_bits,
                             _dev_ptr(w_codes, "w_codes"), _dev_ptr(w_norms, "w_norms"), w_bits,
                             M, N, K, _dev_ptr(out, "y"), _stream(stream))
    _check(rc, "oq_linear")
    return out


def rtn4_prepare_weights(W, *, out=None, scales=None, stream=None):
    """INT4 weight-only RTN of the AdaLN projection weights W [N, K]:
    (uint8 [N, K/2] offset-binary nibbles, float32 scales [N])."""
    import torch
    N, K = W.shape
    if out is None:
        out = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    if scales is None:
        scales = torch.empty((N,), dtype=torch.float32, device=W.device)
    _expect(out, (N, K // 2), torch.uint8, "out")
    _expect(scales, (N,), torch.float32, "scales")
    rc = lib().oq_rtn4_prepare_weights(_dev_ptr(W, "W"), _dtype_code(W), N, K,
                                       _dev_ptr(out, "q4"), _dev_ptr(scales, "scales"),
                                       _stream(stream))
    _check(rc, "oq_rtn4_prepare_weights")
    return out, scales


def rtn4_linear(x, q4, scales, *, out=None, stream=None):
    """bf16 y [M, N] = scale_n sum_k x_mk q_nk (AdaLN projection)."""
    import torch
    M, K = x.shape
    N = q4.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _expect(q4, (N, K // 2), torch.uint8, "q4")
    _expect(scales, (N,), torch.float32, "scales")
    _expect(out, (M, N), torch.bfloat16, "out")
    rc = lib().oq_rtn4_linear(_dev_ptr(x, "x"), _dtype_code(x), M, _dev_ptr(q4, "q4"),
                              _dev_ptr(scales, "scales"), N, K, _dev_ptr(out, "y"),
                              _stream(stream))
    _check(rc, "oq_rtn4_linear")
    return out


def permute_rows(src, seed, *, out=None, stream=None):
    """dst row i = src row pi(i) for the rotation permutation of (d =
    src.shape[0], seed): folds pi into a producer's output rows (any dtype)."""
    import torch
    if out is None:
        out = torch.empty_like(src)
    _expect(out, tuple(src.shape), src.dtype, "out")
    rows = src.shape[0]
    row_bytes = src[0].numel() * src.element_size() if rows else 0
    rc = lib().oq_permute_rows(_dev_ptr(src, "src"), _dev_ptr(out, "dst"), rows, row_bytes,
                               seed, _stream(stream))
    _check(rc, "oq_permute_rows")
    return out


def release_plans():
    _check(lib().oq_release_plans(), "oq_release_plans")


class Plan:
    """Explicitly owned rotation plan of (current device, d, seed): built at
    construction, its device tables freed by close() (or on leaving a
    ``with`` block) once no other handle pins them."""

    def __init__(self, d, seed, *, signs=True):
        h = ctypes.c_void_p()
        flags = 0 if signs else OQ_ROT_NO_SIGNS
        _check(lib().oq_plan_create(d, seed, flags, ctypes.byref(h)), "oq_plan_create")
        self._h = h

    def close(self):
        if self._h is not None and self._h.value:
            h, self._h = self._h, None
            _check(lib().oq_plan_destroy(h), "oq_plan_destroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def diag_mfma_f16(blocks, iters, sink, stream=None):
    """Enqueue the matrix-core probe (orbitquant_diag.h); returns its flop
    count.  sink: float32 CUDA tensor of at least blocks * 512 elements."""
    if sink.numel() < blocks * 512:
        raise ValueError("sink too small")
    _check(lib().oq_diag_mfma_f16(blocks, iters, _dev_ptr(sink, "sink"), _stream(stream)),
           "oq_diag_mfma_f16")
    return blocks * 8 * iters * 32 * 16384
