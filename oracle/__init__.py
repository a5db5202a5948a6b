"""fp64 CPU oracle for the OrbitQuant online quantized-linear path.

TEST INFRASTRUCTURE ONLY.  The test-suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` are the only code allowed to import
this package.  It shares nothing with ``quantization_dit_linear_amd`` (the
HIP product path) and never imports it.

This module is a thin ctypes layer over ``oq_oracle.c`` (plain C, fp64),
built by ``oracle/build.py`` into ``liboq_oracle.so``.  What each function
computes, and the page passage it follows, is documented in the C source.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboq_oracle.so")
_lib = None

F32, BF16 = 0, 1


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    lib.oqo_splitmix64_next.restype = ctypes.c_uint64
    lib.oqo_splitmix64_next.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
    lib.oqo_block_size.restype = ctypes.c_int
    lib.oqo_block_size.argtypes = [ctypes.c_int]
    lib.oqo_plan.restype = None
    lib.oqo_plan.argtypes = [ctypes.c_int, ctypes.c_uint64, P, P]
    lib.oqo_codebook_unit.restype = ctypes.c_int
    lib.oqo_codebook_unit.argtypes = [ctypes.c_int, P, P]
    lib.oqo_codebook.restype = ctypes.c_int
    lib.oqo_codebook.argtypes = [ctypes.c_int, ctypes.c_int, P, P]
    lib.oqo_codebook_mse.restype = ctypes.c_double
    lib.oqo_codebook_mse.argtypes = [ctypes.c_int, P, P]
    lib.oqo_codebook_sphere.restype = ctypes.c_int
    lib.oqo_codebook_sphere.argtypes = [ctypes.c_int, ctypes.c_int, P, P]
    lib.oqo_sphere_mass.restype = ctypes.c_double
    lib.oqo_sphere_mass.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_int]
    lib.oqo_fwht.restype = None
    lib.oqo_fwht.argtypes = [P, ctypes.c_int]
    lib.oqo_hadamard_entry.restype = ctypes.c_int
    lib.oqo_hadamard_entry.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.oqo_rotate_token.restype = None
    lib.oqo_rotate_token.argtypes = [P, ctypes.c_int, P, P, ctypes.c_int, P, P]
    lib.oqo_quantize_one.restype = ctypes.c_int
    lib.oqo_quantize_one.argtypes = [ctypes.c_double, P, ctypes.c_int]
    lib.oqo_slot_of.restype = ctypes.c_int64
    lib.oqo_slot_of.argtypes = [ctypes.c_int64, ctypes.c_int]
    lib.oqo_pack_row.restype = None
    lib.oqo_pack_row.argtypes = [P, ctypes.c_int, ctypes.c_int, P]
    lib.oqo_unpack_row.restype = None
    lib.oqo_unpack_row.argtypes = [P, ctypes.c_int, ctypes.c_int, P]
    lib.oqo_rotate_quantize.restype = ctypes.c_int
    lib.oqo_rotate_quantize.argtypes = [P, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                        ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                        P, P, P]
    lib.oqo_rotate_quantize_ex.restype = ctypes.c_int
    lib.oqo_rotate_quantize_ex.argtypes = [P, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                           ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, P, P, P]
    lib.oqo_linear_ex.restype = ctypes.c_int
    lib.oqo_linear_ex.argtypes = [P, P, ctypes.c_int, P, P, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int64, ctypes.c_int, P, ctypes.c_int64, P]
    lib.oqo_linear.restype = ctypes.c_int
    lib.oqo_linear.argtypes = [P, P, ctypes.c_int, P, P, ctypes.c_int,
                               ctypes.c_int64, ctypes.c_int, P, ctypes.c_int64, P]
    lib.oqo_fake_quantize.restype = ctypes.c_int
    lib.oqo_fake_quantize.argtypes = [P, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                      ctypes.c_uint64, ctypes.c_int, ctypes.c_int, P, P]
    lib.oqo_rtn4_quantize.restype = ctypes.c_int
    lib.oqo_rtn4_quantize.argtypes = [P, ctypes.c_int, ctypes.c_int64, ctypes.c_int, P, P]
    lib.oqo_rtn4_linear.restype = ctypes.c_int
    lib.oqo_rtn4_linear.argtypes = [P, ctypes.c_int, ctypes.c_int64, P, P, ctypes.c_int64,
                                    ctypes.c_int, P]
    lib.oqo_num_threads.restype = ctypes.c_int
    lib.oqo_num_threads.argtypes = []
    lib.oqo_set_threads.restype = None
    lib.oqo_set_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


# ---------------------------------------------------------------- wrappers --

def splitmix64(seed, n):
    """First n outputs of SplitMix64 started from `seed`."""
    lib = _load()
    st = ctypes.c_uint64(seed)
    return [lib.oqo_splitmix64_next(ctypes.byref(st)) for _ in range(n)]


def block_size(d):
    return _load().oqo_block_size(d)


def plan(d, seed):
    """(perm int32[d], sign int8[d]) of the rotation plan."""
    lib = _load()
    perm = np.empty(d, np.int32)
    sign = np.empty(d, np.int8)
    lib.oqo_plan(d, seed, _ptr(perm), _ptr(sign))
    return perm, sign


def codebook_unit(bits):
    """(levels[L], thresholds[L-1], iterations) for N(0,1), fp64."""
    lib = _load()
    L = 1 << bits
    lv = np.zeros(256, np.float64)
    th = np.zeros(256, np.float64)
    it = lib.oqo_codebook_unit(bits, _ptr(lv), _ptr(th))
    return lv[:L].copy(), th[:L - 1].copy(), it


def codebook(d, bits):
    """(levels, thresholds) of C_{d,b}: the unit codebook times 1/sqrt(d)."""
    lib = _load()
    L = 1 << bits
    lv = np.zeros(256, np.float64)
    th = np.zeros(256, np.float64)
    lib.oqo_codebook(d, bits, _ptr(lv), _ptr(th))
    return lv[:L].copy(), th[:L - 1].copy()


def codebook_sphere(d, bits):
    """Lloyd-Max (levels, thresholds) for the exact marginal of a coordinate
    of a uniform point on S^{d-1}, in units of z (fp64), and iterations."""
    L = 1 << bits
    lv = np.zeros(L, np.float64)
    th = np.zeros(max(L - 1, 1), np.float64)
    it = _load().oqo_codebook_sphere(d, bits, _ptr(lv), _ptr(th))
    if it < 0:
        raise ValueError("oracle rejected the arguments")
    return lv, th[:L - 1], it


def sphere_mass(a, b, d):
    """P(a <= T < b) for one coordinate T of a uniform point on S^{d-1}."""
    return _load().oqo_sphere_mass(a, b, d)


def codebook_mse(bits, levels, thresholds):
    lv = np.zeros(256, np.float64)
    th = np.zeros(256, np.float64)
    lv[:len(levels)] = levels
    th[:len(thresholds)] = thresholds
    return _load().oqo_codebook_mse(bits, _ptr(lv), _ptr(th))


def fwht(v):
    """Unnormalised Sylvester-order Walsh-Hadamard transform of a 1-D array."""
    a = np.array(v, dtype=np.float64, copy=True)
    _load().oqo_fwht(_ptr(a), a.shape[0])
    return a


def hadamard_entry(a, b):
    return _load().oqo_hadamard_entry(a, b)


def rotate_token(x, perm, sign, use_signs=True):
    """(z, norm) for one fp64 token."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    d = x.shape[0]
    z = np.empty(d, np.float64)
    nrm = ctypes.c_double(0.0)
    _load().oqo_rotate_token(_ptr(x), d, _ptr(np.ascontiguousarray(perm, np.int32)),
                             _ptr(np.ascontiguousarray(sign, np.int8)), int(use_signs),
                             _ptr(z), ctypes.byref(nrm))
    return z, nrm.value


def quantize_one(z, thresholds):
    th = np.zeros(256, np.float64)
    th[:len(thresholds)] = thresholds
    return _load().oqo_quantize_one(float(z), _ptr(th), len(thresholds) + 1)


def slot_of(i, d):
    """Storage slot of coordinate i in a row of d coordinates."""
    return _load().oqo_slot_of(int(i), int(d))


def pack_row(codes, bits):
    codes = np.ascontiguousarray(codes, np.uint8)
    d = codes.shape[0]
    out = np.empty(d * bits // 8, np.uint8)
    _load().oqo_pack_row(_ptr(codes), d, bits, _ptr(out))
    return out


def unpack_row(packed, d, bits):
    packed = np.ascontiguousarray(packed, np.uint8)
    codes = np.empty(d, np.uint8)
    _load().oqo_unpack_row(_ptr(packed), d, bits, _ptr(codes))
    return codes


def rotate_quantize(x, dtype, d, seed, bits, use_signs=True, want_codes=True, want_z=False,
                    sphere=False):
    """Rotate + quantize every row of x.

    x: np.float32 [rows, d] (dtype=F32) or np.uint16 bf16 bits (dtype=BF16).
    sphere: the exact-sphere-marginal codebook instead of the Gaussian one.
    Returns (codes uint8 [rows, d*bits/8] or None, norms fp64 [rows],
    z fp64 [rows, d] or None)."""
    x = np.ascontiguousarray(x)
    rows = x.shape[0]
    assert x.shape[1] == d
    codes = np.empty((rows, d * bits // 8), np.uint8) if want_codes else None
    norms = np.empty(rows, np.float64)
    z = np.empty((rows, d), np.float64) if want_z else None
    rc = _load().oqo_rotate_quantize_ex(_ptr(x), dtype, rows, d, seed, int(use_signs), bits,
                                        int(sphere), _ptr(codes), _ptr(norms), _ptr(z))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return codes, norms, z


def linear(a_codes, a_norms, ba, w_codes, w_norms, bw, K, rows=None, sphere=False):
    """fp64 y[rows][N] = s_m r_n sum_k C_w[p_nk] C_a[q_mk] (sigma-scaled levels;
    sphere: the exact-sphere-marginal codebooks)."""
    a_codes = np.ascontiguousarray(a_codes, np.uint8)
    w_codes = np.ascontiguousarray(w_codes, np.uint8)
    a_norms = np.ascontiguousarray(a_norms, np.float64)
    w_norms = np.ascontiguousarray(w_norms, np.float64)
    M = a_codes.shape[0]
    N = w_codes.shape[0]
    if rows is None:
        rows = np.arange(M, dtype=np.int64)
    rows = np.ascontiguousarray(rows, np.int64)
    y = np.empty((rows.shape[0], N), np.float64)
    rc = _load().oqo_linear_ex(_ptr(a_codes), _ptr(a_norms), ba, _ptr(w_codes), _ptr(w_norms),
                               bw, int(sphere), N, K, _ptr(rows), rows.shape[0], _ptr(y))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return y


def fake_quantize(x, dtype, d, seed, bits, use_signs=True):
    """Fake quantization: fp64 s * C_{d,bits}[code(z_i)] for every rotated
    coordinate i (coordinate order), and the norms s.  paper.gecl.asia notes,
    Dataset/Evaluation (the pages evaluate with dequantized operands)."""
    x = np.ascontiguousarray(x)
    rows = x.shape[0]
    assert x.shape[1] == d
    out = np.empty((rows, d), np.float64)
    norms = np.empty(rows, np.float64)
    rc = _load().oqo_fake_quantize(_ptr(x), dtype, rows, d, seed, int(use_signs), bits,
                                   _ptr(out), _ptr(norms))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out, norms


def rtn4_quantize(W, dtype, d):
    """INT4 weight-only RTN per row (AdaLN projections): (q int8 [rows, d] in
    [-7, 7], scales float32 [rows]).  paper.gecl.asia notes, Method item 5."""
    W = np.ascontiguousarray(W)
    rows = W.shape[0]
    assert W.shape[1] == d
    q = np.empty((rows, d), np.int8)
    scales = np.empty(rows, np.float32)
    if _load().oqo_rtn4_quantize(_ptr(W), dtype, rows, d, _ptr(q), _ptr(scales)) != 0:
        raise ValueError("oracle rejected the arguments")
    return q, scales


def rtn4_linear(x, dtype, q, scales):
    """fp64 y[m][n] = scale_n sum_k x_mk q_nk."""
    x = np.ascontiguousarray(x)
    q = np.ascontiguousarray(q, np.int8)
    scales = np.ascontiguousarray(scales, np.float32)
    M, K = x.shape
    N = q.shape[0]
    y = np.empty((M, N), np.float64)
    if _load().oqo_rtn4_linear(_ptr(x), dtype, M, _ptr(q), _ptr(scales), N, K, _ptr(y)) != 0:
        raise ValueError("oracle rejected the arguments")
    return y


def num_threads():
    """OpenMP threads the oracle's parallel loops use."""
    return _load().oqo_num_threads()


def set_threads(n):
    """Threads for the oracle's later parallel loops (n <= 0: all
    processors); for timing only, results do not depend on it."""
    _load().oqo_set_threads(int(n))
