"""Helpers for comparing the HIP path with the oracle (test code only).

The acceptance rules (applied element by element):
  * codes: bit-exact, except coordinates whose exact unit-space value
    sqrt(d) z lies within 1e-6 * max(|tau|, 1) of a decision threshold tau;
    at most 1e-4 of all coordinates may differ;
  * norms and rotated values: within 1e-5 relative (rotated values: per
    token ||dz|| <= 1e-5 since ||z|| = 1, and max |dz_i| <= 1e-5 max |z|);
  * linear outputs: relative Frobenius error <= 2e-3 against the oracle's
    fp64 dequantised GEMM;
  * fake-quantized (dequantized) values: within 2^-8 relative (one bf16
    rounding of s * level, plus the norm tolerance), except coordinates
    whose code may differ under the code rule above.
"""
import numpy as np

CODE_WINDOW = 1e-6
CODE_MAX_FRAC = 1e-4
NORM_RTOL = 1e-5
ROT_TOL = 1e-5
LINEAR_FRO = 2e-3
DEQUANT_RTOL = 2.0 ** -8


def slot_index(d):
    """slot_index(d)[i] = storage slot of coordinate i (whole groups of 128
    in the group order, a last partial group in coordinate order)."""
    i = np.arange(d, dtype=np.int64)
    G, r = i // 128, i % 128
    c, p = r // 32, r % 32
    s = 128 * G + 8 * (p % 16) + 4 * (p // 16) + c
    full = (d // 128) * 128
    s[full:] = i[full:]
    return s


def unpack_codes(packed, d, bits):
    """Packed rows [R, d*bits/8] -> codes [R, d] in coordinate order."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    R = packed.shape[0]
    bitarr = np.unpackbits(packed, axis=1, bitorder="little")  # [R, d*bits]
    slots = bitarr.reshape(R, d, bits)
    weights = (1 << np.arange(bits)).astype(np.uint8)
    by_slot = (slots * weights).sum(axis=2).astype(np.uint8)
    return by_slot[:, slot_index(d)]


def code_mismatch_report(gpu_packed, ref_packed, z_ref, d, bits, thr_unit):
    """Returns (n_mismatch, n_outside_window, n_total)."""
    g = unpack_codes(gpu_packed, d, bits)
    r = unpack_codes(ref_packed, d, bits)
    diff = g != r
    n_mis = int(diff.sum())
    if n_mis == 0:
        return 0, 0, g.size
    u = np.sqrt(d) * z_ref[diff]
    tau = np.asarray(thr_unit, np.float64)
    dist = np.abs(u[:, None] - tau[None, :])
    win = CODE_WINDOW * np.maximum(np.abs(tau), 1.0)[None, :]
    inside = (dist <= win).any(axis=1)
    # a code may only be off by one level across the boundary it sits on
    off_by = np.abs(g[diff].astype(int) - r[diff].astype(int))
    outside = int((~inside).sum() + (off_by > 1).sum())
    return n_mis, outside, g.size


def assert_codes_match(gpu_packed, ref_packed, z_ref, d, bits, thr_unit, what=""):
    n_mis, outside, n = code_mismatch_report(gpu_packed, ref_packed, z_ref, d, bits, thr_unit)
    assert outside == 0, f"{what}: {outside} code mismatches outside the boundary window"
    assert n_mis <= CODE_MAX_FRAC * n, f"{what}: {n_mis}/{n} mismatches exceed 1e-4"
    return n_mis


def assert_norms_match(gpu, ref, what=""):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref)
    ok = err <= NORM_RTOL * np.abs(ref)
    assert ok.all(), f"{what}: norm rel err {np.max(err / np.maximum(ref, 1e-300)):.3e}"


def assert_rotated_match(z_gpu, z_ref, what=""):
    z_gpu = np.asarray(z_gpu, np.float64)
    dz = z_gpu - z_ref
    per_tok = np.linalg.norm(dz, axis=1)
    assert per_tok.max() <= ROT_TOL, f"{what}: max ||dz|| {per_tok.max():.3e}"
    mx = np.abs(z_ref).max(axis=1, keepdims=True)
    assert (np.abs(dz) <= ROT_TOL * np.maximum(mx, 1e-300)).all(), f"{what}: max |dz_i|"


def rel_fro(y, ref):
    y = np.asarray(y, np.float64)
    return float(np.linalg.norm(y - ref) / np.linalg.norm(ref))


def assert_dequant_match(gpu, ref, z_ref, d, thr_unit, what=""):
    """gpu: dequantized values (any float dtype) [R, d]; ref: oracle fp64."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    bad = np.abs(g - r) > DEQUANT_RTOL * np.abs(r)
    n_bad = int(bad.sum())
    if n_bad:
        u = np.sqrt(d) * z_ref[bad]
        tau = np.asarray(thr_unit, np.float64)
        dist = np.abs(u[:, None] - tau[None, :])
        win = CODE_WINDOW * np.maximum(np.abs(tau), 1.0)[None, :]
        outside = int((~(dist <= win).any(axis=1)).sum())
        assert outside == 0, f"{what}: {outside} dequantized values off outside the window"
    assert n_bad <= CODE_MAX_FRAC * g.size, f"{what}: {n_bad}/{g.size} values differ"
    return n_bad
