"""Pins for the oracle's low-bit linear and the whole oracle pipeline.

Pages: llmdb.app Mathematical Formulation (y_hat = Q_w(W R^-1) Q_a(R x),
bias-free layer); paper.gecl.asia notes, Method items 1-2 (norm s per token,
row norm r per weight row, shared rotated basis); hotpaper.ai abstract (the
same quantizer on weight rows, offline).
Pinned against: a brute-force triple loop on tiny shapes, the closed form for
all-top-level codes, and the unquantised limit (exact cancellation to W x)
plus the known quantizer distortion at high bit widths.
"""
import numpy as np
import pytest

import oracle
import workloads as wl


@pytest.mark.parametrize("ba,bw,K", [(4, 4, 128), (4, 2, 128), (3, 2, 128), (4, 3, 128),
                                     (2, 2, 128), (8, 8, 128), (4, 4, 96), (3, 4, 192),
                                     (8, 8, 160)])
def test_linear_brute_force_tiny(ba, bw, K):
    M, N = 3, 5
    ac, an = wl.random_codes(M, K, ba, 1)
    wc, wn = wl.random_codes(N, K, bw, 2)
    la, _ = oracle.codebook(K, ba)
    lw, _ = oracle.codebook(K, bw)
    y = oracle.linear(ac, an, ba, wc, wn, bw, K)
    for m in range(M):
        qa = oracle.unpack_row(ac[m], K, ba)
        for n in range(N):
            pw = oracle.unpack_row(wc[n], K, bw)
            acc = 0.0
            for k in range(K):
                acc += la[qa[k]] * lw[pw[k]]
            ref = float(an[m]) * float(wn[n]) * acc
            assert abs(y[m, n] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_linear_all_top_codes_closed_form():
    K, ba, bw = 384, 4, 2
    a = oracle.pack_row(np.full(K, 15, np.uint8), ba)[None, :]
    w = oracle.pack_row(np.full(K, 3, np.uint8), bw)[None, :]
    la, _ = oracle.codebook(K, ba)
    lw, _ = oracle.codebook(K, bw)
    y = oracle.linear(a, np.array([2.0]), ba, w, np.array([0.5]), bw, K)
    assert abs(y[0, 0] - 2.0 * 0.5 * K * la[-1] * lw[-1]) < 1e-12


def test_linear_sampled_rows_match_full():
    M, N, K = 40, 24, 256
    ac, an = wl.random_codes(M, K, 4, 3)
    wc, wn = wl.random_codes(N, K, 4, 4)
    full = oracle.linear(ac, an, 4, wc, wn, 4, K)
    rows = np.array([0, 7, 39])
    part = oracle.linear(ac, an, 4, wc, wn, 4, K, rows=rows)
    assert np.array_equal(full[rows], part)


def test_pipeline_approaches_exact_product_as_bits_grow():
    """Quantised output -> W x as the codebooks get finer: the relative error
    at W4A4 sits near the two quantizers' distortions combined and shrinks
    from 2 to 4 bits.  (Unquantised cancellation is pinned exactly in the
    rotation tests.)"""
    d, M, N, seed = 512, 64, 48, 17
    rng = np.random.default_rng(0)
    x = rng.standard_normal((M, d)).astype(np.float32)
    W = (rng.standard_normal((N, d)) * 0.02).astype(np.float32)
    ref = x.astype(np.float64) @ W.astype(np.float64).T
    errs = {}
    for b in (2, 3, 4, 8):
        ac, an, _ = oracle.rotate_quantize(x, oracle.F32, d, seed, b)
        wc, wn, _ = oracle.rotate_quantize(W, oracle.F32, d, seed, b)
        y = oracle.linear(ac, an, b, wc, wn, b, d)
        errs[b] = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert errs[2] > errs[3] > errs[4] > errs[8]
    # 8 bits: distortion 4.1e-5 (near Panter-Dite), same sqrt(2 D) law
    assert 0.5 * np.sqrt(2 * 4.12e-5) < errs[8] < 2.0 * np.sqrt(2 * 4.12e-5)
    # unit-variance Lloyd-Max distortions: 0.1175 (2b), 0.0345 (3b), 0.0095 (4b);
    # cosine error of each factor ~ distortion, so the product error ~ sqrt(2 D)
    assert 0.5 * np.sqrt(2 * 0.0095) < errs[4] < 2.0 * np.sqrt(2 * 0.0095)
