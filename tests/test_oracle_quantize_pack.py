"""Pins for nearest-level quantization, the storage slot order and packing.

Pages: llmdb.app Implementation Details (activations rotated, then quantized
with the fixed Lloyd-Max codebook); paper.gecl.asia notes, Core Idea.  The
tie rule, code encoding, slot order and bit packing are readings (the pages
are silent) and are pinned by brute force and hand-built vectors.
"""
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_quantize_is_nearest_level_by_brute_force(bits):
    d = 3072
    lv, th = oracle.codebook(d, bits)
    rng = np.random.default_rng(bits)
    zs = list(rng.standard_normal(2000) / np.sqrt(d) * 1.5)
    zs += [0.0, -0.0, 10.0, -10.0]
    for z in zs:
        got = oracle.quantize_one(z, th)
        dist = [abs(z - c) for c in lv]
        best = min(dist)
        cand = [k for k in range(len(lv)) if dist[k] == best]
        assert got == max(cand)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_ties_go_up_and_signed_zero(bits):
    lv, th = oracle.codebook(256, bits)
    L = 1 << bits
    for k, t in enumerate(th):
        assert oracle.quantize_one(t, th) == k + 1          # exactly on tau_{k+1}
        assert oracle.quantize_one(np.nextafter(t, -1), th) == k
    assert oracle.quantize_one(0.0, th) == L // 2
    assert oracle.quantize_one(-0.0, th) == L // 2


def test_slot_order_is_a_bijection_inside_each_group():
    slots = [oracle.slot_of(i, 512) for i in range(512)]
    for g in range(4):
        assert sorted(slots[128 * g:128 * g + 128]) == list(range(128 * g, 128 * g + 128))
    # hand-worked entries: coordinate 32c + p -> 8 (p mod 16) + 4 (p div 16) + c
    assert [oracle.slot_of(i, 512) for i in (0, 1, 16, 31, 32, 33, 127, 128, 161)] == \
        [0, 8, 4, 124, 1, 9, 127, 128, 137]


@pytest.mark.parametrize("d", [32, 64, 96, 160, 224, 352, 16352])
def test_partial_last_group_keeps_coordinate_order(d):
    """Rows whose length is not a multiple of 128: the whole groups keep the
    group order, the last 32, 64 or 96 coordinates sit at their own index,
    and the whole row is a bijection onto its d slots."""
    slots = np.array([oracle.slot_of(i, d) for i in range(d)])
    full = (d // 128) * 128
    assert np.array_equal(np.sort(slots), np.arange(d))
    assert np.array_equal(slots[full:], np.arange(full, d))
    for i in range(0, full, 37):
        assert slots[i] == oracle.slot_of(i, full + 128)


def _load_pack_golden():
    cases = []
    with open(os.path.join(GOLD, "pack_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            bits, codes, hexbytes = [s.strip() for s in line.split("|")]
            raw = bytearray()
            for tok in hexbytes.split():
                if "*" in tok:
                    v, n = tok.split("*")
                    raw += bytes.fromhex(v) * int(n)
                else:
                    raw += bytes.fromhex(tok)
            cases.append((int(bits), codes, bytes(raw)))
    return cases


def _expand(codes_spec):
    """'i:v i:v ... @ rest=v' -> 128 codes in coordinate order."""
    head, _, rest = codes_spec.partition("@")
    fill = int(rest.split("=")[1]) if rest else 0
    codes = np.full(128, fill, np.uint8)
    for tok in head.split():
        i, v = tok.split(":")
        codes[int(i)] = int(v)
    return codes


def test_pack_hand_built_vectors():
    for bits, spec, expect in _load_pack_golden():
        codes = _expand(spec)
        got = oracle.pack_row(codes, bits)
        assert got.tobytes() == expect, (bits, spec)


def _hex_bytes(spec):
    raw = bytearray()
    for tok in spec.split():
        if "*" in tok:
            v, n = tok.split("*")
            raw += bytes.fromhex(v) * int(n)
        else:
            raw += bytes.fromhex(tok)
    return bytes(raw)


def test_pack_hand_built_partial_groups():
    """Rows of 32, 96, 160 and 224 coordinates (a partial last group of 32,
    96, 32 and 96), worked by hand from the slot rule."""
    n = 0
    with open(os.path.join(GOLD, "pack_examples_partial.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            d, bits, spec, hexbytes = [t.strip() for t in line.split("|")]
            d, bits = int(d), int(bits)
            codes = np.zeros(d, np.uint8)
            for tok in spec.split():
                i, v = tok.split(":")
                codes[int(i)] = int(v)
            expect = _hex_bytes(hexbytes)
            assert len(expect) == d * bits // 8
            got = oracle.pack_row(codes, bits)
            assert got.tobytes() == expect, (d, bits, spec)
            assert np.array_equal(oracle.unpack_row(got, d, bits), codes)
            n += 1
    assert n == 5


@pytest.mark.parametrize("d", [384, 416])
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_pack_unpack_roundtrip(bits, d):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, d).astype(np.uint8)
    packed = oracle.pack_row(codes, bits)
    assert packed.shape[0] == d * bits // 8
    assert np.array_equal(oracle.unpack_row(packed, d, bits), codes)


def test_eight_bit_codes_are_whole_bytes_in_slot_order():
    """At 8 bits the little-endian bitstream is plain byte addressing: byte
    slot(i) of the row is the code of coordinate i."""
    rng = np.random.default_rng(8)
    d = 256
    codes = rng.integers(0, 256, d).astype(np.uint8)
    packed = oracle.pack_row(codes, 8)
    assert packed.shape[0] == d
    for i in range(d):
        assert packed[oracle.slot_of(i, d)] == codes[i]


def test_eight_bit_quantize_matches_sorted_search():
    """#{k : z >= tau_k} is the insertion index of z after equal keys."""
    lv, th = oracle.codebook(3072, 8)
    rng = np.random.default_rng(5)
    zs = np.concatenate([rng.standard_normal(3000) / np.sqrt(3072) * 1.3, th, -th[:5],
                         [0.0, 1.0, -1.0]])
    want = np.searchsorted(th, zs, side="right")
    got = np.array([oracle.quantize_one(z, th) for z in zs])
    assert np.array_equal(got, want)
