"""Pins for the oracle's bitstream packing (O2) and unpacking (O3)."""
import json
import os

import numpy as np
import pytest

import oracle as O

BITS = [2, 3, 4, 5, 6, 8]


def _load(golden_dir):
    with open(os.path.join(golden_dir, "pack_worked.json")) as f:
        return json.load(f)["cases"]


def test_worked_examples(golden_dir):
    for case in _load(golden_dir):
        codes = np.zeros((1, case["k"]), dtype=np.uint8)
        for idx, val in case["codes"].items():
            codes[0, int(idx)] = val
        want = np.array([int(w, 16) for w in case["words"]], dtype=np.uint32)
        got = O.pack(codes, case["bits"])[0]
        assert got.tolist() == want.tolist(), (case, [hex(v) for v in got])
        assert O.unpack(got[None, :], case["bits"], case["k"]).tolist() == codes.tolist()


def _bitstring_pack(codes_row, bits):
    """Independent brute force: write each code as `bits` binary digits, least significant
    first, into one long character string, then read 32-character slices back as words."""
    stream = "".join(format(int(c), "0%db" % bits)[::-1] for c in codes_row)
    return [int(stream[i:i + 32][::-1], 2) for i in range(0, len(stream), 32)]


@pytest.mark.parametrize("bits", BITS)
def test_matches_bitstring_packer(bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, size=(5, 128), dtype=np.uint8)
    got = O.pack(codes, bits)
    for r in range(codes.shape[0]):
        assert got[r].tolist() == _bitstring_pack(codes[r], bits)


@pytest.mark.parametrize("bits", BITS)
def test_unpack_inverts_pack(bits):
    rng = np.random.default_rng(100 + bits)
    codes = rng.integers(0, 1 << bits, size=(7, 256), dtype=np.uint8)
    words = O.pack(codes, bits)
    assert words.shape == (7, 256 * bits // 32)
    assert np.array_equal(O.unpack(words, bits, 256), codes)


@pytest.mark.parametrize("bits", [4, 8])
def test_four_and_eight_bit_match_report_formula(bits):
    """[bits8-report] 3.1: word = g*(gs/(32/bits)) + inG/(32/bits), shift = (inG % (32/bits))*bits."""
    per_word = 32 // bits
    rng = np.random.default_rng(bits)
    gs = 64
    codes = rng.integers(0, 1 << bits, size=(3, 256), dtype=np.uint8)
    words = O.pack(codes, bits)
    mask = (1 << bits) - 1
    for n in range(3):
        for k in range(256):
            g, in_g = divmod(k, gs)
            idx = g * (gs // per_word) + in_g // per_word
            shift = (in_g % per_word) * bits
            assert (int(words[n, idx]) >> shift) & mask == codes[n, k]


def test_chunk_of_32_codes_fills_whole_words():
    """32 codes of `bits` bits occupy exactly `bits` words, so chunks never share a word."""
    for bits in BITS:
        codes = np.zeros((1, 64), dtype=np.uint8)
        codes[0, 32:] = (1 << bits) - 1
        words = O.pack(codes, bits)[0]
        assert all(w == 0 for w in words[:bits])
        assert all(w == 0xFFFFFFFF for w in words[bits:])
