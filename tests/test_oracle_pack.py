"""Pins for the oracle's bit packing and the storage arithmetic (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle.pack import words_per_row


def test_pack_layout_hand_derived(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "pack_layout.json")))
    for case in g["cases"]:
        codes = np.array([case["codes"]])
        words = oracle.pack_ref(codes, case["bits"])
        assert [int(x) for x in words[0]] == [int(w, 16) for w in case["words"]], case


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 8])
@pytest.mark.parametrize("n", [1, 7, 31, 33, 100])
def test_pack_roundtrip(bits, n):
    rng = np.random.default_rng(bits * 100 + n)
    codes = rng.integers(0, 2 ** bits, (5, n))
    packed = oracle.pack_ref(codes, bits)
    assert packed.shape == (5, words_per_row(n, bits))
    assert np.array_equal(oracle.unpack_ref(packed, n, bits), codes)


def test_single_code_bit_positions_brute_force():
    for bits in (3, 4):
        n = 40
        for c in range(n):
            codes = np.zeros((1, n), dtype=np.int64)
            codes[0, c] = 1
            packed = oracle.pack_ref(codes, bits)
            set_bits = [32 * w + k for w in range(packed.shape[1]) for k in range(32)
                        if (int(packed[0, w]) >> k) & 1]
            assert set_bits == [c * bits]


def test_bits_per_weight_matches_printed_values(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "bits_per_weight.json")))
    n = 4096
    for G, expect in g["bits_per_weight"].items():
        G = int(G)
        packed_bits = words_per_row(n, g["bits"]) * 32
        meta_bits = (n // G) * g["group_metadata_bits"]
        assert (packed_bits + meta_bits) / n == pytest.approx(expect)


def test_model_sizes_match_printed_values(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "model_sizes_175b.json")))
    for bits, gb in g["gigabytes"].items():
        size = g["params"] * int(bits) / 8 / 1e9
        assert round(size, g["printed_decimals"]) == pytest.approx(gb, abs=0.05)
