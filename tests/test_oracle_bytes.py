"""Pins of the oracle's byte arithmetic and packing against the numbers the pages
print (tests/golden/page_byte_facts.json) and against a brute-force packer."""
import json
import os

import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import fsq_oracle as orc
from oracle import bruteforce as bf


def load(golden_dir):
    return json.load(open(os.path.join(golden_dir, "page_byte_facts.json")))


def test_full_cache_bytes(golden_dir):
    g = load(golden_dir)
    assert orc.full_cache_bytes(n_kv=8, d_h=128) == g["full_cache_bytes_per_token_per_layer_qwen3"]["value"]
    f = g["qwen3_8b_cache_per_token_all_layers_KiB"]
    assert orc.full_cache_bytes(8, 128) * f["layers"] / 1024 == f["value"]


def test_qwen3_1p7b_200k_entries(golden_dir):
    f = load(golden_dir)["qwen3_1p7b_200k_entries_GiB"]
    gib = orc.full_cache_bytes(8, 128) * f["layers"] * f["entries"] / 2 ** 30
    assert round(gib) == f["value"]          # the page prints a rounded 21 GiB


def test_packed_bytes_and_ratios(golden_dir):
    g = load(golden_dir)
    p = g["packed_bytes_at_32x"]
    assert orc.bytes_per_token(p["G"]) == p["bytes"]
    full = orc.full_cache_bytes(8, 128)
    for r in g["compression_ratios"]:
        ratio = full / orc.bytes_per_token(r["G"])
        # pages print ratios to 3-4 significant digits (97.5 for 97.52, 51 for 51.2)
        assert abs(ratio - r["ratio"]) <= 0.005 * r["ratio"], (r, ratio)


def test_width_bytes_table(golden_dir):
    for row in load(golden_dir)["width_bytes_table"]:
        assert orc.bytes_per_token(row["width"], row["bits"]) == row["bytes"]


def test_bits_per_level_count(golden_dir):
    for row in load(golden_dir)["bits_per_level_count"]:
        if "levels" in row:
            assert int(np.ceil(np.log2(row["levels"]))) == row["bits"]


def test_bytes_per_token_odd_width():
    assert [orc.bytes_per_token(G) for G in (1, 2, 3, 63, 64, 83, 84)] == [1, 1, 2, 32, 32, 42, 42]


@settings(max_examples=100, deadline=None)
@given(st.integers(1, 40), st.integers(0, 5), st.randoms())
def test_pack_matches_bruteforce_and_roundtrips(G, N, r):
    codes = np.array([[r.randrange(16) for _ in range(G)] for _ in range(N)], dtype=np.uint8).reshape(N, G)
    packed = orc.pack_codes(codes)
    assert packed.shape == (N, orc.bytes_per_token(G))
    for t in range(N):
        assert bytes(packed[t]) == bf.pack_row(codes[t])
        assert bf.unpack_row(bytes(packed[t]), G) == codes[t].tolist()
    assert np.array_equal(orc.unpack_codes(packed, G), codes)


def test_pack_nibble_order():
    # byte j = code[2j] | code[2j+1] << 4; odd G leaves the last high nibble zero
    packed = orc.pack_codes(np.array([[1, 2, 3]], dtype=np.uint8))
    assert packed.tolist() == [[0x21, 0x03]]
