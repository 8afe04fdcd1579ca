"""Pins of the oracle at L = 4 and 256 levels per coordinate (2 and 8 bits;
the slides' backup frame "the grid size is an allocation choice"): closed-form
level thresholds of Eq. 2 with the reading h = 1.001 (L - 1) / 2, invariants,
packing round trips and hand-worked bytes, the backup table's bytes-per-token
arithmetic, and the latent decode against materialised K/V at these widths."""
import math

import numpy as np
import pytest

from oracle import fsq_oracle as orc


@pytest.mark.parametrize("L", [4, 16, 256])
def test_level_thresholds_closed_form(L):
    h = orc.H_BOUND if L == 16 else orc.h_of_levels(L)
    s = math.atanh(0.5 / h)
    for k in range(-L // 2, L // 2 - 1):
        u = math.atanh((k + 1) / h) - s          # u~ = k + 1/2 exactly here
        assert orc.fsq_levels(np.array([u - 1e-9]), L)[0] == k
        assert orc.fsq_levels(np.array([u + 1e-9]), L)[0] == k + 1


def test_h_reading_reproduces_the_printed_value():
    assert abs(orc.h_of_levels(16) - 7.5075) < 1e-12


@pytest.mark.parametrize("L", [4, 256])
def test_h_reading_gives_exactly_L_levels(L):
    """h at L = 4 and 256 is a reading and its exact value is parity unpinned:
    the pages print h only for L = 16. What they do fix is that Eq. 2 rounds a
    coordinate to L levels; with delta = 1/2 that holds exactly when h lies in
    (L/2 - 1, L/2]. The reading lies there, and an h just outside gives a
    different number of levels (so the pin fails a reading that does not
    produce an L-level grid, but not one that moves h inside the interval)."""
    h = orc.h_of_levels(L)
    assert L / 2 - 1 < h <= L / 2
    u = np.linspace(-15.0, 15.0, 300001)        # tanh < 1 strictly: the range of u~ stays open

    def count(hh):
        return len(np.unique(np.rint(orc.fsq_bound(u, h=hh))))

    assert count(h) == L
    assert count(L / 2) == L
    assert count(L / 2 + 0.05) != L
    assert count(L / 2 - 1 - 0.05) != L


@pytest.mark.parametrize("L", [4, 256])
def test_level_invariants(L):
    u = np.linspace(-12, 12, 200001)
    c = orc.fsq_codes(u, L)
    assert c.min() == 0 and c.max() == L - 1
    assert len(np.unique(c)) == L                # all L levels are reached (Eq. 3 grid per coordinate)
    assert np.all(np.diff(c.astype(int)) >= 0)   # monotone
    assert orc.fsq_codes(np.array([0.0]), L)[0] == L // 2


def test_pack_bytes_by_hand():
    # 2 bits: byte = c0 | c1 << 2 | c2 << 4 | c3 << 6; the last byte's unused bits are zero
    assert orc.pack_codes(np.array([[1, 2, 3, 0, 3]], np.uint8), bits=2).tolist() == [[1 + 8 + 48, 3]]
    # 8 bits: one code per byte
    assert orc.pack_codes(np.array([[200, 7, 255]], np.uint8), bits=8).tolist() == [[200, 7, 255]]
    with pytest.raises(AssertionError):
        orc.pack_codes(np.array([[4]], np.uint8), bits=2)


@pytest.mark.parametrize("bits,G", [(2, 1), (2, 7), (2, 64), (8, 5), (8, 84)])
def test_pack_round_trip(bits, G):
    g = np.random.default_rng(G * bits)
    codes = g.integers(0, 1 << bits, size=(9, G)).astype(np.uint8)
    packed = orc.pack_codes(codes, bits)
    assert packed.shape == (9, orc.bytes_per_token(G, bits))
    assert np.array_equal(orc.unpack_codes(packed, G, bits), codes)


def test_backup_table_bytes_per_token():
    # levels 4 / 16 / 256 -> bits per coordinate 2 / 4 / 8 (backup table), so a
    # fixed 144- or 80-byte budget buys G = 576 / 288 / 144 or 320 / 160 / 80
    for L, bits in [(4, 2), (16, 4), (256, 8)]:
        assert orc.bits_of_levels(L) == bits == int(math.log2(L))
        assert orc.bytes_per_token(144 * 8 // bits, bits) == 144
        assert orc.bytes_per_token(80 * 8 // bits, bits) == 80


@pytest.mark.parametrize("L", [4, 256])
def test_latent_decode_equals_materialised_at_other_widths(L):
    g = np.random.default_rng(L)
    B, n_q, n_kv, d_h, G, T = 2, 8, 2, 16, 13, 31
    q = g.standard_normal((B, n_q, d_h))
    W = g.standard_normal((2 * n_kv * d_h, G)) / math.sqrt(G)
    bits = orc.bits_of_levels(L)
    codes = g.integers(0, L, size=(B, T, G)).astype(np.uint8)
    packed = np.stack([orc.pack_codes(codes[b], bits) for b in range(B)])
    a = orc.decode_attn(q, packed, W, [T, 5], n_kv, G, levels=L)
    b = orc.decode_attn_materialised(q, packed, W, [T, 5], n_kv, G, levels=L)
    assert np.linalg.norm(a - b) / np.linalg.norm(b) < 1e-12
    # zero query: uniform weights, out = W_v mean(z), z = code - L/2
    out = orc.decode_attn(np.zeros_like(q), packed, W, [T, T], n_kv, G, levels=L)
    z = codes[0].astype(np.float64) - L // 2
    Wv0 = W[n_kv * d_h:n_kv * d_h + d_h]
    assert np.allclose(out[0, 0], Wv0 @ z.mean(axis=0), rtol=1e-12)
