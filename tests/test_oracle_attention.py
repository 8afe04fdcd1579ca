"""Pins of the oracle's latent-space decode (Eq. 5-6 with the absorbed query)
against materialised K/V attention, torch's SDPA in float64 on the CPU,
special cases with closed-form answers, and a pure-Python loop oracle."""
import math

import numpy as np
import pytest
import torch

from oracle import fsq_oracle as orc
from oracle import bruteforce as bf


def make(seed, B=2, n_q=4, n_kv=2, d_h=8, G=6, cap=20, lens=None):
    g = np.random.Generator(np.random.PCG64(seed))
    q = g.standard_normal((B, n_q, d_h))
    W = g.standard_normal((2 * n_kv * d_h, G)) / math.sqrt(G)
    codes = g.integers(0, 16, size=(B, cap, G)).astype(np.uint8)
    packed = np.stack([orc.pack_codes(codes[b]) for b in range(B)])
    lens = np.array(lens if lens is not None else [cap] * B, dtype=np.int32)
    return q, packed, W, lens, codes


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("seed", range(5))
def test_latent_equals_materialised(seed):
    q, packed, W, lens, _ = make(seed, B=3, n_q=8, n_kv=2, d_h=16, G=11, cap=37, lens=[37, 5, 1])
    a = orc.decode_attn(q, packed, W, lens, n_kv=2, G=11)
    b = orc.decode_attn_materialised(q, packed, W, lens, n_kv=2, G=11)
    assert rel(a, b) < 1e-12


@pytest.mark.parametrize("seed", range(3))
def test_matches_torch_sdpa_float64(seed):
    n_q, n_kv, d_h, G, T = 8, 2, 16, 12, 29
    q, packed, W, lens, codes = make(seed, B=1, n_q=n_q, n_kv=n_kv, d_h=d_h, G=G, cap=T)
    Z = torch.tensor(codes[0].astype(np.float64) - 8.0)                   # [T, G]
    Wt = torch.tensor(W)
    K = (Z @ Wt[: n_kv * d_h].T).reshape(T, n_kv, d_h).permute(1, 0, 2)  # [n_kv, T, d_h]
    V = (Z @ Wt[n_kv * d_h:].T).reshape(T, n_kv, d_h).permute(1, 0, 2)
    grp = n_q // n_kv
    K = K.repeat_interleave(grp, dim=0)
    V = V.repeat_interleave(grp, dim=0)
    Q = torch.tensor(q[0]).unsqueeze(1)                                   # [n_q, 1, d_h]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V).squeeze(1).numpy()
    out = orc.decode_attn(q, packed, W, lens, n_kv=n_kv, G=G)[0]
    assert rel(out, ref) < 1e-12


def test_bruteforce_loops_match():
    q, packed, W, lens, _ = make(11, B=2, n_q=4, n_kv=2, d_h=4, G=5, cap=7, lens=[7, 3])
    out = orc.decode_attn(q, packed, W, lens, n_kv=2, G=5)
    Wl = W.tolist()
    for b in range(2):
        rows = [bytes(packed[b, t]) for t in range(int(lens[b]))]
        for h in range(4):
            ref = bf.decode_head(q[b, h].tolist(), rows, Wl, n_kv=2, n_q=4, h=h, G=5)
            assert np.allclose(out[b, h], ref, rtol=1e-12, atol=1e-12)


def test_single_token_is_value_of_that_token():
    q, packed, W, _, codes = make(2, B=1, n_q=4, n_kv=2, d_h=8, G=6, cap=1)
    out = orc.decode_attn(q, packed, W, np.array([1]), n_kv=2, G=6)
    z = codes[0, 0].astype(np.float64) - 8
    for h in range(4):
        _, Wv = orc.decoder_blocks(W, h // 2, 2, 8)
        assert np.allclose(out[0, h], Wv @ z, rtol=0, atol=1e-13)


def test_all_tokens_equal_gives_that_value_for_any_query():
    q, packed, W, _, codes = make(3, B=1, n_q=4, n_kv=2, d_h=8, G=6, cap=9)
    packed[0, :] = packed[0, 4]
    z = codes[0, 4].astype(np.float64) - 8
    out = orc.decode_attn(q * 37.0, packed, W, np.array([9]), n_kv=2, G=6)
    for h in range(4):
        _, Wv = orc.decoder_blocks(W, h // 2, 2, 8)
        assert np.allclose(out[0, h], Wv @ z, atol=1e-12)


def test_zero_query_averages_codes():
    q, packed, W, lens, codes = make(4, B=1, n_q=4, n_kv=2, d_h=8, G=6, cap=13)
    out = orc.decode_attn(np.zeros_like(q), packed, W, lens, n_kv=2, G=6)
    zmean = (codes[0].astype(np.float64) - 8).mean(axis=0)
    for h in range(4):
        _, Wv = orc.decoder_blocks(W, h // 2, 2, 8)
        assert np.allclose(out[0, h], Wv @ zmean, atol=1e-12)


def test_dominant_token_selected():
    """A query whose absorbed form is a large multiple of one token's code,
    with that token's code the unique maximiser of q~.z, returns that token's value."""
    G, d_h, n_kv, n_q = 4, 8, 1, 1
    codes = np.array([[15, 0, 15, 0], [0, 15, 0, 15], [8, 8, 8, 8], [3, 12, 7, 9]], dtype=np.uint8)
    packed = orc.pack_codes(codes)[None]
    Wk = np.zeros((d_h, G)); Wk[:G, :G] = np.eye(G)
    Wv = np.random.Generator(np.random.PCG64(5)).standard_normal((d_h, G))
    W = np.concatenate([Wk, Wv])
    z0 = codes[0].astype(np.float64) - 8
    q = np.zeros((1, 1, d_h)); q[0, 0, :G] = 50.0 * z0        # q~ = Wk^T q = 50 z0
    out = orc.decode_attn(q, packed, W, np.array([4]), n_kv=n_kv, G=G)
    assert np.allclose(out[0, 0], Wv @ z0, atol=1e-9)


def test_token_permutation_invariance():
    q, packed, W, lens, _ = make(6, B=1, n_q=4, n_kv=2, d_h=8, G=7, cap=23)
    perm = np.random.Generator(np.random.PCG64(1)).permutation(23)
    a = orc.decode_attn(q, packed, W, lens, n_kv=2, G=7)
    b = orc.decode_attn(q, packed[:, perm], W, lens, n_kv=2, G=7)
    assert rel(a, b) < 1e-13


def test_gqa_heads_with_equal_query_are_equal():
    q, packed, W, lens, _ = make(7, B=1, n_q=8, n_kv=2, d_h=8, G=6, cap=15)
    q[0, 1] = q[0, 0]     # heads 0, 1 share kv head 0
    q[0, 4] = q[0, 0]     # head 4 reads kv head 1: must differ in general
    out = orc.decode_attn(q, packed, W, lens, n_kv=2, G=6)
    assert np.array_equal(out[0, 0], out[0, 1])
    assert not np.allclose(out[0, 0], out[0, 4])


def test_zero_length_gives_zero():
    q, packed, W, _, _ = make(8, B=2, cap=5)
    out = orc.decode_attn(q, packed, W, np.array([0, 5]), n_kv=2, G=6)
    assert np.all(out[0] == 0) and np.any(out[1] != 0)


@pytest.mark.parametrize("bounds", [[0, 64], [0, 1, 64], [0, 7, 8, 30, 64], list(range(0, 65, 4)), [0, 50, 64]])
def test_split_merge_equals_direct(bounds):
    q, packed, W, lens, _ = make(9, B=2, n_q=4, n_kv=2, d_h=8, G=9, cap=64, lens=[64, 31])
    a = orc.decode_attn(q, packed, W, lens, n_kv=2, G=9)
    b = orc.decode_partials(q, packed, W, lens, n_kv=2, G=9, bounds=bounds)
    assert rel(a, b) < 1e-13


def test_scale_and_gqa_mistakes_are_caught():
    """Planted mistakes (missing 1/sqrt(d_h), wrong kv-head map) change the
    output enough that the SDPA pin above would fail."""
    q, packed, W, lens, _ = make(10, B=1, n_q=4, n_kv=2, d_h=16, G=8, cap=40)
    good = orc.decode_attn(q, packed, W, lens, n_kv=2, G=8)
    orig_sqrt = math.sqrt
    try:
        orc.math.sqrt = lambda x: 1.0
        bad = orc.decode_attn(q, packed, W, lens, n_kv=2, G=8)
    finally:
        orc.math.sqrt = orig_sqrt
    assert rel(bad, good) > 1e-3
    orig = orc._kv_head
    try:
        orc._kv_head = lambda h, n_q, n_kv: h % n_kv
        bad = orc.decode_attn(q, packed, W, lens, n_kv=2, G=8)
    finally:
        orc._kv_head = orig
    assert rel(bad, good) > 1e-3
