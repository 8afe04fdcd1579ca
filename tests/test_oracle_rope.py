"""Pins of the oracle's Eq. 5 keys in full, k^_t = RoPE_t(N_k(W_k z_t))
(decode_attn_rope, rope, rms_norm): closed-form rotations, the algebra that
defines a rotary embedding (norm kept, angles add, scores depend on relative
position), the RMS norm's closed forms, torch's SDPA in float64 on explicitly
built keys, and special cases. The constants gamma, eps and theta are
readings (the pages do not fix them)."""
import math

import numpy as np
import pytest
import torch

from oracle import fsq_oracle as orc


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("t", [0, 1, 3, 17, 1000])
def test_rope_2d_is_the_plane_rotation_by_t(t):
    # d_h = 2: one channel pair at frequency theta^0 = 1, so the angle is t
    out = orc.rope(np.array([[1.0, 0.0], [0.0, 1.0]]), [t, t], theta=1e6)
    assert np.allclose(out[0], [math.cos(t), math.sin(t)], atol=1e-15)
    assert np.allclose(out[1], [-math.sin(t), math.cos(t)], atol=1e-15)


def test_rope_4d_pairs_and_frequencies():
    # d_h = 4, theta = 100: pairs (0, 2) at angle t and (1, 3) at t * 100^(-1/2) = t / 10
    k = np.array([[1.0, 2.0, 3.0, 4.0]])
    t = 7
    out = orc.rope(k, [t], theta=100.0)[0]
    a0, a1 = t, t / 10.0
    exp = [1 * math.cos(a0) - 3 * math.sin(a0), 2 * math.cos(a1) - 4 * math.sin(a1),
           3 * math.cos(a0) + 1 * math.sin(a0), 4 * math.cos(a1) + 2 * math.sin(a1)]
    assert np.allclose(out, exp, atol=1e-13)


def test_rope_keeps_norms_and_angles_add():
    g = np.random.default_rng(1)
    k = g.standard_normal((5, 16))
    pos = np.array([0, 3, 10, 999, 123456])
    r = orc.rope(k, pos, theta=1e6)
    assert np.allclose(np.linalg.norm(r, axis=1), np.linalg.norm(k, axis=1), rtol=1e-13)
    r2 = orc.rope(orc.rope(k, pos, 1e6), pos + 7, 1e6)
    assert np.allclose(r2, orc.rope(k, 2 * pos + 7, 1e6), atol=1e-9)


def test_rope_scores_depend_only_on_relative_position():
    g = np.random.default_rng(2)
    a, b = g.standard_normal((1, 32)), g.standard_normal((1, 32))
    for t, s, c in [(10, 3, 100), (0, 0, 5000), (77, 900, 13)]:
        x = (orc.rope(a, [t], 1e4) * orc.rope(b, [s], 1e4)).sum()
        y = (orc.rope(a, [t + c], 1e4) * orc.rope(b, [s + c], 1e4)).sum()
        assert abs(x - y) < 1e-9 * max(1.0, abs(x))


def test_rms_norm_closed_forms():
    g = np.random.default_rng(3)
    k = g.standard_normal((4, 64)) * 3.0
    ms = np.mean(k * k, axis=1)
    y = orc.rms_norm(k, np.ones(64), 1e-6)
    assert np.allclose(np.mean(y * y, axis=1), ms / (ms + 1e-6), rtol=1e-13)
    # scale invariance (eps = 0) and the per-channel gain
    gam = g.standard_normal(64)
    assert np.allclose(orc.rms_norm(5.0 * k, gam, 0.0), orc.rms_norm(k, gam, 0.0), rtol=1e-12)
    assert np.allclose(orc.rms_norm(k, gam, 0.0) / orc.rms_norm(k, np.ones(64), 0.0), gam)


def case(seed, B=1, n_q=8, n_kv=2, d_h=16, G=12, T=29):
    g = np.random.default_rng(seed)
    q = g.standard_normal((B, n_q, d_h))
    W = g.standard_normal((2 * n_kv * d_h, G)) / math.sqrt(G)
    codes = g.integers(0, 16, size=(B, T, G)).astype(np.uint8)
    packed = np.stack([orc.pack_codes(codes[b]) for b in range(B)])
    gam = 1.0 + 0.1 * g.standard_normal(d_h)
    return q, W, codes, packed, gam


@pytest.mark.parametrize("seed", range(3))
def test_rope_decode_matches_torch_sdpa_on_built_keys(seed):
    n_q, n_kv, d_h, G, T = 8, 2, 16, 12, 29
    q, W, codes, packed, gam = case(seed, n_q=n_q, n_kv=n_kv, d_h=d_h, G=G, T=T)
    Z = codes[0].astype(np.float64) - 8.0
    Ks, Vs = [], []
    for g_ in range(n_kv):
        K = Z @ W[g_ * d_h:(g_ + 1) * d_h].T
        K = orc.rope(orc.rms_norm(K, gam, 1e-6), np.arange(T), 1e4)
        Ks.append(K)
        Vs.append(Z @ W[n_kv * d_h + g_ * d_h:n_kv * d_h + (g_ + 1) * d_h].T)
    grp = n_q // n_kv
    K = torch.tensor(np.stack(Ks)).repeat_interleave(grp, dim=0)
    V = torch.tensor(np.stack(Vs)).repeat_interleave(grp, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.tensor(q[0]).unsqueeze(1), K, V)
    out = orc.decode_attn_rope(q, packed, W, [T], n_kv, G, gam, 1e-6, 1e4)[0]
    assert rel(out, ref.squeeze(1).numpy()) < 1e-12


def test_rope_decode_single_token_is_its_value():
    q, W, codes, packed, gam = case(4, T=1)
    out = orc.decode_attn_rope(q, packed, W, [1], 2, 12, gam, 1e-6, 1e6)
    z = codes[0, 0].astype(np.float64) - 8.0
    for h in range(8):
        g_ = h // 4
        assert np.allclose(out[0, h], W[2 * 16 + g_ * 16:2 * 16 + (g_ + 1) * 16] @ z, rtol=1e-12)


def test_rope_decode_differs_from_plain_keys_and_zero_length():
    q, W, codes, packed, gam = case(5, B=2, T=40)
    a = orc.decode_attn_rope(q, packed, W, [40, 0], 2, 12, gam, 1e-6, 1e4)
    b = orc.decode_attn(q, packed, W, [40, 0], 2, 12)
    assert rel(a[0], b[0]) > 1e-3          # norm and rotation change the scores
    assert np.all(a[1] == 0)


# --------------------------------------------------------------- mutants
def _rope_pins_hold(rope_fn):
    """The closed-form RoPE pins above, as one predicate over a rope function."""
    for t in [1, 3, 17]:
        out = rope_fn(np.array([[1.0, 0.0], [0.0, 1.0]]), [t, t], 1e6)
        if not (np.allclose(out[0], [math.cos(t), math.sin(t)], atol=1e-12)
                and np.allclose(out[1], [-math.sin(t), math.cos(t)], atol=1e-12)):
            return False
    k, t = np.array([[1.0, 2.0, 3.0, 4.0]]), 7
    a0, a1 = t, t / 10.0
    exp = [1 * math.cos(a0) - 3 * math.sin(a0), 2 * math.cos(a1) - 4 * math.sin(a1),
           3 * math.cos(a0) + 1 * math.sin(a0), 4 * math.cos(a1) + 2 * math.sin(a1)]
    return bool(np.allclose(rope_fn(k, [t], 100.0)[0], exp, atol=1e-12))


def _rope_interleaved(k, positions, theta):
    # pairs (2i, 2i + 1) instead of (i, i + d_h/2)
    k = np.asarray(k, dtype=np.float64)
    d_h = k.shape[-1]
    inv = theta ** (-2.0 * np.arange(d_h // 2) / d_h)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    a, b = k[..., 0::2], k[..., 1::2]
    out = np.empty_like(k)
    out[..., 0::2] = a * np.cos(ang) - b * np.sin(ang)
    out[..., 1::2] = b * np.cos(ang) + a * np.sin(ang)
    return out


def _rope_mutant(kind):
    def fn(k, positions, theta):
        k = np.asarray(k, dtype=np.float64)
        d_h = k.shape[-1]
        half = d_h // 2
        e = np.arange(half, dtype=np.float64)
        inv = theta ** (-(e if kind == "freq_exponent" else 2.0 * e) / d_h)
        ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
        c, s = np.cos(ang), np.sin(ang)
        if kind == "sign":
            s = -s
        a, b = k[..., :half], k[..., half:]
        return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
    return fn


def test_rope_pins_hold_for_the_oracle():
    assert _rope_pins_hold(orc.rope)


@pytest.mark.parametrize("kind", ["interleaved", "sign", "freq_exponent"])
def test_rope_pins_catch_planted_mistakes(kind):
    fn = _rope_interleaved if kind == "interleaved" else _rope_mutant(kind)
    assert not _rope_pins_hold(fn)


def _rms_pins_hold(fn):
    g = np.random.default_rng(3)
    k = g.standard_normal((4, 64)) * 3.0
    ms = np.mean(k * k, axis=1)
    gam = g.standard_normal(64)
    return bool(np.allclose(np.mean(fn(k, np.ones(64), 1e-6) ** 2, axis=1), ms / (ms + 1e-6), rtol=1e-13)
                and np.allclose(fn(k, gam, 0.0) / fn(k, np.ones(64), 0.0), gam))


@pytest.mark.parametrize("kind", ["sum_not_mean", "no_gamma", "eps_outside", "gamma_inverted"])
def test_rms_norm_pins_catch_planted_mistakes(kind):
    def fn(k, gamma, eps):
        k = np.asarray(k, dtype=np.float64)
        gamma = np.asarray(gamma, dtype=np.float64)
        if kind == "sum_not_mean":
            return k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps) * gamma
        ms = np.mean(k * k, axis=-1, keepdims=True)
        if kind == "no_gamma":
            return k / np.sqrt(ms + eps)
        if kind == "eps_outside":
            return k / (np.sqrt(ms) + eps) * gamma
        return k / np.sqrt(ms + eps) / gamma
    assert _rms_pins_hold(orc.rms_norm)
    assert not _rms_pins_hold(fn)
