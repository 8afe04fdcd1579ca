"""Plain, slow fp64 CPU oracle for Transformer-FSQ latent decode.

TEST INFRASTRUCTURE ONLY. Only the test-suite, the smoke check and the CPU
baseline leg of the bench may import this module. The product path (the HIP
library and its binding) never calls it and shares no code with it.

What it computes, and where the pages define it (page titles as cited):
  * "Transformer-FSQ: Discrete Latents for Extreme KV-Cache Compression"
    (picx.dev summary), Theoretical Basis, Eq. 2 (the FSQ bound and round) and
    Eq. 3 (the implicit product grid); Architecture, Eq. 4 (z = Q_FSQ(E x)) and
    Eq. 5 (k = W_k z, v = W_v z, here without key norm and RoPE);
    Key Design Innovation, Eq. 6 (values decoded once after pooling codes);
    Byte Budgeting (c_full = 2 n_kv d_h sizeof(fp16)).
  * Slides "Transformer-FSQ" (slides.en.tex), frame "A wide product code uses
    four bits per coordinate": h = 7.5075, delta = 0.5 for L = 16, and the cache
    size ceil(G b / 8) bytes per token per layer; frame "Attention pools codes
    before decoding values" (Eq. 5-6 again).
  * Query absorption q~_h = W_k,g(h)^T q_h is not on the pages; it is exact for
    the linear key map W_k z used here and is pinned against materialised K/V.

  * Eq. 5 in full, k^_t = RoPE_t(N_k(W_k z_t)) (Architecture, Eq. 5; slides,
    frame "Attention pools codes before decoding values": keys are rebuilt per
    position because RoPE depends on it), in decode_attn_rope.

Readings of points the pages leave open:
  * level values are the integers round(u~) in {-8..7}; code = level + 8;
  * rounding is to nearest with ties to even (numpy.rint);
  * byte j of a token holds code[2j] in its low nibble and code[2j+1] in its
    high nibble; for odd G the last high nibble is zero;
  * attention scale 1/sqrt(d_h); q head h reads kv head h // (n_q // n_kv);
  * W_kv rows are [W_k; W_v], each kv-head-major with d_h rows per head;
  * a sequence of length 0 produces a zero output;
  * Eq. 5's N_k is the model's per-head key RMS norm, k * gamma / sqrt(mean(k^2)
    + eps), with gamma over the d_h channels shared by the heads; RoPE_t is the
    rotate-half form on channel pairs (i, i + d_h/2) at angle t * theta^(-2i/d_h),
    t the 0-based cache position; the pages fix neither gamma, eps nor theta
    (the tests use gamma from a seed, eps = 1e-6, theta = 1e6); the query is
    taken as already normalised and rotated at its own position.

Every computation is fp64 on the exact values of the bf16 inputs.

Parity unpinned: h_of_levels at L = 4 and 256 (the exact value of the bound h
of Eq. 2 away from L = 16; only the interval that gives L levels is pinned).
Every other function here is pinned by closed forms, invariants, library
routines or brute force in tests/test_oracle_*.py.
"""
from __future__ import annotations

import math

import numpy as np

# L = 16 levels per coordinate -> 4 bits; constants printed on the slides,
# frame "A wide product code uses four bits per coordinate" (footnote).
LEVELS = 16
BITS = 4
H_BOUND = 7.5075
DELTA = 0.5
CODE_OFFSET = LEVELS // 2     # code = level + 8


# ----------------------------------------------------------------- Eq. 2 / 3
def fsq_bound(u, h: float = H_BOUND, delta: float = DELTA) -> np.ndarray:
    """Bounded coordinate of Eq. 2: u~ = h * tanh(u + atanh(delta / h)) - delta."""
    u = np.asarray(u, dtype=np.float64)
    return h * np.tanh(u + math.atanh(delta / h)) - delta


def h_of_levels(levels: int) -> float:
    """Bound h of Eq. 2 for L levels. The pages print h only for L = 16 (7.5075,
    slides footnote); reading for L = 4 and 256 (the slides' backup frame "the
    grid size is an allocation choice"): h = 1.001 (L - 1) / 2, which gives
    7.5075 at L = 16, with delta = 0.5 and levels -L/2 .. L/2 - 1.

    PARITY UNPINNED at L = 4 and 256: no page value fixes h there. The tests pin
    only that h lies in (L/2 - 1, L/2], the interval in which Eq. 2 yields
    exactly L levels; any h inside it would pass them."""
    return 1.001 * (levels - 1) / 2.0


def fsq_levels(u, levels: int = LEVELS) -> np.ndarray:
    """Forward value of Eq. 2: the rounded bounded coordinate round(u~).

    The straight-through term sg(round(u~) - u~) only changes gradients; in the
    forward pass u^ equals round(u~) exactly. Result is an int64 level in
    -L/2 .. L/2 - 1 (-8..7 for L = 16)."""
    h = H_BOUND if levels == LEVELS else h_of_levels(levels)
    lv = np.rint(fsq_bound(u, h=h))
    if lv.size and (lv.min() < -(levels // 2) or lv.max() > levels // 2 - 1):
        raise AssertionError("FSQ level outside the grid")
    return lv.astype(np.int64)


def fsq_codes(u, levels: int = LEVELS) -> np.ndarray:
    """Code of each coordinate: level + L/2, a value in 0..L-1 (uint8)."""
    return (fsq_levels(u, levels) + levels // 2).astype(np.uint8)


def encode(x, E, levels: int = LEVELS) -> np.ndarray:
    """Eq. 4: z_t = Q_FSQ(E x_t) for every row x_t of x.

    x [N, C] and E [G, C] as float64 (the exact bf16 values). Returns codes
    [N, G] uint8. The projection is the fp64 matrix product u = x E^T."""
    x = np.asarray(x, dtype=np.float64)
    E = np.asarray(E, dtype=np.float64)
    u = x @ E.T
    return fsq_codes(u, levels)


def projection(x, E) -> np.ndarray:
    """u = x E^T in fp64 (the argument of the quantiser in Eq. 4)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(E, dtype=np.float64).T


# --------------------------------------------------------------- bytes, packing
def bytes_per_token(G: int, bits: int = BITS) -> int:
    """Cache size per token per layer, ceil(G * b / 8) bytes (slides, frame
    "A wide product code uses four bits per coordinate")."""
    return -(-(G * bits) // 8)


def full_cache_bytes(n_kv: int, d_h: int, elem_bytes: int = 2) -> int:
    """Uncompressed K/V bytes per token per layer, 2 * n_kv * d_h * sizeof(fp16)
    (picx.dev summary, Byte Budgeting)."""
    return 2 * n_kv * d_h * elem_bytes


def pack_codes(codes, bits: int = BITS) -> np.ndarray:
    """[N, G] codes of b bits -> [N, ceil(G b/8)] bytes; byte j holds codes
    c[k j + i], i < k = 8 / b, at bits b i (4 bits: c[2j] | c[2j+1] << 4)."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, G = codes.shape
    if codes.size and int(codes.max()) >= (1 << bits):
        raise AssertionError("code outside the b-bit range")
    k = 8 // bits
    P = bytes_per_token(G, bits)
    padded = np.zeros((N, k * P), dtype=np.uint8)
    padded[:, :G] = codes
    out = np.zeros((N, P), dtype=np.uint8)
    for j in range(P):
        for i in range(k):
            out[:, j] |= (padded[:, k * j + i] << (bits * i)).astype(np.uint8)
    return out


def unpack_codes(packed, G: int, bits: int = BITS) -> np.ndarray:
    """Inverse of pack_codes: [N, ceil(G b/8)] bytes -> [N, G] codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    N, P = packed.shape
    if P != bytes_per_token(G, bits):
        raise ValueError("packed width does not match G")
    k = 8 // bits
    mask = (1 << bits) - 1
    out = np.zeros((N, k * P), dtype=np.uint8)
    for j in range(P):
        for i in range(k):
            out[:, k * j + i] = (packed[:, j] >> (bits * i)) & mask
    return out[:, :G]


def levels_of_codes(codes, levels: int = LEVELS) -> np.ndarray:
    """Latent values z = code - L/2 as float64 (the grid points of Eq. 3)."""
    return np.asarray(codes, dtype=np.float64) - levels // 2


def bits_of_levels(levels: int) -> int:
    """b = log2 L for L = 4, 16, 256."""
    return {4: 2, 16: 4, 256: 8}[levels]


# ------------------------------------------------------- latent-space decode
def _kv_head(h: int, n_q: int, n_kv: int) -> int:
    return h // (n_q // n_kv)


def decoder_blocks(W_kv, g: int, n_kv: int, d_h: int):
    """W_k,g and W_v,g: the d_h rows of kv head g in the key and value halves
    of W_kv = [W_k; W_v] (picx.dev summary, Eq. 8 row order)."""
    W_kv = np.asarray(W_kv, dtype=np.float64)
    Wk = W_kv[g * d_h:(g + 1) * d_h, :]
    Wv = W_kv[n_kv * d_h + g * d_h:n_kv * d_h + (g + 1) * d_h, :]
    return Wk, Wv


def decode_attn(q, packed, W_kv, seq_lens, n_kv: int, G: int, levels: int = LEVELS) -> np.ndarray:
    """One decode step of latent-space attention.

    q [B, n_q, d_h], packed [B, cap, ceil(G/2)] bytes, W_kv [2 n_kv d_h, G],
    seq_lens [B]. For each sequence b and query head h (kv head g):
      q~ = W_k,g^T q                 (absorbed query; exact for k = W_k z)
      s_t = q~ . z_t / sqrt(d_h)     for t < seq_lens[b]
      p = softmax(s)
      zbar = sum_t p_t z_t           (pool codes, Eq. 6)
      out = W_v,g zbar               (values decoded once, Eq. 6)
    A sequence of length 0 gives out = 0. With L = levels per coordinate the
    codes are b = log2 L bits wide and z = code - L/2. Returns float64 [B, n_q, d_h]."""
    q = np.asarray(q, dtype=np.float64)
    B, n_q, d_h = q.shape
    out = np.zeros((B, n_q, d_h), dtype=np.float64)
    for b in range(B):
        T = int(seq_lens[b])
        if T == 0:
            continue
        Z = levels_of_codes(unpack_codes(packed[b, :T], G, bits_of_levels(levels)), levels)   # [T, G]
        for h in range(n_q):
            Wk, Wv = decoder_blocks(W_kv, _kv_head(h, n_q, n_kv), n_kv, d_h)
            qt = Wk.T @ q[b, h]
            s = (Z @ qt) / math.sqrt(d_h)
            p = np.exp(s - s.max())
            p /= p.sum()
            zbar = Z.T @ p
            out[b, h] = Wv @ zbar
    return out


def decode_attn_materialised(q, packed, W_kv, seq_lens, n_kv: int, G: int,
                             levels: int = LEVELS) -> np.ndarray:
    """The same step with keys and values written out, Eq. 5 without N_k and
    RoPE: K = Z W_k,g^T, V = Z W_v,g^T, then textbook softmax(K q / sqrt(d_h))^T V."""
    q = np.asarray(q, dtype=np.float64)
    B, n_q, d_h = q.shape
    out = np.zeros((B, n_q, d_h), dtype=np.float64)
    for b in range(B):
        T = int(seq_lens[b])
        if T == 0:
            continue
        Z = levels_of_codes(unpack_codes(packed[b, :T], G, bits_of_levels(levels)), levels)
        for h in range(n_q):
            Wk, Wv = decoder_blocks(W_kv, _kv_head(h, n_q, n_kv), n_kv, d_h)
            K = Z @ Wk.T
            V = Z @ Wv.T
            s = K @ q[b, h] / math.sqrt(d_h)
            w = np.exp(s - s.max())
            w /= w.sum()
            out[b, h] = w @ V
    return out


def decode_partials(q, packed, W_kv, seq_lens, n_kv: int, G: int, bounds):
    """Split form of decode_attn over token ranges [bounds[i], bounds[i+1]).

    Returns per split (m, l, acc) with m = max s, l = sum exp(s - m),
    acc = sum exp(s - m) z, each per (b, h), and the merged output
      M = max m_i, zbar = sum_i e^(m_i - M) acc_i / sum_i e^(m_i - M) l_i,
      out = W_v,g zbar.
    This is the "merge partials" step of the slides' kernel frame; it must equal
    decode_attn for any split points (a test checks that)."""
    q = np.asarray(q, dtype=np.float64)
    B, n_q, d_h = q.shape
    out = np.zeros((B, n_q, d_h), dtype=np.float64)
    for b in range(B):
        T = int(seq_lens[b])
        if T == 0:
            continue
        Z = levels_of_codes(unpack_codes(packed[b, :T], G))
        for h in range(n_q):
            Wk, Wv = decoder_blocks(W_kv, _kv_head(h, n_q, n_kv), n_kv, d_h)
            qt = Wk.T @ q[b, h]
            parts = []
            for lo, hi in zip(bounds[:-1], bounds[1:]):
                lo, hi = min(lo, T), min(hi, T)
                if hi <= lo:
                    continue
                s = Z[lo:hi] @ qt / math.sqrt(d_h)
                m = s.max()
                e = np.exp(s - m)
                parts.append((m, e.sum(), Z[lo:hi].T @ e))
            M = max(m for m, _, _ in parts)
            l = sum(math.exp(m - M) * li for m, li, _ in parts)
            acc = sum(math.exp(m - M) * a for m, _, a in parts)
            out[b, h] = Wv @ (acc / l)
    return out


# ------------------------------------------------- Eq. 5 keys: N_k and RoPE
def rms_norm(k, gamma, eps: float) -> np.ndarray:
    """N_k of Eq. 5 (reading): k * gamma / sqrt(mean(k^2) + eps) over the last
    axis (the d_h channels of one key head)."""
    k = np.asarray(k, dtype=np.float64)
    ms = np.mean(k * k, axis=-1, keepdims=True)
    return k / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def rope(k, positions, theta: float) -> np.ndarray:
    """RoPE_t of Eq. 5 (reading: rotate-half pairs). k [..., T, d_h], positions [T].
    Channel i < d_h/2 and i + d_h/2 form a pair rotated by angle t * theta^(-2i/d_h):
      out_i        = k_i cos a - k_{i+d_h/2} sin a
      out_{i+d_h/2} = k_{i+d_h/2} cos a + k_i sin a."""
    k = np.asarray(k, dtype=np.float64)
    d_h = k.shape[-1]
    half = d_h // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / d_h)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]      # [T, half]
    c, s = np.cos(ang), np.sin(ang)
    a, b = k[..., :half], k[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def decode_attn_rope(q, packed, W_kv, seq_lens, n_kv: int, G: int, gamma, eps: float,
                     theta: float) -> np.ndarray:
    """One decode step with the keys of Eq. 5 in full: for each sequence b and
    query head h (kv head g), over t < seq_lens[b],
      k^_t = RoPE_t(N_k(W_k,g z_t)),  s_t = q . k^_t / sqrt(d_h),  p = softmax(s),
      out = W_v,g sum_t p_t z_t       (values still pooled as codes, Eq. 6).
    Keys are materialised per position (absorption does not apply: N_k is
    nonlinear and RoPE_t depends on t). Length 0 gives 0. float64 [B, n_q, d_h]."""
    q = np.asarray(q, dtype=np.float64)
    B, n_q, d_h = q.shape
    out = np.zeros((B, n_q, d_h), dtype=np.float64)
    for b in range(B):
        T = int(seq_lens[b])
        if T == 0:
            continue
        Z = levels_of_codes(unpack_codes(packed[b, :T], G))
        for g in range(n_kv):
            Wk, Wv = decoder_blocks(W_kv, g, n_kv, d_h)
            K = rope(rms_norm(Z @ Wk.T, gamma, eps), np.arange(T), theta)      # [T, d_h]
            for h in range(g * (n_q // n_kv), (g + 1) * (n_q // n_kv)):
                s = K @ q[b, h] / math.sqrt(d_h)
                p = np.exp(s - s.max())
                p /= p.sum()
                out[b, h] = Wv @ (Z.T @ p)
    return out
