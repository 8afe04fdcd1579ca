"""Pure-Python loop forms of the oracle for tiny inputs.

TEST INFRASTRUCTURE ONLY (see fsq_oracle). These functions restate the same
definitions with scalar loops and the math module, in a different order from
the NumPy oracle, so that a slip in either shows up when the two are compared:
  * quantiser as "nearest of the 16 levels to u~" (picx.dev summary, Eq. 2:
    u^ lies on the level set L_i; the forward value is the nearest level);
  * codes written to bytes nibble by nibble with shifts on Python ints;
  * attention with materialised per-position keys and values (Eq. 5 without
    N_k and RoPE) and a two-pass softmax.
Use only for tiny shapes (T, G, d_h of a few dozen).
"""
from __future__ import annotations

import math

H_BOUND = 7.5075
DELTA = 0.5


def quantise_scalar(u: float) -> int:
    """Nearest level in {-8..7} to u~ = h tanh(u + atanh(delta/h)) - delta.
    Exact ties between two levels resolve to the even level."""
    ut = H_BOUND * math.tanh(u + math.atanh(DELTA / H_BOUND)) - DELTA
    best, best_d = None, None
    for lv in range(-8, 8):
        d = abs(ut - lv)
        if best is None or d < best_d or (d == best_d and lv % 2 == 0):
            best, best_d = lv, d
    return best


def pack_row(codes) -> bytes:
    """One token's codes -> bytes: nibble i lives at bit 4*(i % 2) of byte i // 2."""
    nbytes = (len(codes) * 4 + 7) // 8
    acc = 0
    for i, c in enumerate(codes):
        acc |= (int(c) & 0xF) << (4 * i)
    return acc.to_bytes(nbytes, "little") if nbytes else b""


def unpack_row(row: bytes, G: int):
    acc = int.from_bytes(bytes(row), "little")
    return [(acc >> (4 * i)) & 0xF for i in range(G)]


def decode_head(q, rows, W_kv, n_kv: int, n_q: int, h: int, G: int):
    """Output of query head h for one sequence. q: list of d_h floats; rows:
    list of packed token rows (bytes); W_kv: nested lists [2 n_kv d_h][G]."""
    d_h = len(q)
    g = h // (n_q // n_kv)
    if not rows:
        return [0.0] * d_h
    Z = [[c - 8 for c in unpack_row(r, G)] for r in rows]
    K = [[sum(W_kv[g * d_h + d][j] * z[j] for j in range(G)) for d in range(d_h)] for z in Z]
    V = [[sum(W_kv[n_kv * d_h + g * d_h + d][j] * z[j] for j in range(G)) for d in range(d_h)] for z in Z]
    scale = 1.0 / math.sqrt(d_h)
    s = [sum(k[d] * q[d] for d in range(d_h)) * scale for k in K]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    tot = sum(w)
    return [sum(w[t] * V[t][d] for t in range(len(rows))) / tot for d in range(d_h)]
