"""Seeded synthetic inputs shared by the oracle-side tests, the GPU tests and the bench.

This module draws random numbers and lays them out in the input formats the
library consumes (bf16 bit patterns, packed code bytes, int32 lengths). It holds
none of the method's arithmetic: no projection, no quantiser, no packing of
codes from levels, no attention. Both the oracle and the HIP path receive the
same arrays from here and compute everything else on their own.

Seeds: every tensor comes from ``numpy.random.Generator(PCG64(SeedSequence(
[workload_id, layer, tensor_id])))`` so that any tensor of any layer can be
regenerated in isolation (the bench and the tests draw the same bytes).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# tensor ids inside a (workload, layer) seed
T_X = 1          # residual states x for the append
T_E = 2          # encoder E
T_WKV = 3        # shared decoder W_kv
T_Q = 4          # decode queries q
T_CODES = 5      # uniform cache code bytes
T_LENS = 6       # ragged sequence lengths
T_XNEW = 7       # the one new residual state appended per decode step


def rng(workload_id: int, layer: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload_id, layer, tensor_id])))


# ---------------------------------------------------------------- bf16 formats
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns as uint16. Inputs here are finite; their bit
    patterns are at most 0xFF7FFFFF, so the 32-bit sum below cannot wrap."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact: every bfloat16 value is a float64 value."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def normal_bf16(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) drawn in float32, rounded to bf16, returned as uint16 bits."""
    return f32_to_bf16_bits(g.standard_normal(shape, dtype=np.float32) * np.float32(std))


# ----------------------------------------------------------- code-byte inputs
def bytes_per_token(G: int, bits: int = 4) -> int:
    """Storage width of one token's codes at b bits per coordinate (4 by default)."""
    return (G * bits + 7) // 8


def uniform_code_bytes(g: np.random.Generator, shape_tokens, G: int, bits: int = 4) -> np.ndarray:
    """Random cache bytes whose b-bit fields are i.i.d. uniform codes in 0..2^b - 1.

    Codes share bytes, so uniform codes are uniform bytes. The unused high bits
    of each token's last byte (when G b is not a multiple of 8) are zero, the
    storage convention of the packed cache."""
    P = bytes_per_token(G, bits)
    shape = tuple(np.atleast_1d(shape_tokens)) + (P,)
    out = g.integers(0, 256, size=shape, dtype=np.uint8)
    used = G * bits - 8 * (P - 1)
    if used < 8:
        out[..., -1] &= np.uint8((1 << used) - 1)
    return out


def loguniform_lengths(g: np.random.Generator, batch: int, lo: int, hi: int) -> np.ndarray:
    """floor(exp(U[ln lo, ln hi))) as int32."""
    v = np.floor(np.exp(g.uniform(math.log(lo), math.log(hi), size=batch))).astype(np.int64)
    return np.clip(v, lo, hi).astype(np.int32)


# ---------------------------------------------------------------- workloads
@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes of one synthetic workload (Qwen3-shaped attention layers)."""
    wid: int
    name: str
    layers: int
    C: int
    n_q: int
    n_kv: int
    d_h: int
    G: int
    batch: int
    context: int            # tokens per sequence (max for ragged)
    ragged: bool = False
    append_tokens: int = 0  # prefill chunk appended through E + FSQ (0 = none)
    codes_from_fsq: bool = False
    levels: int = 16        # L levels per coordinate (4, 16 or 256: 2, 4 or 8 bits)

    @property
    def bits(self) -> int:
        return {4: 2, 16: 4, 256: 8}[self.levels]

    @property
    def P(self) -> int:
        return bytes_per_token(self.G, self.bits)


WORKLOADS = {
    "tiny": Workload(0, "tiny", 1, 1024, 16, 8, 128, 64, 1, 1024, append_tokens=1024),
    "qwen3_8b_g256": Workload(1, "qwen3_8b_g256", 36, 4096, 32, 8, 128, 256, 1, 32768),
    "qwen3_8b_g84": Workload(2, "qwen3_8b_g84", 36, 4096, 32, 8, 128, 84, 1, 131072,
                             append_tokens=8192),
    "qwen3_1p7b_ragged": Workload(3, "qwen3_1p7b_ragged", 28, 2048, 16, 8, 128, 256, 16, 65536,
                                  ragged=True),
    "qwen3_8b_g84_1m": Workload(4, "qwen3_8b_g84_1m", 36, 4096, 32, 8, 128, 84, 1, 1048576,
                                codes_from_fsq=True),
    # other operating points of the same shapes: G = 32 (256x, 16 B/token) and
    # G = 20 (409.6x, 10 B/token) at 4 bits; the G = 84 byte budget (42 B) spent
    # on 2-bit (L = 4, G = 168) or 8-bit (L = 256, G = 42) codes
    "qwen3_8b_g32": Workload(5, "qwen3_8b_g32", 36, 4096, 32, 8, 128, 32, 1, 131072),
    "qwen3_8b_g20": Workload(6, "qwen3_8b_g20", 36, 4096, 32, 8, 128, 20, 1, 131072),
    "qwen3_8b_l4_g168": Workload(7, "qwen3_8b_l4_g168", 36, 4096, 32, 8, 128, 168, 1, 131072, levels=4),
    "qwen3_8b_l256_g42": Workload(8, "qwen3_8b_l256_g42", 36, 4096, 32, 8, 128, 42, 1, 131072,
                                  levels=256),
}


def seq_lens(w: Workload, layer: int = 0) -> np.ndarray:
    if w.ragged:
        # one set of lengths per workload (shared by all layers of a step)
        return loguniform_lengths(rng(w.wid, 0, T_LENS), w.batch, 4096, w.context)
    return np.full(w.batch, w.context, dtype=np.int32)


def layer_weights(w: Workload, layer: int):
    """E [G, C] ~ N(0, 1/C) and W_kv [2 n_kv d_h, G] ~ N(0, 1/G), bf16 bits."""
    E = normal_bf16(rng(w.wid, layer, T_E), (w.G, w.C), 1.0 / math.sqrt(w.C))
    W_kv = normal_bf16(rng(w.wid, layer, T_WKV), (2 * w.n_kv * w.d_h, w.G), 1.0 / math.sqrt(w.G))
    return E, W_kv


def layer_query(w: Workload, layer: int) -> np.ndarray:
    return normal_bf16(rng(w.wid, layer, T_Q), (w.batch, w.n_q, w.d_h), 1.0)


def layer_x(w: Workload, layer: int, n_tokens: int, tensor_id: int = T_X) -> np.ndarray:
    return normal_bf16(rng(w.wid, layer, tensor_id), (n_tokens, w.C), 1.0)


def layer_x_chunk(w: Workload, layer: int, chunk: int, chunk_tokens: int = 8192) -> np.ndarray:
    """Residual states of prefill chunk `chunk` (tokens chunk * chunk_tokens ..), for
    caches built by appending chunk after chunk (the million-token workload);
    each chunk has its own seed [workload, layer, T_X, chunk]."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.wid, layer, T_X, chunk])))
    return normal_bf16(g, (chunk_tokens, w.C), 1.0)


def layer_codes(w: Workload, layer: int, lens: np.ndarray | None = None, cap: int | None = None) -> np.ndarray:
    """Uniform cache bytes [batch, cap, P]; rows at t >= seq_lens[b] are zero."""
    cap = w.context if cap is None else cap
    out = uniform_code_bytes(rng(w.wid, layer, T_CODES), (w.batch, cap), w.G, w.bits)
    if lens is not None:
        for b, T in enumerate(lens):
            out[b, int(T):] = 0
    return out
