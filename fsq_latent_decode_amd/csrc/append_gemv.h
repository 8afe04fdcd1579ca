// Append of a few tokens (u = E x, Eq. 4; the Eq. 2 bound and round; 4-bit
// packing) as a device-side body shared by the append kernel and the fused
// decode-step kernel, so both produce bit-identical codes.
#pragma once

#include "common.h"

namespace fsq {

constexpr int kGemvWaves = 4;      // 256 threads
constexpr int kGemvTokens = 8;     // tokens per CTA at most

__device__ inline float dot8_bf16(u32x4 a, u32x4 b) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s += __uint_as_float(a[i] << 16) * __uint_as_float(b[i] << 16);
        s += __uint_as_float(a[i] & 0xFFFF0000u) * __uint_as_float(b[i] & 0xFFFF0000u);
    }
    return s;
}

// Output byte j (coordinates 2j, 2j+1) of tokens tb .. tb + NT - 1 (< n).
// Destination row of token i: row i of a dense [n, P] array when lens is null;
// otherwise row lens[i] - 1 of sequence i in a [n, seq_cap, P] cache, skipped
// unless 1 <= lens[i] <= seq_cap. The per-token arithmetic does not depend on NT.
template <int NT>
__device__ __attribute__((always_inline)) inline void append_gemv_body(int j, int tb, const uint16_t *__restrict__ x,
                                        const uint16_t *__restrict__ E, uint8_t *__restrict__ codes,
                                        int n, int C, int G, float shift,
                                        const int32_t *__restrict__ lens, int64_t seq_cap) {
    __shared__ float red[kGemvWaves][NT][2];
    const int nt = (n - tb) < NT ? (n - tb) : NT;
    const int c0 = 2 * j, c1 = 2 * j + 1;
    const bool has1 = c1 < G;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float acc[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t][0] = acc[t][1] = 0.0f;
    const int nv = C / 8;
    const u32x4 *e0p = reinterpret_cast<const u32x4 *>(E + (size_t)c0 * C);
    const u32x4 *e1p = reinterpret_cast<const u32x4 *>(E + (size_t)(has1 ? c1 : c0) * C);
    // two vectors per thread and pass, all loads issued before the first use
    // (clamped indices); each thread accumulates its vectors in index order
    constexpr int U = 2;
    const int nthr = kGemvWaves * 64;
    for (int v0 = threadIdx.x; v0 < nv; v0 += U * nthr) {
        u32x4 e0[U], e1[U], xv[U][NT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * nthr < nv ? v0 + u * nthr : nv - 1;
            e0[u] = e0p[v];
            e1[u] = has1 ? e1p[v] : u32x4{};
#pragma unroll
            for (int t = 0; t < NT; ++t)
                if (t < nt) xv[u][t] = reinterpret_cast<const u32x4 *>(x + (size_t)(tb + t) * C)[v];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (v0 + u * nthr < nv) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    if (t < nt) {
                        acc[t][0] += dot8_bf16(e0[u], xv[u][t]);
                        acc[t][1] += dot8_bf16(e1[u], xv[u][t]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            float a = acc[t][c];
            for (int off = 32; off > 0; off >>= 1) a += __shfl_xor(a, off);
            if (lane == 0) red[wave][t][c] = a;
        }
    __syncthreads();
    if (threadIdx.x < nt) {
        const int t = threadIdx.x;
        float u0 = 0.0f, u1 = 0.0f;
        for (int w = 0; w < kGemvWaves; ++w) {
            u0 += red[w][t][0];
            u1 += red[w][t][1];
        }
        const uint32_t q0 = fsq_code(u0, shift);
        const uint32_t q1 = has1 ? fsq_code(u1, shift) : 0u;
        const int P = bytes_per_token(G);
        size_t row;
        if (lens == nullptr) {
            row = (size_t)(tb + t);
        } else {
            const int64_t len = lens[tb + t];
            if (len < 1 || len > seq_cap) return;
            row = (size_t)(tb + t) * (size_t)seq_cap + (size_t)(len - 1);
        }
        codes[row * P + j] = (uint8_t)(q0 | (q1 << 4));
    }
}

// Tokens per CTA for n tokens (n < 32 in the append path, the batch in a decode step).
inline int gemv_tokens_per_cta(int64_t n) { return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : kGemvTokens; }

}  // namespace fsq
