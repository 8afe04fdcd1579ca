// Append of a few tokens (u = E x, Eq. 4; the Eq. 2 bound and round; packing
// at 2, 4 or 8 bits per code) as a device-side body shared by the append kernel and the fused
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

// Sum over the 64 lanes of a wave, in every lane, without LDS: quad swaps and
// the half-row and row mirrors (DPP) leave each 16-lane row's sum in all of its
// lanes; v_permlane16_swap and v_permlane32_swap then pair rows l, l ^ 1 and
// halves l, l ^ 2 (each returns the two operands with rows exchanged).
template <int CTRL>
__device__ inline float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ inline float wave_sum_dpp(float a) {
    a += dpp_f32<0xB1>(a);    // quad_perm [1, 0, 3, 2]
    a += dpp_f32<0x4E>(a);    // quad_perm [2, 3, 0, 1]
    a += dpp_f32<0x141>(a);   // row_half_mirror
    a += dpp_f32<0x140>(a);   // row_mirror
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
    a = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
    return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// Output byte j of tokens tb .. tb + NT - 1 (< n): the CPB = 8 / bits codes of
// coordinates CPB j .. CPB j + CPB - 1 (past G: zero bits), code i of the byte
// at bits i * bits (little-endian within the byte).
// Destination row of token i: row i of a dense [n, P] array when lens is null;
// otherwise row lens[i] - 1 of sequence i in a [n, seq_cap, P] cache, skipped
// unless 1 <= lens[i] <= seq_cap. The per-token arithmetic does not depend on NT.
template <int NT, int CPB>
__device__ __attribute__((always_inline)) inline void append_gemv_body(int j, int tb, const uint16_t *__restrict__ x,
                                        const uint16_t *__restrict__ E, uint8_t *__restrict__ codes,
                                        int n, int C, int G, const FsqQuant &fq,
                                        const int32_t *__restrict__ lens, int64_t seq_cap) {
    constexpr int BITS = 8 / CPB;
    __shared__ float red[kGemvWaves][NT][CPB];
    const int nt = (n - tb) < NT ? (n - tb) : NT;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float acc[NT][CPB];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int c = 0; c < CPB; ++c) acc[t][c] = 0.0f;
    // the destination row's length, requested ahead of the dot products' loads
    // (a volatile read keeps it there rather than next to its use after the
    // barrier, where its latency would add to the step)
    const int64_t len_t = (lens != nullptr && (int)threadIdx.x < nt)
                              ? *reinterpret_cast<const volatile int32_t *>(lens + tb + threadIdx.x)
                              : 0;
    const int nv = C / 8;
    const u32x4 *ep[CPB];
    bool has[CPB];
#pragma unroll
    for (int c = 0; c < CPB; ++c) {
        has[c] = CPB * j + c < G;
        ep[c] = reinterpret_cast<const u32x4 *>(E + (size_t)(has[c] ? CPB * j + c : CPB * j) * C);
    }
    // two vectors per thread and pass, all loads issued before the first use
    // (clamped indices); each thread accumulates its vectors in index order
    constexpr int U = 2;
    const int nthr = kGemvWaves * 64;
    for (int v0 = threadIdx.x; v0 < nv; v0 += U * nthr) {
        u32x4 ev[U][CPB], xv[U][NT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * nthr < nv ? v0 + u * nthr : nv - 1;
#pragma unroll
            for (int c = 0; c < CPB; ++c) ev[u][c] = has[c] ? ep[c][v] : u32x4{};
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
#pragma unroll
                        for (int c = 0; c < CPB; ++c) acc[t][c] += dot8_bf16(ev[u][c], xv[u][t]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int c = 0; c < CPB; ++c) {
            const float a = wave_sum_dpp(acc[t][c]);
            if (lane == 0) red[wave][t][c] = a;
        }
    __syncthreads();
    if ((int)threadIdx.x < nt) {
        const int t = threadIdx.x;
        uint32_t byte = 0;
#pragma unroll
        for (int c = 0; c < CPB; ++c) {
            float u = 0.0f;
            for (int w = 0; w < kGemvWaves; ++w) u += red[w][t][c];
            if (has[c]) byte |= fsq_code(u, fq) << (BITS * c);
        }
        const int P = bytes_per_token_b(G, BITS);
        size_t row;
        if (lens == nullptr) {
            row = (size_t)(tb + t);
        } else {
            if (len_t < 1 || len_t > seq_cap) return;
            row = (size_t)(tb + t) * (size_t)seq_cap + (size_t)(len_t - 1);
        }
        codes[row * P + j] = (uint8_t)byte;
    }
}

// Tokens per CTA for n tokens (n < 32 in the append path, the batch in a decode step).
inline int gemv_tokens_per_cta(int64_t n) { return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : kGemvTokens; }

}  // namespace fsq
