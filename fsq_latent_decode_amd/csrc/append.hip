// Append path: u = E x (Eq. 4), the Eq. 2 bound and round in fp32, and 4-bit
// packing (slides "Transformer-FSQ", frame "A wide product code uses four bits
// per coordinate": ceil(G b / 8) bytes per token, no metadata).
//
// Two kernels, chosen by the number of tokens:
//   append_mfma_kernel  n >= 32: one CTA per 32 tokens, bf16 MFMA 32x32x16 with
//                       fp32 accumulation; the 4 waves split the C dimension and
//                       are summed in a fixed order; FSQ + packing in the epilogue.
//   append_gemv_kernel  n < 32 (a decode step appends one token per sequence):
//                       one CTA per output byte (a pair of coordinates) and up to
//                       8 tokens, 16-byte vector loads of E and x, tree reduction.
#include "common.h"

namespace fsq {

constexpr int kAppendWaves = 4;
constexpr int kGemvTokens = 8;

__device__ inline float dot8_bf16(u32x4 a, u32x4 b) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s += __uint_as_float(a[i] << 16) * __uint_as_float(b[i] << 16);
        s += __uint_as_float(a[i] & 0xFFFF0000u) * __uint_as_float(b[i] & 0xFFFF0000u);
    }
    return s;
}

template <int NT>
__global__ __launch_bounds__(256) void append_gemv_kernel(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ E,
                                                          uint8_t *__restrict__ codes, int n, int C,
                                                          int G, float shift) {
    __shared__ float red[kAppendWaves][NT][2];
    const int j = blockIdx.x;            // output byte = coordinates 2j, 2j+1
    const int tb = blockIdx.y * NT;      // first token of this CTA
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
    for (int v = threadIdx.x; v < nv; v += blockDim.x) {
        const u32x4 e0 = e0p[v];
        const u32x4 e1 = has1 ? e1p[v] : u32x4{};
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < nt) {
                const u32x4 xv = reinterpret_cast<const u32x4 *>(x + (size_t)(tb + t) * C)[v];
                acc[t][0] += dot8_bf16(e0, xv);
                acc[t][1] += dot8_bf16(e1, xv);
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
        for (int w = 0; w < kAppendWaves; ++w) {
            u0 += red[w][t][0];
            u1 += red[w][t][1];
        }
        const uint32_t q0 = fsq_code(u0, shift);
        const uint32_t q1 = has1 ? fsq_code(u1, shift) : 0u;
        codes[(size_t)(tb + t) * bytes_per_token(G) + j] = (uint8_t)(q0 | (q1 << 4));
    }
}

template <int GP>
__global__ __launch_bounds__(kAppendWaves * 64) void append_mfma_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ E, uint8_t *__restrict__ codes,
    int64_t n, int C, int G, float shift) {
    constexpr int CB = GP / 32;
    constexpr int ROW = GP + 1;
    __shared__ float U[32 * ROW];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t tile0 = (int64_t)blockIdx.x * 32;
    const int rows = (n - tile0) < 32 ? (int)(n - tile0) : 32;
    const int r = lane & 31, hh = lane >> 5;
    floatx16 acc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb] = floatx16{};
    const uint16_t *xrow = x + (size_t)(tile0 + (r < rows ? r : 0)) * C;
    const int nks = (C + 15) / 16;
    for (int ks = wave; ks < nks; ks += kAppendWaves) {
        const int k = ks * 16 + hh * 8;
        const bool kin = k < C;
        const u32x4 av = (kin && r < rows) ? *reinterpret_cast<const u32x4 *>(xrow + k) : u32x4{};
        const bf16x8 a = __builtin_bit_cast(bf16x8, av);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const int g = cb * 32 + r;
            const u32x4 ev = (kin && g < G) ? *reinterpret_cast<const u32x4 *>(E + (size_t)g * C + k)
                                            : u32x4{};
            acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, ev),
                                                              acc[cb], 0, 0, 0);
        }
    }
    // fixed-order sum of the 4 waves' partial products in LDS
    for (int w = 0; w < kAppendWaves; ++w) {
        if (wave == w) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int tok = (i >> 2) * 8 + hh * 4 + (i & 3);
                    float &dst = U[tok * ROW + cb * 32 + r];
                    dst = (w == 0) ? acc[cb][i] : dst + acc[cb][i];
                }
        }
        __syncthreads();
    }
    // FSQ + pack: one thread per output byte
    const int P = bytes_per_token(G);
    uint8_t *dst = codes + (size_t)tile0 * P;
    for (int idx = threadIdx.x; idx < rows * P; idx += blockDim.x) {
        const int tok = idx / P, j = idx - tok * P;
        const uint32_t q0 = fsq_code(U[tok * ROW + 2 * j], shift);
        const uint32_t q1 = (2 * j + 1 < G) ? fsq_code(U[tok * ROW + 2 * j + 1], shift) : 0u;
        dst[idx] = (uint8_t)(q0 | (q1 << 4));
    }
}

template <int GP>
static hipError_t launch_append_mfma(const uint16_t *x, const uint16_t *E, uint8_t *codes,
                                     int64_t n, int C, int G, float shift, hipStream_t st) {
    const int64_t tiles = (n + 31) / 32;
    append_mfma_kernel<GP><<<dim3((unsigned)tiles), kAppendWaves * 64, 0, st>>>(x, E, codes, n, C, G,
                                                                               shift);
    return hipGetLastError();
}

hipError_t launch_append(const uint16_t *x, const uint16_t *E, uint8_t *codes, int64_t n, int C,
                         int G, hipStream_t st) {
    const float shift = (float)atanh((double)kDelta / (double)kH);
    if (n < 32) {
        const int nt = n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : kGemvTokens;
        dim3 grid(bytes_per_token(G), (unsigned)((n + nt - 1) / nt));
        switch (nt) {
            case 1: append_gemv_kernel<1><<<grid, 256, 0, st>>>(x, E, codes, (int)n, C, G, shift); break;
            case 2: append_gemv_kernel<2><<<grid, 256, 0, st>>>(x, E, codes, (int)n, C, G, shift); break;
            case 4: append_gemv_kernel<4><<<grid, 256, 0, st>>>(x, E, codes, (int)n, C, G, shift); break;
            default:
                append_gemv_kernel<kGemvTokens><<<grid, 256, 0, st>>>(x, E, codes, (int)n, C, G, shift);
        }
        return hipGetLastError();
    }
    const int GP = (G + 31) / 32 * 32;
    switch (GP) {
#define FSQ_APPEND_CASE(X) \
    case X:                \
        return launch_append_mfma<X>(x, E, codes, n, C, G, shift, st);
        FSQ_APPEND_CASE(32)
        FSQ_APPEND_CASE(64)
        FSQ_APPEND_CASE(96)
        FSQ_APPEND_CASE(128)
        FSQ_APPEND_CASE(160)
        FSQ_APPEND_CASE(192)
        FSQ_APPEND_CASE(224)
        FSQ_APPEND_CASE(256)
#undef FSQ_APPEND_CASE
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace fsq
