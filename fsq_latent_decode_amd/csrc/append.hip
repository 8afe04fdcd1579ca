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
#include "append_gemv.h"
#include "common.h"

namespace fsq {

constexpr int kAppendWaves = 4;

template <int NT>
__global__ __launch_bounds__(kGemvWaves * 64) void append_gemv_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ E, uint8_t *__restrict__ codes, int n,
    int C, int G, float shift) {
    append_gemv_body<NT>(blockIdx.x, blockIdx.y * NT, x, E, codes, n, C, G, shift, nullptr, 0);
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
    const float shift = host_fsq_shift();
    if (n < 32) {
        const int nt = gemv_tokens_per_cta(n);
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
