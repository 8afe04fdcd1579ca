// Shared device/host definitions of the FSQ latent-decode library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace fsq {

// L = 16 levels, 4 bits per coordinate; bound constants for L = 16 from the
// slides "Transformer-FSQ", frame "A wide product code uses four bits per
// coordinate" (h = 7.5075, delta = 0.5).
constexpr float kH = 7.5075f;
constexpr float kDelta = 0.5f;
constexpr int kCodeOffset = 8;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;   // LDS pointer of direct-to-LDS loads
typedef __attribute__((address_space(1))) void glb_void_t;   // global pointer of direct-to-LDS loads

__host__ __device__ inline int bytes_per_token(int G) { return (G + 1) / 2; }
__host__ __device__ inline int round_up(int a, int b) { return (a + b - 1) / b * b; }

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bf16 bits, round to nearest even (inputs are finite here).
__device__ inline uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Quantiser of Eq. 2 for L levels per coordinate, L = 4, 16 or 256 (2, 4 or 8
// bits; the slides' backup table "the grid size is an allocation choice").
// The pages print h only for L = 16 (7.5075 with delta = 0.5); for the other L
// the reading h = 1.001 (L - 1) / 2 is used, which reproduces 7.5075 at L = 16.
// Levels are -L/2 .. L/2 - 1 and code = level + L/2.
struct FsqQuant {
    float h, shift, lo, hi;   // shift = atanh(delta / h); lo = -L/2, hi = L/2 - 1
    int half;                 // L / 2
};
inline FsqQuant host_fsq_quant(int levels) {
    const double h = 1.001 * (levels - 1) / 2.0;
    FsqQuant q;
    q.h = (float)h;
    q.shift = (float)atanh((double)kDelta / h);
    q.lo = (float)(-levels / 2);
    q.hi = (float)(levels / 2 - 1);
    q.half = levels / 2;
    return q;
}
__host__ __device__ inline int bits_of_levels(int levels) { return levels == 4 ? 2 : levels == 256 ? 8 : 4; }
__host__ __device__ inline int bytes_per_token_b(int G, int bits) { return (G * bits + 7) / 8; }

// Eq. 2 forward value in fp32 and the code = level + L/2.
__device__ inline uint32_t fsq_code(float u, const FsqQuant &q) {
    float ut = q.h * tanhf(u + q.shift) - kDelta;
    float lv = rintf(ut);
    lv = fminf(fmaxf(lv, q.lo), q.hi);
    return (uint32_t)((int)lv + q.half);
}

// Position of latent coordinate k inside the fp16 operand order of the decode
// kernels (GP = G padded to a multiple of 32, KB = GP / 16 score k-blocks of 8
// coordinates per lane half). Each lane half reads one contiguous run of its
// token's packed dwords; operand kb of half hh holds 8 coordinates:
//   4 bits: dword D = hh KB + kb, fp16 pairs (c0,c4) (c1,c5) (c2,c6) (c3,c7);
//   8 bits: dwords 2 kb, 2 kb + 1 of the half, pairs (c0,c2) (c1,c3) each;
//   2 bits: half of dword kb / 2 of the half (coordinates 0..15 of it), pairs
//           (c_i, c_i+8) for i = 0..3 or 4..7.
__host__ __device__ inline int coord_to_pos(int k, int GP, int bits = 4) {
    const int KB = GP / 16;
    if (bits == 8) {
        const int D = k >> 2, e = k & 3, hh = D / (2 * KB), dh = D % (2 * KB);
        return 16 * (dh >> 1) + 8 * hh + 4 * (dh & 1) + (((e & 1) << 1) | (e >> 1));
    }
    if (bits == 2) {
        const int D = k >> 4, e = k & 15, hh = D / (KB / 2), dh = D % (KB / 2), i = e & 7;
        return 16 * (2 * dh + (i >> 2)) + 8 * hh + (((i & 3) << 1) | (e >> 3));
    }
    const int D = k >> 3, e = k & 7;
    return 16 * (D % KB) + 8 * (D / KB) + (((e & 3) << 1) | (e >> 2));
}
__host__ __device__ inline int pos_to_coord(int p, int GP, int bits = 4) {
    const int KB = GP / 16, kb = p >> 4, hh = (p >> 3) & 1, j = p & 7;
    if (bits == 8) {
        const int r = j & 3;
        return 4 * (hh * 2 * KB + 2 * kb + (j >> 2)) + (((r & 1) << 1) | (r >> 1));
    }
    if (bits == 2)
        return 16 * (hh * (KB / 2) + (kb >> 1)) + 4 * (kb & 1) + (j >> 1) + 8 * (j & 1);
    return 8 * (kb + hh * KB) + (((j & 1) << 2) | (j >> 1));
}

}  // namespace fsq
