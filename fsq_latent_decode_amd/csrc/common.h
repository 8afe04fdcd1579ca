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

// atanh(delta / h), the Eq. 2 shift, evaluated in double on the host and
// passed to the kernels as fp32.
inline float host_fsq_shift() { return (float)atanh((double)kDelta / (double)kH); }

// Eq. 2 forward value in fp32 and the code = level + 8.
__device__ inline uint32_t fsq_code(float u, float shift) {
    float ut = kH * tanhf(u + shift) - kDelta;
    float lv = rintf(ut);
    lv = fminf(fmaxf(lv, -8.0f), 7.0f);
    return (uint32_t)((int)lv + kCodeOffset);
}

// Position of latent coordinate k inside the fp16 operand order of the decode
// kernel (GP = G padded to a multiple of 32, KB = GP / 16 score k-blocks).
// Packed dword D of a token (coordinates 8D..8D+7) feeds k-block D % KB from
// lane half D / KB, so each half reads one contiguous run of dwords; inside a
// dword the fp16 pairs are (c0,c4) (c1,c5) (c2,c6) (c3,c7).
__host__ __device__ inline int coord_to_pos(int k, int GP) {
    const int KB = GP / 16, D = k >> 3, e = k & 7;
    return 16 * (D % KB) + 8 * (D / KB) + (((e & 3) << 1) | (e >> 2));
}
__host__ __device__ inline int pos_to_coord(int p, int GP) {
    const int KB = GP / 16, kb = p >> 4, hh = (p >> 3) & 1, j = p & 7;
    return 8 * (kb + hh * KB) + (((j & 1) << 2) | (j >> 1));
}

}  // namespace fsq
