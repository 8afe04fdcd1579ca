// Load-only kernel with the prefill append's memory traffic, for measuring the
// floor its structure sets (a measurement aid of the benchmark, built as its own
// library; nothing in the FSQ library calls it).
//
// Like append_stage_kernel, a CTA of 8 waves covers 32 tokens and reads, in
// k-batches of 256 starting at batch (CTA index mod batches), the 512-byte
// segments of its 32 x rows and of the GP rows of E (rows past G clamped to row
// G - 1), two rows per 16-byte-per-lane load instruction, 16 instructions in
// flight per wave. mode 0 reads x and E, mode 1 x only, mode 2 E only. The words
// read are XOR-folded into out[cta * 512 + thread] so that no load is dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kWaves = 8;
constexpr int kQ = 16;

// NI load instructions per batch (two tile rows each) from tile row ROW0 on:
// ROW0 = 0, NI = (32 + GP) / 2 reads x and E; NI = 16 x only; ROW0 = 32,
// NI = GP / 2 E only (compile-time, so the index arithmetic per load is a few
// operations, as in the append kernel)
template <int NI, int ROW0>
__global__ __launch_bounds__(kWaves * 64) void append_loads_kernel(const uint16_t *__restrict__ x,
                                                                   const uint16_t *__restrict__ E,
                                                                   uint32_t *__restrict__ out, int C, int G) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 31, hh = lane >> 5;
    const int64_t tile0 = (int64_t)blockIdx.x * 32;
    const int nb = C / 256;
    const int rot = (int)(blockIdx.x % (unsigned)nb);
    constexpr int ni = NI, row0 = ROW0;
    const int per = nb * ni / kWaves;                                         // per wave
    auto addr = [&](int j) -> const u32x4 * {
        j = j < per ? j : per - 1;
        const int f = wave + kWaves * j, jb = f / ni, q = f - jb * ni;
        const int kb = (jb + rot < nb ? jb + rot : jb + rot - nb) * 256;
        const int row = row0 + 2 * q + hh;
        const uint16_t *p = row < 32 ? x + (tile0 + row) * C : E + (int64_t)(row - 32 < G ? row - 32 : G - 1) * C;
        return reinterpret_cast<const u32x4 *>(p + kb + 8 * r);
    };
    u32x4 v[kQ];
    uint32_t acc = 0;
#pragma unroll
    for (int s = 0; s < kQ; ++s) v[s] = *addr(s);
    for (int j0 = kQ; j0 < per; j0 += kQ) {
#pragma unroll
        for (int s = 0; s < kQ; ++s) {
            acc ^= v[s][0] ^ v[s][1] ^ v[s][2] ^ v[s][3];
            v[s] = *addr(j0 + s);
        }
    }
#pragma unroll
    for (int s = 0; s < kQ; ++s) acc ^= v[s][0] ^ v[s][1] ^ v[s][2] ^ v[s][3];
    out[blockIdx.x * (kWaves * 64) + threadIdx.x] = acc;
}

}  // namespace

// x [n, C] bf16, E [G, C] bf16, device pointers, 16-byte aligned; out: n / 32 x
// 512 u32, device. Requires n % 32 == 0, C % 256 == 0, GP = G rounded up to 32
// with (C / 256) * ((32 + GP) / 2) a multiple of 8. Returns 0, or -1 for sizes
// it does not take, or the HIP error of the launch.
extern "C" int fsq_probe_append_loads(int mode, const void *x, const void *E, int64_t n, int C, int G,
                                      void *out, void *stream) {
    const int GP = (G + 31) / 32 * 32;
    if (mode < 0 || mode > 2 || n <= 0 || n % 32 || C <= 0 || C % 256 || G <= 0 || GP > 256 || !x || !E ||
        !out || ((C / 256) * ((32 + GP) / 2)) % kWaves || ((C / 256) * 16) % kWaves ||
        ((C / 256) * (GP / 2)) % kWaves)
        return -1;
    const dim3 grid((unsigned)(n / 32));
    const uint16_t *xp = (const uint16_t *)x, *ep = (const uint16_t *)E;
    uint32_t *op = (uint32_t *)out;
    hipStream_t st = (hipStream_t)stream;
    if (mode == 1) {
        append_loads_kernel<16, 0><<<grid, kWaves * 64, 0, st>>>(xp, ep, op, C, G);
        return (int)hipGetLastError();
    }
    switch (GP) {
#define FSQ_PROBE_CASE(X)                                                                            \
    case X:                                                                                          \
        if (mode == 0)                                                                               \
            append_loads_kernel<(32 + X) / 2, 0><<<grid, kWaves * 64, 0, st>>>(xp, ep, op, C, G);    \
        else                                                                                         \
            append_loads_kernel<X / 2, 32><<<grid, kWaves * 64, 0, st>>>(xp, ep, op, C, G);          \
        break;
        FSQ_PROBE_CASE(32)
        FSQ_PROBE_CASE(64)
        FSQ_PROBE_CASE(96)
        FSQ_PROBE_CASE(128)
        FSQ_PROBE_CASE(160)
        FSQ_PROBE_CASE(192)
        FSQ_PROBE_CASE(224)
        FSQ_PROBE_CASE(256)
#undef FSQ_PROBE_CASE
        default:
            return -1;
    }
    return (int)hipGetLastError();
}
