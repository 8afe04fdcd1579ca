// Append path: u = E x (Eq. 4), the Eq. 2 bound and round in fp32, and packing
// at b = 4 bits per code (slides "Transformer-FSQ", frame "A wide product code
// uses four bits per coordinate": ceil(G b / 8) bytes per token, no metadata),
// or 2 / 8 bits for L = 4 / 256 levels (backup frame "the grid size is an
// allocation choice").
//
// Two kernels, chosen by the number of tokens:
//   append_stage_kernel n >= 32: one CTA of 8 waves per 32 tokens, bf16 MFMA
//                       32x32x16 with fp32 accumulation over CTA-wide k-batches
//                       staged in registers several batches ahead; the 8 waves'
//                       sums added in a fixed order; FSQ + packing in the
//                       epilogue.
//   append_gemv_kernel  n < 32 (a decode step appends one token per sequence):
//                       one CTA per output byte (a pair of coordinates) and up to
//                       8 tokens, 16-byte vector loads of E and x, tree reduction.
#include "append_gemv.h"
#include "common.h"

namespace fsq {

template <int NT, int CPB>
__global__ __launch_bounds__(kGemvWaves * 64) void append_gemv_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ E, uint8_t *__restrict__ codes, int n,
    int C, int G, FsqQuant fq) {
    append_gemv_body<NT, CPB>(blockIdx.x, blockIdx.y * NT, x, E, codes, n, C, G, fq, nullptr, 0);
}

// Prefill path. A CTA of 8 waves computes u = E x for 32 tokens over k-batches
// of KPB (256 for GP <= 128, else 128): the batch's tile is the 32 x rows and
// the GP E rows, 2 KPB bytes each (x rows clamped to the last token, E rows to
// row G - 1: their outputs are never used). Every load instruction moves whole
// row segments (16 bytes per lane, 1 KB per instruction) into registers; a
// wave's loads run D batches ahead of their use, so a CU keeps D tiles of
// loads in flight in its register file instead of the few that fit LDS beside
// the tiles being multiplied. The x rows are loaded non-temporally (read once).
// When a batch's registers arrive they are written to one of two LDS tiles
// (16-byte chunk c of row rho at c ^ (rho & 15): the 16 lanes of one pass of a
// 16-byte LDS access touch 16 distinct 16-byte bank groups, for the row-wise
// writes and the column-wise operand reads alike), one barrier hands the tile to
// the CTA, and wave w runs its share of the batch's k-steps (KPB / 128 of them)
// for all output blocks, reading its MFMA operands with ds_read_b128 (lane =
// row; k-step s takes chunks 2s and 2s + 1). k past C (the last batch when
// C % KPB != 0, and the batches that round the count up to a multiple of D) is
// zeroed in the tile. After the last batch the waves store their sums to LDS,
// 128 coordinates at a time, and every output coordinate is the sum over waves
// 0..7 in that order.
constexpr int kStageWaves = 8;

// Workgroup barrier for an LDS hand-off: waits for this wave's LDS operations
// only (__syncthreads would also wait for the staged global loads in flight).
__device__ __attribute__((always_inline)) inline void stage_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int GP>
struct StageCfg {
    static constexpr int KPB = GP <= 128 ? 256 : 128;        // k per batch
    static constexpr int RL = 2 * KPB;                       // bytes per tile row
    static constexpr int CPR = RL / 16;                      // 16-byte chunks per row (32 or 16)
    static constexpr int RPI = 64 / CPR;                     // rows per load instruction (2 or 4)
    static constexpr int ROWS = 32 + GP;                     // x rows, then E rows
    static constexpr int TILE = ROWS * RL;                   // bytes per LDS tile
    static constexpr int LPW = ROWS / (RPI * kStageWaves);   // load instructions per wave and batch
    static constexpr int XT = 32 / (RPI * kStageWaves);      // of which x rows (t < XT)
    static constexpr int KSW = KPB / 16 / kStageWaves;       // k-steps per wave and batch
    static constexpr int D = GP <= 96 ? 4 : 2;               // batches in flight per wave
    static constexpr int CB = GP / 32;                       // 32-wide output blocks
    static constexpr int EPB = CB < 4 ? CB : 4;              // output blocks per epilogue pass
    static constexpr int NPASS = (CB + EPB - 1) / EPB;
    static constexpr int PS = 32 * EPB + 8;                  // row stride of the waves' sums (floats)
    static_assert(ROWS % (RPI * kStageWaves) == 0 && XT * RPI * kStageWaves == 32, "whole rows per load instruction");
    static constexpr int SUMS = kStageWaves * 32 * PS * 4;   // bytes of the waves' sums (one pass)
    static constexpr int LDS = 2 * TILE > SUMS ? 2 * TILE : SUMS;
    static_assert(LDS <= 160 * 1024, "two tiles, or one pass of sums, fit LDS");
    static_assert(KSW * kStageWaves * 16 == KPB && CPR <= 32, "k-steps shared out evenly");
    static_assert(D % 2 == 0, "tile of batch jb is jb & 1");
};

template <int GP>
__global__ __launch_bounds__(kStageWaves * 64) void append_stage_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ E, uint8_t *__restrict__ codes,
    int64_t n, int C, int G, FsqQuant fq, int bits) {
    using S = StageCfg<GP>;
    constexpr int KPB = S::KPB, RL = S::RL, CPR = S::CPR, RPI = S::RPI, TILE = S::TILE, LPW = S::LPW;
    constexpr int XT = S::XT, KSW = S::KSW, D = S::D, CB = S::CB, EPB = S::EPB, PS = S::PS;
    __shared__ __attribute__((aligned(16))) uint8_t lds[S::LDS];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tile0 = (int64_t)blockIdx.x * 32;
    const int rows = (n - tile0) < 32 ? (int)(n - tile0) : 32;
    const int r = lane & 31, hh = lane >> 5;

    // Load instruction t of this wave moves tile rows RPI (wave + 8 t) + lr,
    // 16-byte chunk lc of their batch segment. (RPI * 8 t) & 15 == 0, so the
    // swizzle of a lane's rows is the same for every t.
    const int lc = lane % CPR, lr = lane / CPR;
    const uint16_t *src[LPW];
#pragma unroll
    for (int t = 0; t < LPW; ++t) {
        const int row = RPI * (wave + kStageWaves * t) + lr;
        src[t] = row < 32 ? x + (tile0 + (row < rows ? row : rows - 1)) * (int64_t)C + 8 * lc
                          : E + (int64_t)(row - 32 < G ? row - 32 : G - 1) * C + 8 * lc;
    }
    const int wrow0 = RPI * wave + lr;
    const int woff = wrow0 * RL + 16 * (lc ^ (wrow0 & 15));   // + t * RPI * kStageWaves * RL
    // operand reads: row r of the x block / of E block cb, chunk 2 KSW wave + 2 s + hh
    const int sw = r & 15;

    floatx16 acc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb] = floatx16{};

    const int nb = (C + KPB - 1) / KPB;
    const int nbp = (nb + D - 1) / D * D;
    // CTA b takes the batches in the order b mod nb, b + 1 mod nb, ...: at any
    // moment the CTAs read different columns of x and E, which spreads their
    // requests over the memory channels (batches past nb are the all-zero
    // padding and keep their index)
    const int rot = (int)(blockIdx.x % (unsigned)nb);
    auto batch_k = [&](int jb) { return (jb < nb ? (jb + rot < nb ? jb + rot : jb + rot - nb) : jb) * KPB; };
    u32x4 st[D][LPW];
    auto load = [&](u32x4(&v)[LPW], int jb) {
        // lanes whose chunk lies past C read their row's first chunk (zeroed later)
        const int kb = batch_k(jb);
        const int ko = kb + 8 * lc < C ? kb : -8 * lc;
#pragma unroll
        for (int t = 0; t < LPW; ++t) {
            if (t < XT)   // x rows: read once, kept out of the caches' reuse
                v[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src[t] + ko));
            else
                v[t] = *reinterpret_cast<const u32x4 *>(src[t] + ko);
        }
    };
    auto stage = [&](const u32x4(&v)[LPW], int jb, uint8_t *tile) {
        const int kb = batch_k(jb);
        if (kb + KPB <= C) {
#pragma unroll
            for (int t = 0; t < LPW; ++t)
                *reinterpret_cast<u32x4 *>(tile + woff + t * RPI * kStageWaves * RL) = v[t];
        } else {
            const bool kin = kb + 8 * lc < C;
#pragma unroll
            for (int t = 0; t < LPW; ++t)
                *reinterpret_cast<u32x4 *>(tile + woff + t * RPI * kStageWaves * RL) = kin ? v[t] : u32x4{};
        }
    };
    auto compute = [&](const uint8_t *tile) {
#pragma unroll
        for (int s = 0; s < KSW; ++s) {
            const int ch = 16 * ((2 * KSW * wave + 2 * s + hh) ^ sw);
            const u32x4 av = *reinterpret_cast<const u32x4 *>(tile + r * RL + ch);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const u32x4 ev = *reinterpret_cast<const u32x4 *>(tile + (32 + 32 * cb + r) * RL + ch);
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                                  __builtin_bit_cast(bf16x8, ev), acc[cb], 0,
                                                                  0, 0);
            }
        }
    };
    // Stage s of the registers holds batch j0 + s; the tile of batch jb is
    // jb & 1 (D is even and j0 a multiple of D). Writing tile jb & 1 is safe
    // once every wave has passed the barrier of batch jb - 1, which each wave
    // reaches after its reads of batch jb - 2.
#pragma unroll
    for (int s = 0; s < D; ++s) load(st[s], s);
    int j0 = 0;
    for (; j0 < nbp - D; j0 += D) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
            uint8_t *tile = lds + (s & 1) * TILE;
            stage(st[s], j0 + s, tile);
            stage_barrier();
            compute(tile);
            load(st[s], j0 + s + D);
        }
    }
#pragma unroll
    for (int s = 0; s < D; ++s) {
        uint8_t *tile = lds + (s & 1) * TILE;
        stage(st[s], j0 + s, tile);
        stage_barrier();
        compute(tile);
    }
    // Epilogue, in passes of EPB output blocks (128 coordinates): the waves'
    // sums to LDS ([wave][token][PS]; the two lane halves, tokens 4 apart, on
    // opposite bank halves), then FSQ + pack of the bytes whose codes lie in the
    // pass, one thread per output byte (8 / bits codes, little-endian).
    float *P = reinterpret_cast<float *>(lds);
    const int cpb = 8 / bits;
    const int Pb = bytes_per_token_b(G, bits);
    uint8_t *dst = codes + (size_t)tile0 * Pb;
#pragma unroll
    for (int pass = 0; pass < S::NPASS; ++pass) {
        stage_barrier();   // the tiles, or the previous pass's sums, are no longer read
#pragma unroll
        for (int e = 0; e < EPB; ++e) {
            const int cb = pass * EPB + e;
            if (cb < CB) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int tok = (i >> 2) * 8 + hh * 4 + (i & 3);
                    P[(wave * 32 + tok) * PS + e * 32 + r] = acc[cb][i];
                }
            }
        }
        stage_barrier();
        const int k0 = pass * 32 * EPB;                              // first coordinate of the pass
        const int jlo = k0 / cpb;
        const int jhi0 = (k0 + 32 * EPB) / cpb;
        const int jhi = jhi0 < Pb ? jhi0 : Pb;
        const int nbt = jhi - jlo;                                   // bytes per token in the pass
        for (int idx = threadIdx.x; idx < rows * nbt; idx += kStageWaves * 64) {
            const int tok = idx / nbt, j = jlo + (idx - tok * nbt);
            uint32_t byte = 0;
            for (int c = 0; c < cpb; ++c) {
                const int k = cpb * j + c;
                if (k < G) {
                    const int kk = k - k0;
                    float u = P[tok * PS + kk];
#pragma unroll
                    for (int w = 1; w < kStageWaves; ++w) u += P[(w * 32 + tok) * PS + kk];
                    byte |= fsq_code(u, fq) << (bits * c);
                }
            }
            dst[(size_t)tok * Pb + j] = (uint8_t)byte;
        }
    }
}

template <int GP>
static hipError_t launch_append_stage(const uint16_t *x, const uint16_t *E, uint8_t *codes,
                                     int64_t n, int C, int G, const FsqQuant &fq, int bits,
                                     hipStream_t st) {
    const int64_t tiles = (n + 31) / 32;
    append_stage_kernel<GP><<<dim3((unsigned)tiles), kStageWaves * 64, 0, st>>>(x, E, codes, n, C, G,
                                                                               fq, bits);
    return hipGetLastError();
}

template <int CPB>
static void launch_append_gemv(const uint16_t *x, const uint16_t *E, uint8_t *codes, int n, int C,
                               int G, const FsqQuant &fq, hipStream_t st) {
    const int nt = gemv_tokens_per_cta(n);
    dim3 grid(bytes_per_token_b(G, 8 / CPB), (unsigned)((n + nt - 1) / nt));
    switch (nt) {
        case 1: append_gemv_kernel<1, CPB><<<grid, 256, 0, st>>>(x, E, codes, n, C, G, fq); break;
        case 2: append_gemv_kernel<2, CPB><<<grid, 256, 0, st>>>(x, E, codes, n, C, G, fq); break;
        case 4: append_gemv_kernel<4, CPB><<<grid, 256, 0, st>>>(x, E, codes, n, C, G, fq); break;
        default: append_gemv_kernel<kGemvTokens, CPB><<<grid, 256, 0, st>>>(x, E, codes, n, C, G, fq);
    }
}

hipError_t launch_append(const uint16_t *x, const uint16_t *E, uint8_t *codes, int64_t n, int C,
                         int G, int levels, hipStream_t st) {
    const FsqQuant fq = host_fsq_quant(levels);
    const int bits = bits_of_levels(levels);
    if (n < 32) {
        if (bits == 2)
            launch_append_gemv<4>(x, E, codes, (int)n, C, G, fq, st);
        else if (bits == 8)
            launch_append_gemv<1>(x, E, codes, (int)n, C, G, fq, st);
        else
            launch_append_gemv<2>(x, E, codes, (int)n, C, G, fq, st);
        return hipGetLastError();
    }
    const int GP = (G + 31) / 32 * 32;
    switch (GP) {
#define FSQ_APPEND_CASE(X) \
    case X:                \
        return launch_append_stage<X>(x, E, codes, n, C, G, fq, bits, st);
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
