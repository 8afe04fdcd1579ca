// Append path: u = E x (Eq. 4), the Eq. 2 bound and round in fp32, and packing
// at b = 4 bits per code (slides "Transformer-FSQ", frame "A wide product code
// uses four bits per coordinate": ceil(G b / 8) bytes per token, no metadata),
// or 2 / 8 bits for L = 4 / 256 levels (backup frame "the grid size is an
// allocation choice").
//
// Three kernels, chosen by the number of tokens and the width:
//   append_stage_kernel n >= 32, GP <= 128: one CTA of 8 waves per 32 tokens,
//                       bf16 MFMA 32x32x16 with fp32 accumulation over
//                       CTA-wide k-batches staged in registers several batches
//                       ahead; the 8 waves' sums added in a fixed order; FSQ +
//                       packing in the epilogue.
//   append_mfma_kernel  n >= 32, GP > 128: one CTA of 4 waves per 32 tokens,
//                       the waves split the C dimension, tiles staged by
//                       direct-to-LDS loads; the same epilogue.
//   append_gemv_kernel  n < 32 (a decode step appends one token per sequence):
//                       one CTA per output byte (a pair of coordinates) and up to
//                       8 tokens, 16-byte vector loads of E and x, tree reduction.
#include "append_gemv.h"
#include "common.h"

namespace fsq {

constexpr int kAppendWaves = 4;

template <int NT, int CPB>
__global__ __launch_bounds__(kGemvWaves * 64) void append_gemv_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ E, uint8_t *__restrict__ codes, int n,
    int C, int G, FsqQuant fq) {
    append_gemv_body<NT, CPB>(blockIdx.x, blockIdx.y * NT, x, E, codes, n, C, G, fq, nullptr, 0);
}

// Prefill path. A CTA of 4 waves computes u = E x for 32 tokens; the waves
// split C into batches of KPB (wave w takes batches w, w + 4, ...). Each wave
// stages its batches through a private ring of NB LDS slots holding the x tile
// [32 rows x KPB] and the E tile [GP rows x KPB]: every load instruction moves
// one 16-byte chunk per lane straight into LDS (global_load_lds_dwordx4, LDS
// address = slot base + 16 * lane), so that the lanes of an instruction read
// whole row segments (8 or 4 lanes per row) and the loads coalesce. A chunk c
// of row r sits at slot position c ^ swz(r); the MFMA operands are then read
// back with ds_read_b128 in their register layout (lane = row, k-step i = chunks
// 2i and 2i + 1), 16 consecutive rows on distinct banks.
template <int GP>
struct AppendCfg {
    static constexpr int CB = GP / 32;                  // 32-wide output blocks
    static constexpr int KPB = GP <= 96 ? 64 : 32;      // k per batch
    static constexpr int RL = KPB * 2;                  // tile row bytes
    static constexpr int CPR = RL / 16;                 // 16-byte chunks per row
    static constexpr int RPI = 64 / CPR;                // rows per load instruction
    static constexpr int SWS = CPR == 8 ? 1 : 2;        // rows sharing a 256-byte bank window: 2^SWS
    static constexpr int XI = 32 / RPI;                 // x load instructions per batch
    static constexpr int EI = GP / RPI;                 // E load instructions per batch
    static constexpr int KS = KPB / 16;                 // MFMA k-steps per batch
    static constexpr int NB = 2;                        // slots per wave
    static constexpr int SLOT = (32 + GP) * RL;         // bytes per slot
    static constexpr int LDS = kAppendWaves * NB * SLOT;
    static_assert(LDS + 0 <= 160 * 1024, "ring fits LDS");
    static_assert(32 * (GP + 1) * 4 <= LDS, "the epilogue's sums fit the ring");
};

template <int GP>
__device__ inline int append_swz(int row) {
    using A = AppendCfg<GP>;
    return (row >> A::SWS) & (A::CPR - 1);
}


template <int GP>
__global__ __launch_bounds__(kAppendWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void append_mfma_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ E, uint8_t *__restrict__ codes,
    int64_t n, int C, int G, FsqQuant fq, int bits) {
    using A = AppendCfg<GP>;
    constexpr int CB = A::CB, KPB = A::KPB, RL = A::RL, CPR = A::CPR, RPI = A::RPI;
    constexpr int XI = A::XI, EI = A::EI, KS = A::KS, NB = A::NB, SLOT = A::SLOT;
    constexpr int ROW = GP + 1;
    // s_waitcnt immediate (gfx9 layout): vmcnt <= XI + EI, expcnt and lgkmcnt not waited on
    constexpr int kWaitLoads = XI + EI;
    static_assert(kWaitLoads < 64, "vmcnt field");
    constexpr int kWaitOneSlot = (kWaitLoads & 0xF) | (0x7 << 4) | (0xF << 8) | ((kWaitLoads >> 4) << 14);
    __shared__ __attribute__((aligned(16))) uint8_t ring[A::LDS];
    float *U = reinterpret_cast<float *>(ring);   // the epilogue's sums, after the ring is drained
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tile0 = (int64_t)blockIdx.x * 32;
    const int rows = (n - tile0) < 32 ? (int)(n - tile0) : 32;
    const int r = lane & 31, hh = lane >> 5;
    floatx16 acc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb] = floatx16{};
    bool ein[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) ein[cb] = cb * 32 + r < G;
    uint8_t *myring = ring + wave * NB * SLOT;

    const int nbatch = (C + KPB - 1) / KPB;
    const int nbw = nbatch > wave ? (nbatch - wave + kAppendWaves - 1) / kAppendWaves : 0;
    // the row and 16-byte chunk this lane moves in each load instruction
    const int lrow = lane / CPR, lslot = lane % CPR;
    auto issue = [&](int s, int jw) {
        const int kb = (wave + kAppendWaves * jw) * KPB;
        uint8_t *xs = myring + s * SLOT, *es = xs + 32 * RL;
#pragma unroll
        for (int j = 0; j < XI; ++j) {
            const int row = j * RPI + lrow;
            const int k = kb + 8 * (lslot ^ append_swz<GP>(row));
            const uint16_t *src = x + (size_t)(tile0 + (row < rows ? row : rows - 1)) * C + (k < C ? k : 0);
            __builtin_amdgcn_global_load_lds((glb_void_t *)src, (lds_void_t *)(xs + j * 1024), 16, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < EI; ++j) {
            const int row = j * RPI + lrow;
            const int k = kb + 8 * (lslot ^ append_swz<GP>(row));
            const uint16_t *src = E + (size_t)(row < G ? row : G - 1) * C + (k < C ? k : 0);
            __builtin_amdgcn_global_load_lds((glb_void_t *)src, (lds_void_t *)(es + j * 1024), 16, 0, 0);
        }
    };
    auto compute = [&](int s, int jw) {
        const int kb = (wave + kAppendWaves * jw) * KPB;
        const bool jin = jw < nbw;   // batches past this wave's last contribute zero
        const uint8_t *xs = myring + s * SLOT, *es = xs + 32 * RL;
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            const int c = 2 * i + hh;
            const bool kin = jin && kb + 8 * c < C;
            u32x4 av = *reinterpret_cast<const u32x4 *>(xs + r * RL + 16 * (c ^ append_swz<GP>(r)));
            av = (kin && r < rows) ? av : u32x4{};
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const int er = cb * 32 + r;
                u32x4 ev = *reinterpret_cast<const u32x4 *>(es + er * RL + 16 * (c ^ append_swz<GP>(er)));
                ev = (kin && ein[cb]) ? ev : u32x4{};
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                                  __builtin_bit_cast(bf16x8, ev), acc[cb], 0,
                                                                  0, 0);
            }
        }
    };
    // Straight-line steady state: slot s holds batch j0 + s; after its MFMAs
    // have read it, the slot is refilled with batch j0 + s + NB (batches past
    // the last are fetched from the last batch's addresses and zeroed in use).
    if (nbw > 0) {
#pragma unroll
        for (int s = 0; s < NB; ++s) issue(s, s < nbw ? s : nbw - 1);
        for (int j0 = 0; j0 < nbw; j0 += NB) {
#pragma unroll
            for (int s = 0; s < NB; ++s) {
                // slot s holds the oldest of the NB batches in flight: wait until
                // at most one slot's loads (the next batch's) are outstanding
                __builtin_amdgcn_s_waitcnt(kWaitOneSlot);
                compute(s, j0 + s);
                const int jn = j0 + s + NB;
                issue(s, jn < nbw ? jn : nbw - 1);
            }
        }
    }
    __syncthreads();   // every wave is done with its ring before it becomes U
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
    // FSQ + pack: one thread per output byte (8 / bits codes, little-endian)
    const int cpb = 8 / bits;
    const int P = bytes_per_token_b(G, bits);
    uint8_t *dst = codes + (size_t)tile0 * P;
    for (int idx = threadIdx.x; idx < rows * P; idx += blockDim.x) {
        const int tok = idx / P, j = idx - tok * P;
        uint32_t byte = 0;
        for (int c = 0; c < cpb; ++c) {
            const int k = cpb * j + c;
            if (k < G) byte |= fsq_code(U[tok * ROW + k], fq) << (bits * c);
        }
        dst[idx] = (uint8_t)byte;
    }
}

// Prefill path for GP <= 128. A CTA of 8 waves computes u = E x for 32 tokens
// over k-batches of 256: the batch's tile is the 32 x rows and the GP E rows,
// 512 bytes each (x rows clamped to the last token, E rows to row G - 1: their
// outputs are never used). Every load instruction moves two whole 512-byte row
// segments (16 bytes per lane) into registers; a wave's loads run D batches
// ahead of their use, so a CU keeps D tiles of loads in flight in its register
// file instead of the few that fit LDS beside the tiles being multiplied. The
// x rows are loaded non-temporally (read once).
// When a batch's registers arrive they are written to one of two LDS tiles
// (16-byte chunk c of row rho at c ^ (rho & 15): the 16 lanes of one pass of a
// 16-byte LDS access touch 16 distinct 16-byte bank groups, for the row-wise
// writes and the column-wise operand reads alike), one barrier hands the tile to
// the CTA, and wave w runs the batch's k-steps 2w and 2w + 1 for all output
// blocks, reading its MFMA operands with ds_read_b128 (lane = row; k-step s
// takes chunks 2s and 2s + 1). k past C (the last batch when C % 256 != 0, and
// the batches that round the count up to a multiple of D) is zeroed in the
// tile. After the last batch each wave stores its sums to LDS and every output
// coordinate is the sum over waves 0..7 in that order.
constexpr int kStageWaves = 8;

// Workgroup barrier for an LDS hand-off: waits for this wave's LDS operations
// only (__syncthreads would also wait for the staged global loads in flight).
__device__ __attribute__((always_inline)) inline void stage_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int GP>
struct StageCfg {
    static constexpr int KPB = 256;                          // k per batch
    static constexpr int RL = 2 * KPB;                       // bytes per tile row
    static constexpr int ROWS = 32 + GP;                     // x rows, then E rows
    static constexpr int TILE = ROWS * RL;                   // bytes per LDS tile
    static constexpr int LPW = ROWS / (2 * kStageWaves);     // load instructions per wave and batch
    static constexpr int D = GP <= 96 ? 4 : 2;               // batches in flight per wave
    static constexpr int CB = GP / 32;                       // 32-wide output blocks
    static_assert(ROWS % (2 * kStageWaves) == 0, "two rows per load instruction");
    static_assert(2 * TILE <= 160 * 1024, "two tiles fit LDS");
    static constexpr int PS = GP + 8;                        // row stride of the waves' sums (floats)
    static_assert(kStageWaves * 32 * PS * 4 <= 2 * TILE, "the waves' sums fit the tiles");
    static_assert(KPB / 16 == 2 * kStageWaves, "two k-steps per wave and batch");
};

template <int GP>
__global__ __launch_bounds__(kStageWaves * 64) void append_stage_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ E, uint8_t *__restrict__ codes,
    int64_t n, int C, int G, FsqQuant fq, int bits) {
    using S = StageCfg<GP>;
    constexpr int KPB = S::KPB, RL = S::RL, TILE = S::TILE, LPW = S::LPW, D = S::D, CB = S::CB;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * TILE];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tile0 = (int64_t)blockIdx.x * 32;
    const int rows = (n - tile0) < 32 ? (int)(n - tile0) : 32;
    const int r = lane & 31, hh = lane >> 5;

    // Load instruction t of this wave moves tile rows 2 (wave + 8 t) + hh,
    // 16-byte chunk `r` of their batch segment. (2 * 8 t) & 15 == 0, so the
    // swizzle of a lane's rows is the same for every t.
    const uint16_t *src[LPW];
#pragma unroll
    for (int t = 0; t < LPW; ++t) {
        const int row = 2 * (wave + kStageWaves * t) + hh;
        src[t] = row < 32 ? x + (tile0 + (row < rows ? row : rows - 1)) * (int64_t)C + 8 * r
                          : E + (int64_t)(row - 32 < G ? row - 32 : G - 1) * C + 8 * r;
    }
    const int wrow0 = 2 * wave + hh;
    const int woff = wrow0 * RL + 16 * (r ^ (wrow0 & 15));   // + t * 2 * kStageWaves * RL
    // operand reads: row r of the x block / of E block cb, chunk 4 wave + 2 s + hh
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
        const int ko = kb + 8 * r < C ? kb : -8 * r;
#pragma unroll
        for (int t = 0; t < LPW; ++t) {
            if (t < 32 / (2 * kStageWaves)) {   // x rows: read once, kept out of the caches' reuse
                v[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src[t] + ko));
            } else {
                v[t] = *reinterpret_cast<const u32x4 *>(src[t] + ko);
            }
        }
    };
    auto stage = [&](const u32x4(&v)[LPW], int jb, uint8_t *tile) {
        const int kb = batch_k(jb);
        if (kb + KPB <= C) {
#pragma unroll
            for (int t = 0; t < LPW; ++t)
                *reinterpret_cast<u32x4 *>(tile + woff + t * 2 * kStageWaves * RL) = v[t];
        } else {
            const bool kin = kb + 8 * r < C;
#pragma unroll
            for (int t = 0; t < LPW; ++t)
                *reinterpret_cast<u32x4 *>(tile + woff + t * 2 * kStageWaves * RL) = kin ? v[t] : u32x4{};
        }
    };
    auto compute = [&](const uint8_t *tile) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int ch = 16 * ((4 * wave + 2 * s + hh) ^ sw);
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
    stage_barrier();   // every wave is done with the tiles before they hold the sums
    // [wave][token][PS]: the two lane halves (tokens 4 apart) on opposite bank halves
    constexpr int PS = S::PS;
    float *P = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int tok = (i >> 2) * 8 + hh * 4 + (i & 3);
            P[(wave * 32 + tok) * PS + cb * 32 + r] = acc[cb][i];
        }
    stage_barrier();
    // FSQ + pack: one thread per output byte (8 / bits codes, little-endian)
    const int cpb = 8 / bits;
    const int Pb = bytes_per_token_b(G, bits);
    uint8_t *dst = codes + (size_t)tile0 * Pb;
    for (int idx = threadIdx.x; idx < rows * Pb; idx += kStageWaves * 64) {
        const int tok = idx / Pb, j = idx - tok * Pb;
        uint32_t byte = 0;
        for (int c = 0; c < cpb; ++c) {
            const int k = cpb * j + c;
            if (k < G) {
                float u = P[tok * PS + k];
#pragma unroll
                for (int w = 1; w < kStageWaves; ++w) u += P[(w * 32 + tok) * PS + k];
                byte |= fsq_code(u, fq) << (bits * c);
            }
        }
        dst[idx] = (uint8_t)byte;
    }
}

template <int GP>
static hipError_t launch_append_mfma(const uint16_t *x, const uint16_t *E, uint8_t *codes,
                                     int64_t n, int C, int G, const FsqQuant &fq, int bits,
                                     hipStream_t st) {
    const int64_t tiles = (n + 31) / 32;
    if constexpr (GP <= 128) {
        append_stage_kernel<GP><<<dim3((unsigned)tiles), kStageWaves * 64, 0, st>>>(x, E, codes, n, C, G,
                                                                                   fq, bits);
        return hipGetLastError();
    }
    append_mfma_kernel<GP><<<dim3((unsigned)tiles), kAppendWaves * 64, 0, st>>>(x, E, codes, n, C, G,
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
        return launch_append_mfma<X>(x, E, codes, n, C, G, fq, bits, st);
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
