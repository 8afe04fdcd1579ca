// Split-K latent-space decode attention over a packed 4-bit FSQ cache (gfx950).
//
// Pages: "Transformer-FSQ: Discrete Latents for Extreme KV-Cache Compression"
// (picx.dev summary), Eq. 5 (k = W_k z, v = W_v z; key norm and RoPE not applied
// here) and Eq. 6 (sum_t a_t W_v z_t = W_v sum_t a_t z_t: pool the codes, then
// apply W_v once); slides "Transformer-FSQ", frame "The kernel reads codes and
// never writes reconstructed K/V" (read packed codes, unpack to registers,
// scores + online softmax, accumulate attention-weighted codes, merge partials,
// apply W_v once). Unlike the pages' kernel, keys are never rebuilt: the query
// is absorbed into latent space, q~ = W_k^T q, so a score is q~ . z.
//
// Three launches per call, all on the caller's stream:
//   absorb_kernel       q~ = (log2 e / sqrt d_h) W_k,g^T q -> fp16, operand order
//                       (step_prep_kernel in a decode step: the same absorption
//                       plus the append of each sequence's new token)
//   decode_split_kernel one CTA per (token chunk, sequence, 32-head group):
//                       codes -> registers (prefetched one round ahead) -> fp16
//                       operands -> MFMA scores (all heads share z); the codes
//                       to an LDS tile (4-bit: the packed nibbles, read back
//                       transposed by ds_read_b64_tr_b4; 2 and 8 bits: fp16)
//                       -> online softmax (exp2) -> MFMA latent pooling ->
//                       (m, l, zbar fp16); for long chunks decode_stream_kernel
//                       (below) instead, split on the device for batches
//   decode_merge1_kernel one 16-wave CTA per (sequence, head) (or up to four
//                       sharing a head's W_v rows): log-sum-exp merge of the
//                       chunks' zbar by cross-lane reductions, one barrier, then
//                       out = W_v,g zbar (decode_merge_kernel, two LDS levels,
//                       when a sequence has more than 4 splits per lane)
#include <hip/hip_ext.h>

#include <type_traits>

#include "append_gemv.h"
#include "common.h"
#include "decode_plan.h"

namespace fsq {

constexpr int kTile = 32;        // tokens per wave and round (the score MFMA's M)

// Lazy online softmax: the reference max m of a head is raised (and the
// accumulators rescaled) only when a tile's max exceeds it by more than this
// many log2 units, so the weights p = 2^(s - m) stay below 2^kRescaleSlack,
// inside fp16's range (65504).
#ifndef FSQ_RESCALE_SLACK
#define FSQ_RESCALE_SLACK 15
#endif
constexpr float kRescaleSlack = (float)FSQ_RESCALE_SLACK;
static_assert(FSQ_RESCALE_SLACK >= 1 && FSQ_RESCALE_SLACK <= 15, "p must stay below fp16's largest value");

// Lane l's value combined with lane l ^ 32's through v_permlane32_swap (a VALU
// exchange of the wave's halves; a shuffle would go through the LDS crossbar).
// The swap returns the pair in an order that is the same for both lanes, so
// both compute the same bits.
__device__ inline float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Codes of one packed dword (8 codes, nibble i = coordinate 8D + i) as fp16
// operands in the order (c0,c4)(c1,c5)(c2,c6)(c3,c7). The bit pattern n of a
// code is the fp16 subnormal n * 2^-24, exact, so no bias is subtracted here:
// with z = n - 8 and n' = n * 2^-24,
//   q~ . z = 2^24 (q~ . n') - 8 sum_k q~_k,
// where the last term is the same for every token of a head and cancels in the
// softmax (and in the merge of splits, which share it), and
//   sum_t p_t z_t / sum_t p_t = 2^24 sum_t p_t n'_t / sum_t p_t - 8
// when the denominator sums the same fp16 p_t that the pooling MFMA uses.
constexpr float kCodeScale = 16777216.0f;   // 2^24
__device__ inline half8 unpack_codes(uint32_t w) {
    const uint32_t m = 0x000F000Fu;
    const u32x4 t = {w & m, (w >> 4) & m, (w >> 8) & m, (w >> 12) & m};
    return __builtin_bit_cast(half8, t);
}
// 8-bit codes (L = 256): two packed dwords, 4 codes each, as fp16 subnormals
// n * 2^-24 in the order (c0,c2) (c1,c3) (c4,c6) (c5,c7).
__device__ inline half8 unpack_codes8(uint32_t w0, uint32_t w1) {
    const uint32_t m = 0x00FF00FFu;
    const u32x4 t = {w0 & m, (w0 >> 8) & m, w1 & m, (w1 >> 8) & m};
    return __builtin_bit_cast(half8, t);
}
// 2-bit codes (L = 4): half of a packed dword of 16 codes (upper = 0: codes
// 0..3 and 8..11, upper = 1: 4..7 and 12..15) in the order (c_i, c_i+8).
__device__ inline half8 unpack_codes2(uint32_t w, int upper) {
    const uint32_t m = 0x00030003u, v = upper ? w >> 8 : w;
    const u32x4 t = {v & m, (v >> 2) & m, (v >> 4) & m, (v >> 6) & m};
    return __builtin_bit_cast(half8, t);
}

// Codes of one packed dword as fp16 operands with five operations: nibbles at
// bits 4..7 of each 16-bit half are masked in place rather than shifted down,
// so the operand order is (c0,c4) (16 c1,16 c5) (c2,c6) (16 c3,16 c7) - the
// order of unpack_codes with odd coordinates (or, for a transposed read, odd
// source rows) 16 times larger; the other operand carries a factor 1/16 there.
__device__ inline half8 unpack_codes_x16(uint32_t w) {
    const uint32_t lo = 0x000F000Fu, hi = 0x00F000F0u, w8 = w >> 8;
    const u32x4 t = {w & lo, w & hi, w8 & lo, w8 & hi};
    return __builtin_bit_cast(half8, t);
}

// The same operands as unpack_codes_x16, but as normal fp16 numbers 1024 + n
// (1024 + 16 n at the odd positions): the nibbles are placed under the
// exponent of 1024 by an AND-OR, as cheap as the AND. Against q~ this adds
// 1024 sum_k q~_k to every score of a head, a constant that cancels in the
// softmax and in the merge of splits; in exchange the product is in log2 units
// already (no 2^24 scale before the exponential).
// v_and_or_b32 takes no literal operands on this target: with the three
// constants as literals the compiler emits a separate AND and OR per operand
// dword. Made opaque (x16n_const) they stay in registers (the masks in scalar
// registers, the exponent bits in a vector register: an instruction may read
// one scalar register), and the compiler selects one v_and_or_b32 for the C
// expression. It is written in C, not inline asm, on purpose: an MFMA that
// reads a VGPR written by an ordinary VALU instruction needs two wait states
// after it, and the compiler inserts them only for instructions it can see
// (behind inline asm the MFMA could read the operand's old value).
__device__ inline uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) { return (a & m) | o; }
struct X16nConst {
    uint32_t lo, hi, e;
};
__device__ inline X16nConst x16n_const() {
    // opaque to the compiler, so the values stay in registers instead of being
    // re-materialised as literals next to every use
    X16nConst c{0x000F000Fu, 0x00F000F0u, 0x64006400u};
    asm volatile("" : "+s"(c.lo), "+s"(c.hi), "+v"(c.e));
    return c;
}
__device__ inline half8 unpack_codes_x16n(uint32_t w, const X16nConst &c) {
    const uint32_t w8 = w >> 8;
    const u32x4 t = {and_or(w, c.lo, c.e), and_or(w, c.hi, c.e), and_or(w8, c.lo, c.e), and_or(w8, c.hi, c.e)};
    return __builtin_bit_cast(half8, t);
}

// Row of token r (0..31) in the nibble tile: the 16 tokens a transposed read
// gathers for one lane half are rows 16 hh .. 16 hh + 15.
__device__ inline int tile_row(int r) { return ((r >> 3) << 2) | (r & 3) | (((r >> 2) & 1) << 4); }

typedef int v2i32 __attribute__((vector_size(8)));

// ---------------------------------------------------------------- absorb
// q~[b, h, pos(k)] = scale * sum_d W_k[g d_h + d, k] q[b, h, d] for the heads h
// of kv head g. One CTA per (kv head, 64 latent columns, sequence). A thread
// holds VW adjacent columns (one VW x bf16 load per row) for the rows
// d = dg, dg + DG, ...; the DG row groups are summed through LDS.
constexpr int kAbsorbCols = 64;
constexpr int kAbsorbHeads = 4;    // heads reduced per LDS pass

template <int VW>
struct AbsorbCfg {
    static constexpr int CG = kAbsorbCols / VW;   // column groups per CTA
    static constexpr int DG = 256 / CG;           // row groups
    static constexpr int RMAX = kMaxDh / DG;      // rows per thread at most
};

template <int VW> struct VecT;
template <> struct VecT<8> { typedef u32x4 T; };
template <> struct VecT<4> { typedef uint2 T; };
template <> struct VecT<2> { typedef uint32_t T; };
template <> struct VecT<1> { typedef uint16_t T; };

template <int VW>
__device__ inline void bf16_vec_to_f32(const typename VecT<VW>::T &v, float *f) {
    if constexpr (VW == 1) {
        f[0] = __uint_as_float((uint32_t)v << 16);
    } else {
        const uint32_t *u = reinterpret_cast<const uint32_t *>(&v);
#pragma unroll
        for (int i = 0; i < VW / 2; ++i) {
            f[2 * i] = __uint_as_float(u[i] << 16);
            f[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
        }
    }
}

// LDS of the absorption, one instance per vector width (shared by both row counts)
template <int VW>
struct AbsorbSmem {
    float qs[kAbsorbHeads][kMaxDh];
    // row-group partials; a row group's stride is one float past a multiple of
    // the bank count, so a wave's 8 row groups x 8 column groups write distinct banks
    float red[AbsorbCfg<VW>::DG][kAbsorbHeads * kAbsorbCols + 1];
};
template <int VW>
__device__ inline AbsorbSmem<VW> &absorb_smem() {
    __shared__ AbsorbSmem<VW> sm;
    return sm;
}

// RR rows per thread: A::RMAX covers d_h = kMaxDh, A::RMAX / 2 covers d_h <= kMaxDh / 2
// qlo > 0 (8-bit codes): q~ is also stored as a second fp16 term, the rounding
// residual q~ - fp16(q~), at qt + qlo. With 256 levels the scores spread over
// about a hundred log2 units and the softmax is nearly an argmax, where one
// fp16 rounding of q~ (relative 2^-12) moves the leading weights by about 1%;
// the two terms carry q~ to about 2^-22.
template <int VW, int RR>
__device__ __attribute__((always_inline)) inline void absorb_rows(int g, int cblk, int b, const uint16_t *__restrict__ q,
                                   const uint16_t *__restrict__ W_kv, _Float16 *__restrict__ qt,
                                   int G, int GP, int n_q, int nqp, int n_kv, int d_h, float scale,
                                   float odd_scale, int bits, size_t qlo) {
    using A = AbsorbCfg<VW>;
    using VT = typename VecT<VW>::T;
    auto &qs = absorb_smem<VW>().qs;
    auto &red = absorb_smem<VW>().red;
    const int tid = threadIdx.x, cg = tid % A::CG, dg = tid / A::CG;
    const int k0 = cblk * kAbsorbCols + cg * VW;
    const bool kin = k0 < G;                  // G % VW == 0: the group is all in or all out
    const int grp = n_q / n_kv;
    // q rows of heads hb .. hb + 3 of this kv head, kAbsorbHeads * kMaxDh values
    // over the 256 threads, from clamped addresses (masked when staged)
    static_assert(kAbsorbHeads * kMaxDh == 4 * 256, "4 q values per thread");
    uint16_t qr[4];
    auto load_q = [&](int hb) {
        const int nh = (grp - hb) < kAbsorbHeads ? (grp - hb) : kAbsorbHeads;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = tid + 256 * u, j = i / kMaxDh, d = i - j * kMaxDh;
            const int jj = j < nh ? j : nh - 1, dd = d < d_h ? d : d_h - 1;
            qr[u] = q[((size_t)b * n_q + (size_t)g * grp + hb + jj) * d_h + dd];
        }
    };
    load_q(0);
    // this thread's output in every pass: head j_t of the pass, column col_t;
    // its operand position (integer divisions by runtime sizes) is computed
    // here, while the loads are in flight, and pinned there
    static_assert(kAbsorbHeads * kAbsorbCols == 256, "one output per thread and pass");
    const int j_t = tid / kAbsorbCols, col_t = tid % kAbsorbCols, k_t = cblk * kAbsorbCols + col_t;
    int pos_t = k_t < GP ? coord_to_pos(k_t, GP, bits) : 0;
    asm volatile("" : "+v"(pos_t));
    const float sk_t = (k_t & 1) ? scale * odd_scale : scale;
    // W_k rows of this thread: loads issued unconditionally from clamped addresses
    const uint16_t *wk = W_kv + (size_t)g * d_h * G + (kin ? k0 : 0);
    VT wr[RR];
#pragma unroll
    for (int i = 0; i < RR; ++i) {
        const int d = dg + A::DG * i;
        wr[i] = *reinterpret_cast<const VT *>(wk + (size_t)(d < d_h ? d : d_h - 1) * G);
    }
    // rows past n_q up to the 32-head padding are zero: the CTAs of kv head 0
    // clear this column block of them, one 16-byte store per thread (at most
    // 31 rows x 8 chunks; the block's columns are a contiguous 128-byte run)
    if (g == 0) {
        const int npad = nqp - n_q, pr = tid >> 3, pc = cblk * kAbsorbCols + 8 * (tid & 7);
        if (pr < npad && pc < GP) {
            const size_t o = ((size_t)b * nqp + n_q + pr) * GP + pc;
            *reinterpret_cast<u32x4 *>(qt + o) = u32x4{};
            if (qlo) *reinterpret_cast<u32x4 *>(qt + qlo + o) = u32x4{};
        }
    }
    float w[RR][VW];
#pragma unroll
    for (int i = 0; i < RR; ++i) {
        bf16_vec_to_f32<VW>(wr[i], w[i]);
        const bool ok = kin && dg + A::DG * i < d_h;
#pragma unroll
        for (int c = 0; c < VW; ++c) w[i][c] = ok ? w[i][c] : 0.0f;
    }
    for (int hb = 0; hb < grp; hb += kAbsorbHeads) {
        const int nh = (grp - hb) < kAbsorbHeads ? (grp - hb) : kAbsorbHeads;
        if (hb > 0) load_q(hb);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = tid + 256 * u, j = i / kMaxDh, d = i - j * kMaxDh;
            qs[j][d] = (j < nh && d < d_h) ? bf16_to_f32(qr[u]) : 0.0f;
        }
        __syncthreads();
        // every head of the pass at once, straight-line (staged rows of heads
        // past nh are zero; their partials are written and never read)
        float a[kAbsorbHeads][VW];
#pragma unroll
        for (int j = 0; j < kAbsorbHeads; ++j)
#pragma unroll
            for (int c = 0; c < VW; ++c) a[j][c] = 0.0f;
#pragma unroll
        for (int i = 0; i < RR; ++i) {
            const int d = dg + A::DG * i;
#pragma unroll
            for (int j = 0; j < kAbsorbHeads; ++j) {
                const float qv = qs[j][d < kMaxDh ? d : kMaxDh - 1];
#pragma unroll
                for (int c = 0; c < VW; ++c) a[j][c] += w[i][c] * qv;
            }
        }
#pragma unroll
        for (int j = 0; j < kAbsorbHeads; ++j)
#pragma unroll
            for (int c = 0; c < VW; ++c) red[dg][j * kAbsorbCols + cg * VW + c] = a[j][c];
        __syncthreads();
        if (j_t < nh && k_t < GP) {
            float sum = 0.0f;
            for (int r = 0; r < A::DG; ++r) sum += red[r][j_t * kAbsorbCols + col_t];
            const int h = g * grp + hb + j_t;
            // the fp32 product is kept as such (not folded with the fp16
            // conversion into one mixed-precision FMA, which rounds once), so
            // that every instantiation - with or without the second term -
            // rounds q~ the same way: the decode step and the two-call path
            // must give identical bits
            float v = k_t < G ? sum * sk_t : 0.0f;
            asm volatile("" : "+v"(v));
            const _Float16 hi = (_Float16)v;
            qt[((size_t)b * nqp + h) * GP + pos_t] = hi;
            if (qlo) qt[qlo + ((size_t)b * nqp + h) * GP + pos_t] = (_Float16)(v - (float)hi);
        }
        __syncthreads();
    }
}

template <int VW>
__device__ __attribute__((always_inline)) inline void absorb_body(int g, int cblk, int b, const uint16_t *__restrict__ q,
                                   const uint16_t *__restrict__ W_kv, _Float16 *__restrict__ qt,
                                   int G, int GP, int n_q, int nqp, int n_kv, int d_h, float scale,
                                   float odd_scale, int bits, size_t qlo) {
    using A = AbsorbCfg<VW>;
    if (d_h <= A::DG * (A::RMAX / 2))   // uniform
        absorb_rows<VW, A::RMAX / 2>(g, cblk, b, q, W_kv, qt, G, GP, n_q, nqp, n_kv, d_h, scale, odd_scale, bits, qlo);
    else
        absorb_rows<VW, A::RMAX>(g, cblk, b, q, W_kv, qt, G, GP, n_q, nqp, n_kv, d_h, scale, odd_scale, bits, qlo);
}

// Absorption launch of fsq_decode_attn: one CTA per (kv head, 64-column
// block, sequence), in a 1-D grid.
template <int VW>
__global__ __launch_bounds__(256) void absorb_kernel(const uint16_t *__restrict__ q,
                                                     const uint16_t *__restrict__ W_kv,
                                                     _Float16 *__restrict__ qt, int G, int GP,
                                                     int n_q, int nqp, int n_kv, int d_h, float scale,
                                                     float odd_scale, int bits, size_t qlo) {
    const int ncb = (GP + kAbsorbCols - 1) / kAbsorbCols;
    int r = blockIdx.x;
    const int g = r % n_kv;
    r /= n_kv;
    absorb_body<VW>(g, r % ncb, r / ncb, q, W_kv, qt, G, GP, n_q, nqp, n_kv, d_h, scale, odd_scale, bits, qlo);
}

// ---------------------------------------------------------- decode step
// One launch for the two independent first stages of a decode step: CTAs
// [0, n_app) append the new token of each sequence (output byte j = bx % P of
// tokens (bx / P) NT ..) at row seq_lens[b] - 1 of its cache, the rest absorb
// the queries (kv head, 64-column block, sequence). The split kernel that
// follows sees the appended rows. CPB codes per byte: 2 (4-bit codes), 4
// (2-bit) or 1 (8-bit, whose absorption also writes the second term of q~ at
// qt + qlo).
struct StepAppend {
    const uint16_t *x_new, *E;
    uint8_t *codes;
    int C;
    FsqQuant fq;   // the code width's L
};

template <int NT, int VW, int CPB>
__global__ __launch_bounds__(256) void step_prep_kernel(StepAppend ap, const int32_t *__restrict__ seq_lens,
                                                        int64_t seq_cap, int batch, int n_app,
                                                        const uint16_t *__restrict__ q,
                                                        const uint16_t *__restrict__ W_kv,
                                                        _Float16 *__restrict__ qt, int G, int GP,
                                                        int n_q, int nqp, int n_kv, int d_h, float scale,
                                                        float odd_scale, size_t qlo) {
    const int bx = blockIdx.x;
    const int P = bytes_per_token_b(G, 8 / CPB);
    if (bx < n_app) {
        append_gemv_body<NT, CPB>(bx % P, (bx / P) * NT, ap.x_new, ap.E, ap.codes, batch, ap.C, G, ap.fq,
                                  seq_lens, seq_cap);
    } else {
        const int ncb = (GP + kAbsorbCols - 1) / kAbsorbCols;
        int r = bx - n_app;
        const int g = r % n_kv;
        r /= n_kv;
        absorb_body<VW>(g, r % ncb, r / ncb, q, W_kv, qt, G, GP, n_q, nqp, n_kv, d_h, scale, odd_scale, 8 / CPB,
                        qlo);
    }
}

template <int NT, int CPB>
static void launch_step_prep_nt(int vw, dim3 grid, hipStream_t st, const StepAppend &ap,
                                const int32_t *seq_lens, int64_t seq_cap, int batch, int n_app,
                                const uint16_t *q, const uint16_t *W_kv, _Float16 *qt, int G, int GP,
                                int n_q, int nqp, int n_kv, int d_h, float scale, float odd_scale,
                                size_t qlo) {
#define FSQ_PREP_ARGS ap, seq_lens, seq_cap, batch, n_app, q, W_kv, qt, G, GP, n_q, nqp, n_kv, d_h, scale, odd_scale, qlo
    switch (vw) {
        case 8: step_prep_kernel<NT, 8, CPB><<<grid, 256, 0, st>>>(FSQ_PREP_ARGS); break;
        case 4: step_prep_kernel<NT, 4, CPB><<<grid, 256, 0, st>>>(FSQ_PREP_ARGS); break;
        case 2: step_prep_kernel<NT, 2, CPB><<<grid, 256, 0, st>>>(FSQ_PREP_ARGS); break;
        default: step_prep_kernel<NT, 1, CPB><<<grid, 256, 0, st>>>(FSQ_PREP_ARGS);
    }
#undef FSQ_PREP_ARGS
}

// ----------------------------------------------------------------- split
// One CTA = NW waves (8 or 4) working through its token chunk in rounds of
// NW x 32 tokens.
// In a round each wave loads (one round ahead, straight into registers),
// unpacks and scores its own 32-token tile against all 32 heads; the waves then
// agree on a per-head reference max and normaliser through LDS, and every wave
// pools all 4 tiles but only for its own latent coordinate blocks (block cb
// belongs to wave cb % NW). The softmax state is therefore identical in all
// waves and the pooled sums need no cross-wave combine.
template <int GP, int NW>
struct SplitCfg {
    static constexpr int KB = GP / 16;                 // score k-blocks = dwords per lane half
    static constexpr int CB = GP / 32;                 // pooling coordinate blocks
    static constexpr int CBW = (CB + NW - 1) / NW;   // blocks per wave
    static constexpr int RS = (GP / 2 + 63) / 64 * 64; // dwords per fp16 tile row
    static constexpr int kTileDw = kTile * RS;
    static constexpr int kZBytes = NW * kTileDw * 4;
    // 4-bit codes: per-wave nibble tiles (the packed rows, read back by
    // ds_read_b64_tr_b4) instead of fp16 copies, a quarter of the LDS bytes
    static constexpr int TSN = GP / 2 + 8;             // nibble-tile row stride: an odd number of 8-byte units
    static constexpr int kNibBytes = NW * kTile * TSN;
    // the probability region also stages Q~ (32 rows of GP + 8 halves) before
    // the first round: its first writes follow the max barrier, after every
    // wave has read its Q~ operands, so the tiles need no barrier of their own
    static constexpr int kPBytes = (NW * 2 * 64 * 16) > (32 * (GP + 8) * 2) ? (NW * 2 * 64 * 16) : (32 * (GP + 8) * 2);
};

// XOR swizzle (dword granularity) of the fp16 tile: the 16-byte row writes of
// 16 consecutive rows and the transposing 8-byte reads of 4 rows x 16 dwords
// both fall on distinct LDS banks.
__device__ inline int zt_swz(int row) { return 16 * (row & 3) + 4 * ((row >> 2) & 3); }

template <int GP, int NW, bool AL, int BITS>
__global__ __launch_bounds__(NW * 64) void decode_split_kernel(
    const _Float16 *__restrict__ qt, const uint8_t *__restrict__ codes,
    const int32_t *__restrict__ seq_lens, _Float16 *__restrict__ part_z,
    float *__restrict__ part_ml, int64_t seq_cap, int G, int n_q, int nqp, int chunk, int S, size_t qlo) {
    using C = SplitCfg<GP, NW>;
    constexpr int KB = C::KB, CB = C::CB, CBW = C::CBW, RS = C::RS;
    constexpr int HB = GP * BITS / 16;       // bytes of a lane's half of a token row
    constexpr int ND = HB / 4;               // packed dwords per half (KB operands of 8 codes)
    constexpr int NLD = AL ? ND : ND + 1;   // dwords loaded per lane per tile
    static_assert(!AL || ND % 2 == 0, "8-byte loads of whole halves");
    __shared__ __attribute__((aligned(16))) uint32_t zsm[(BITS == 4 ? C::kNibBytes : C::kZBytes) / 4];
    __shared__ __attribute__((aligned(16))) uint8_t psm[C::kPBytes];
    __shared__ float tmax_s[NW][32], tsum_s[NW][32];

    const int P = bytes_per_token_b(G, BITS);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int s = blockIdx.x, b = blockIdx.y, hg = blockIdx.z;
    const int64_t c0 = (int64_t)s * chunk;   // < seq_cap: the grid has ceil(seq_cap / chunk) chunks
    // The first round's loads are issued before the sequence length is known,
    // bounded by the cache capacity (rows up to seq_cap - 1 are inside the
    // buffer); rows past the length are masked once it has arrived.
    int64_t c1 = (c0 + chunk < seq_cap) ? c0 + chunk : seq_cap;
    const int t = lane & 31, hh = lane >> 5;
    const uint8_t *seq = codes + (size_t)b * seq_cap * P;
    // the sequence length is requested first and used after the Q~ barrier
    const int32_t T_raw = seq_lens[b];

    // ---- per-lane loads of one tile (this lane's half of token t)
    uint32_t ld[NLD];
    int ld_ntok = 0, ld_sh = 0;
    // Every load is unconditional (tiles past the chunk re-read its first row,
    // and are never used), so that a wait for one load counts exactly the loads
    // issued after it.
    auto issue = [&](int64_t t0) {
        const int64_t rem = c1 - t0;
        ld_ntok = rem <= 0 ? 0 : (rem < kTile ? (int)rem : kTile);
        const int64_t tb = ld_ntok == 0 ? c0 : t0;
        const int nr = ld_ntok == 0 ? 1 : ld_ntok;
        const int tc = t < nr ? t : nr - 1;
        if (AL) {
            // G == GP and P % 16 == 0: the half is ND whole, 8-byte aligned dwords
            const uint2 *src = reinterpret_cast<const uint2 *>(seq + (size_t)(tb + tc) * P + hh * HB);
#pragma unroll
            for (int i = 0; i < ND / 2; ++i) {
                const uint2 v = src[i];
                ld[2 * i] = v.x;
                ld[2 * i + 1] = v.y;
            }
        } else {
            // aligned dwords around the half, clamped to the tile's last dword
            const uint8_t *a = seq + (size_t)(tb + tc) * P + hh * HB;
            ld_sh = (int)((uintptr_t)a & 3) * 8;
            const uint32_t *a0 = reinterpret_cast<const uint32_t *>(a - ((uintptr_t)a & 3));
            const uint8_t *lastb = seq + (size_t)(tb + nr) * P - 1;
            const uint32_t *last = reinterpret_cast<const uint32_t *>(lastb - ((uintptr_t)lastb & 3));
#pragma unroll
            for (int i = 0; i < NLD; ++i) ld[i] = *(a0 + i <= last ? a0 + i : last);
        }
    };

    // Q~ rows of this head group (32 x GP fp16, contiguous) are read from global
    // once per CTA into LDS (rows padded to GP + 8 halves for conflict-free
    // 16-byte reads), then each wave takes its B operands from there. They are
    // requested first, so that staging them waits for them alone while the
    // first tile's codes are still in flight.
    constexpr int NQ16 = 32 * GP / 8;                    // 16-byte chunks
    constexpr int NQI = (NQ16 + NW * 64 - 1) / (NW * 64);
    u32x4 qreg[NQI];
    {
        const u32x4 *qsrc = reinterpret_cast<const u32x4 *>(qt + ((size_t)b * nqp + hg * 32) * GP);
#pragma unroll
        for (int u = 0; u < NQI; ++u) {
            const int i = threadIdx.x + u * NW * 64;
            qreg[u] = qsrc[i < NQ16 ? i : NQ16 - 1];
        }
    }
    half8 qv[KB];
    // 8-bit codes: the residual term of q~ (see absorb_rows), B operands read
    // straight from global memory
    half8 qvl[BITS == 8 ? KB : 1];
    if constexpr (BITS == 8) {
        const _Float16 *ql = qt + qlo + ((size_t)b * nqp + hg * 32 + t) * GP + 8 * hh;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) qvl[kb] = *reinterpret_cast<const half8 *>(ql + 16 * kb);
    }
    // issue order pinned: Q~, then the first tile (the compiler would move the
    // tile's loads behind the Q~ barrier, or ahead of the Q~ loads)
    __builtin_amdgcn_sched_barrier(0);
    issue(c0 + wave * kTile);
    __builtin_amdgcn_sched_barrier(0);

    {
        constexpr int QROW = GP + 8;
        _Float16 *qsm = reinterpret_cast<_Float16 *>(psm);   // free until the first max barrier
#pragma unroll
        for (int u = 0; u < NQI; ++u) {
            // threads past the last chunk rewrite it with the same data (no
            // branch, so that its load stays where it was issued)
            const int i0 = threadIdx.x + u * NW * 64, i = i0 < NQ16 ? i0 : NQ16 - 1;
            const int r = i / (GP / 8), c = i - r * (GP / 8);
            *reinterpret_cast<u32x4 *>(qsm + r * QROW + 8 * c) = qreg[u];
        }
        __syncthreads();
        // the sequence length: leave if this chunk is past it (uniform), else
        // bound the chunk and recount the first round's tokens
        int64_t T = T_raw;
        T = T < 0 ? 0 : (T > seq_cap ? seq_cap : T);
        if (c0 >= T) {
            // the first tile's words are used on this path too (waited for,
            // harmlessly, before leaving), so that their loads stay ahead of
            // the Q~ barrier instead of being sunk behind this branch
            asm volatile("" ::"v"(ld[0]));
            return;
        }
        c1 = (c0 + chunk < T) ? c0 + chunk : T;
        const int64_t rem0 = c1 - (c0 + wave * kTile);
        ld_ntok = rem0 <= 0 ? 0 : (rem0 < kTile ? (int)rem0 : kTile);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            qv[kb] = *reinterpret_cast<const half8 *>(qsm + t * QROW + 16 * kb + 8 * hh);
    }

    float m_ref = -INFINITY, l_run = 0.0f;
    floatx16 acc[CBW];
#pragma unroll
    for (int j = 0; j < CBW; ++j) acc[j] = floatx16{};

    uint32_t *zt_own = zsm + wave * C::kTileDw;
    const int i16 = lane & 15, g16 = (lane >> 4) & 1;
    const int mrow = i16 >> 2, pcol = i16 & 3;
    typedef __attribute__((address_space(3))) shortx4 lds_s4;
    typedef short short8 __attribute__((ext_vector_type(8)));

    for (int64_t r0 = c0; r0 < c1; r0 += NW * kTile) {
        // ---- phase 1: own tile -> fp16 codes -> LDS tile + scores
        uint32_t cur[ND];
        const int ntok = ld_ntok;
        const int sh = ld_sh;
        if (AL) {
#pragma unroll
            for (int i = 0; i < ND; ++i) cur[i] = ld[i];
        } else {
#pragma unroll
            for (int i = 0; i < ND; ++i)
                cur[i] = (uint32_t)((((uint64_t)ld[i + 1] << 32) | ld[i]) >> sh);
        }
        issue(r0 + NW * kTile + wave * kTile);

        // No masking of the loaded words: tokens past the chunk's end (rows
        // clamped into the cache) get probability 0 below, and coordinates in
        // the padding G..GP-1 (bytes of the next row) meet zero q~ entries and
        // are never read back from the pooled sums; all codes are finite.
        // Scores are accumulated in units of 2^-24 (unpack_codes) and scaled
        // when they enter the max and the exponent. 4-bit codes go to the
        // wave's nibble tile as loaded (row tile_row(t), this lane's half) and
        // are scored by unpack_codes_x16 against q~ with odd coordinates / 16.
        if constexpr (BITS == 4) {
            uint8_t *tdst = reinterpret_cast<uint8_t *>(zsm) + (wave * kTile + tile_row(t)) * C::TSN + hh * (GP / 4);
#pragma unroll
            for (int i = 0; i < KB / 2; ++i)
                *reinterpret_cast<uint2 *>(tdst + 8 * i) = uint2{cur[2 * i], cur[2 * i + 1]};
        }
        floatx16 sc = floatx16{};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const half8 z = BITS == 8   ? unpack_codes8(cur[2 * kb], cur[2 * kb + 1])
                            : BITS == 2 ? unpack_codes2(cur[kb >> 1], kb & 1)
                                        : unpack_codes_x16(cur[kb]);
            if constexpr (BITS != 4)
                *reinterpret_cast<half8 *>(zt_own + t * RS + ((8 * kb + 4 * hh) ^ zt_swz(t))) = z;
            sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(z, qv[kb], sc, 0, 0, 0);
            if constexpr (BITS == 8) sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(z, qvl[kb], sc, 0, 0, 0);
        }
        float sv[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int tok = (r >> 2) * 8 + hh * 4 + (r & 3);
            sv[r] = tok < ntok ? sc[r] : -INFINITY;
            tmax = fmaxf(tmax, sv[r]);
        }
        tmax = halves_max(tmax) * kCodeScale;
        if (lane < 32) tmax_s[wave][t] = tmax;
        __syncthreads();

        // ---- phase 2: common reference max (lazy), probabilities, row sums
        float rmax = tmax_s[0][t];
#pragma unroll
        for (int w = 1; w < NW; ++w) rmax = fmaxf(rmax, tmax_s[w][t]);
        const bool bump = rmax > m_ref + kRescaleSlack;
        const float m_new = bump ? rmax : m_ref;
        const float alpha = bump ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
        const bool rescale = bump && m_ref != -INFINITY;
        m_ref = m_new;
        float psum = 0.0f;
        _Float16 p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            p[r] = (_Float16)__builtin_amdgcn_exp2f(fmaf(sv[r], kCodeScale, -m_new));
            psum += (float)p[r];   // the normaliser sums the fp16 weights the pooling uses
        }
        psum = halves_sum(psum);
        if (lane < 32) tsum_s[wave][t] = psum;
        // pooling operands: with nibble tiles, in the order of unpack_codes_x16
        // applied to a transposed read (pairs of rows, the second pair's
        // weights / 16: they meet codes read 16x)
        const _Float16 w16 = BITS == 4 ? (_Float16)0.0625f : (_Float16)1.0f;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const half8 pv = {p[ks * 8 + 0], p[ks * 8 + 1], p[ks * 8 + 2] * w16, p[ks * 8 + 3] * w16,
                              p[ks * 8 + 4], p[ks * 8 + 5], p[ks * 8 + 6] * w16, p[ks * 8 + 7] * w16};
            *reinterpret_cast<half8 *>(psm + ((wave * 2 + ks) * 64 + lane) * 16) = pv;
        }
        __syncthreads();
        float rsum = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) rsum += tsum_s[w][t];
        l_run = l_run * alpha + rsum;
        if (__any(rescale)) {
#pragma unroll
            for (int j = 0; j < CBW; ++j) acc[j] *= alpha;
        }

        // ---- phase 3: pool the round's tiles for this wave's coordinate blocks.
        // Block cb = wave + NW j; when CB is a multiple of NW every wave owns CBW
        // blocks (known at compile time), otherwise ownership is wave-uniform.
        // A tile past the chunk's end holds finite codes and zero probabilities
        // (phases 1 and 2 wrote them), so all NW tiles are pooled and the LDS
        // operand reads of tile w2 + 1 are issued before the MFMAs of tile w2.
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        if constexpr (BITS == 4) {
            // transposed nibble reads: lane l addresses row 16 hh + (d & 8) +
            // sigma^-1(d & 7) (d = l & 15; sigma as in tile_row) of a wave's
            // tile, bytes 16 cb + 8 ((l >> 4) & 1): the A operand of block cb
            // for the tile's 32 tokens in two k-steps, coordinates in natural
            // order, matched by the probabilities' order above
            const int dsrc = lane & 15;
            const int rsrc = 16 * hh + (dsrc & 8) + (((dsrc & 3) << 1) | ((dsrc >> 2) & 1));
            const uint8_t *trb = reinterpret_cast<const uint8_t *>(zsm) + rsrc * C::TSN + 8 * ((lane >> 4) & 1);
            typedef __attribute__((address_space(3))) v2i32 lds_v2;
            half8 pn[2][2];
            v2i32 zn[2][CBW];
            auto read_nib = [&](int w2, half8 (&pbo)[2], v2i32 (&zo)[CBW]) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    pbo[ks] = *reinterpret_cast<const half8 *>(psm + ((w2 * 2 + ks) * 64 + lane) * 16);
#pragma unroll
                for (int j = 0; j < CBW; ++j) {
                    const int cb = wv + NW * j;
                    if (CB % NW == 0 || cb < CB)
                        zo[j] = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
                            (lds_v2 *)(trb + w2 * kTile * C::TSN + 16 * cb));
                }
            };
            read_nib(0, pn[0], zn[0]);
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) {
                const int cur_b = w2 & 1;
                if (w2 + 1 < NW) read_nib(w2 + 1, pn[cur_b ^ 1], zn[cur_b ^ 1]);
#pragma unroll
                for (int j = 0; j < CBW; ++j) {
                    if (CB % NW == 0 || wv + NW * j < CB) {
                        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(unpack_codes_x16((uint32_t)zn[cur_b][j][0]),
                                                                        pn[cur_b][0], acc[j], 0, 0, 0);
                        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(unpack_codes_x16((uint32_t)zn[cur_b][j][1]),
                                                                        pn[cur_b][1], acc[j], 0, 0, 0);
                    }
                }
            }
        } else {
        half8 pb[2][2];
        shortx4 za[2][2][CBW][2];
        auto read_ops = [&](int w2, half8 (&pbo)[2], shortx4 (&zao)[2][CBW][2]) {
            const uint32_t *zt = zsm + w2 * C::kTileDw;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                pbo[ks] = *reinterpret_cast<const half8 *>(psm + ((w2 * 2 + ks) * 64 + lane) * 16);
                const int ra = ks * 16 + hh * 4 + mrow, rb = ra + 8;
#pragma unroll
                for (int j = 0; j < CBW; ++j) {
                    const int cb = wv + NW * j;
                    if (CB % NW == 0 || cb < CB) {
                        const int cdw = cb * 16 + g16 * 8 + pcol * 2;
                        zao[ks][j][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_s4 *)(zt + ra * RS + (cdw ^ zt_swz(ra))));
                        zao[ks][j][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_s4 *)(zt + rb * RS + (cdw ^ zt_swz(rb))));
                    }
                }
            }
        };
        read_ops(0, pb[0], za[0]);
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) {
            const int cur_b = w2 & 1;
            if (w2 + 1 < NW) read_ops(w2 + 1, pb[cur_b ^ 1], za[cur_b ^ 1]);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int j = 0; j < CBW; ++j) {
                    if (CB % NW == 0 || wv + NW * j < CB) {
                        const shortx4 lo = za[cur_b][ks][j][0], hi = za[cur_b][ks][j][1];
                        const short8 zs = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, zs),
                                                                        pb[cur_b][ks], acc[j], 0, 0, 0);
                    }
                }
        }
        }
        __syncthreads();   // the next round overwrites the tiles and probabilities
    }

    // ---- epilogue: zbar = acc / l, fp16, stored from registers: each lane
    // holds head t and, per block, 4 runs of 4 positions (natural coordinate
    // order from nibble tiles; operand-position order from fp16 tiles)
    const float zscale = kCodeScale / l_run;   // codes n * 2^-24 pooled: zbar = 2^24 acc / l - L/2
    constexpr float kLevelOffset = (float)(1 << (BITS - 1));
    const int heads = (n_q - hg * 32) < 32 ? (n_q - hg * 32) : 32;
    // partials are head-major: row ((b n_q + h) S + s), so a head's rows are contiguous
    const size_t pbase = ((size_t)b * n_q + hg * 32) * S + s;
    typedef _Float16 half4 __attribute__((ext_vector_type(4)));
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    if (t < heads) {
        _Float16 *dst = part_z + (pbase + (size_t)t * S) * GP;
#pragma unroll
        for (int j = 0; j < CBW; ++j) {
            const int cb = wv + NW * j;
            if (CB % NW == 0 || cb < CB) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const half4 v = {(_Float16)fmaf(acc[j][4 * r4 + 0], zscale, -kLevelOffset),
                                     (_Float16)fmaf(acc[j][4 * r4 + 1], zscale, -kLevelOffset),
                                     (_Float16)fmaf(acc[j][4 * r4 + 2], zscale, -kLevelOffset),
                                     (_Float16)fmaf(acc[j][4 * r4 + 3], zscale, -kLevelOffset)};
                    *reinterpret_cast<half4 *>(dst + cb * 32 + r4 * 8 + hh * 4) = v;
                }
            }
        }
    }
    if (wave == 0 && lane < heads) {
        part_ml[(pbase + (size_t)lane * S) * 2 + 0] = m_ref;
        part_ml[(pbase + (size_t)lane * S) * 2 + 1] = l_run;
    }
}

// ----------------------------------------------------------- streaming split

// The split kernel above makes its waves agree on one softmax state per round,
// which costs three barriers and an fp16 copy of every tile in LDS per round;
// that is the right trade when a CTA covers one or two rounds (short caches,
// where launch and dependent latency dominate), not when it streams many.
// decode_stream_kernel is the variant for long chunks. Each wave is an
// independent flash-decoding unit over the tiles k = wave, wave + NW, ... of
// the CTA's chunk with its own (m, l, acc) for all 32 heads and all GP latent
// coordinates; the waves combine once, at the end of the chunk. Per tile:
//   1. global -> LDS: the tile's packed bytes (one contiguous range of the
//      sequence) arrive by 16-byte direct-to-LDS loads into a ring of D slots
//      per wave, issued D - 1 tiles ahead, so each wave keeps D - 1 tiles of
//      codes in flight without holding them in registers;
//   2. scores: each lane reads its half of its token's row from the slot,
//      unpacks to fp16 operands (codes as subnormals, see unpack_codes), and
//      the waves' MFMAs compute all 32 heads' scores (K = latent coordinates);
//   3. the same packed half-rows are written, still as nibbles, to a per-wave
//      tile whose rows are 8-byte aligned and padded to an odd number of
//      8-byte units;
//   4. pooling: ds_read_b64_tr_b4 transposes 16 x 16 nibble blocks of that
//      tile, so a lane receives 16 tokens of one latent coordinate, which is
//      the operand layout of the pooling MFMA (K = tokens). The tokens behind
//      the 16 nibbles are chosen (through the tile's row order) to be exactly
//      the tokens whose probabilities the lane already holds from step 2, so
//      no probability crosses lanes.
// LDS traffic per code byte: DMA write 1, row read 1, tile write 1, transposed
// read 1. Pooled sums come out in natural coordinate order.
template <int GP, int NW, int D, bool AL>
struct StreamCfg {
    static constexpr int KB = GP / 16;                 // score k-blocks = dwords per lane half
    static constexpr int CB = GP / 32;                 // pooling coordinate blocks
    static constexpr int RB = GP / 2;                  // bytes of a token's row window
    static constexpr int TS = RB + 8;                  // nibble-tile row stride: an odd number of 8-byte units
    static constexpr int NEED = AL ? 32 * RB : 32 * RB + 32;   // a tile's bytes + alignment slack + read overrun
    static constexpr int SLOTB = NEED < 1024 ? 1024 : (NEED + 127) / 128 * 128;
    static constexpr int NI = (SLOTB + 1023) / 1024;   // direct-to-LDS loads per tile (64 lanes x 16 B)
    static constexpr int RING = NW * D * SLOTB;
    static constexpr bool PAIR = GP < 128;             // tiles taken two at a time (absorbed queries)
    static constexpr int TILE = NW * 32 * TS * (PAIR ? 2 : 1);   // per-wave nibble tile(s)
    static constexpr int QST = 32 * (GP + 8) * 2;      // Q~ staging, prologue only (aliases the tiles)
    static constexpr int CBYTES = NW * 64 * 16 * 4;    // one coordinate block of every wave's sums
    static constexpr int BPP0 = RING / CBYTES;
    static constexpr int BPP = BPP0 < 1 ? 1 : (BPP0 > CB ? CB : BPP0);   // blocks per combine pass
    static constexpr int COMB = BPP * CBYTES;          // the combine reuses the ring
    static constexpr int RINGA = RING > COMB ? RING : COMB;
    static_assert(QST <= TILE, "Q~ staging must fit in the tile region");
    static_assert((D - 1) * NI < 64, "vmcnt field");
    static_assert(KB % 2 == 0 && (!AL || KB % 4 == 0), "row halves in whole 8 / 16-byte units");
};

// Byte offset inside a ring slot of logical byte L of the tile: 16-byte chunks
// are XOR-permuted inside each 128-byte line by the line index, so that the
// same chunk of 8 consecutive 128-byte rows falls on distinct LDS banks.
// The permutation is its own inverse.
__device__ inline int slot_phys(int L) { return L ^ (((L >> 7) & 7) << 4); }

// Reads of a ring slot, written in asm. The slot is filled by direct-to-LDS
// loads, and before any ordinary LDS read of that LDS object the compiler
// waits for every such load in flight (vmcnt(0)), since it cannot tell which
// slot a load targets: that would drain the ring on every tile. The kernel's
// own s_waitcnt vmcnt already guarantees the slot being read is complete.
// Each block waits for its own reads (lgkmcnt) before returning them.
// a: LDS byte addresses.
template <int N>
__device__ __attribute__((always_inline)) inline void slot_read_b32(const uint32_t (&a)[N], uint32_t (&v)[N]) {
    static_assert(N >= 1, "");
    if constexpr (N >= 4) {
        asm volatile("ds_read_b32 %0, %4\n\tds_read_b32 %1, %5\n\tds_read_b32 %2, %6\n\tds_read_b32 %3, %7\n\t"
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
                     : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
                     : "memory");
        if constexpr (N > 4) {
            uint32_t ar[N - 4], vr[N - 4];
#pragma unroll
            for (int i = 0; i < N - 4; ++i) ar[i] = a[4 + i];
            slot_read_b32<N - 4>(ar, vr);
#pragma unroll
            for (int i = 0; i < N - 4; ++i) v[4 + i] = vr[i];
        }
    } else if constexpr (N == 3) {
        asm volatile("ds_read_b32 %0, %3\n\tds_read_b32 %1, %4\n\tds_read_b32 %2, %5\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2])
                     : "v"(a[0]), "v"(a[1]), "v"(a[2])
                     : "memory");
    } else if constexpr (N == 2) {
        asm volatile("ds_read_b32 %0, %2\n\tds_read_b32 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(v[0]), "=&v"(v[1])
                     : "v"(a[0]), "v"(a[1])
                     : "memory");
    } else {
        asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v[0]) : "v"(a[0]) : "memory");
    }
}
template <int N>
__device__ __attribute__((always_inline)) inline void slot_read_b128(const uint32_t (&a)[N], u32x4 (&v)[N]) {
    static_assert(N >= 1 && N <= 4, "1..4 reads");
    if constexpr (N == 4) {
        asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
                     : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
                     : "memory");
    } else if constexpr (N == 3) {
        asm volatile("ds_read_b128 %0, %3\n\tds_read_b128 %1, %4\n\tds_read_b128 %2, %5\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2])
                     : "v"(a[0]), "v"(a[1]), "v"(a[2])
                     : "memory");
    } else if constexpr (N == 2) {
        asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(v[0]), "=&v"(v[1])
                     : "v"(a[0]), "v"(a[1])
                     : "memory");
    } else {
        asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v[0]) : "v"(a[0]) : "memory");
    }
}
__device__ inline uint32_t lds_addr(const uint8_t *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
}

// This lane's half of token t's row (GP / 4 bytes, KB dwords) out of a ring
// slot: 16-byte reads when rows are 16-byte aligned (AL), else the KB + 1
// dwords around the half, funnel-shifted by the row's misalignment.
template <int GP, bool AL>
__device__ __attribute__((always_inline)) inline void slot_row(const uint8_t *slot, int t, int hh, int P, int mis,
                                                               uint32_t (&cur)[GP / 16]) {
    constexpr int KB = GP / 16;
    if constexpr (AL) {
        uint32_t a[KB / 4];
        u32x4 v[KB / 4];
#pragma unroll
        for (int i = 0; i < KB / 4; ++i) a[i] = lds_addr(slot + slot_phys(t * P + hh * (GP / 4) + 16 * i));
        slot_read_b128<KB / 4>(a, v);
#pragma unroll
        for (int i = 0; i < KB / 4; ++i) {
            cur[4 * i + 0] = v[i].x;
            cur[4 * i + 1] = v[i].y;
            cur[4 * i + 2] = v[i].z;
            cur[4 * i + 3] = v[i].w;
        }
    } else {
        const int ab = mis + t * P + hh * (GP / 4);
        const int a0 = ab & ~3, sh = (ab & 3) * 8;
        uint32_t a[KB + 1], ld[KB + 1];
#pragma unroll
        for (int i = 0; i < KB + 1; ++i) a[i] = lds_addr(slot + slot_phys(a0 + 4 * i));
        slot_read_b32<KB + 1>(a, ld);
#pragma unroll
        for (int i = 0; i < KB; ++i) cur[i] = (uint32_t)((((uint64_t)ld[i + 1] << 32) | ld[i]) >> sh);
    }
}


// N transposed nibble reads (ds_read_b64_tr_b4) at LDS byte address a + 16 i,
// issued back to back and waited for in the same asm block. Written in asm
// because the compiler makes the builtin form wait for every direct-to-LDS
// load in flight (to any LDS object), which would drain the code ring.
// Result i: lane l of a 16-lane group receives nibble (l & 15) of the 8 bytes
// that lane 16 (l / 16) + d of the group addresses, as nibble d (d = 0..15).
template <int N>
__device__ __attribute__((always_inline)) inline void tr4_reads(uint32_t a, v2i32 (&v)[N]);
template <>
__device__ __attribute__((always_inline)) inline void tr4_reads<1>(uint32_t a, v2i32 (&v)[1]) {
    asm volatile("ds_read_b64_tr_b4 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v[0]) : "v"(a) : "memory");
}
template <>
__device__ __attribute__((always_inline)) inline void tr4_reads<2>(uint32_t a, v2i32 (&v)[2]) {
    asm volatile("ds_read_b64_tr_b4 %0, %2\n\tds_read_b64_tr_b4 %1, %2 offset:16\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]) : "v"(a) : "memory");
}
template <>
__device__ __attribute__((always_inline)) inline void tr4_reads<3>(uint32_t a, v2i32 (&v)[3]) {
    asm volatile("ds_read_b64_tr_b4 %0, %3\n\tds_read_b64_tr_b4 %1, %3 offset:16\n\t"
                 "ds_read_b64_tr_b4 %2, %3 offset:32\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]) : "v"(a) : "memory");
}
template <>
__device__ __attribute__((always_inline)) inline void tr4_reads<4>(uint32_t a, v2i32 (&v)[4]) {
    asm volatile("ds_read_b64_tr_b4 %0, %4\n\tds_read_b64_tr_b4 %1, %4 offset:16\n\t"
                 "ds_read_b64_tr_b4 %2, %4 offset:32\n\tds_read_b64_tr_b4 %3, %4 offset:48\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]) : "v"(a) : "memory");
}
template <int N>
__device__ __attribute__((always_inline)) inline void tr4_reads(uint32_t a, v2i32 (&v)[N]) {
    static_assert(N > 4 && N <= 8, "1..8 reads");
    v2i32 lo[4], hi[N - 4];
    tr4_reads<4>(a, lo);
    tr4_reads<N - 4>(a + 64, hi);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = lo[i];
#pragma unroll
    for (int i = 0; i < N - 4; ++i) v[4 + i] = hi[i];
}

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// operations, not for its global loads (__syncthreads would also wait for the
// direct-to-LDS loads in flight, draining the ring) nor its global stores.
__device__ __attribute__((always_inline)) inline void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Inputs of the key-reconstruction variants (RC = 1, 2): instead of absorbed
// queries, each CTA serves the heads of one kv head g and rebuilds the tile's
// keys K = Z W_k,g^T (d_h <= 128, d_h % 32 == 0) before scoring them against
// q. RC = 2 also applies the rest of Eq. 5: the key RMS norm (gamma, eps) and
// rotate-half RoPE at each key's cache position, with the rotation of channel
// pair (i, i + d_h/2) for position t being t * rope_f[i] / 2^64 revolutions.
struct ReconArgs {
    const uint16_t *q, *W_kv;
    int n_kv, d_h;
    float scale;
    const uint16_t *gamma;   // RC = 2: [d_h] bf16
    float eps;               // RC = 2
    uint64_t rope_f[64];     // RC = 2: theta^(-2i/d_h) / (2 pi) in units of 2^-64, i < d_h/2
};
constexpr int kReconMaxDh = 128;

// Codes of one packed dword as fp16 levels n - 8 (exact) in the order of
// unpack_codes: the nibble is placed under the exponent of 1024.0 and 1032 is
// subtracted.
__device__ inline half8 unpack_codes_centered(uint32_t w) {
    const uint32_t m = 0x000F000Fu, e = 0x64006400u;
    const u32x4 t = {(w & m) | e, ((w >> 4) & m) | e, ((w >> 8) & m) | e, ((w >> 12) & m) | e};
    const _Float16 c = (_Float16)1032.0f;
    return __builtin_bit_cast(half8, t) - half8{c, c, c, c, c, c, c, c};
}

// Device-side split of the streaming kernel (kDynMaxBatch sequences or fewer):
// the chunk is chosen from the actual lengths, so that the sum of all
// sequences' tokens spreads over ncta CTAs in whole rounds of q tokens (the
// CTA's waves x 32), at least chunk_min (which bounds a sequence's split count by the
// workspace's). Sequence b then has ceil(T_b / chunk) work items, numbered
// consecutively over the sequences; CTA i takes item i. Every wave of a CTA
// computes this the same way: lane b holds T_b (one vector load), a wave sum
// gives the total, a prefix scan of the item counts locates item i.
__device__ inline int stream_dyn_chunk(int64_t total, int ncta, int nseq, int chunk_min, int64_t q) {
    // chunk >= total / n with n = ncta - nseq + 1: sequence b has
    // ceil(T_b / chunk) <= (T_b + chunk - 1) / chunk items, so all of them
    // number at most total / chunk + nseq - nseq / chunk < n + nseq = ncta + 1,
    // i.e. at most ncta, and every item has a CTA of the one resident set
    // (nseq <= 64 <= ncta / 4). One sequence gets exactly ncta items when its
    // length is a multiple of ncta rounds.
    // By an fp64 division: total < 2^37 and n <= 2^10, so the correctly rounded
    // quotient is within 2^-15 of the exact one, whose fraction is 0 or at
    // least 2^-10: its floor is the integer quotient
    // rounded up to whole rounds by a mask: q, a round of 32 tokens times the
    // streaming kernel's 4 or 8 waves, is a power of two (a 64-bit division by
    // a runtime value costs dozens of instructions in every wave)
    const int n = ncta - nseq + 1;
    int64_t c = (int64_t)floor((double)(total + n - 1) / (double)n);
    c = (c + q - 1) & ~(q - 1);
    return (int)(c < chunk_min ? chunk_min : c);
}
// Cross-lane arithmetic without LDS (DPP and lane swaps; the compiler adds the
// DPP hazard waits). update_dpp writes 0 where a lane is masked off or its
// source lane lies outside the row.
template <int CTRL, int ROWS = 0xF, int BANKS = 0xF>
__device__ inline uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, BANKS, true);
}
// Sum over the 64 lanes, in every lane: quad swaps, half-row and row mirrors
// leave each 16-lane row's sum in all its lanes; v_permlane16_swap and
// v_permlane32_swap return the operand with rows (halves) exchanged.
__device__ inline uint32_t wave_sum_u32(uint32_t a) {
    a += dpp_u32<0xB1>(a);    // quad_perm [1, 0, 3, 2]
    a += dpp_u32<0x4E>(a);    // quad_perm [2, 3, 0, 1]
    a += dpp_u32<0x141>(a);   // row_half_mirror
    a += dpp_u32<0x140>(a);   // row_mirror
    const auto r16 = __builtin_amdgcn_permlane16_swap(a, a, false, false);
    a = r16[0] + r16[1];
    const auto r32 = __builtin_amdgcn_permlane32_swap(a, a, false, false);
    return r32[0] + r32[1];
}
// Sum of 64 lengths 0 <= v < 2^31 (exact: 16-bit halves summed in 32 bits)
__device__ inline int64_t wave_sum64(int64_t v) {
    const uint32_t lo = wave_sum_u32((uint32_t)v & 0xFFFFu), hi = wave_sum_u32((uint32_t)((uint64_t)v >> 16));
    return ((int64_t)hi << 16) + (int64_t)lo;
}
// Inclusive prefix sum over lanes 0..l: within rows by shifts 1, 2, 3 of the
// input, then 4 and 8 of the partial sums (upper banks only), then each row's
// last lane added to the rows after it (row_bcast:15 to rows 1, 3;
// row_bcast:31 to rows 2, 3).
__device__ inline uint32_t wave_scan_u32(uint32_t v) {
    uint32_t x = v + dpp_u32<0x111>(v);
    x += dpp_u32<0x112>(v);
    x += dpp_u32<0x113>(v);
    x += dpp_u32<0x114, 0xF, 0xE>(x);
    x += dpp_u32<0x118, 0xF, 0xC>(x);
    x += dpp_u32<0x142, 0xA, 0xF>(x);
    x += dpp_u32<0x143, 0xC, 0xF>(x);
    return x;
}
// lane's clamped length T_lane (0 past the batch) and the chunk
__device__ inline int stream_dyn_lens(const int32_t *__restrict__ seq_lens, int batch, int64_t seq_cap, int64_t q,
                                      int ncta, int chunk_min, int lane, int64_t &t_lane) {
    int64_t T = lane < batch ? (int64_t)seq_lens[lane] : 0;
    T = T < 0 ? 0 : (T > seq_cap ? seq_cap : T);
    t_lane = T;
    return stream_dyn_chunk(wave_sum64(T), ncta, batch, chunk_min, q);
}

template <int GP, int NW, int D, bool AL, int RC>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(RC ? 1 : 2))) void decode_stream_kernel(
    const _Float16 *__restrict__ qt, const uint8_t *__restrict__ codes,
    const int32_t *__restrict__ seq_lens, _Float16 *__restrict__ part_z,
    float *__restrict__ part_ml, int64_t seq_cap, int G, int n_q, int nqp, int chunk_arg, int S,
    int dyn_batch, int ncta, ReconArgs ra) {
    // dyn_batch > 0: device-side split (stream_dyn_lens), 1-D grid of CTAs over
    // work items; chunk_arg is then the smallest chunk. Otherwise CTA (s, b)
    // takes tokens [s chunk_arg, (s + 1) chunk_arg) of sequence b.
    using C = StreamCfg<GP, NW, D, AL>;
    constexpr int KB = C::KB, CB = C::CB, TS = C::TS, SLOTB = C::SLOTB, NI = C::NI;
    // scores arrive in units of 2^-24 from absorbed queries (codes as fp16
    // subnormals), in plain log2 units from rebuilt keys (rescaled below)
    constexpr float kSS = RC ? 1.0f : kCodeScale;
    // absorbed queries below GP 128: scores computed in the wave's frame (see
    // weigh); wider latents keep the running max (no registers to spare for
    // the frame's constants, whose spills cost more than they save)
    constexpr bool FRAME = !RC && GP < 128;
    constexpr int WROW = GP + 8;   // rebuilt-key operand rows (halves), RC only
    // s_waitcnt immediates (gfx9 layout), only vmcnt waited on
    constexpr int kWaitAhead = (((D - 1) * NI) & 0xF) | (0x7 << 4) | (0xF << 8) | ((((D - 1) * NI) >> 4) << 14);
    constexpr int kWaitAll = (0x7 << 4) | (0xF << 8);
    // The ring (the only target of direct-to-LDS loads) and the nibble tiles are
    // distinct LDS objects, so the compiler's waits for those loads do not
    // extend to the tile stores.
    // REG (below GP 128, absorbed queries) uses this space only to combine the
    // waves, all coordinate blocks at once
    constexpr bool REGC = C::PAIR && !RC;
    constexpr int RING_BYTES = REGC ? C::CB * C::CBYTES : C::RINGA;
    __shared__ __attribute__((aligned(16))) uint8_t ring_lds[RING_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t tile_lds[C::TILE];
    __shared__ __attribute__((aligned(16))) _Float16 wk_lds[RC ? kReconMaxDh * WROW : 8];
    __shared__ float gam_lds[RC == 2 ? kReconMaxDh : 1];
    __shared__ uint64_t rope_lds[RC == 2 ? kReconMaxDh / 2 : 1];
    __shared__ float ms[NW][32], ls[NW][32];

    const int P = (G + 1) / 2;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hg = blockIdx.z;
    // Q~ rows of head group hg of a sequence (32 x GP fp16, contiguous): NQI
    // 16-byte loads per thread, issued first for the sequence known before the
    // split is (the only one of a one-sequence call, or CTA row blockIdx.y) and
    // again once it is known if it differs
    constexpr int QROW = GP + 8;
    constexpr int NQ16 = 32 * GP / 8;
    constexpr int NQI = (NQ16 + NW * 64 - 1) / (NW * 64);
    u32x4 qreg[RC ? 1 : NQI];
    auto load_q = [&](int bq) {
        if constexpr (!RC) {
            const u32x4 *qsrc = reinterpret_cast<const u32x4 *>(qt + ((size_t)bq * nqp + hg * 32) * GP);
#pragma unroll
            for (int u = 0; u < NQI; ++u) {
                const int i = threadIdx.x + u * NW * 64;
                qreg[u] = qsrc[i < NQ16 ? i : NQ16 - 1];
            }
        }
    };
    const int b_early = dyn_batch > 0 ? 0 : (int)blockIdx.y;
    load_q(b_early);
    int s, b, chunk;
    int64_t T_dyn = 0;
    if (dyn_batch == 1) {   // one sequence: item i is chunk i of it
        int64_t T0 = seq_lens[0];
        T0 = T0 < 0 ? 0 : (T0 > seq_cap ? seq_cap : T0);
        chunk = stream_dyn_chunk(T0, ncta, 1, chunk_arg, 32 * NW);
        b = 0;
        s = blockIdx.x;
        if ((int64_t)s * chunk >= T0) return;   // no work left (uniform)
        T_dyn = T0;
    } else if (dyn_batch > 0) {
        int64_t t_lane;
        chunk = stream_dyn_lens(seq_lens, dyn_batch, seq_cap, 32 * NW, ncta, chunk_arg, lane, t_lane);
        const int n = (int)(((uint32_t)t_lane + (uint32_t)chunk - 1u) / (uint32_t)chunk);   // this lane's sequence's items (T < 2^31)
        const int incl = (int)wave_scan_u32((uint32_t)n);
        const int item = blockIdx.x;
        b = __builtin_popcountll(__ballot(incl <= item));   // sequences wholly before the item
        if (b >= dyn_batch) return;                         // no work left (uniform)
        // wave-uniform values kept in scalar registers (b is uniform: lane reads)
        chunk = __builtin_amdgcn_readfirstlane(chunk);
        s = item - (__builtin_amdgcn_readlane(incl, b) - __builtin_amdgcn_readlane(n, b));
        T_dyn = (int64_t)(uint32_t)__builtin_amdgcn_readlane((int)t_lane, b);   // T < 2^31
        if ((int64_t)s * chunk >= T_dyn) return;   // never taken (s < the sequence's items); keeps every tile inside it
        if (b != b_early) load_q(b);   // uniform
    } else {
        s = blockIdx.x;
        b = blockIdx.y;
        chunk = chunk_arg;
    }
    const int64_t c0 = (int64_t)s * chunk;   // < seq_cap: the grid has ceil(seq_cap / chunk) chunks
    // until the sequence length arrives, tiles are bounded by the cache capacity
    // (the device-side split knows it already)
    const int64_t cap_b = dyn_batch > 0 ? T_dyn : seq_cap;
    int64_t cend = (c0 + chunk < cap_b) ? c0 + chunk : cap_b;
    const int t = lane & 31, hh = lane >> 5;
    const uint8_t *seq = codes + (size_t)b * seq_cap * P;
    // the sequence length is requested first and used once Q~ is in LDS
    const int32_t T_raw = dyn_batch > 0 ? (int32_t)T_dyn : seq_lens[b];
    uint8_t *ring = ring_lds + wave * D * SLOTB;
    uint8_t *tile = tile_lds + wave * 32 * TS * (C::PAIR ? 2 : 1);

    auto tiles_before = [&](int64_t e) -> int {   // this wave's tiles starting before token e
        const int64_t first = c0 + (int64_t)kTile * wave;
        return e <= first ? 0 : (int)((e - first + (int64_t)kTile * NW - 1) / ((int64_t)kTile * NW));
    };
    auto tile_t0 = [&](int j) -> int64_t { return c0 + (int64_t)kTile * (wave + NW * j); };
    // direct-to-LDS loads of tile j (which starts before cend) into slot j % D:
    // NI loads of 64 x 16 bytes; the last load's window is moved back to end at
    // the slot's end (overlapping windows write the same bytes), and chunks
    // past the tile's last byte repeat that byte's chunk
    auto issue = [&](int j) {
        int64_t t0 = tile_t0(j);
        int64_t rem = cend - t0;
        if (rem <= 0) {   // prologue only: a tile past the chunk re-reads its first row
            t0 = c0;
            rem = 1;
        }
        const int n = rem < kTile ? (int)rem : kTile;
        const uintptr_t A = (uintptr_t)(seq + (size_t)t0 * P);
        const uintptr_t a0 = A & ~(uintptr_t)15;
        const uintptr_t last = (A + (uintptr_t)n * P - 1) & ~(uintptr_t)15;
        uint8_t *slot = ring + (j % D) * SLOTB;
        // byte offsets from a0 (wave-uniform) in 32 bits: one clamp per load
        const uint32_t lim = (uint32_t)(last - a0);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int pb = (i * 1024 < SLOTB - 1024) ? i * 1024 : SLOTB - 1024;
            const uint32_t off = (uint32_t)slot_phys(pb + 16 * lane);
            const uint8_t *src = reinterpret_cast<const uint8_t *>(a0) + (off < lim ? off : lim);
            __builtin_amdgcn_global_load_lds((glb_void_t *)src, (lds_void_t *)(slot + pb), 16, 0, 0);
        }
    };

    // Below GP 128 (absorbed queries) the codes bypass the ring: each lane loads
    // the dwords around its half of its token's row straight into registers,
    // four tiles ahead (REG below); the ring and its LDS reads serve the wider
    // latents and the key-reconstruction variants.
    constexpr bool REG = REGC;
    // dwords per lane and tile (REG): the KB + 1 aligned dwords around the
    // lane's half (funnel-shifted by its byte offset) for every row alignment
    constexpr int NLD = KB + 1;
    // lane window: byte loff of the 4-byte aligned sequence base sb, relative to
    // each tile's first row (t0 P is a multiple of 4: t0 is a multiple of 32)
    const uint32_t loff = (uint32_t)(((uintptr_t)seq & 3u) + (uint32_t)(t * P + hh * (GP / 4)));
    const uint32_t voff = loff & ~3u, fsh = (loff & 3u) * 8u;
    // (pointer arithmetic rather than integer casts, so that the compiler keeps
    // these global-memory pointers and emits global, not flat, loads)
    const uint8_t *sb = seq - ((uintptr_t)seq & 3u);
    // the last dword holding bytes of this sequence's rows (clamp of the tiles
    // that end near the cache capacity)
    const uint8_t *lastb = seq + (size_t)seq_cap * P - 1;
    const uint8_t *lastdw = lastb - ((uintptr_t)lastb & 3u);
    uint32_t rb[REG ? 4 : 1][REG ? NLD : 1];
    // tile jt of this wave into registers. The loads need no bounds checks
    // while the windows end inside the next row (t0 + 32 < seq_cap); a tile
    // past the chunk, or the one tile that ends at the cache capacity, loads
    // the sequence's first tile instead (a valid address; that data is never
    // used: the capacity-end tile is reloaded with clamped addresses when it
    // is processed). The plan takes this kernel only for seq_cap >= 64.
    auto load_tile = [&](int jt, auto &dst) {
        if constexpr (REG) {
            int64_t t0 = tile_t0(jt);
            if (t0 >= cend || t0 + kTile >= seq_cap) t0 = 0;
            const uint32_t *src = reinterpret_cast<const uint32_t *>(sb + (size_t)t0 * P + voff);
#pragma unroll
            for (int i = 0; i < NLD; ++i) dst[i] = src[i];
        }
    };
    // Q~ rows of this head group -> LDS (rows padded to GP + 8 halves) -> each
    // lane's B operands, as in the split kernel. Only the first tile is loaded
    // alongside (the compiler waits for all loads before the Q~ stores); the
    // ring's other D - 2 tiles are issued once Q~ is in place, so they are in
    // flight while the first tile is processed. (REG: the first four tiles,
    // into registers.)
    if constexpr (REG) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < 4; ++k) load_tile(k, rb[k]);
        __builtin_amdgcn_sched_barrier(0);
    } else {
        issue(0);
    }
    half8 qv[RC ? 1 : KB];
    half8 qb[RC ? 4 : 1][2];   // RC: B operands q[head][d] * scale per 32-row block of d and half
    const int grp = RC ? n_q / ra.n_kv : 32;
    if constexpr (RC) {
        // W_k,g (bf16, [d_h][G]) -> fp16 rows of WROW halves in operand order
        // (RC = 1: odd coordinates scaled 1/16, they meet codes read 16x); zero
        // past G
        const int g = hg, DB = ra.d_h / 32;
        const uint16_t *wk = ra.W_kv + (size_t)g * ra.d_h * G;
        for (int it = threadIdx.x; it < ra.d_h * (GP / 8); it += NW * 64) {
            const int d = it / (GP / 8), Dw = it - d * (GP / 8);   // 8 coordinates 8 Dw .. 8 Dw + 7
            half8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = 8 * Dw + e;
                const float x = c < G ? bf16_to_f32(wk[(size_t)d * G + c]) : 0.0f;
                v[((e & 3) << 1) | (e >> 2)] = (_Float16)((RC == 1 && (e & 1)) ? x * 0.0625f : x);
            }
            *reinterpret_cast<half8 *>(wk_lds + d * WROW + 16 * (Dw % KB) + 8 * (Dw / KB)) = v;
        }
        if constexpr (RC == 2) {
            for (int i = threadIdx.x; i < ra.d_h; i += NW * 64) gam_lds[i] = bf16_to_f32(ra.gamma[i]);
            for (int i = threadIdx.x; i < ra.d_h / 2; i += NW * 64) rope_lds[i] = ra.rope_f[i];
        }
        // q operands: lane = head n of this kv head, K slot (hh, jj) of block
        // (db, e) = d 32 db + (2 e + jj / 4) 8 + 4 hh + jj % 4
        // (lanes past the group's heads and blocks past d_h read in-bounds
        // elements and zero them)
        const bool hv = t < grp;
        const uint16_t *qh = ra.q + ((size_t)b * n_q + (size_t)g * grp + (hv ? t : 0)) * ra.d_h;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int d = 32 * db + (2 * e + (jj >> 2)) * 8 + 4 * hh + (jj & 3);
                    const bool ok = hv && db < DB;
                    const float x = bf16_to_f32(qh[ok ? d : 0]) * ra.scale;
                    qb[db][e][jj] = (_Float16)(ok ? x : 0.0f);
                }
        lds_barrier();
        int64_t T = T_raw;
        T = T < 0 ? 0 : (T > seq_cap ? seq_cap : T);
        if (c0 >= T) {   // uniform: nothing to do; no load may still target the LDS
            __builtin_amdgcn_s_waitcnt(kWaitAll);
            return;
        }
        cend = (c0 + chunk < T) ? c0 + chunk : T;
    } else {
        _Float16 *qsm = reinterpret_cast<_Float16 *>(tile_lds);   // the tiles are free here
#pragma unroll
        for (int u = 0; u < NQI; ++u) {
            // threads past the last chunk rewrite it with the same data (no
            // branch, so the loads stay ahead of the ring's)
            const int i0 = threadIdx.x + u * NW * 64, i = i0 < NQ16 ? i0 : NQ16 - 1;
            const int r = i / (GP / 8), c = i - r * (GP / 8);
            *reinterpret_cast<u32x4 *>(qsm + r * QROW + 8 * c) = qreg[u];
        }
        lds_barrier();
        int64_t T = T_raw;
        T = T < 0 ? 0 : (T > seq_cap ? seq_cap : T);
        if (c0 >= T) {   // uniform: nothing to do; no load may still target the LDS
            __builtin_amdgcn_s_waitcnt(kWaitAll);
            return;
        }
        cend = (c0 + chunk < T) ? c0 + chunk : T;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            qv[kb] = *reinterpret_cast<const half8 *>(qsm + t * QROW + 16 * kb + 8 * hh);
        lds_barrier();   // before the tile region is reused
    }
    const int nt = tiles_before(cend);
    if constexpr (!REG) {
#pragma unroll
        for (int j = 1; j < D - 1; ++j) issue(j);   // a static number of loads (see issue)
    }

    float m_ref = -INFINITY, l_run = 0.0f;
    floatx16 acc[CB];
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[j] = floatx16{};

    // Absorbed queries below GP 128 (FRAME): scores come out of the MFMAs already shifted
    // into the wave's frame. With codes as 1024 + n (unpack_codes_x16n) the
    // product sum S of a head is in log2 units; the score MFMAs start from cfr
    // instead of zero, so element r of a lane ends as S + fr - 4 o(r), where fr
    // is the head's frame and o(r) = 1 for the token slots the pooling reads 16x
    // (elements 2, 3, 6, 7, 10, 11, 14, 15): exp2 of it is the weight p = 2^(S +
    // fr), or p / 16 at those slots, with no subtraction or scaling on the VALU.
    // The frame is set by the first step's maximum and lowered only when a
    // weight would leave fp16 (p >= 65520 is converted to infinity, which makes
    // the step's normaliser infinite): then the step is redone against its own
    // maximum (a rare path). Weights stay below 2^16 x 16, the frame never rises
    // above the running maximum, and -fr plays the part of the running max m.
    float fr = 0.0f;
    bool fresh = true;   // no step seen yet (wave-uniform)
    const X16nConst xc = x16n_const();
    floatx16 cfr_keep;
    auto set_cfr = [&]() {
#pragma unroll
        for (int r = 0; r < 16; ++r) cfr_keep[r] = ((r >> 1) & 1) ? fr - 4.0f : fr;
    };
    auto cfr = [&]() { return cfr_keep; };
    set_cfr();
    // weights of NTL scored tiles (ph[u][i] = elements 2i, 2i + 1 of tile u, in
    // fp16), the normaliser of exactly those fp16 values (x16 at the 1/16
    // slots), the frame's rare updates
    auto weigh = [&](auto ntl_c, auto &sc, const auto &ntok, auto &ph) {
        constexpr int NTL = decltype(ntl_c)::value;
#pragma unroll
        for (int u = 0; u < NTL; ++u)
            if (ntok[u] < kTile) {   // the chunk's last tile only (uniform)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int tok = (r >> 2) * 8 + hh * 4 + (r & 3);
                    sc[u][r] = tok < ntok[u] ? sc[u][r] : -INFINITY;
                }
            }
        const half2 one2 = {(_Float16)1.0f, (_Float16)1.0f}, c16 = {(_Float16)16.0f, (_Float16)16.0f};
        float psum = 0.0f;
#pragma unroll
        for (int u = 0; u < NTL; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float e0 = __builtin_amdgcn_exp2f(sc[u][2 * i]), e1 = __builtin_amdgcn_exp2f(sc[u][2 * i + 1]);
                ph[u][i] = half2{(_Float16)e0, (_Float16)e1};
                psum = __builtin_amdgcn_fdot2(ph[u][i], (i & 1) ? c16 : one2, psum, false);
            }
        if (__builtin_expect(fresh || __any(!(psum < INFINITY)), 0)) {
            // the step's maximum of S + fr per head (slot offsets undone)
            float tm = -INFINITY;
#pragma unroll
            for (int u = 0; u < NTL; ++u)
#pragma unroll
                for (int r = 0; r < 16; ++r) tm = fmaxf(tm, ((r >> 1) & 1) ? sc[u][r] + 4.0f : sc[u][r]);
            tm = halves_max(tm);
            const float fr_new = (fresh || tm > kRescaleSlack) ? fr - tm : fr;
            const float d = fr_new - fr;
            if (!fresh) {
                const float alpha = __builtin_amdgcn_exp2f(d);
                l_run *= alpha;
                if (__any(d != 0.0f)) {
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) acc[cb] *= alpha;
                }
            }
            fr = fr_new;
            fresh = false;
            set_cfr();
            psum = 0.0f;
#pragma unroll
            for (int u = 0; u < NTL; ++u)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float e0 = __builtin_amdgcn_exp2f(sc[u][2 * i] + d);
                    const float e1 = __builtin_amdgcn_exp2f(sc[u][2 * i + 1] + d);
                    ph[u][i] = half2{(_Float16)e0, (_Float16)e1};
                    psum = __builtin_amdgcn_fdot2(ph[u][i], (i & 1) ? c16 : one2, psum, false);
                }
        }
        l_run += psum;
    };

    // transposed-read source row of this lane: nibble d of the result is token
    // row (16 hh + (d & 8) + sigma^-1(d & 7)); see the unpack order
    const int dsrc = lane & 15;
    const int rsrc = 16 * hh + (dsrc & 8) + (((dsrc & 3) << 1) | ((dsrc >> 2) & 1));
    const uint8_t *trsrc = tile + rsrc * TS + 8 * ((lane >> 4) & 1);
    const uint32_t tr_addr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)trsrc;
    uint8_t *tdst = tile + tile_row(t) * TS + hh * (GP / 4);

    if constexpr (REG) {
        // Two tiles per step: two independent score chains, one softmax update
        // for 64 tokens, and pooling from two nibble tiles, which gives a wave
        // twice the independent work between its waits. The registers hold
        // four tiles: a step takes tiles j, j + 1 from one pair of buffers and
        // refills that pair with tiles j + 4, j + 5, so two steps of codes are
        // in flight; the compiler's waits count exactly those loads.
        auto step = [&](auto ntl_c, int j, auto &x0, auto &x1) {
            constexpr int NTL = decltype(ntl_c)::value;
            uint32_t cur[NTL][KB];
            int ntok[NTL];
#pragma unroll
            for (int u = 0; u < NTL; ++u) {
                const int64_t rem = cend - tile_t0(j + u);
                ntok[u] = rem < kTile ? (int)rem : kTile;
                const auto &x = u == 0 ? x0 : x1;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)   // (v_alignbit: no register pairs)
                    cur[u][kb] = __builtin_amdgcn_alignbit(x[kb + 1], x[kb], fsh);
#pragma unroll
                for (int i = 0; i < KB / 2; ++i)
                    *reinterpret_cast<uint2 *>(tdst + u * 32 * TS + 8 * i) = uint2{cur[u][2 * i], cur[u][2 * i + 1]};
            }
            if constexpr (NTL == 2) {
                load_tile(j + 4, x0);
                load_tile(j + 5, x1);
            }
            // scores, the tiles' chains interleaved, each started from the frame
            floatx16 sc[NTL];
#pragma unroll
            for (int u = 0; u < NTL; ++u)
                sc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(unpack_codes_x16n(cur[u][0], xc), qv[0], cfr(), 0, 0, 0);
#pragma unroll
            for (int kb = 1; kb < KB; ++kb)
#pragma unroll
                for (int u = 0; u < NTL; ++u)
                    sc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(unpack_codes_x16n(cur[u][kb], xc), qv[kb], sc[u], 0, 0, 0);
            // weights of the step's tokens (lane: head t, tokens tok(r))
            half2 ph[NTL][8];
            weigh(ntl_c, sc, ntok, ph);
            // pooling (B operands as in the one-tile loop below)
            v2i32 zt[NTL][CB];
#pragma unroll
            for (int u = 0; u < NTL; ++u) tr4_reads<CB>(tr_addr + u * 32 * TS, zt[u]);
#pragma unroll
            for (int u = 0; u < NTL; ++u) {
                const half8 pv0 = {ph[u][0].x, ph[u][0].y, ph[u][1].x, ph[u][1].y, ph[u][2].x, ph[u][2].y, ph[u][3].x, ph[u][3].y};
                const half8 pv1 = {ph[u][4].x, ph[u][4].y, ph[u][5].x, ph[u][5].y, ph[u][6].x, ph[u][6].y, ph[u][7].x, ph[u][7].y};
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(unpack_codes_x16((uint32_t)zt[u][cb][0]), pv0, acc[cb], 0, 0, 0);
                    acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(unpack_codes_x16((uint32_t)zt[u][cb][1]), pv1, acc[cb], 0, 0, 0);
                }
            }
        };
        constexpr std::integral_constant<int, 2> two{};
        constexpr std::integral_constant<int, 1> one{};
        // tiles with no bounds concerns: all but (possibly) the capacity-end one
        const int64_t fast_end = seq_cap - kTile < cend ? seq_cap - kTile : cend;
        const int nf = tiles_before(fast_end);
        int j = 0;
        for (; j + 3 < nf; j += 4) {
            step(two, j, rb[0], rb[1]);
            step(two, j + 2, rb[2], rb[3]);
        }
        if (j + 1 < nf) {
            step(two, j, rb[0], rb[1]);
            if (j + 2 < nf) step(one, j + 2, rb[2], rb[3]);
        } else if (j < nf) {
            step(one, j, rb[0], rb[1]);
        }
        if (nf < nt) {   // the capacity-end tile (this wave's last): dwords past
                         // the sequence's last one are clamped to it
            const uint8_t *tb = sb + (size_t)tile_t0(nt - 1) * P + voff;
            uint32_t rx[NLD];
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const uint8_t *a = tb + 4 * i;
                rx[i] = *reinterpret_cast<const uint32_t *>(a < lastdw ? a : lastdw);
            }
            step(one, nt - 1, rx, rx);
        }
    } else
    for (int j = 0; j < nt; ++j) {
        const bool ahead = j + D - 1 < nt;
        if (ahead) issue(j + D - 1);   // into the slot tile j - 1 used
        if (ahead)
            __builtin_amdgcn_s_waitcnt(kWaitAhead);
        else
            __builtin_amdgcn_s_waitcnt(kWaitAll);
        const int64_t t0 = tile_t0(j);
        const int64_t rem = cend - t0;
        const int ntok = rem < kTile ? (int)rem : kTile;
        const uint8_t *slot = ring + (j % D) * SLOTB;

        // ---- this lane's half of token t's row (GP / 4 bytes) -> KB dwords.
        // Rows past the tile's tokens and padding coordinates G..GP-1 hold
        // finite codes (stale slot bytes or the next row's): the former get
        // probability 0, the latter meet zero q~ entries and are never read back.
        uint32_t cur[KB];
        slot_row<GP, AL>(slot, t, hh, P, AL ? 0 : (int)((uintptr_t)(seq + (size_t)t0 * P) & 15), cur);
#pragma unroll
        for (int i = 0; i < KB / 2; ++i)
            *reinterpret_cast<uint2 *>(tdst + 8 * i) = uint2{cur[2 * i], cur[2 * i + 1]};

        // ---- scores of the tile's 32 tokens for the 32 heads (units of 2^-24)
        floatx16 sc = floatx16{};
        if constexpr (FRAME) {   // started from the frame (see weigh), accumulated in place
            sc = cfr();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(unpack_codes_x16n(cur[kb], xc), qv[kb], sc, 0, 0, 0);
        } else if constexpr (!RC) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(unpack_codes_x16(cur[kb]), qv[kb], sc, 0, 0, 0);
        } else {
            // rebuilt keys, 32-row blocks of K^T[d][token] = sum_c W_k[d][c] z_c;
            // lane (token t, half hh) holds d = 32 db + (r/4) 8 + 4 hh + r%4.
            // RC = 1: codes as subnormals (units of 2^-24, levels + 8: the
            // offset adds 8 rowsum_d, a per-head score constant that cancels in
            // the softmax). RC = 2: the levels themselves, as N_k needs them.
            const int DB = ra.d_h / 32;
            half8 zb[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                zb[kb] = RC == 2 ? unpack_codes_centered(cur[kb]) : unpack_codes_x16(cur[kb]);
            floatx16 kt[4];
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                kt[db] = floatx16{};
                if (db < DB) {
                    const _Float16 *wr = wk_lds + (32 * db + t) * WROW + 8 * hh;
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
                        kt[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            *reinterpret_cast<const half8 *>(wr + 16 * kb), zb[kb], kt[db], 0, 0, 0);
                }
            }
            if constexpr (RC == 2) {
                // N_k: k * gamma / sqrt(mean(k^2) + eps) over the token's d_h
                // channels (this lane's half, then the other half's sum)
                float ss = 0.0f;
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) ss = fmaf(kt[db][r], kt[db][r], ss);
                ss = halves_sum(ss);
                const float inv = __builtin_amdgcn_rsqf(ss / (float)ra.d_h + ra.eps);
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int d = 32 * db + (r >> 2) * 8 + 4 * hh + (r & 3);
                        kt[db][r] *= inv * gam_lds[d < ra.d_h ? d : 0];
                    }
                // RoPE_t on pairs (d, d + d_h/2): blocks db and db + DB/2, same r
                // (d_h is 64 or 128, so DB is 2 or 4)
                const uint64_t pos = (uint64_t)(t0 + t);
                auto rot = [&](floatx16 &x, floatx16 &y, int db) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int d = 32 * db + (r >> 2) * 8 + 4 * hh + (r & 3);
                        const uint64_t ph = pos * rope_lds[d];   // revolutions mod 1, units of 2^-64
                        const float rev = (float)(uint32_t)(ph >> 40) * 5.9604645e-8f;   // 2^-24
                        const float cs = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
                        const float a = x[r], bb = y[r];
                        x[r] = a * cs - bb * sn;
                        y[r] = bb * cs + a * sn;
                    }
                };
                if (DB == 4) {
                    rot(kt[0], kt[2], 0);
                    rot(kt[1], kt[3], 1);
                } else {
                    rot(kt[0], kt[1], 0);
                }
            }
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                if (db < DB) {
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        half8 ka;
#pragma unroll
                        for (int jj = 0; jj < 8; ++jj)
                            ka[jj] = (_Float16)(RC == 1 ? kt[db][8 * e + jj] * kCodeScale : kt[db][8 * e + jj]);
                        sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qb[db][e], sc, 0, 0, 0);
                    }
                }
            }
        }

        half8 pv0, pv1;
        if constexpr (FRAME) {
            floatx16 sc1[1] = {sc};
            const int nt1[1] = {ntok};
            half2 ph[1][8];
            weigh(std::integral_constant<int, 1>{}, sc1, nt1, ph);
            pv0 = half8{ph[0][0].x, ph[0][0].y, ph[0][1].x, ph[0][1].y, ph[0][2].x, ph[0][2].y, ph[0][3].x, ph[0][3].y};
            pv1 = half8{ph[0][4].x, ph[0][4].y, ph[0][5].x, ph[0][5].y, ph[0][6].x, ph[0][6].y, ph[0][7].x, ph[0][7].y};
        } else {
        // ---- online softmax of this wave (lane: head t, tokens tok(r))
        float sv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[r] = sc[r];
        if (ntok < kTile) {   // the chunk's last tile only (uniform)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int tok = (r >> 2) * 8 + hh * 4 + (r & 3);
                sv[r] = tok < ntok ? sv[r] : -INFINITY;
            }
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sv[r]);
        tmax = halves_max(tmax) * kSS;
        const bool bump = tmax > m_ref + kRescaleSlack;
        const float m_new = bump ? tmax : m_ref;
        const float alpha = bump ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
        const bool rescale = bump && m_ref != -INFINITY;
        m_ref = m_new;
        // weights p in fp16, pairwise; the normaliser sums exactly those fp16
        // values (v_dot2 with (1, 1) accumulates in fp32)
        half2 ph[8];
        float psum = 0.0f;
        const half2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float e0 = __builtin_amdgcn_exp2f(fmaf(sv[2 * i], kSS, -m_new));
            const float e1 = __builtin_amdgcn_exp2f(fmaf(sv[2 * i + 1], kSS, -m_new));
            ph[i] = half2{(_Float16)e0, (_Float16)e1};
            psum = __builtin_amdgcn_fdot2(ph[i], one2, psum, false);
        }
        l_run = l_run * alpha + psum;
        if (__any(rescale)) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) acc[cb] *= alpha;
        }
        // pooling B operands: K slots 2, 3, 6, 7 meet codes read 16x (odd
        // source rows of the transposed read), so their weights are scaled by 1/16
        const half2 s16 = {(_Float16)0.0625f, (_Float16)0.0625f};
        const half2 q1 = ph[1] * s16, q3 = ph[3] * s16, q5 = ph[5] * s16, q7 = ph[7] * s16;
        pv0 = half8{ph[0].x, ph[0].y, q1.x, q1.y, ph[2].x, ph[2].y, q3.x, q3.y};
        pv1 = half8{ph[4].x, ph[4].y, q5.x, q5.y, ph[6].x, ph[6].y, q7.x, q7.y};
        }

        // ---- pooling: acc[cb][coordinate 32 cb + m][head] += z^T p
        v2i32 zt[CB];
        tr4_reads<CB>(tr_addr, zt);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(unpack_codes_x16((uint32_t)zt[cb][0]), pv0, acc[cb], 0, 0, 0);
            acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(unpack_codes_x16((uint32_t)zt[cb][1]), pv1, acc[cb], 0, 0, 0);
        }
    }

    // ---- combine the waves: M = max m_w, c_w = 2^(m_w - M), L = sum c_w l_w,
    // zbar = 2^24 sum c_w acc_w / L - 8, summed in wave order
    const int heads = RC ? grp : ((n_q - hg * 32) < 32 ? (n_q - hg * 32) : 32);
    const size_t pbase = ((size_t)b * n_q + hg * (RC ? grp : 32)) * S + s;   // head-major partial rows
    typedef _Float16 half4 __attribute__((ext_vector_type(4)));
    if constexpr (REG) {
        // Every wave's (m, l) and unscaled sums go to LDS (which nothing else
        // uses here) before one barrier; wave cb % NW then weighs and sums
        // block cb of all waves.
        m_ref = fresh ? -INFINITY : -fr;
        const float l_w = halves_sum(l_run);
        if (lane < 32) {
            ms[wave][lane] = m_ref;
            ls[wave][lane] = l_w;
        }
        floatx4 *cbuf = reinterpret_cast<floatx4 *>(ring_lds);   // [block][wave][4][64 lanes]
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                cbuf[((cb * NW + wave) * 4 + e) * 64 + lane] =
                    floatx4{acc[cb][4 * e], acc[cb][4 * e + 1], acc[cb][4 * e + 2], acc[cb][4 * e + 3]};
        __builtin_amdgcn_s_waitcnt(kWaitAll);   // the loads of tiles past the chunk
        lds_barrier();
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, ms[w][t]);
        float L = 0.0f, cw[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float mw = ms[w][t];
            cw[w] = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
            L += cw[w] * ls[w][t];
        }
        const float zscale = kCodeScale / L;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            if (cb % NW == wave && t < heads) {
                _Float16 *dst = part_z + (pbase + (size_t)t * S) * GP + cb * 32 + hh * 4;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    floatx4 sum = cbuf[((cb * NW + 0) * 4 + e) * 64 + lane] * cw[0];
#pragma unroll
                    for (int w = 1; w < NW; ++w) sum += cbuf[((cb * NW + w) * 4 + e) * 64 + lane] * cw[w];
                    const half4 v = {(_Float16)fmaf(sum[0], zscale, -8.0f), (_Float16)fmaf(sum[1], zscale, -8.0f),
                                     (_Float16)fmaf(sum[2], zscale, -8.0f), (_Float16)fmaf(sum[3], zscale, -8.0f)};
                    *reinterpret_cast<half4 *>(dst + 8 * e) = v;
                }
            }
        }
        if (wave == 0 && lane < heads) {
            part_ml[(pbase + (size_t)lane * S) * 2 + 0] = M;
            part_ml[(pbase + (size_t)lane * S) * 2 + 1] = L;
        }
        return;
    }
    __builtin_amdgcn_s_waitcnt(kWaitAll);   // prologue loads past the length may be in flight
    lds_barrier();                          // every wave is done with its ring and tile
    if constexpr (FRAME) m_ref = fresh ? -INFINITY : -fr;
    const float l_w = halves_sum(l_run);
    if (lane < 32) {
        ms[wave][lane] = m_ref;
        ls[wave][lane] = l_w;
    }
    lds_barrier();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, ms[w][t]);
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const float mw = ms[w][t];
        L += mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M) * ls[w][t];
    }
    const float cw = m_ref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_ref - M);
    const float zscale = kCodeScale / L;
    floatx4 *cbuf = reinterpret_cast<floatx4 *>(ring_lds);   // [block][wave][4][64 lanes]
#pragma unroll
    for (int p0 = 0; p0 < CB; p0 += C::BPP) {
#pragma unroll
        for (int i = 0; i < C::BPP; ++i) {
            if (p0 + i < CB) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    cbuf[((i * NW + wave) * 4 + e) * 64 + lane] =
                        floatx4{acc[p0 + i][4 * e], acc[p0 + i][4 * e + 1], acc[p0 + i][4 * e + 2],
                                acc[p0 + i][4 * e + 3]} * cw;
            }
        }
        lds_barrier();
#pragma unroll
        for (int i = 0; i < C::BPP; ++i) {
            const int cb = p0 + i;
            if (cb < CB && cb % NW == wave) {
                floatx4 sum[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) sum[e] = cbuf[((i * NW + 0) * 4 + e) * 64 + lane];
#pragma unroll
                for (int w = 1; w < NW; ++w)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sum[e] += cbuf[((i * NW + w) * 4 + e) * 64 + lane];
                if (t < heads) {
                    _Float16 *dst = part_z + (pbase + (size_t)t * S) * GP + cb * 32 + hh * 4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const half4 v = {(_Float16)fmaf(sum[e][0], zscale, -8.0f),
                                         (_Float16)fmaf(sum[e][1], zscale, -8.0f),
                                         (_Float16)fmaf(sum[e][2], zscale, -8.0f),
                                         (_Float16)fmaf(sum[e][3], zscale, -8.0f)};
                        *reinterpret_cast<half4 *>(dst + 8 * e) = v;
                    }
                }
            }
        }
        lds_barrier();
    }
    if (wave == 0 && lane < heads) {
        part_ml[(pbase + (size_t)lane * S) * 2 + 0] = M;
        part_ml[(pbase + (size_t)lane * S) * 2 + 1] = L;
    }
}

// ----------------------------------------------------------------- merge
// One CTA of 16 waves per (head, sequence): out = W_v,g zbar with
//   zbar = sum_i c_i zbar_i / sum_i c_i,  c_i = l_i 2^(m_i - M),  M = max_i m_i.
// Every global load (this thread's part of its W_v row, VW bf16 per load, and R
// partial rows per thread with their (m, l)) is issued before any is used; 16
// waves keep more of them in flight per CU than 4 would, which is what bounds
// this kernel. The sum is taken in two levels, each against its own reference
// max, so only two barriers are needed: a thread (8-position group kg, split
// group sg: rows sg + u SG) sums its rows against their max m_sg; TPP threads
// per position then sum the split groups against their own max and combine by
// shuffles. With few heads, blockIdx.z = c of NC CTAs per head each apply rows
// [c d_h / NC, (c + 1) d_h / NC) of W_v (zbar is formed by each of them).
constexpr int kMergeThreads = 1024;

// Merge geometry of a launch, computed on the host so that the kernel's way to
// its first loads has no integer division by runtime values. Quotients by
// small divisors use q = (n ceil(2^k / d)) >> k, exact while n (d - 1) < 2^k.
struct MergeGeom {
    int DR;         // W_v rows per CTA (d_h / NC)
    int tpr_log2;   // threads per W_v row: 1 << tpr_log2
    int KG, SG;     // 8-coordinate groups of a partial row; split groups 1024 / KG
    int kg_mul;     // ceil(2^16 / KG): tid / KG for tid < 1024 (KG <= 32)
    int tpp_log2;   // level-two threads per position: 1 << tpp_log2
    int ZS;         // zpart row stride (floats)
    int g_mul;      // ceil(2^20 / (n_q / n_kv)): kv head of query head h < 64
    int dyn_q;      // device split: the streaming CTA's round (waves x 32 tokens)
};
constexpr int kMergeMaxS = 1024;

template <int VW, int R, int NVW>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(
    const _Float16 *__restrict__ part_z, const float *__restrict__ part_ml,
    const uint16_t *__restrict__ W_kv, const int32_t *__restrict__ seq_lens,
    uint16_t *__restrict__ out, int64_t seq_cap, int G, int GP, int n_q, int n_kv, int d_h,
    int chunk_arg, int S, int natural, int bits, int dyn_batch, int ncta, MergeGeom geo) {
    using VT = typename VecT<VW>::T;
    __shared__ __attribute__((aligned(16))) float zpart[9216];   // [split group][ZS]: ZS * SG <= 9216
    __shared__ float gm[256], gl[256];                            // per split group: SG <= 256
    __shared__ __attribute__((aligned(16))) float zbar[kMaxG];
    const int h = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x;
    const int DR = geo.DR, d0 = (int)blockIdx.z * DR;   // this CTA's rows of W_v
    uint16_t *o = out + ((size_t)b * n_q + h) * d_h;
    const size_t srow = 1;   // rows between splits (head-major partials)
    // ---- loads, all unconditional (clamped indices), so that a wait for one
    // counts exactly the loads issued after it: the batch's lengths (device-side
    // split of a batch), the first R partial rows of this thread and their
    // (m, l) over the workspace's S splits (entries at or past the sequence's
    // split count ns are discarded by selects once it is known), then the W_v
    // rows, which are used last and stay in flight meanwhile
    const int32_t tl_raw = seq_lens[min(tid & 63, (dyn_batch > 1 ? dyn_batch : 1) - 1)];
    const int KG = geo.KG, SG = geo.SG;
    // level 2 uses TPP threads per position; zpart rows are padded to ZS floats,
    // ZS = 64 / TPP (mod 32), so a wave's 64 reads fall on distinct bank pairs
    const int TPP = 1 << geo.tpp_log2;
    const int ZS = geo.ZS;
    const int sg = (int)(((uint32_t)tid * (uint32_t)geo.kg_mul) >> 16), kg = tid - sg * KG;
    const bool zthr = sg < SG;
    const _Float16 *zp = part_z + ((size_t)b * n_q + h) * S * GP + kg * 8;
    const float2 *ml = reinterpret_cast<const float2 *>(part_ml) + ((size_t)b * n_q + h) * S;
    half8 v[R];
    float2 mr[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int ic = min(sg + u * SG, S - 1);
        v[u] = *reinterpret_cast<const half8 *>(zp + (size_t)ic * srow * GP);
        mr[u] = ml[(size_t)ic * srow];
    }
    const int g = (int)(((uint32_t)h * (uint32_t)geo.g_mul) >> 20);
    const uint16_t *Wv = W_kv + ((size_t)n_kv * d_h + (size_t)g * d_h) * G;
    const int TPR = 1 << geo.tpr_log2;
    const int NV = G / VW;
    const int d = d0 + (tid >> geo.tpr_log2), part = tid & (TPR - 1);
    const bool drow = (tid >> geo.tpr_log2) < DR;
    const VT *wrow = reinterpret_cast<const VT *>(Wv + (size_t)(drow ? d : 0) * G);
    VT wv[NVW];
#pragma unroll
    for (int i = 0; i < NVW; ++i) wv[i] = wrow[min(part + TPR * i, NV - 1)];
    // the chunk of the split kernel: the plan's, or the device-side split's
    const int32_t T_raw = seq_lens[b];
    int chunk = chunk_arg;
    if (dyn_batch > 0) {
        const int64_t tb = T_raw < 0 ? 0 : (T_raw > seq_cap ? seq_cap : (int64_t)T_raw);
        const int64_t tl = (tid & 63) >= dyn_batch || tl_raw < 0 ? 0 : (tl_raw > seq_cap ? seq_cap : (int64_t)tl_raw);
        chunk = stream_dyn_chunk(dyn_batch == 1 ? tb : wave_sum64(tl), ncta, dyn_batch, chunk_arg, geo.dyn_q);
    }
    // T < 2^31 and chunk < 2^30: the split count in 32-bit arithmetic
    const uint32_t T = T_raw < 0 ? 0u : (T_raw > seq_cap ? (uint32_t)seq_cap : (uint32_t)T_raw);
    const int ns = (int)((T + (uint32_t)chunk - 1u) / (uint32_t)chunk);
    if (ns == 0) {   // empty sequence (uniform): the output is zero
        for (int dd = tid; dd < DR; dd += kMergeThreads) o[d0 + dd] = 0;
        return;
    }

    // ---- level 1: this thread's rows against their own max
    if (zthr) {
        float m = -INFINITY;
#pragma unroll
        for (int u = 0; u < R; ++u)
            if (sg + u * SG < ns) m = fmaxf(m, mr[u].x);
        float a[8] = {0, 0, 0, 0, 0, 0, 0, 0}, l = 0.0f;
#pragma unroll
        for (int u = 0; u < R; ++u) {
            // rows of splits past the sequence's end hold stale workspace
            // contents (possibly not finite): selected out, not multiplied by 0
            const bool ok = sg + u * SG < ns;
            const float c = ok ? mr[u].y * __builtin_amdgcn_exp2f(mr[u].x - m) : 0.0f;
            l += c;
#pragma unroll
            for (int j = 0; j < 8; ++j) a[j] += ok ? c * (float)v[u][j] : 0.0f;
        }
        for (int i0 = sg + R * SG; i0 < ns; i0 += R * SG) {   // more splits than one batch covers
#pragma unroll
            for (int u = 0; u < R; ++u) {
                const int i = i0 + u * SG, ic = i < ns ? i : ns - 1;
                v[u] = *reinterpret_cast<const half8 *>(zp + (size_t)ic * srow * GP);
                mr[u] = ml[(size_t)ic * srow];
            }
            float mb = m;
#pragma unroll
            for (int u = 0; u < R; ++u)
                if (i0 + u * SG < ns) mb = fmaxf(mb, mr[u].x);
            const float alpha = __builtin_amdgcn_exp2f(m - mb);   // m is finite here (row sg < ns)
            l *= alpha;
#pragma unroll
            for (int j = 0; j < 8; ++j) a[j] *= alpha;
            m = mb;
#pragma unroll
            for (int u = 0; u < R; ++u) {
                const float c = i0 + u * SG < ns ? mr[u].y * __builtin_amdgcn_exp2f(mr[u].x - m) : 0.0f;
                l += c;
#pragma unroll
                for (int j = 0; j < 8; ++j) a[j] += c * (float)v[u][j];
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) zpart[sg * ZS + kg * 8 + j] = a[j];
        if (kg == 0) {
            gm[sg] = m;   // -inf: no rows of the sequence in this group (l = 0, a = 0)
            gl[sg] = l;
        }
    }
    __syncthreads();
    // ---- level 2: TPP threads per position (TPP GP <= 1024), split groups
    // r + TPP k, k < SG / TPP <= kL2 (all LDS reads issued before use)
    {
        constexpr int kL2 = 16;   // SG / TPP <= 13 for every GP
        const int p = tid >> geo.tpp_log2, r = tid & (TPP - 1);
        const int pc = p < GP ? p : 0;
        float gv[kL2], lv[kL2], zv[kL2];
#pragma unroll
        for (int k = 0; k < kL2; ++k) {
            const int uc = r + TPP * k < SG ? r + TPP * k : 0;
            gv[k] = gm[uc];
            lv[k] = gl[uc];
            zv[k] = zpart[uc * ZS + pc];
        }
#pragma unroll
        for (int k = 0; k < kL2; ++k)
            if (r + TPP * k >= SG) gv[k] = -INFINITY;
        float m = gv[0];
#pragma unroll
        for (int k = 1; k < kL2; ++k) m = fmaxf(m, gv[k]);
        float z = 0.0f, l = 0.0f;
        if (m != -INFINITY) {
#pragma unroll
            for (int k = 0; k < kL2; ++k) {
                const float c = __builtin_amdgcn_exp2f(gv[k] - m);   // 0 for empty groups
                z += c * zv[k];
                l += c * lv[k];
            }
        }
        float M = m;
        for (int off = 1; off < TPP; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));   // finite: split 0 is in group 0
        const float e = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
        z *= e;
        l *= e;
        for (int off = 1; off < TPP; off <<= 1) {
            z += __shfl_xor(z, off);
            l += __shfl_xor(l, off);
        }
        if (p < GP && r == 0) zbar[natural ? p : pos_to_coord(p, GP, bits)] = z / l;
    }
    __syncthreads();

    // ---- out = W_v,g zbar
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < NVW; ++i) {
        const int vi = part + TPR * i;
        float wf[VW];
        bf16_vec_to_f32<VW>(wv[i], wf);
        if (vi < NV) {
#pragma unroll
            for (int c = 0; c < VW; ++c) acc += wf[c] * zbar[vi * VW + c];
        }
    }
    for (int vi = part + TPR * NVW; vi < NV; vi += TPR) {
        float wf[VW];
        bf16_vec_to_f32<VW>(wrow[vi], wf);
#pragma unroll
        for (int c = 0; c < VW; ++c) acc += wf[c] * zbar[vi * VW + c];
    }
    for (int off = TPR >> 1; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (part == 0 && drow) o[d] = f32_to_bf16(acc);
}

// Max over the 64 lanes of a wave, in every lane (the pattern of wave_sum_dpp).
__device__ inline float wave_max_f32(float a) {
    a = fmaxf(a, dpp_f32<0xB1>(a));
    a = fmaxf(a, dpp_f32<0x4E>(a));
    a = fmaxf(a, dpp_f32<0x141>(a));
    a = fmaxf(a, dpp_f32<0x140>(a));
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
    a = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
    return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Sum over the SEG lanes of each SEG-lane segment of a wave (SEG = 64: the
// whole wave; 32: each half), in every lane of the segment.
template <int SEG>
__device__ inline float seg_sum(float a) {
    if constexpr (SEG == 64) {
        return wave_sum_dpp(a);
    } else {
        static_assert(SEG == 32, "segments of 32 or 64 lanes");
        a += dpp_f32<0xB1>(a);
        a += dpp_f32<0x4E>(a);
        a += dpp_f32<0x141>(a);
        a += dpp_f32<0x140>(a);
        const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
        return __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    }
}

// Merge with a single barrier. Each SEG-lane segment of a wave merges one
// 8-coordinate group of the head's partial rows (segment k of wave w: group
// w 64/SEG + k), its lane l holding splits l, l + SEG, ... (RS of them). Every
// wave reads the (m, l) pairs of those splits and forms the common max M by a
// wave-wide reduction in registers, the weights c_s = l_s 2^(m_s - M) and
// L = sum_s c_s by segment reductions; then zbar = sum_s c_s zbar_s / L per
// coordinate, reduced the same way, goes to LDS. After the one barrier,
// out = W_v,g zbar as in the two-level kernel (same W_v rows per CTA).
template <int VW, int RS, int SEG, int NVW>
__global__ __launch_bounds__(kMergeThreads) void decode_merge1_kernel(
    const _Float16 *__restrict__ part_z, const float *__restrict__ part_ml,
    const uint16_t *__restrict__ W_kv, const int32_t *__restrict__ seq_lens,
    uint16_t *__restrict__ out, int64_t seq_cap, int G, int GP, int n_q, int n_kv, int d_h,
    int chunk_arg, int S, int natural, int bits, int dyn_batch, int ncta, MergeGeom geo) {
    using VT = typename VecT<VW>::T;
    constexpr int NSEG = 64 / SEG;
    __shared__ __attribute__((aligned(16))) float zbar[kMaxG];
    const int h = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int sl = lane % SEG;
    const int kg = wave * NSEG + lane / SEG;   // this lane's coordinate group
    const int DR = geo.DR, d0 = (int)blockIdx.z * DR;
    uint16_t *o = out + ((size_t)b * n_q + h) * d_h;
    // ---- loads, all unconditional (clamped indices), so that a wait for one
    // counts exactly the loads issued after it: the batch's lengths (device-side
    // split of a batch), this lane's (m, l) pairs and partial rows (bounded by
    // the workspace's S rows, not by the sequence length, which is not known
    // yet), then the W_v rows, which are used last and stay in flight meanwhile
    const int32_t tl_raw = seq_lens[min(lane, (dyn_batch > 1 ? dyn_batch : 1) - 1)];
    const float2 *ml = reinterpret_cast<const float2 *>(part_ml) + ((size_t)b * n_q + h) * S;
    const _Float16 *zp = part_z + ((size_t)b * n_q + h) * S * GP;
    const int KG = GP / 8;
    const int kgc = kg < KG ? kg : 0;
    float2 mr[RS];
    half8 v[RS];
#pragma unroll
    for (int i = 0; i < RS; ++i) {
        const int sc = min(sl + SEG * i, S - 1);
        mr[i] = ml[sc];
        v[i] = *reinterpret_cast<const half8 *>(zp + (size_t)sc * GP + kgc * 8);
    }
    const int g = (int)(((uint32_t)h * (uint32_t)geo.g_mul) >> 20);
    const uint16_t *Wv = W_kv + ((size_t)n_kv * d_h + (size_t)g * d_h) * G;
    const int TPR = 1 << geo.tpr_log2;
    const int NV = G / VW;
    const int d = d0 + (tid >> geo.tpr_log2), part = tid & (TPR - 1);
    const bool drow = (tid >> geo.tpr_log2) < DR;
    const VT *wrow = reinterpret_cast<const VT *>(Wv + (size_t)(drow ? d : 0) * G);
    VT wv[NVW];
#pragma unroll
    for (int i = 0; i < NVW; ++i) wv[i] = wrow[min(part + TPR * i, NV - 1)];
    // ---- the sequence's split count
    const int32_t T_raw = seq_lens[b];
    int chunk = chunk_arg;
    if (dyn_batch > 0) {
        const int64_t tb = T_raw < 0 ? 0 : (T_raw > seq_cap ? seq_cap : (int64_t)T_raw);
        const int64_t tl = lane >= dyn_batch || tl_raw < 0 ? 0 : (tl_raw > seq_cap ? seq_cap : (int64_t)tl_raw);
        chunk = stream_dyn_chunk(dyn_batch == 1 ? tb : wave_sum64(tl), ncta, dyn_batch, chunk_arg, geo.dyn_q);
    }
    const uint32_t T = T_raw < 0 ? 0u : (T_raw > seq_cap ? (uint32_t)seq_cap : (uint32_t)T_raw);
    const int ns = (int)((T + (uint32_t)chunk - 1u) / (uint32_t)chunk);
    if (ns == 0) {   // empty sequence (uniform): the output is zero
        for (int dd = tid; dd < DR; dd += kMergeThreads) o[d0 + dd] = 0;
        return;
    }
    // ---- common max, weights and normaliser (the same bits in every wave)
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < RS; ++i) m = fmaxf(m, sl + SEG * i < ns ? mr[i].x : -INFINITY);
    m = wave_max_f32(m);   // finite: split 0 is in every sequence with ns > 0
    float c[RS], l = 0.0f;
#pragma unroll
    for (int i = 0; i < RS; ++i) {
        // rows past the sequence's splits hold stale workspace contents (possibly
        // not finite): selected out, not multiplied by 0
        c[i] = sl + SEG * i < ns ? mr[i].y * __builtin_amdgcn_exp2f(mr[i].x - m) : 0.0f;
        l += c[i];
    }
    l = seg_sum<SEG>(l);
    const float inv = 1.0f / l;
    // ---- this segment's coordinate group
    float a[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < RS; ++i) {
        if constexpr (SEG == 32) {
            // widths above 128: a row past the sequence's splits (weight 0) is
            // cleared before use, once per row rather than per product, so that
            // each term is one mixed-precision FMA of the fp16 value (measured
            // faster there, slower with 64-lane segments)
            const half8 vi = sl + SEG * i < ns ? v[i] : half8{};
#pragma unroll
            for (int j = 0; j < 8; ++j) a[j] = fmaf(c[i], (float)vi[j], a[j]);
        } else {
            const bool ok = sl + SEG * i < ns;
#pragma unroll
            for (int j = 0; j < 8; ++j) a[j] += ok ? c[i] * (float)v[i][j] : 0.0f;
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = seg_sum<SEG>(a[j]);
    if (sl == 0 && kg < KG) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int pp = kg * 8 + j;
            zbar[natural ? pp : pos_to_coord(pp, GP, bits)] = a[j] * inv;
        }
    }
    __syncthreads();
    // ---- out = W_v,g zbar (vectors part + TPR i; past NVW of them, read here)
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < NVW; ++i) {
        const int vi = part + TPR * i;
        float wf[VW];
        bf16_vec_to_f32<VW>(wv[i], wf);
        if (vi < NV) {
#pragma unroll
            for (int cc = 0; cc < VW; ++cc) acc += wf[cc] * zbar[vi * VW + cc];
        }
    }
    for (int vi = part + TPR * NVW; vi < NV; vi += TPR) {
        float wf[VW];
        bf16_vec_to_f32<VW>(wrow[vi], wf);
#pragma unroll
        for (int cc = 0; cc < VW; ++cc) acc += wf[cc] * zbar[vi * VW + cc];
    }
    for (int off = TPR >> 1; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (part == 0 && drow) o[d] = f32_to_bf16(acc);
}

// Merge launch: the widest bf16 vector that divides G and the W_kv alignment,
// and the fewest partial rows per thread that cover S in one batch (at most 8).
static hipError_t launch_merge(const _Float16 *pz, const float *pml, const uint16_t *W_kv,
                               const int32_t *seq_lens, uint16_t *out, int64_t seq_cap, int G,
                               int GP, int n_q, int n_kv, int d_h, int batch, int chunk, int S,
                               int natural, int bits, int dyn_batch, int ncta, hipStream_t st) {
    if (S < 1 || S > kMergeMaxS || GP > kMaxG || d_h > kMaxDh) return hipErrorInvalidValue;
    const int vw = ((G & 7) == 0 && ((uintptr_t)W_kv & 15) == 0)  ? 8
                   : ((G & 3) == 0 && ((uintptr_t)W_kv & 7) == 0) ? 4
                   : ((G & 1) == 0 && ((uintptr_t)W_kv & 3) == 0) ? 2
                                                                   : 1;
    const int SG = kMergeThreads / (GP / 8);
    const int rows = (S + SG - 1) / SG;
    const int r = rows <= 2 ? 2 : rows <= 4 ? 4 : 8;   // more: the kernel loops
    // NC CTAs per head while the grid stays within 256 CTAs and each applies
    // at least 16 rows of W_v
    int nc = 1;
    while (nc < 4 && (int64_t)n_q * batch * nc * 2 <= 256 && d_h % (nc * 2) == 0 && d_h / (nc * 2) >= 16) nc *= 2;
    const dim3 mg(n_q, batch, nc);
    MergeGeom geo;
    geo.DR = d_h / nc;
    geo.tpr_log2 = 2;   // TPR = 4, doubled while two rows' threads fit
    while ((2 << geo.tpr_log2) * geo.DR <= kMergeThreads && (1 << geo.tpr_log2) < 64) ++geo.tpr_log2;
    geo.KG = GP / 8;
    geo.SG = SG;
    geo.kg_mul = ((1 << 16) + geo.KG - 1) / geo.KG;
    geo.tpp_log2 = GP <= 32 ? 5 : GP <= 64 ? 4 : GP <= 128 ? 3 : 2;
    geo.ZS = GP + (geo.tpp_log2 == 5 ? 4 : 64 >> geo.tpp_log2);
    const int grp = n_q / n_kv;
    geo.g_mul = ((1 << 20) + grp - 1) / grp;
    geo.dyn_q = 32 * stream_waves(GP);
    // the one-barrier merge: one coordinate group per 64-lane wave (widths up to
    // 128) or per 32-lane half (up to 256), at most 4 splits per lane; more
    // splits (long single sequences) take the two-level kernel
    const int seg = GP <= 128 ? 64 : 32;
    const int rs = (S + seg - 1) / seg;
    if (rs <= 4) {
        const int rs2 = rs <= 1 ? 1 : rs <= 2 ? 2 : 4;
        const int nv = G / vw, tpr = 1 << geo.tpr_log2;
        const int nvw_need = (nv + tpr - 1) / tpr;
        const int nvw = nvw_need <= 1 ? 1 : nvw_need <= 2 ? 2 : 4;   // more: read in the dot loop
#define FSQ_MERGE1_CASE(VWX, RSX, SEGX, NVWX)                                                               \
    if (vw == VWX && rs2 == RSX && seg == SEGX && nvw == NVWX) {                                           \
        decode_merge1_kernel<VWX, RSX, SEGX, NVWX><<<mg, kMergeThreads, 0, st>>>(                          \
            pz, pml, W_kv, seq_lens, out, seq_cap, G, GP, n_q, n_kv, d_h, chunk, S, natural, bits,         \
            dyn_batch, ncta, geo);                                                                         \
        return hipGetLastError();                                                                          \
    }
#define FSQ_MERGE1_RS(VWX, NVWX)                                                                           \
    FSQ_MERGE1_CASE(VWX, 1, 64, NVWX) FSQ_MERGE1_CASE(VWX, 2, 64, NVWX) FSQ_MERGE1_CASE(VWX, 4, 64, NVWX)  \
    FSQ_MERGE1_CASE(VWX, 1, 32, NVWX) FSQ_MERGE1_CASE(VWX, 2, 32, NVWX) FSQ_MERGE1_CASE(VWX, 4, 32, NVWX)
#define FSQ_MERGE1_VW(VWX) FSQ_MERGE1_RS(VWX, 1) FSQ_MERGE1_RS(VWX, 2) FSQ_MERGE1_RS(VWX, 4)
        FSQ_MERGE1_VW(8)
        FSQ_MERGE1_VW(4)
        FSQ_MERGE1_VW(2)
        FSQ_MERGE1_VW(1)
#undef FSQ_MERGE1_VW
#undef FSQ_MERGE1_RS
#undef FSQ_MERGE1_CASE
    }
    const int nv2 = G / vw, tpr2 = 1 << geo.tpr_log2;
    const int nvw2_need = (nv2 + tpr2 - 1) / tpr2;
    const int nvw2 = nvw2_need <= 1 ? 1 : nvw2_need <= 2 ? 2 : 4;   // more: read in the dot loop
#define FSQ_MERGE_CASE(VWX, RX, NVWX)                                                                      \
    if (vw == VWX && r == RX && nvw2 == NVWX) {                                                           \
        decode_merge_kernel<VWX, RX, NVWX><<<mg, kMergeThreads, 0, st>>>(pz, pml, W_kv, seq_lens, out,    \
                                                                         seq_cap, G, GP, n_q, n_kv, d_h,  \
                                                                         chunk, S, natural, bits,         \
                                                                         dyn_batch, ncta, geo);           \
        return hipGetLastError();                                                                         \
    }
#define FSQ_MERGE_R(VWX, NVWX) FSQ_MERGE_CASE(VWX, 2, NVWX) FSQ_MERGE_CASE(VWX, 4, NVWX) FSQ_MERGE_CASE(VWX, 8, NVWX)
#define FSQ_MERGE_VW(VWX) FSQ_MERGE_R(VWX, 1) FSQ_MERGE_R(VWX, 2) FSQ_MERGE_R(VWX, 4)
    FSQ_MERGE_VW(8)
    FSQ_MERGE_VW(4)
    FSQ_MERGE_VW(2)
    FSQ_MERGE_VW(1)
#undef FSQ_MERGE_VW
#undef FSQ_MERGE_R
#undef FSQ_MERGE_CASE
    return hipErrorInvalidValue;
}

template <int GP, int NW, int BITS>
static hipError_t launch_split_nw(const DecodePlan &pl, const _Float16 *qt, const uint8_t *codes,
                                  const int32_t *seq_lens, _Float16 *pz, float *pml, int64_t seq_cap,
                                  int G, int n_q, int batch, hipStream_t st, hipEvent_t ev0,
                                  hipEvent_t ev1) {
    const size_t qlo = BITS == 8 ? (size_t)batch * pl.nqp * pl.GP : 0;
    dim3 grid(pl.S, batch, pl.nqp / 32);
    dim3 block(NW * 64);
    // whole-dword vector loads when every token row starts on a 16-byte boundary
    constexpr bool kCanAl = (GP * BITS / 64) % 2 == 0;
    const bool al = kCanAl && G == GP && (bytes_per_token_b(G, BITS) % 16) == 0 &&
                    ((uintptr_t)codes & 15) == 0;
    auto k = al ? decode_split_kernel<GP, NW, kCanAl, BITS> : decode_split_kernel<GP, NW, false, BITS>;
    if (ev0 && ev1)   // timed launch: events bracket this kernel's execution
        hipExtLaunchKernelGGL(k, grid, block, 0, st, ev0, ev1, 0, qt, codes, seq_lens, pz, pml,
                              seq_cap, G, n_q, pl.nqp, pl.chunk, pl.S, qlo);
    else
        k<<<grid, block, 0, st>>>(qt, codes, seq_lens, pz, pml, seq_cap, G, n_q, pl.nqp, pl.chunk,
                                  pl.S, qlo);
    return hipGetLastError();
}

template <int GP, int D>
static hipError_t launch_stream_d(const DecodePlan &pl, const _Float16 *qt, const uint8_t *codes,
                                  const int32_t *seq_lens, _Float16 *pz, float *pml, int64_t seq_cap,
                                  int G, int n_q, int batch, hipStream_t st, hipEvent_t ev0,
                                  hipEvent_t ev1) {
    constexpr int NW = GP < 128 ? 8 : 4;   // stream_waves(GP)
    // device-side split: ncta + batch CTAs cover every work item (the per-sequence
    // rounding up adds at most one item per sequence)
    dim3 grid(pl.dyn ? pl.ncta + batch : pl.S, pl.dyn ? 1 : batch, pl.nqp / 32);
    dim3 block(NW * 64);
    const int dyn_batch = pl.dyn ? batch : 0;
    // 16-byte row reads when every token row starts on a 16-byte boundary and a
    // lane half is whole 16-byte chunks
    constexpr bool kCanAl = GP % 64 == 0;
    const bool al = kCanAl && G == GP && ((uintptr_t)codes & 15) == 0;
    auto k = al ? decode_stream_kernel<GP, NW, D, kCanAl, false> : decode_stream_kernel<GP, NW, D, false, false>;
    const ReconArgs ra{};
    if (ev0 && ev1)
        hipExtLaunchKernelGGL(k, grid, block, 0, st, ev0, ev1, 0, qt, codes, seq_lens, pz, pml,
                              seq_cap, G, n_q, pl.nqp, pl.chunk, pl.S, dyn_batch, pl.ncta, ra);
    else
        k<<<grid, block, 0, st>>>(qt, codes, seq_lens, pz, pml, seq_cap, G, n_q, pl.nqp, pl.chunk,
                                  pl.S, dyn_batch, pl.ncta, ra);
    return hipGetLastError();
}

// Key-reconstruction variant: grid (chunks, sequences, kv heads), chunk and
// split count from recon_split (at most the plan's split count, so the same
// workspace holds the partials).
template <int GP, int RC>
static hipError_t launch_recon(int chunk, int S, const uint8_t *codes, const int32_t *seq_lens,
                               _Float16 *pz, float *pml, int64_t seq_cap, int G, int n_q, int batch,
                               const ReconArgs &ra, hipStream_t st) {
    constexpr int NW = kStreamWaves;
    constexpr int D = GP >= 128 ? 3 : 4;
    dim3 grid(S, batch, ra.n_kv);
    dim3 block(NW * 64);
    constexpr bool kCanAl = GP % 64 == 0;
    const bool al = kCanAl && G == GP && ((uintptr_t)codes & 15) == 0;
    auto k = al ? decode_stream_kernel<GP, NW, D, kCanAl, RC> : decode_stream_kernel<GP, NW, D, false, RC>;
    k<<<grid, block, 0, st>>>(nullptr, codes, seq_lens, pz, pml, seq_cap, G, n_q, 0, chunk, S, 0, 0, ra);
    return hipGetLastError();
}

template <int GP>
static hipError_t launch_split(const DecodePlan &pl, const _Float16 *qt, const uint8_t *codes,
                               const int32_t *seq_lens, _Float16 *pz, float *pml, int64_t seq_cap,
                               int G, int n_q, int batch, hipStream_t st, hipEvent_t ev0,
                               hipEvent_t ev1, int bits) {
    // split kernel: 8-wave CTAs from GP 64 up, 4-wave CTAs below GP 128 (the plan's choice)
    const bool nw8 = pl.waves == 8 && GP >= 64, nw4 = pl.waves == 4 && GP < 128;
    if (bits != 4) {   // 2- and 8-bit codes: the split kernel only
        if (pl.stream || !(nw8 || nw4)) return hipErrorInvalidValue;
        if (bits == 2)
            return nw8 ? launch_split_nw<GP, (GP >= 64 ? 8 : 4), 2>(pl, qt, codes, seq_lens, pz, pml, seq_cap, G, n_q, batch, st, ev0, ev1)
                       : launch_split_nw<GP, (GP < 128 ? 4 : 8), 2>(pl, qt, codes, seq_lens, pz, pml, seq_cap, G, n_q,
                                                                     batch, st, ev0, ev1);
        return nw8 ? launch_split_nw<GP, (GP >= 64 ? 8 : 4), 8>(pl, qt, codes, seq_lens, pz, pml, seq_cap, G, n_q, batch, st, ev0, ev1)
                   : launch_split_nw<GP, (GP < 128 ? 4 : 8), 8>(pl, qt, codes, seq_lens, pz, pml, seq_cap, G, n_q,
                                                                 batch, st, ev0, ev1);
    }
    if (pl.stream) {
        if (pl.waves != stream_waves(GP)) return hipErrorInvalidValue;
        constexpr int D = GP >= 128 ? 3 : 4;   // stream_depth(GP)
        if (stream_depth(GP) != D) return hipErrorInvalidValue;
        return launch_stream_d<GP, D>(pl, qt, codes, seq_lens, pz, pml, seq_cap, G, n_q, batch, st,
                                      ev0, ev1);
    }
    if (!(nw8 || nw4)) return hipErrorInvalidValue;
    return nw8 ? launch_split_nw<GP, (GP >= 64 ? 8 : 4), 4>(pl, qt, codes, seq_lens, pz, pml, seq_cap, G, n_q, batch, st, ev0, ev1)
               : launch_split_nw<GP, (GP < 128 ? 4 : 8), 4>(pl, qt, codes, seq_lens, pz, pml, seq_cap, G, n_q,
                                                             batch, st, ev0, ev1);
}

hipError_t launch_decode(const DecodePlan &pl, const uint16_t *q, const uint8_t *codes,
                         const uint16_t *W_kv, const int32_t *seq_lens, uint16_t *out, int batch,
                         int n_q, int n_kv, int d_h, int G, int64_t seq_cap, void *workspace,
                         hipStream_t st, hipEvent_t ev0, hipEvent_t ev1, const uint16_t *x_new,
                         const uint16_t *E, int C, int levels) {
    const int bits = bits_of_levels(levels);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    _Float16 *qt = reinterpret_cast<_Float16 *>(ws + pl.off_qt);
    _Float16 *pz = reinterpret_cast<_Float16 *>(ws + pl.off_acc);
    float *pml = reinterpret_cast<float *>(ws + pl.off_ml);
    const float scale = 1.4426950408889634f / sqrtf((float)d_h);
    // 4-bit codes are read with odd coordinates 16x (unpack_codes_x16) by both
    // split-K kernels, whose pooled sums then come out in natural coordinate order
    const float odd = bits == 4 ? 0.0625f : 1.0f;
    const int natural = bits == 4 ? 1 : 0;
    // 8-bit codes: the second term of q~ follows the first (the workspace's
    // q~ region holds two)
    const size_t qlo = bits == 8 ? (size_t)batch * pl.nqp * pl.GP : 0;
    hipError_t e;
    // widest bf16 vector that divides G and the W_kv alignment
    const int vw = ((G & 7) == 0 && ((uintptr_t)W_kv & 15) == 0)  ? 8
                   : ((G & 3) == 0 && ((uintptr_t)W_kv & 7) == 0) ? 4
                   : ((G & 1) == 0 && ((uintptr_t)W_kv & 3) == 0) ? 2
                                                                   : 1;
    if (pl.S > 0 && x_new) {
        // decode step: append + absorb in one launch
        const StepAppend ap{x_new, E, const_cast<uint8_t *>(codes), C, host_fsq_quant(levels)};
        const int nt = gemv_tokens_per_cta(batch);
        const int n_app = bytes_per_token_b(G, bits) * ((batch + nt - 1) / nt);
        const int n_abs = n_kv * ((pl.GP + kAbsorbCols - 1) / kAbsorbCols) * batch;
        const dim3 grid((unsigned)(n_app + n_abs));
#define FSQ_PREP_CALL(NT, CPB) \
    launch_step_prep_nt<NT, CPB>(vw, grid, st, ap, seq_lens, seq_cap, batch, n_app, q, W_kv, qt, G, pl.GP, n_q, pl.nqp, n_kv, d_h, scale, odd, qlo)
#define FSQ_PREP_NT(CPB)                                  \
        switch (nt) {                                     \
            case 1: FSQ_PREP_CALL(1, CPB); break;         \
            case 2: FSQ_PREP_CALL(2, CPB); break;         \
            case 4: FSQ_PREP_CALL(4, CPB); break;         \
            default: FSQ_PREP_CALL(kGemvTokens, CPB);     \
        }
        if (bits == 2) {
            FSQ_PREP_NT(4)
        } else if (bits == 8) {
            FSQ_PREP_NT(1)
        } else {
            FSQ_PREP_NT(2)
        }
#undef FSQ_PREP_NT
#undef FSQ_PREP_CALL
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if (pl.S > 0) {
        const int n_abs = n_kv * ((pl.GP + kAbsorbCols - 1) / kAbsorbCols) * batch;
        const dim3 ag((unsigned)n_abs);
        switch (vw) {
            case 8: absorb_kernel<8><<<ag, 256, 0, st>>>(q, W_kv, qt, G, pl.GP, n_q, pl.nqp, n_kv, d_h, scale, odd, bits, qlo); break;
            case 4: absorb_kernel<4><<<ag, 256, 0, st>>>(q, W_kv, qt, G, pl.GP, n_q, pl.nqp, n_kv, d_h, scale, odd, bits, qlo); break;
            case 2: absorb_kernel<2><<<ag, 256, 0, st>>>(q, W_kv, qt, G, pl.GP, n_q, pl.nqp, n_kv, d_h, scale, odd, bits, qlo); break;
            default: absorb_kernel<1><<<ag, 256, 0, st>>>(q, W_kv, qt, G, pl.GP, n_q, pl.nqp, n_kv, d_h, scale, odd, bits, qlo);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (pl.S > 0) {
        switch (pl.GP) {
#define FSQ_SPLIT_CASE(X)                                                                             \
    case X:                                                                                           \
        e = launch_split<X>(pl, qt, codes, seq_lens, pz, pml, seq_cap, G, n_q, batch, st, ev0, ev1, bits); \
        break;
            FSQ_SPLIT_CASE(32)
            FSQ_SPLIT_CASE(64)
            FSQ_SPLIT_CASE(96)
            FSQ_SPLIT_CASE(128)
            FSQ_SPLIT_CASE(160)
            FSQ_SPLIT_CASE(192)
            FSQ_SPLIT_CASE(224)
            FSQ_SPLIT_CASE(256)
#undef FSQ_SPLIT_CASE
            default:
                return hipErrorInvalidValue;
        }
        if (e != hipSuccess) return e;
    }
    return launch_merge(pz, pml, W_kv, seq_lens, out, seq_cap, G, pl.GP, n_q, n_kv, d_h, batch, pl.chunk,
                        pl.S > 0 ? pl.S : 1, natural, bits, pl.dyn ? batch : 0, pl.ncta, st);
}

// The key-reconstruction comparison: no absorption launch; the split kernel
// rebuilds keys per tile, then the same merge applies W_v once.
hipError_t launch_decode_recon(const DecodePlan &pl, const uint16_t *q, const uint8_t *codes,
                               const uint16_t *W_kv, const int32_t *seq_lens, uint16_t *out,
                               int batch, int n_q, int n_kv, int d_h, int G, int64_t seq_cap,
                               void *workspace, hipStream_t st, const uint16_t *gamma, float eps,
                               float theta) {
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    _Float16 *pz = reinterpret_cast<_Float16 *>(ws + pl.off_acc);
    float *pml = reinterpret_cast<float *>(ws + pl.off_ml);
    // about 512 CTAs over (chunks, sequences, kv heads); chunks no shorter than
    // the plan's, so the split count (and the partials) fit its workspace
    const int64_t quantum = 32 * kStreamWaves;
    int64_t per = ((int64_t)batch * n_kv * seq_cap + 511) / 512;
    per = (per + quantum - 1) / quantum * quantum;
    int64_t chunk = per > pl.chunk ? per : pl.chunk;
    const int S = seq_cap > 0 ? (int)((seq_cap + chunk - 1) / chunk) : 0;
    ReconArgs ra{};
    ra.q = q;
    ra.W_kv = W_kv;
    ra.n_kv = n_kv;
    ra.d_h = d_h;
    ra.scale = 1.4426950408889634f / sqrtf((float)d_h);
    ra.gamma = gamma;
    ra.eps = eps;
    if (gamma) {
        // rotation rate of channel pair i in revolutions per position, as a
        // 64-bit fraction: t * rope_f[i] mod 2^64 is the angle of position t
        // without rounding growth in t
        for (int i = 0; i < d_h / 2; ++i) {
            const long double f = powl((long double)theta, -2.0L * i / d_h) / (2.0L * 3.141592653589793238462643383279L);
            ra.rope_f[i] = (uint64_t)llroundl(ldexpl(f, 64));
        }
    }
    hipError_t e = hipSuccess;
    if (S > 0) {
        switch (pl.GP) {
#define FSQ_RECON_CASE(X)                                                                                   \
    case X:                                                                                                 \
        e = gamma ? launch_recon<X, 2>((int)chunk, S, codes, seq_lens, pz, pml, seq_cap, G, n_q, batch, ra, st) \
                  : launch_recon<X, 1>((int)chunk, S, codes, seq_lens, pz, pml, seq_cap, G, n_q, batch, ra, st); \
        break;
            FSQ_RECON_CASE(32)
            FSQ_RECON_CASE(64)
            FSQ_RECON_CASE(96)
            FSQ_RECON_CASE(128)
            FSQ_RECON_CASE(160)
            FSQ_RECON_CASE(192)
            FSQ_RECON_CASE(224)
            FSQ_RECON_CASE(256)
#undef FSQ_RECON_CASE
            default:
                return hipErrorInvalidValue;
        }
        if (e != hipSuccess) return e;
    }
    const int chunk_i = S > 0 ? (int)chunk : pl.chunk;
    return launch_merge(pz, pml, W_kv, seq_lens, out, seq_cap, G, pl.GP, n_q, n_kv, d_h, batch, chunk_i,
                        S > 0 ? S : 1, 1, 4, 0, 0, st);
}

}  // namespace fsq
