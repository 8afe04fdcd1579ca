// Split-K plan and workspace layout of the decode call. Pure host arithmetic:
// the plan depends only on the call's sizes, so the workspace size can be
// queried without a device.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace fsq {

constexpr int kMaxG = 256;     // largest latent width the decode kernels are built for
constexpr int kMaxDh = 256;    // largest head dimension
constexpr int kMaxNq = 64;     // largest number of query heads
// Split-K CTAs have 8 waves when the padded latent width is >= 128 (about 256
// CTAs, one per CU, are aimed for) and 4 waves below (about 512 CTAs, two or
// more per CU), except for widths 64 and 96 once the work (batch x cache
// capacity) reaches 2 x 256 x 256 tokens: there 8-wave CTAs, each taking two or
// more rounds, halve the partials to write and merge (measured on the MI355X:
// a G=84 layer over 131k tokens 19.1 vs 21.3 us; one-round chunks and width 32
// are faster with 4 waves). A CTA covers whole rounds of waves x 32 tokens.
inline int split_waves(int GP, int64_t work) {
    return (GP >= 128 || (GP >= 64 && work >= (int64_t)2 * 256 * 256)) ? 8 : 4;
}

// Streaming split (long chunks). GP >= 128: 4-wave CTAs, each wave keeping
// stream_depth - 1 tiles of codes in flight through an LDS ring; registers and
// LDS allow two CTAs per CU, so 512 CTAs (one resident set) are aimed for.
// Below GP 128: 8-wave CTAs whose waves keep four tiles in registers, one CTA
// per CU (two waves per SIMD), 256 CTAs: half the partial rows of 4-wave CTAs
// at the same occupancy. It is chosen when every wave gets at least
// kStreamMinTiles tiles of 32 tokens. (The key-reconstruction variants use
// 4-wave CTAs at every width: kStreamWaves.)
constexpr int kStreamWaves = 4;
inline int stream_waves(int GP) { return GP < 128 ? 8 : 4; }   // 32 x this is a power of two (the device split rounds by masks)
constexpr int kStreamMinTiles = 4;
// Streaming calls of up to kDynMaxBatch sequences split on the device from the
// actual lengths (one lane per sequence there); the chunk is then at least
// kStreamMinTiles rounds and at least seq_cap / kDynMaxSplits, which bounds a
// sequence's split count for the workspace.
constexpr int kDynMaxBatch = 64;
constexpr int kDynMaxSplits = 1024;
inline int stream_depth(int GP) { return GP >= 128 ? 3 : 4; }
inline int stream_target(int GP) { return GP >= 128 ? 512 : 256; }
// Work items of the device-side split: one resident set of CTAs (512 of 4
// waves at GP >= 128, 256 of 8 waves below; measured on the MI355X with 4-wave
// CTAs: a 1M-token G=84 layer 38.8 us with 512 items vs 41.5 with 768).
inline int dyn_ctas(int GP) { return GP >= 128 ? 512 : 256; }
static_assert(kDynMaxBatch * 4 <= 256, "the device split spreads over ncta - batch + 1 CTAs");

struct DecodePlan {
    int GP = 0;       // G padded to a multiple of 32 (MFMA blocks)
    int nqp = 0;      // n_q padded to a multiple of 32 (head groups)
    int chunk = 0;    // tokens per split
    int S = 0;        // splits per sequence (0 when seq_cap == 0)
    int waves = 0;    // waves per split-K CTA
    int stream = 0;   // 1: decode_stream_kernel (partials in natural coordinate order)
    int dyn = 0;      // 1: streaming with the device-side split; chunk and S are then
                      // the smallest chunk and the largest split count per sequence
    int ncta = 0;     // dyn: CTAs the tokens of all sequences are spread over
    size_t off_qt = 0, off_acc = 0, off_ml = 0, total = 0;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// allow_stream = false (codes of 2 or 8 bits) keeps the split kernel; its split
// count never exceeds the default plan's, so the default workspace suffices.
inline DecodePlan make_decode_plan(int batch, int n_q, int G, int64_t seq_cap, bool allow_stream = true) {
    DecodePlan p;
    p.GP = (G + 31) / 32 * 32;
    p.nqp = (n_q + 31) / 32 * 32;
    const int64_t work = int64_t(batch) * seq_cap;
    const int squant = 32 * stream_waves(p.GP);
    const int starget = stream_target(p.GP);
    int64_t sper = (work + starget - 1) / starget;
    sper = (sper + squant - 1) / squant * squant;
    // (and only for caches of 64 rows or more: below GP 128 its unchecked
    // register loads may read into the row after a tile)
    p.stream = allow_stream && sper >= (int64_t)kStreamMinTiles * squant && seq_cap >= 64 ? 1 : 0;
    p.waves = p.stream ? stream_waves(p.GP) : split_waves(p.GP, work);
    const int quantum = 32 * p.waves;
    const int target = p.stream ? starget : (p.waves == 8 ? 256 : 512);
    int64_t per = (work + target - 1) / target;
    if (per < quantum) per = quantum;
    per = (per + quantum - 1) / quantum * quantum;
    if (p.stream && batch <= kDynMaxBatch) {
        p.dyn = 1;
        p.ncta = dyn_ctas(p.GP);
        int64_t cmin = (seq_cap + kDynMaxSplits - 1) / kDynMaxSplits;
        if (cmin < (int64_t)kStreamMinTiles * squant) cmin = (int64_t)kStreamMinTiles * squant;
        per = (cmin + squant - 1) / squant * squant;
    }
    if (per > (int64_t)1 << 30) per = (int64_t)1 << 30;
    p.chunk = (int)per;
    p.S = (int)((seq_cap + p.chunk - 1) / p.chunk);
    // device split: the chunk is at least ceil(sum of lengths / ncta), so no
    // sequence has more than ncta work items
    if (p.dyn && p.S > p.ncta) p.S = p.ncta;
    const int S1 = p.S > 0 ? p.S : 1;
    p.off_qt = 0;
    // q~ in fp16, two terms (8-bit codes use the second: the rounding residual)
    p.off_acc = align256((size_t)batch * p.nqp * p.GP * 2 * 2);
    p.off_ml = p.off_acc + align256((size_t)batch * S1 * n_q * p.GP * 2);   // fp16 zbar
    p.total = p.off_ml + align256((size_t)batch * S1 * n_q * 2 * 4);
    return p;
}

}  // namespace fsq
