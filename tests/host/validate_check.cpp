// Host-only check of the C ABI's argument validation (csrc/validate.h) and of
// the decode split plan (csrc/decode_plan.h): no HIP, no device. Built by
// tests/test_host_sanitized.py with g++ -fsanitize=address,undefined (every
// report fatal) and run there; any overflow, out-of-bounds access or failed
// expectation ends the program with a nonzero status.
#include <algorithm>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../fsq_latent_decode_amd/csrc/validate.h"

using fsq::DecodePlan;

static int n_checks = 0;
#define EXPECT(cond)                                                          \
    do {                                                                      \
        ++n_checks;                                                           \
        if (!(cond)) {                                                        \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
            exit(1);                                                          \
        }                                                                     \
    } while (0)

// Stand-in pointer values (never dereferenced): aligned to 256 bytes, and one
// that is 16-byte but not 256-byte aligned, and one that is misaligned.
static const void *const P = reinterpret_cast<const void *>(uintptr_t(0x100000));
static const void *const P16 = reinterpret_cast<const void *>(uintptr_t(0x100010));
static const void *const P2 = reinterpret_cast<const void *>(uintptr_t(0x100002));

// Invariants of a plan that fsq_decode_attn would launch with.
static void check_plan(const DecodePlan &p, int32_t batch, int32_t n_q, int32_t G, int64_t cap, bool stream_ok) {
    EXPECT(p.GP % 32 == 0 && p.GP >= G && p.GP < G + 32);
    EXPECT(p.nqp % 32 == 0 && p.nqp >= n_q && p.nqp < n_q + 32);
    EXPECT(p.waves == 4 || p.waves == 8);
    EXPECT(p.chunk > 0 && p.chunk % (32 * p.waves) == 0);
    if (cap == 0) EXPECT(p.S == 0);
    else if (!p.dyn) EXPECT((int64_t)p.S * p.chunk >= cap && (int64_t)(p.S - 1) * p.chunk < cap);
    // device split: S bounds the work items of any sequence, ceil(T / chunk)
    // with chunk >= max(chunk_min, sum of lengths / ncta): at most ncta
    else EXPECT(p.S == std::min<int64_t>((cap + p.chunk - 1) / p.chunk, p.ncta));
    EXPECT(!p.stream || stream_ok);
    EXPECT(!p.stream || p.waves == fsq::stream_waves(p.GP));
    EXPECT(!p.dyn || (p.stream && batch <= fsq::kDynMaxBatch && p.ncta == fsq::dyn_ctas(p.GP)));
    if (p.dyn) EXPECT(p.chunk >= fsq::kStreamMinTiles * 32 * p.waves && (int64_t)p.chunk * fsq::kDynMaxSplits >= cap);
    // workspace: q~ rows, then fp16 zbar partials, then (m, l) pairs, each
    // region 256-byte aligned and large enough for every split of the plan
    const size_t S1 = p.S > 0 ? (size_t)p.S : 1;
    EXPECT(p.off_qt == 0);
    EXPECT(p.off_acc % 256 == 0 && p.off_ml % 256 == 0 && p.total % 256 == 0);
    EXPECT(p.off_acc >= (size_t)batch * p.nqp * p.GP * 2 * 2);   // q~ in two fp16 terms
    EXPECT(p.off_ml - p.off_acc >= (size_t)batch * S1 * n_q * p.GP * 2);
    EXPECT(p.total - p.off_ml >= (size_t)batch * S1 * n_q * 2 * 4);
}

static void append_cases() {
    EXPECT(fsq::validate_append(P, P, P, 1, 4096, 84, 16) == FSQ_OK);
    EXPECT(fsq::validate_append(nullptr, nullptr, nullptr, 0, 4096, 84, 16) == FSQ_OK);   // nothing to do
    EXPECT(fsq::validate_append(P, P, P, -1, 4096, 84, 16) == FSQ_ERR_SHAPE);
    EXPECT(fsq::validate_append(P, P, P, 1, 0, 84, 16) == FSQ_ERR_SHAPE);
    EXPECT(fsq::validate_append(P, P, P, 1, 4096, 0, 16) == FSQ_ERR_SHAPE);
    EXPECT(fsq::validate_append(P, P, P, 1, 4096, FSQ_MAX_G + 1, 16) == FSQ_ERR_UNSUPPORTED);
    EXPECT(fsq::validate_append(P, P, P, 1, 4100, 84, 16) == FSQ_ERR_UNSUPPORTED);
    EXPECT(fsq::validate_append(P, P, P, 1, 4096, 84, 8) == FSQ_ERR_UNSUPPORTED);
    EXPECT(fsq::validate_append(P, P, P, 1, 4096, 84, 4) == FSQ_OK);
    EXPECT(fsq::validate_append(P, P, P, 1, 4096, 84, 256) == FSQ_OK);
    EXPECT(fsq::validate_append(nullptr, P, P, 1, 4096, 84, 16) == FSQ_ERR_NULL);
    EXPECT(fsq::validate_append(P, nullptr, P, 1, 4096, 84, 16) == FSQ_ERR_NULL);
    EXPECT(fsq::validate_append(P, P, nullptr, 1, 4096, 84, 16) == FSQ_ERR_NULL);
    EXPECT(fsq::validate_append(P2, P, P, 1, 4096, 84, 16) == FSQ_ERR_UNSUPPORTED);
    EXPECT(fsq::validate_append(P, P2, P, 1, 4096, 84, 16) == FSQ_ERR_UNSUPPORTED);
    EXPECT(fsq::validate_append(P, P, P2, 1, 4096, 84, 16) == FSQ_OK);        // codes: any byte alignment
    EXPECT(fsq::validate_append(P, P, P, ((int64_t)1 << 36) + 1, 8, 1, 16) == FSQ_ERR_UNSUPPORTED);
    EXPECT(fsq::validate_append(P, P, P, INT64_MAX, INT32_MAX - 7, FSQ_MAX_G, 16) == FSQ_ERR_UNSUPPORTED);
}

static int decode(int32_t batch, int32_t n_q, int32_t n_kv, int32_t d_h, int32_t G, int64_t cap, size_t ws_bytes,
                  int32_t levels = 16, const void *codes = P, const void *ws = P, DecodePlan *pl = nullptr) {
    return fsq::validate_decode(P, codes, P, P, P, batch, n_q, n_kv, d_h, G, cap, ws, ws_bytes, levels, pl);
}

static void decode_cases() {
    const size_t big = (size_t)1 << 40;
    EXPECT(decode(1, 32, 8, 128, 256, 32768, big) == FSQ_OK);
    EXPECT(decode(0, 32, 8, 128, 256, 32768, big) == FSQ_ERR_SHAPE);
    EXPECT(decode(1, 0, 8, 128, 256, 32768, big) == FSQ_ERR_SHAPE);
    EXPECT(decode(1, 32, 0, 128, 256, 32768, big) == FSQ_ERR_SHAPE);
    EXPECT(decode(1, 32, 8, 0, 256, 32768, big) == FSQ_ERR_SHAPE);
    EXPECT(decode(1, 32, 8, 128, 0, 32768, big) == FSQ_ERR_SHAPE);
    EXPECT(decode(1, 32, 8, 128, 256, -1, big) == FSQ_ERR_SHAPE);
    EXPECT(decode(1, 32, 7, 128, 256, 32768, big) == FSQ_ERR_SHAPE);              // n_q % n_kv
    EXPECT(decode(1, 96, 8, 128, 256, 32768, big) == FSQ_ERR_UNSUPPORTED);        // n_q > 64
    EXPECT(decode(1, 32, 8, 512, 256, 32768, big) == FSQ_ERR_UNSUPPORTED);        // d_h > 256
    EXPECT(decode(1, 32, 8, 128, 257, 32768, big) == FSQ_ERR_UNSUPPORTED);        // G > 256
    EXPECT(decode(1, 32, 8, 128, 84, 32768, big, 8) == FSQ_ERR_UNSUPPORTED);      // levels
    EXPECT(decode(1, 32, 8, 128, 84, 32768, big, 16, P2) == FSQ_ERR_UNSUPPORTED);  // codes alignment
    EXPECT(decode(1, 32, 8, 128, 84, 0, big, 16, nullptr) == FSQ_OK);             // no cache at all
    EXPECT(decode(1, 32, 8, 128, 84, 1, big, 16, nullptr) == FSQ_ERR_NULL);
    EXPECT(fsq::validate_decode(nullptr, P, P, P, P, 1, 32, 8, 128, 84, 10, P, big, 16, nullptr) == FSQ_ERR_NULL);
    EXPECT(fsq::validate_decode(P, P, nullptr, P, P, 1, 32, 8, 128, 84, 10, P, big, 16, nullptr) == FSQ_ERR_NULL);
    EXPECT(fsq::validate_decode(P, P, P, nullptr, P, 1, 32, 8, 128, 84, 10, P, big, 16, nullptr) == FSQ_ERR_NULL);
    EXPECT(fsq::validate_decode(P, P, P, P, nullptr, 1, 32, 8, 128, 84, 10, P, big, 16, nullptr) == FSQ_ERR_NULL);
    EXPECT(decode(1, 32, 8, 128, 84, 10, big, 16, P, nullptr) == FSQ_ERR_WORKSPACE);
    EXPECT(decode(1, 32, 8, 128, 84, 10, big, 16, P, P16) == FSQ_ERR_WORKSPACE);   // not 256-byte aligned
    const size_t need = fsq::make_decode_plan(1, 32, 84, 131072).total;
    EXPECT(decode(1, 32, 8, 128, 84, 131072, need) == FSQ_OK);
    EXPECT(decode(1, 32, 8, 128, 84, 131072, need - 1) == FSQ_ERR_WORKSPACE);
    EXPECT(decode(65536, 8, 8, 64, 32, 1, big) == FSQ_ERR_UNSUPPORTED);          // batch limit
    EXPECT(decode(2, 32, 8, 128, 84, ((int64_t)1 << 40) / 2 + 1, big) == FSQ_ERR_UNSUPPORTED);
    EXPECT(decode(INT32_MAX, FSQ_MAX_NQ, 1, FSQ_MAX_DH, FSQ_MAX_G, INT64_MAX, SIZE_MAX) == FSQ_ERR_UNSUPPORTED);
    // the allocation-free entry point's capacity check: the per-layer
    // workloads fit its scratch area, the layer-batched G=256 call does not
    size_t ws_need = 0;
    EXPECT(fsq::validate_decode_args(P, P, P, P, P, 16, 16, 8, 128, 256, 65536, 16, nullptr, &ws_need) == FSQ_OK);
    EXPECT(ws_need <= FSQ_NOALLOC_SCRATCH_BYTES);
    EXPECT(fsq::validate_decode_args(P, P, P, P, P, 1, 32, 8, 128, 84, 1 << 20, 16, nullptr, &ws_need) == FSQ_OK);
    EXPECT(ws_need <= FSQ_NOALLOC_SCRATCH_BYTES);
    EXPECT(fsq::validate_decode_args(P, P, P, P, P, 36, 32, 8, 128, 256, 32768, 16, nullptr, &ws_need) == FSQ_OK);
    EXPECT(ws_need > FSQ_NOALLOC_SCRATCH_BYTES);
    // the step's extra arguments
    EXPECT(fsq::validate_step_append(P, P, 1, 4096, 32, 8, 128, 84, 10) == FSQ_OK);
    EXPECT(fsq::validate_step_append(P, P, 1, 0, 32, 8, 128, 84, 10) == FSQ_ERR_SHAPE);
    EXPECT(fsq::validate_step_append(P, P, 1, 4100, 32, 8, 128, 84, 10) == FSQ_ERR_UNSUPPORTED);
    EXPECT(fsq::validate_step_append(nullptr, P, 1, 4096, 32, 8, 128, 84, 10) == FSQ_ERR_NULL);
    EXPECT(fsq::validate_step_append(P2, P, 1, 4096, 32, 8, 128, 84, 10) == FSQ_ERR_UNSUPPORTED);
    // the reconstruction variants' further limits
    EXPECT(fsq::validate_recon(P, P, P, P, P, 1, 32, 8, 128, 84, 1000, P, big, nullptr) == FSQ_OK);
    EXPECT(fsq::validate_recon(P, P, P, P, P, 1, 32, 8, 96, 84, 1000, P, big, nullptr) == FSQ_OK);
    EXPECT(fsq::validate_recon(P, P, P, P, P, 1, 32, 8, 100, 84, 1000, P, big, nullptr) == FSQ_ERR_UNSUPPORTED);
    EXPECT(fsq::validate_recon(P, P, P, P, P, 1, 64, 1, 128, 84, 1000, P, big, nullptr) == FSQ_ERR_UNSUPPORTED);
    EXPECT(fsq::validate_rope_extra(P, 1, 32, 8, 128, 84, 10, 1e6f, 1e-6f) == FSQ_OK);
    EXPECT(fsq::validate_rope_extra(P, 1, 32, 8, 96, 84, 10, 1e6f, 1e-6f) == FSQ_ERR_UNSUPPORTED);
    EXPECT(fsq::validate_rope_extra(P, 1, 32, 8, 128, 84, 10, 1.0f, 1e-6f) == FSQ_ERR_SHAPE);
    EXPECT(fsq::validate_rope_extra(P, 1, 32, 8, 128, 84, 10, 1e6f, -1.0f) == FSQ_ERR_SHAPE);
    EXPECT(fsq::validate_rope_extra(nullptr, 1, 32, 8, 128, 84, 10, 1e6f, 1e-6f) == FSQ_ERR_NULL);
}

// The workloads' own shapes: the plans the kernels are launched with.
static void workload_plans() {
    struct W { int32_t batch, n_q, G; int64_t cap; const char *name; };
    const W ws[] = {{1, 16, 64, 1024, "tiny"},       {1, 32, 256, 32768, "qwen3_8b_g256"},
                    {1, 32, 84, 131072, "qwen3_8b_g84"}, {16, 16, 256, 65536, "qwen3_1p7b_ragged"},
                    {1, 32, 84, 1048576, "qwen3_8b_g84_1m"}, {1, 32, 32, 131072, "g32"},
                    {1, 32, 20, 131072, "g20"},      {1, 32, 168, 131072, "l4_g168"},
                    {1, 32, 42, 131072, "l256_g42"}, {36, 32, 256, 32768, "layer-batched g256"},
                    {36, 32, 84, 131072, "layer-batched g84"}};
    for (const W &w : ws) {
        DecodePlan pl;
        EXPECT(decode(w.batch, w.n_q, 8, 128, w.G, w.cap, (size_t)1 << 40, 16, P, P, &pl) == FSQ_OK);
        check_plan(pl, w.batch, w.n_q, w.G, w.cap, true);
        printf("%-20s kernel=%s%s waves=%d S=%d chunk=%d workspace=%zu\n", w.name, pl.stream ? "stream" : "split",
               pl.dyn ? "(device split)" : "", pl.waves, pl.S, pl.chunk, pl.total);
    }
}

// Pseudo-random sizes over the accepted range and past it (a fixed 64-bit LCG):
// validation and planning must not overflow or read out of bounds anywhere, and
// every accepted call's plan must satisfy the invariants.
static void random_sizes() {
    uint64_t s = 0x9E3779B97F4A7C15ull;
    auto next = [&](uint64_t mod) {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        return (s >> 17) % mod;
    };
    int accepted = 0;
    for (int i = 0; i < 200000; ++i) {
        const int32_t batch = (int32_t)next(4) == 0 ? (int32_t)next(70000) : 1 + (int32_t)next(70);
        const int32_t n_kv = 1 + (int32_t)next(16);
        const int32_t n_q = n_kv * (1 + (int32_t)next(10));
        const int32_t d_h = 1 + (int32_t)next(300);
        const int32_t G = 1 + (int32_t)next(300);
        const int64_t cap = next(8) == 0 ? (int64_t)next((uint64_t)1 << 41) : (int64_t)next(1 << 22);
        const int32_t levels = next(3) == 0 ? 4 : next(2) ? 16 : 256;
        const size_t need = fsq::decode_sizes_ok(batch, n_q, G, cap) ? fsq::make_decode_plan(batch, n_q, G, cap).total : 0;
        DecodePlan pl;
        const int v = decode(batch, n_q, n_kv, d_h, G, cap, need, levels, P, P, &pl);
        if (v == FSQ_OK) {
            ++accepted;
            check_plan(pl, batch, n_q, G, cap, levels == 16);
            EXPECT(decode(batch, n_q, n_kv, d_h, G, cap, need - 1, levels) == FSQ_ERR_WORKSPACE);
        }
    }
    EXPECT(accepted > 10000);
    printf("random sizes: %d accepted\n", accepted);
}

int main() {
    append_cases();
    decode_cases();
    workload_plans();
    random_sizes();
    printf("ok: %d checks\n", n_checks);
    return 0;
}
