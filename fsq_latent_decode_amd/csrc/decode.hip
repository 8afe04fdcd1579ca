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
//   decode_split_kernel one CTA per (token chunk, sequence, 32-head group):
//                       codes -> registers (prefetched one tile ahead) -> LDS ->
//                       fp16 levels -> MFMA scores (all heads share z) -> online
//                       softmax (exp2) -> MFMA latent pooling -> (m, l, zbar fp16)
//   decode_merge_kernel one CTA per (sequence, head): log-sum-exp merge of the
//                       chunks' zbar, then out = W_v,g zbar
#include <hip/hip_ext.h>

#include "common.h"
#include "decode_plan.h"

namespace fsq {

constexpr int kTile = 32;     // tokens per wave iteration (the score MFMA's M)
constexpr int kWaves = 4;     // waves per CTA, each on its own token tiles

// fp16 levels of one packed dword (8 codes, nibble i = coordinate 8D + i), in
// the operand order (c0,c4)(c1,c5)(c2,c6)(c3,c7): 0x6400 | n is the fp16 value
// 1024 + n, so subtracting 1032 gives the level n - 8 exactly.
__device__ inline half8 unpack_levels(uint32_t w) {
    typedef _Float16 half2v __attribute__((ext_vector_type(2)));
    const uint32_t m = 0x000F000Fu, e = 0x64006400u;
    const uint32_t t0 = (w & m) | e;
    const uint32_t t1 = ((w >> 4) & m) | e;
    const uint32_t t2 = ((w >> 8) & m) | e;
    const uint32_t t3 = ((w >> 12) & m) | e;
    const half2v bias = {(_Float16)1032.0f, (_Float16)1032.0f};
    const half2v h0 = __builtin_bit_cast(half2v, t0) - bias;
    const half2v h1 = __builtin_bit_cast(half2v, t1) - bias;
    const half2v h2 = __builtin_bit_cast(half2v, t2) - bias;
    const half2v h3 = __builtin_bit_cast(half2v, t3) - bias;
    const half8 r = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
    return r;
}

// ---------------------------------------------------------------- absorb
// q~[b, h, pos(k)] = scale * sum_d W_k[g d_h + d, k] q[b, h, d] for the grp heads
// h of kv head g. One CTA per (kv head, 64 latent columns, sequence); the 256
// threads are 64 columns x 4 quarters of d, each thread holding its W_k values
// in registers while it forms the grp dot products.
constexpr int kAbsorbCols = 64;
constexpr int kMergeWvElems = 128 * 272;   // LDS for W_v blocks up to 128 padded rows of 256
constexpr int kAbsorbHeadBatch = 8;

__global__ __launch_bounds__(256) void absorb_kernel(const uint16_t *__restrict__ q,
                                                     const uint16_t *__restrict__ W_kv,
                                                     _Float16 *__restrict__ qt, int G, int GP,
                                                     int n_q, int nqp, int n_kv, int d_h,
                                                     float scale) {
    extern __shared__ float qs[];   // [grp][d_h]
    __shared__ float red[4][kAbsorbHeadBatch][kAbsorbCols];
    const int g = blockIdx.x, b = blockIdx.z;
    const int col = threadIdx.x & (kAbsorbCols - 1), qd = threadIdx.x >> 6;
    const int k = blockIdx.y * kAbsorbCols + col;
    const int grp = n_q / n_kv;
    for (int i = threadIdx.x; i < grp * d_h; i += blockDim.x)
        qs[i] = bf16_to_f32(q[((size_t)b * n_q + (size_t)g * grp) * d_h + i]);
    // rows past n_q up to the 32-head padding are zero (written once, by kv head 0)
    if (g == 0 && k < GP && qd == 0)
        for (int h = n_q; h < nqp; ++h) qt[((size_t)b * nqp + h) * GP + k] = (_Float16)0.0f;
    __syncthreads();
    const int dq = (d_h + 3) / 4;
    const int d0 = qd * dq, d1 = (d0 + dq < d_h) ? d0 + dq : d_h;
    float w[kMaxDh / 4];
    const bool kin = k < G;
    // every load is issued unconditionally from a clamped (valid) address so that
    // all of them are in flight together; out-of-range values are zeroed after
    const int kc = kin ? k : G - 1;
    const uint16_t *wcol = W_kv + (size_t)g * d_h * G + kc;
    uint16_t wr[kMaxDh / 4];
#pragma unroll
    for (int i = 0; i < kMaxDh / 4; ++i) {
        const int d = (d0 + i < d_h) ? d0 + i : d_h - 1;
        wr[i] = wcol[(size_t)d * G];
    }
#pragma unroll
    for (int i = 0; i < kMaxDh / 4; ++i) w[i] = (kin && d0 + i < d1) ? bf16_to_f32(wr[i]) : 0.0f;
    for (int hb = 0; hb < grp; hb += kAbsorbHeadBatch) {
        const int nh = (grp - hb) < kAbsorbHeadBatch ? (grp - hb) : kAbsorbHeadBatch;
        for (int j = 0; j < nh; ++j) {
            // w[i] is zero past this thread's d range; the clamped q index keeps
            // the LDS reads in range without a per-element branch
            const float *qj = qs + (hb + j) * d_h;
            float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
            for (int i = 0; i < kMaxDh / 4; i += 2) {
                a0 += w[i] * qj[(d0 + i) < d_h ? d0 + i : d_h - 1];
                a1 += w[i + 1] * qj[(d0 + i + 1) < d_h ? d0 + i + 1 : d_h - 1];
            }
            red[qd][j][col] = a0 + a1;
        }
        __syncthreads();
        if (qd == 0 && k < GP) {
            for (int j = 0; j < nh; ++j) {
                const float a = red[0][j][col] + red[1][j][col] + red[2][j][col] + red[3][j][col];
                const int h = g * grp + hb + j;
                qt[((size_t)b * nqp + h) * GP + coord_to_pos(k, GP)] = (_Float16)(kin ? a * scale : 0.0f);
            }
        }
        __syncthreads();
    }
}

// ----------------------------------------------------------------- split
// One CTA = 4 waves working through its token chunk in rounds of 4 x 32 tokens.
// In a round each wave loads (one round ahead, straight into registers),
// unpacks and scores its own 32-token tile against all 32 heads; the waves then
// agree on a per-head reference max and normaliser through LDS, and every wave
// pools all 4 tiles but only for its own latent coordinate blocks (block cb
// belongs to wave cb % 4). The softmax state is therefore identical in all
// waves and the pooled sums need no cross-wave combine.
template <int GP>
struct SplitCfg {
    static constexpr int KB = GP / 16;                 // score k-blocks = dwords per lane half
    static constexpr int CB = GP / 32;                 // pooling coordinate blocks
    static constexpr int CBW = (CB + kWaves - 1) / kWaves;   // blocks per wave
    static constexpr int RS = (GP / 2 + 63) / 64 * 64; // dwords per fp16 tile row
    static constexpr int kTileDw = kTile * RS;
    static constexpr int kZBytes = kWaves * kTileDw * 4;
    static constexpr int kPBytes = kWaves * 2 * 64 * 16;
    static constexpr int kCbufBytes = 32 * (GP + 1) * 4;
    static_assert(kCbufBytes <= kZBytes, "epilogue buffer must fit in the tile region");
};

// XOR swizzle (dword granularity) of the fp16 tile: the 16-byte row writes of
// 16 consecutive rows and the transposing 8-byte reads of 4 rows x 16 dwords
// both fall on distinct LDS banks.
__device__ inline int zt_swz(int row) { return 16 * (row & 3) + 4 * ((row >> 2) & 3); }

template <int GP, bool AL>
__global__ __launch_bounds__(kWaves * 64) void decode_split_kernel(
    const _Float16 *__restrict__ qt, const uint8_t *__restrict__ codes,
    const int32_t *__restrict__ seq_lens, _Float16 *__restrict__ part_z,
    float *__restrict__ part_ml, int64_t seq_cap, int G, int n_q, int nqp, int chunk, int S) {
    using C = SplitCfg<GP>;
    constexpr int KB = C::KB, CB = C::CB, CBW = C::CBW, RS = C::RS;
    constexpr int NLD = AL ? KB : KB + 1;   // dwords loaded per lane per tile
    // the reference max may lag the true max by this much (log2 units) before the
    // accumulators are rescaled: p = 2^(s - m) stays <= 256, exact range for fp16
    constexpr float kRescaleSlack = 8.0f;
    __shared__ __attribute__((aligned(16))) uint32_t zsm[C::kZBytes / 4];
    __shared__ __attribute__((aligned(16))) uint8_t psm[C::kPBytes];
    __shared__ float tmax_s[kWaves][32], tsum_s[kWaves][32];

    const int P = (G + 1) / 2;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int s = blockIdx.x, b = blockIdx.y, hg = blockIdx.z;
    int64_t T = seq_lens[b];
    T = T < 0 ? 0 : (T > seq_cap ? seq_cap : T);
    const int64_t c0 = (int64_t)s * chunk;
    if (c0 >= T) return;
    const int64_t c1 = (c0 + chunk < T) ? c0 + chunk : T;
    const int t = lane & 31, hh = lane >> 5;
    const uint8_t *seq = codes + (size_t)b * seq_cap * P;

    // ---- per-lane loads of one tile (this lane's half of token t)
    uint32_t ld[NLD];
    int ld_ntok = 0, ld_sh = 0;
    auto issue = [&](int64_t t0) {
        const int64_t rem = c1 - t0;
        ld_ntok = rem <= 0 ? 0 : (rem < kTile ? (int)rem : kTile);
        if (ld_ntok == 0) return;
        const int tc = t < ld_ntok ? t : ld_ntok - 1;
        if (AL) {
            // P == GP / 2 and P % 16 == 0: the half is KB whole, 8-byte aligned dwords
            const uint2 *src = reinterpret_cast<const uint2 *>(seq + (size_t)(t0 + tc) * P + hh * (GP / 4));
#pragma unroll
            for (int i = 0; i < KB / 2; ++i) {
                const uint2 v = src[i];
                ld[2 * i] = v.x;
                ld[2 * i + 1] = v.y;
            }
        } else {
            // aligned dwords around the half, clamped to the tile's last dword
            const uint8_t *a = seq + (size_t)(t0 + tc) * P + hh * (GP / 4);
            ld_sh = (int)((uintptr_t)a & 3) * 8;
            const uint32_t *a0 = reinterpret_cast<const uint32_t *>(a - ((uintptr_t)a & 3));
            const uint8_t *lastb = seq + (size_t)(t0 + ld_ntok) * P - 1;
            const uint32_t *last = reinterpret_cast<const uint32_t *>(lastb - ((uintptr_t)lastb & 3));
#pragma unroll
            for (int i = 0; i < NLD; ++i) ld[i] = *(a0 + i <= last ? a0 + i : last);
        }
    };

    issue(c0 + wave * kTile);

    half8 qv[KB];
    {
        const _Float16 *qrow = qt + ((size_t)b * nqp + hg * 32 + t) * GP + hh * 8;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) qv[kb] = *reinterpret_cast<const half8 *>(qrow + 16 * kb);
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

    for (int64_t r0 = c0; r0 < c1; r0 += kWaves * kTile) {
        // ---- phase 1: own tile -> levels -> fp16 tile + scores
        uint32_t cur[KB];
        const int ntok = ld_ntok;
        const int sh = ld_sh;
        if (AL) {
#pragma unroll
            for (int i = 0; i < KB; ++i) cur[i] = ld[i];
        } else {
#pragma unroll
            for (int i = 0; i < KB; ++i)
                cur[i] = (uint32_t)((((uint64_t)ld[i + 1] << 32) | ld[i]) >> sh);
        }
        issue(r0 + kWaves * kTile + wave * kTile);

        const bool live = t < ntok;
        floatx16 sc0 = floatx16{}, sc1 = floatx16{};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            uint32_t w = cur[kb];
            if (!AL) {
                const int nvalid = P - hh * (GP / 4) - 4 * kb;
                w &= nvalid <= 0 ? 0u : nvalid >= 4 ? 0xFFFFFFFFu : (1u << (8 * nvalid)) - 1u;
            }
            w = live ? w : 0u;
            const half8 z = unpack_levels(w);
            *reinterpret_cast<half8 *>(zt_own + t * RS + ((8 * kb + 4 * hh) ^ zt_swz(t))) = z;
            if (kb & 1)
                sc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(z, qv[kb], sc1, 0, 0, 0);
            else
                sc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(z, qv[kb], sc0, 0, 0, 0);
        }
        const floatx16 sc = sc0 + sc1;
        float sv[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int tok = (r >> 2) * 8 + hh * 4 + (r & 3);
            sv[r] = tok < ntok ? sc[r] : -INFINITY;
            tmax = fmaxf(tmax, sv[r]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        if (lane < 32) tmax_s[wave][t] = tmax;
        __syncthreads();

        // ---- phase 2: common reference max (lazy), probabilities, row sums
        float rmax = tmax_s[0][t];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) rmax = fmaxf(rmax, tmax_s[w][t]);
        const bool bump = rmax > m_ref + kRescaleSlack;
        const float m_new = bump ? rmax : m_ref;
        const float alpha = bump ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
        const bool rescale = bump && m_ref != -INFINITY;
        m_ref = m_new;
        float psum = 0.0f;
        _Float16 p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float e = __builtin_amdgcn_exp2f(sv[r] - m_new);
            psum += e;
            p[r] = (_Float16)e;
        }
        psum += __shfl_xor(psum, 32);
        if (lane < 32) tsum_s[wave][t] = psum;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const half8 pv = {p[ks * 8 + 0], p[ks * 8 + 1], p[ks * 8 + 2], p[ks * 8 + 3],
                              p[ks * 8 + 4], p[ks * 8 + 5], p[ks * 8 + 6], p[ks * 8 + 7]};
            *reinterpret_cast<half8 *>(psm + ((wave * 2 + ks) * 64 + lane) * 16) = pv;
        }
        __syncthreads();
        float rsum = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) rsum += tsum_s[w][t];
        l_run = l_run * alpha + rsum;
        if (__any(rescale)) {
#pragma unroll
            for (int j = 0; j < CBW; ++j) acc[j] *= alpha;
        }

        // ---- phase 3: pool the round's tiles for this wave's coordinate blocks
#pragma unroll
        for (int w2 = 0; w2 < kWaves; ++w2) {
            if (r0 + w2 * kTile >= c1) break;     // empty tile (uniform)
            const uint32_t *zt = zsm + w2 * C::kTileDw;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const half8 pb = *reinterpret_cast<const half8 *>(psm + ((w2 * 2 + ks) * 64 + lane) * 16);
                const int ra = ks * 16 + hh * 4 + mrow, rb = ra + 8;
#pragma unroll
                for (int j = 0; j < CBW; ++j) {
                    const int cb = wave + kWaves * j;
                    if (cb < CB) {
                        const int cdw = cb * 16 + g16 * 8 + pcol * 2;
                        const shortx4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_s4 *)(zt + ra * RS + (cdw ^ zt_swz(ra))));
                        const shortx4 a2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_s4 *)(zt + rb * RS + (cdw ^ zt_swz(rb))));
                        const short8 zs = {a1[0], a1[1], a1[2], a1[3], a2[0], a2[1], a2[2], a2[3]};
                        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, zs),
                                                                        pb, acc[j], 0, 0, 0);
                    }
                }
            }
        }
        __syncthreads();   // the next round overwrites the tiles and probabilities
    }

    // ---- epilogue: zbar = acc / l (operand-position order) via LDS, fp16 out
    const float invL = 1.0f / l_run;
    float *cbuf = reinterpret_cast<float *>(zsm);   // [32 heads][GP + 1]
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
        const int cb = wave + kWaves * j;
        if (cb < CB) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int pos = cb * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
                cbuf[t * (GP + 1) + pos] = acc[j][r] * invL;
            }
        }
    }
    __syncthreads();
    const int heads = (n_q - hg * 32) < 32 ? (n_q - hg * 32) : 32;
    const size_t pbase = ((size_t)b * S + s) * n_q + hg * 32;
    typedef _Float16 half4 __attribute__((ext_vector_type(4)));
    for (int idx = threadIdx.x; idx < heads * (GP / 4); idx += blockDim.x) {
        const int hd = idx / (GP / 4), p4 = idx - hd * (GP / 4);
        const float *src = cbuf + hd * (GP + 1) + p4 * 4;
        const half4 v = {(_Float16)src[0], (_Float16)src[1], (_Float16)src[2], (_Float16)src[3]};
        *reinterpret_cast<half4 *>(part_z + (pbase + hd) * GP + p4 * 4) = v;
    }
    if (wave == 0 && lane < heads) {
        part_ml[(pbase + lane) * 2 + 0] = m_ref;
        part_ml[(pbase + lane) * 2 + 1] = l_run;
    }
}

// ----------------------------------------------------------------- merge
// One CTA per (head, sequence): M = max_i m_i, c_i = l_i 2^(m_i - M),
// zbar = sum_i c_i zbar_i / sum_i c_i, out = W_v,g zbar. The partials are read
// with 16-byte loads spread over (8-position group x split group) threads.
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const _Float16 *__restrict__ part_z, const float *__restrict__ part_ml,
    const uint16_t *__restrict__ W_kv, const int32_t *__restrict__ seq_lens,
    uint16_t *__restrict__ out, int64_t seq_cap, int G, int GP, int n_q, int n_kv, int d_h,
    int chunk, int S) {
    extern __shared__ float coef[];   // [S]
    __shared__ float zpart[256 * 8];   // [split group][GP]
    __shared__ __attribute__((aligned(16))) float zbar[kMaxG];
    __shared__ __attribute__((aligned(16))) uint16_t wv_s[kMergeWvElems];
    __shared__ float red[8];
    const int h = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint16_t *o = out + ((size_t)b * n_q + h) * d_h;
    int64_t T = seq_lens[b];
    T = T < 0 ? 0 : (T > seq_cap ? seq_cap : T);
    const int ns = (int)((T + chunk - 1) / chunk);
    if (ns == 0) {
        for (int d = tid; d < d_h; d += blockDim.x) o[d] = 0;
        return;
    }
    // stage this kv head's W_v block (d_h x G bf16, contiguous in memory) in LDS
    // rows of WS dwords; the loads are issued first so that they overlap the
    // partial-state loads below. TPR threads share an output row; WS / 4 = TPR
    // (mod 16) puts the 16-byte reads of one pass (16 / TPR rows x TPR chunks)
    // on distinct banks.
    const int g = h / (n_q / n_kv);
    const uint16_t *Wv = W_kv + ((size_t)n_kv * d_h + (size_t)g * d_h) * G;
    int TPR = 1;
    while (TPR * 2 * d_h <= 256 && TPR < 16) TPR *= 2;
    int WS = ((G + 1) / 2 + 3) / 4 * 4;
    while (((WS / 4) & 15) != (TPR & 15)) WS += 4;
    const bool wv_lds = d_h * WS * 2 <= kMergeWvElems;
    if (wv_lds) {
        if ((G & 7) == 0 && ((uintptr_t)Wv & 15) == 0) {
            const int nc = G / 8;
            for (int i = tid; i < d_h * nc; i += blockDim.x) {
                const int d = i / nc, c = i - d * nc;
                *reinterpret_cast<u32x4 *>(wv_s + d * 2 * WS + 8 * c) =
                    reinterpret_cast<const u32x4 *>(Wv)[i];
            }
        } else if ((G & 1) == 0 && ((uintptr_t)Wv & 3) == 0) {
            const int nc = G / 2;
            for (int i = tid; i < d_h * nc; i += blockDim.x) {
                const int d = i / nc, c = i - d * nc;
                *reinterpret_cast<uint32_t *>(wv_s + d * 2 * WS + 2 * c) =
                    reinterpret_cast<const uint32_t *>(Wv)[i];
            }
        } else {
            for (int i = tid; i < d_h * G; i += blockDim.x) {
                const int d = i / G, c = i - d * G;
                wv_s[d * 2 * WS + c] = Wv[i];
            }
        }
    }
    const size_t sstride = (size_t)n_q;                       // rows between splits
    const float *ml = part_ml + ((size_t)b * S * n_q + h) * 2;
    float M = -INFINITY;
    for (int i = tid; i < ns; i += blockDim.x) M = fmaxf(M, ml[i * sstride * 2]);
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    if (lane == 0) red[wave] = M;
    __syncthreads();
    M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float Lp = 0.0f;
    for (int i = tid; i < ns; i += blockDim.x) {
        const float c = ml[i * sstride * 2 + 1] * __builtin_amdgcn_exp2f(ml[i * sstride * 2] - M);
        coef[i] = c;
        Lp += c;
    }
    for (int off = 32; off > 0; off >>= 1) Lp += __shfl_xor(Lp, off);
    if (lane == 0) red[wave] = Lp;
    __syncthreads();
    const float invL = 1.0f / ((red[0] + red[1]) + (red[2] + red[3]));

    // zbar in operand-position order: thread = (8-position group kg, split group sg)
    const int KG = GP / 8, SG = 256 / KG;
    const int kg = tid % KG, sg = tid / KG;
    float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (sg < SG) {
        // up to 16 partial rows per thread in flight at once (indices clamped,
        // coefficients of the clamped rows zero)
        constexpr int U = 16;
        const _Float16 *zp = part_z + ((size_t)b * S * n_q + h) * GP + kg * 8;
        for (int i0 = sg; i0 < ns; i0 += U * SG) {
            half8 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + u * SG;
                v[u] = *reinterpret_cast<const half8 *>(zp + (size_t)(i < ns ? i : ns - 1) * sstride * GP);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + u * SG;
                const float c = i < ns ? coef[i] : 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j) a[j] += c * (float)v[u][j];
            }
        }
    }
    // reduce over split groups in a fixed order
    if (sg < SG)
#pragma unroll
        for (int j = 0; j < 8; ++j) zpart[sg * GP + kg * 8 + j] = a[j];
    __syncthreads();
    for (int p = tid; p < GP; p += blockDim.x) {
        float z = 0.0f;
        for (int u = 0; u < SG; ++u) z += zpart[u * GP + p];
        zbar[pos_to_coord(p, GP)] = z * invL;
    }
    __syncthreads();

    // out = W_v,g zbar: TPR threads per output row (from LDS when staged)
    const int rows_per_pass = 256 / TPR;
    const int part = tid % TPR;
    for (int dbase = 0; dbase < d_h; dbase += rows_per_pass) {
        const int d = dbase + tid / TPR;
        float acc = 0.0f;
        if (d < d_h) {
            if (wv_lds && (G & 7) == 0) {
                const uint16_t *row = wv_s + d * 2 * WS;
#pragma unroll 4
                for (int v = part; v < G / 8; v += TPR) {
                    const u32x4 wv = *reinterpret_cast<const u32x4 *>(row + 8 * v);
                    const floatx4 z0 = *reinterpret_cast<const floatx4 *>(zbar + 8 * v);
                    const floatx4 z1 = *reinterpret_cast<const floatx4 *>(zbar + 8 * v + 4);
                    acc += __uint_as_float(wv[0] << 16) * z0[0] + __uint_as_float(wv[0] & 0xFFFF0000u) * z0[1];
                    acc += __uint_as_float(wv[1] << 16) * z0[2] + __uint_as_float(wv[1] & 0xFFFF0000u) * z0[3];
                    acc += __uint_as_float(wv[2] << 16) * z1[0] + __uint_as_float(wv[2] & 0xFFFF0000u) * z1[1];
                    acc += __uint_as_float(wv[3] << 16) * z1[2] + __uint_as_float(wv[3] & 0xFFFF0000u) * z1[3];
                }
            } else {
                const uint16_t *row = wv_lds ? wv_s + d * 2 * WS : Wv + (size_t)d * G;
#pragma unroll 8
                for (int k = part; k < G; k += TPR) acc += bf16_to_f32(row[k]) * zbar[k];
            }
        }
        for (int off = TPR >> 1; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
        if (part == 0 && d < d_h) o[d] = f32_to_bf16(acc);
    }
}

template <int GP>
static hipError_t launch_split(const DecodePlan &pl, const _Float16 *qt, const uint8_t *codes,
                               const int32_t *seq_lens, _Float16 *pz, float *pml, int64_t seq_cap,
                               int G, int n_q, int batch, hipStream_t st, hipEvent_t ev0,
                               hipEvent_t ev1) {
    dim3 grid(pl.S, batch, pl.nqp / 32);
    dim3 block(kWaves * 64);
    // whole-dword vector loads when every token row starts on a 16-byte boundary
    const bool al = G == GP && ((G / 2) % 16) == 0 && ((uintptr_t)codes & 15) == 0;
    auto k = al ? decode_split_kernel<GP, true> : decode_split_kernel<GP, false>;
    if (ev0 && ev1)   // timed launch: events bracket this kernel's execution
        hipExtLaunchKernelGGL(k, grid, block, 0, st, ev0, ev1, 0, qt, codes, seq_lens, pz, pml,
                              seq_cap, G, n_q, pl.nqp, pl.chunk, pl.S);
    else
        k<<<grid, block, 0, st>>>(qt, codes, seq_lens, pz, pml, seq_cap, G, n_q, pl.nqp, pl.chunk,
                                  pl.S);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodePlan &pl, const uint16_t *q, const uint8_t *codes,
                         const uint16_t *W_kv, const int32_t *seq_lens, uint16_t *out, int batch,
                         int n_q, int n_kv, int d_h, int G, int64_t seq_cap, void *workspace,
                         hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    _Float16 *qt = reinterpret_cast<_Float16 *>(ws + pl.off_qt);
    _Float16 *pz = reinterpret_cast<_Float16 *>(ws + pl.off_acc);
    float *pml = reinterpret_cast<float *>(ws + pl.off_ml);
    const float scale = 1.4426950408889634f / sqrtf((float)d_h);
    hipError_t e;
    if (pl.S > 0) {
        const int grp = n_q / n_kv;
        dim3 ag(n_kv, (pl.GP + kAbsorbCols - 1) / kAbsorbCols, batch);
        absorb_kernel<<<ag, 256, (size_t)grp * d_h * sizeof(float), st>>>(q, W_kv, qt, G, pl.GP, n_q,
                                                                         pl.nqp, n_kv, d_h, scale);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        switch (pl.GP) {
#define FSQ_SPLIT_CASE(X)                                                                     \
    case X:                                                                                   \
        e = launch_split<X>(pl, qt, codes, seq_lens, pz, pml, seq_cap, G, n_q, batch, st, ev0, ev1); \
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
    decode_merge_kernel<<<dim3(n_q, batch), 256, (size_t)(pl.S > 0 ? pl.S : 1) * sizeof(float), st>>>(
        pz, pml, W_kv, seq_lens, out, seq_cap, G, pl.GP, n_q, n_kv, d_h, pl.chunk, pl.S);
    return hipGetLastError();
}

}  // namespace fsq
