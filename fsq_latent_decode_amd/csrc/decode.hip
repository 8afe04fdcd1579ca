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
//   absorb_kernel       q~ = (log2 e / sqrt d_h) W_k,g^T q  -> fp16, operand order
//   decode_split_kernel one CTA per (token chunk, sequence, 32-head group):
//                       codes -> LDS -> fp16 levels -> MFMA scores (all heads share
//                       z) -> online softmax (exp2) -> MFMA latent pooling -> (m, l, acc)
//   decode_merge_kernel log-sum-exp merge of the chunks, zbar = acc / l, out = W_v,g zbar
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
    uint32_t t0 = (w & m) | e;
    uint32_t t1 = ((w >> 4) & m) | e;
    uint32_t t2 = ((w >> 8) & m) | e;
    uint32_t t3 = ((w >> 12) & m) | e;
    const half2v bias = {(_Float16)1032.0f, (_Float16)1032.0f};
    half2v h0 = __builtin_bit_cast(half2v, t0) - bias;
    half2v h1 = __builtin_bit_cast(half2v, t1) - bias;
    half2v h2 = __builtin_bit_cast(half2v, t2) - bias;
    half2v h3 = __builtin_bit_cast(half2v, t3) - bias;
    half8 r = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
    return r;
}

// Little-endian dword at any byte offset of an LDS byte array.
__device__ inline uint32_t lds_dword(const uint8_t *p, int off) {
    if ((off & 3) == 0) return *reinterpret_cast<const uint32_t *>(p + off);
    if ((off & 1) == 0) {
        const uint16_t *s = reinterpret_cast<const uint16_t *>(p + off);
        return (uint32_t)s[0] | ((uint32_t)s[1] << 16);
    }
    return (uint32_t)p[off] | ((uint32_t)p[off + 1] << 8) | ((uint32_t)p[off + 2] << 16) |
           ((uint32_t)p[off + 3] << 24);
}

__global__ __launch_bounds__(256) void absorb_kernel(const uint16_t *__restrict__ q,
                                                     const uint16_t *__restrict__ W_kv,
                                                     _Float16 *__restrict__ qt, int G, int GP,
                                                     int n_q, int nqp, int n_kv, int d_h,
                                                     float scale) {
    __shared__ float qs[kMaxDh];
    const int h = blockIdx.x, b = blockIdx.y;
    _Float16 *row = qt + ((size_t)b * nqp + h) * GP;
    if (h >= n_q) {
        for (int k = threadIdx.x; k < GP; k += blockDim.x) row[k] = (_Float16)0.0f;
        return;
    }
    const int g = h / (n_q / n_kv);
    for (int d = threadIdx.x; d < d_h; d += blockDim.x)
        qs[d] = bf16_to_f32(q[((size_t)b * n_q + h) * d_h + d]);
    __syncthreads();
    for (int k = threadIdx.x; k < GP; k += blockDim.x) {
        float acc = 0.0f;
        if (k < G) {
            const uint16_t *w = W_kv + (size_t)g * d_h * G + k;
            for (int d = 0; d < d_h; ++d) acc += bf16_to_f32(w[(size_t)d * G]) * qs[d];
        }
        row[coord_to_pos(k)] = (_Float16)(acc * scale);
    }
}

template <int GP>
struct SplitSmem {
    static constexpr int kRawBytes = kTile * (GP / 2) + 32;   // >= tile bytes + 16-byte lead
    static constexpr int kRow = GP + 8;                        // fp16 row stride (16-byte pad)
    static constexpr int kZHalves = kTile * kRow;
    static constexpr int kWaveBytes = ((kRawBytes + 15) / 16) * 16 + kZHalves * 2;
    static constexpr int kBytes = kWaveBytes * kWaves;
    static_assert(kBytes >= 32 * GP * 4, "combine buffer must fit in the tile region");
};

template <int GP>
__global__ __launch_bounds__(kWaves * 64) void decode_split_kernel(
    const _Float16 *__restrict__ qt, const uint8_t *__restrict__ codes,
    const int32_t *__restrict__ seq_lens, float *__restrict__ part_acc,
    float *__restrict__ part_ml, int64_t seq_cap, int G, int n_q, int nqp, int chunk, int S) {
    constexpr int KB = GP / 16;   // score k-blocks
    constexpr int CB = GP / 32;   // pooling coordinate blocks
    using SM = SplitSmem<GP>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[SM::kBytes];
    __shared__ float wm[kWaves][32], wl[kWaves][32];

    const int P = (G + 1) / 2;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int s = blockIdx.x, b = blockIdx.y, hg = blockIdx.z;
    int64_t T = seq_lens[b];
    T = T < 0 ? 0 : (T > seq_cap ? seq_cap : T);
    const int64_t c0 = (int64_t)s * chunk;
    if (c0 >= T) return;
    const int64_t c1 = (c0 + chunk < T) ? c0 + chunk : T;

    uint8_t *raw = smem + wave * SM::kWaveBytes;
    _Float16 *zt = reinterpret_cast<_Float16 *>(raw + ((SM::kRawBytes + 15) / 16) * 16);

    const int t = lane & 31, hh = lane >> 5;

    half8 qv[KB];
    {
        const _Float16 *qrow = qt + ((size_t)b * nqp + hg * 32 + t) * GP + hh * 8;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) qv[kb] = *reinterpret_cast<const half8 *>(qrow + 16 * kb);
    }

    float m_run = -INFINITY, l_run = 0.0f;
    floatx16 acc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb] = floatx16{};

    const uint8_t *seq = codes + (size_t)b * seq_cap * P;
    for (int64_t t0 = c0 + wave * kTile; t0 < c1; t0 += kWaves * kTile) {
        const int ntok = (int)((c1 - t0) < kTile ? (c1 - t0) : kTile);
        // 1. stage the tile's bytes in LDS with aligned 16-byte loads
        const uint8_t *src = seq + (size_t)t0 * P;
        const uintptr_t base = (uintptr_t)src & ~(uintptr_t)15;
        const int lead = (int)((uintptr_t)src - base);
        const int n16 = (lead + ntok * P + 15) >> 4;
        for (int i = lane; i < n16; i += 64)
            reinterpret_cast<u32x4 *>(raw)[i] = reinterpret_cast<const u32x4 *>(base)[i];

        // 2. unpack levels, score MFMA S^T = Z Q~^T, keep the fp16 tile for pooling
        floatx16 sc = floatx16{};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int d = 2 * kb + hh;
            const int nvalid = P - 4 * d;
            uint32_t w = 0;
            if (t < ntok && nvalid > 0) {
                w = lds_dword(raw, lead + t * P + 4 * d);
                if (nvalid < 4) w &= (1u << (8 * nvalid)) - 1u;
            }
            const half8 z = unpack_levels(w);
            *reinterpret_cast<half8 *>(zt + t * SM::kRow + 16 * kb + 8 * hh) = z;
            sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(z, qv[kb], sc, 0, 0, 0);
        }

        // 3. online softmax in the log2 domain (scores already carry log2 e / sqrt d_h)
        float sv[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int tok = (r >> 2) * 8 + hh * 4 + (r & 3);
            sv[r] = tok < ntok ? sc[r] : -INFINITY;
            tmax = fmaxf(tmax, sv[r]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float psum = 0.0f;
        _Float16 p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float e = __builtin_amdgcn_exp2f(sv[r] - m_new);
            psum += e;
            p[r] = (_Float16)e;
        }
        psum += __shfl_xor(psum, 32);
        l_run = l_run * alpha + psum;
        m_run = m_new;
        if (alpha != 1.0f) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) acc[cb] *= alpha;
        }

        // 4. latent pooling O^T = Z^T P^T; Z^T comes from the fp16 tile by
        //    transposing LDS reads (4 tokens x 1 coordinate per 64-bit read)
        const int i16 = lane & 15, g16 = (lane >> 4) & 1;
        const int mrow = i16 >> 2, pcol = i16 & 3;
        typedef __attribute__((address_space(3))) shortx4 lds_s4;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const half8 pb = {p[ks * 8 + 0], p[ks * 8 + 1], p[ks * 8 + 2], p[ks * 8 + 3],
                              p[ks * 8 + 4], p[ks * 8 + 5], p[ks * 8 + 6], p[ks * 8 + 7]};
            const _Float16 *r1 = zt + (ks * 16 + hh * 4 + mrow) * SM::kRow + g16 * 16 + pcol * 4;
            const _Float16 *r2 = r1 + 8 * SM::kRow;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const shortx4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(r1 + cb * 32));
                const shortx4 a2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(r2 + cb * 32));
                typedef short short8 __attribute__((ext_vector_type(8)));
                const short8 zs = {a1[0], a1[1], a1[2], a1[3], a2[0], a2[1], a2[2], a2[3]};
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, zs), pb,
                                                                 acc[cb], 0, 0, 0);
            }
        }
    }

    // combine the waves of this CTA: common max, then a fixed-order sum in LDS
    __syncthreads();
    if (lane < 32) {
        wm[wave][lane] = m_run;
        wl[wave][lane] = l_run;
    }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wm[w][t]);
    const float scale = __builtin_amdgcn_exp2f(m_run - M);
    float *cbuf = reinterpret_cast<float *>(smem);   // [32 heads][GP], LDS positions
    for (int w = 0; w < kWaves; ++w) {
        if (wave == w) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int pos = cb * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
                    const float v = acc[cb][r] * scale;
                    float &dst = cbuf[t * GP + pos];
                    dst = (w == 0) ? v : dst + v;
                }
        }
        __syncthreads();
    }
    const int heads = (n_q - hg * 32) < 32 ? (n_q - hg * 32) : 32;
    const size_t pbase = ((size_t)b * S + s) * n_q + hg * 32;
    for (int idx = threadIdx.x; idx < heads * GP; idx += blockDim.x) {
        const int hd = idx / GP, k = idx - hd * GP;
        if (k < G) part_acc[(pbase + hd) * GP + k] = cbuf[hd * GP + coord_to_pos(k)];
    }
    if (threadIdx.x < heads) {
        const int hd = threadIdx.x;
        float Mh = -INFINITY;
        for (int w = 0; w < kWaves; ++w) Mh = fmaxf(Mh, wm[w][hd]);
        float L = 0.0f;
        for (int w = 0; w < kWaves; ++w) L += wl[w][hd] * __builtin_amdgcn_exp2f(wm[w][hd] - Mh);
        part_ml[(pbase + hd) * 2 + 0] = Mh;
        part_ml[(pbase + hd) * 2 + 1] = L;
    }
}

__global__ __launch_bounds__(256) void decode_merge_kernel(
    const float *__restrict__ part_acc, const float *__restrict__ part_ml,
    const uint16_t *__restrict__ W_kv, const int32_t *__restrict__ seq_lens,
    uint16_t *__restrict__ out, int64_t seq_cap, int G, int GP, int n_q, int n_kv, int d_h,
    int chunk, int S) {
    extern __shared__ float wsplit[];   // [S]
    __shared__ float zbar[kMaxG];
    __shared__ float red[8];
    const int h = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    uint16_t *o = out + ((size_t)b * n_q + h) * d_h;
    int64_t T = seq_lens[b];
    T = T < 0 ? 0 : (T > seq_cap ? seq_cap : T);
    const int ns = (int)((T + chunk - 1) / chunk);
    if (ns == 0) {
        for (int d = threadIdx.x; d < d_h; d += blockDim.x) o[d] = 0;
        return;
    }
    const size_t stride = (size_t)n_q;   // between splits, in (head) rows
    const float *ml = part_ml + ((size_t)b * S * n_q + h) * 2;
    // max over splits
    float M = -INFINITY;
    for (int i = threadIdx.x; i < ns; i += blockDim.x) M = fmaxf(M, ml[(size_t)i * stride * 2]);
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    if (lane == 0) red[wave] = M;
    __syncthreads();
    M = red[0];
    for (int w = 1; w < nw; ++w) M = fmaxf(M, red[w]);
    __syncthreads();
    for (int i = threadIdx.x; i < ns; i += blockDim.x)
        wsplit[i] = __builtin_amdgcn_exp2f(ml[(size_t)i * stride * 2] - M);
    __syncthreads();
    // l = sum_i w_i l_i in a fixed order (thread 0), shared through LDS
    if (threadIdx.x == 0) {
        float L = 0.0f;
        for (int i = 0; i < ns; ++i) L += wsplit[i] * ml[(size_t)i * stride * 2 + 1];
        red[0] = L;
    }
    __syncthreads();
    const float invL = 1.0f / red[0];
    const float *acc = part_acc + ((size_t)b * S * n_q + h) * GP;
    for (int k = threadIdx.x; k < G; k += blockDim.x) {
        float a = 0.0f;
        for (int i = 0; i < ns; ++i) a += wsplit[i] * acc[(size_t)i * stride * GP + k];
        zbar[k] = a * invL;
    }
    __syncthreads();
    // out = W_v,g zbar: one wave per output row, lanes across the latent
    const int g = h / (n_q / n_kv);
    const uint16_t *Wv = W_kv + ((size_t)n_kv * d_h + (size_t)g * d_h) * G;
    for (int d = wave; d < d_h; d += nw) {
        float a = 0.0f;
        for (int k = lane; k < G; k += 64) a += bf16_to_f32(Wv[(size_t)d * G + k]) * zbar[k];
        for (int off = 32; off > 0; off >>= 1) a += __shfl_xor(a, off);
        if (lane == 0) o[d] = f32_to_bf16(a);
    }
}

template <int GP>
static hipError_t launch_split(const DecodePlan &pl, const _Float16 *qt, const uint8_t *codes,
                               const int32_t *seq_lens, float *pacc, float *pml, int64_t seq_cap,
                               int G, int n_q, int batch, hipStream_t st) {
    dim3 grid(pl.S, batch, pl.nqp / 32);
    decode_split_kernel<GP><<<grid, kWaves * 64, 0, st>>>(qt, codes, seq_lens, pacc, pml, seq_cap,
                                                          G, n_q, pl.nqp, pl.chunk, pl.S);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodePlan &pl, const uint16_t *q, const uint8_t *codes,
                         const uint16_t *W_kv, const int32_t *seq_lens, uint16_t *out, int batch,
                         int n_q, int n_kv, int d_h, int G, int64_t seq_cap, void *workspace,
                         hipStream_t st) {
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    _Float16 *qt = reinterpret_cast<_Float16 *>(ws + pl.off_qt);
    float *pacc = reinterpret_cast<float *>(ws + pl.off_acc);
    float *pml = reinterpret_cast<float *>(ws + pl.off_ml);
    const float scale = 1.4426950408889634f / sqrtf((float)d_h);
    hipError_t e;
    if (pl.S > 0) {
        absorb_kernel<<<dim3(pl.nqp, batch), 256, 0, st>>>(q, W_kv, qt, G, pl.GP, n_q, pl.nqp, n_kv,
                                                          d_h, scale);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        switch (pl.GP) {
#define FSQ_SPLIT_CASE(X)                                                                       \
    case X:                                                                                     \
        e = launch_split<X>(pl, qt, codes, seq_lens, pacc, pml, seq_cap, G, n_q, batch, st); \
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
        pacc, pml, W_kv, seq_lens, out, seq_cap, G, pl.GP, n_q, n_kv, d_h, pl.chunk, pl.S);
    return hipGetLastError();
}

}  // namespace fsq
