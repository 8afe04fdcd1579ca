/*
 * fsq.h - C ABI of the Transformer-FSQ latent-decode library for AMD MI355X (gfx950).
 *
 * The cache stores, per token and layer, G four-bit finite-scalar-quantised
 * codes of z = FSQ(E x) and nothing else. Keys and values exist only through a
 * shared decoder W_kv = [W_k; W_v]. Definitions are those of the pages
 * "Transformer-FSQ: Discrete Latents for Extreme KV-Cache Compression"
 * (picx.dev summary: Eq. 2 quantiser, Eq. 4 encoder, Eq. 5-6 keys/values and
 * values decoded after pooling; Byte Budgeting) and the slides "Transformer-FSQ"
 * (frame "A wide product code uses four bits per coordinate": L = 16, h = 7.5075,
 * delta = 0.5, ceil(G b / 8) bytes per token per layer; frame "The kernel reads
 * codes and never writes reconstructed K/V": the decode kernel's steps).
 *
 * Conventions shared by every call
 *   - Tensor pointers are DEVICE pointers owned by the caller. The library
 *     allocates no device memory, keeps no pointer after returning, and holds
 *     no per-call state; calls on different streams may run concurrently as
 *     long as they use distinct output and workspace buffers.
 *   - bf16 tensors are passed as uint16_t bit patterns, row-major, contiguous.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream). Calls only
 *     enqueue work on it and return; nothing synchronises with the host. A
 *     device-side fault surfaces at the caller's next synchronisation.
 *   - Arguments are validated before any HIP call. On a validation failure
 *     nothing is enqueued and no output is touched.
 *   - Returns an fsq_status; fsq_status_string() names it. No C++ exception
 *     crosses this interface.
 *
 * Code layout (a reading of the pages, which fix only the byte count):
 *   level  = round-half-even(h * tanh(u + atanh(delta / h)) - delta) in -8..7,
 *   code   = level + 8 in 0..15,
 *   byte j of a token = code[2j] | (code[2j+1] << 4), j < ceil(G/2); for odd G
 *   the last high nibble is zero. A token row is exactly ceil(G/2) bytes; rows
 *   of one sequence are contiguous.
 * The *_levels entry points take L = 4, 16 or 256 levels (b = 2, 4, 8 bits per
 * code; the slides' backup frame "the grid size is an allocation choice"):
 * h = 1.001 (L - 1) / 2 (a reading: the pages print h only for L = 16, where
 * this gives 7.5075), delta = 0.5, levels -L/2 .. L/2 - 1, code = level + L/2,
 * code i of a token at bits (i b) mod 8 of byte floor(i b / 8), unused high
 * bits of the last byte zero; a row is ceil(G b / 8) bytes.
 */
#ifndef FSQ_H
#define FSQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fsq_status {
    FSQ_OK = 0,
    FSQ_ERR_NULL = 1,        /* a required pointer is NULL                         */
    FSQ_ERR_SHAPE = 2,       /* a size is negative, zero where it must not be, or  */
                             /* the sizes are inconsistent (n_q % n_kv != 0, ...)  */
    FSQ_ERR_UNSUPPORTED = 3, /* valid but outside what the kernels implement       */
    FSQ_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required            */
    FSQ_ERR_HIP = 5          /* a HIP runtime call (device query, launch) failed   */
} fsq_status;

/* Static name of a status code ("FSQ_OK", ...; "FSQ_UNKNOWN" otherwise). */
const char *fsq_status_string(int status);

/* Limits enforced by validation. */
#define FSQ_MAX_G 256          /* latent width G: 1..FSQ_MAX_G                       */
#define FSQ_MAX_NQ 64          /* query heads per sequence: 1..FSQ_MAX_NQ            */
#define FSQ_MAX_DH 256         /* head dimension d_h: 1..FSQ_MAX_DH                  */

/*
 * fsq_append - encode residual states and write their packed codes.
 *
 * Computes z_t = Q_FSQ(E x_t) (Eq. 4 with the Eq. 2 forward value) for each of
 * the n_tokens rows of x and stores the packed codes.
 *   x      [n_tokens, C]        bf16, row-major, 16-byte aligned.
 *   E      [G, C]               bf16, row-major (the encoder), 16-byte aligned.
 *   codes  [n_tokens, ceil(G/2)] u8 destination rows (the caller points at the
 *                               first row to write, e.g. cache + T * ceil(G/2));
 *                               any byte alignment is accepted.
 *   n_tokens >= 0 (0 enqueues nothing), C >= 1 with C % 8 == 0, 1 <= G <= FSQ_MAX_G.
 * Arithmetic: bf16 products accumulated in fp32 (MFMA for n_tokens >= 32,
 * vector FMA below), bound and round in fp32. Compared with an exact fp64
 * evaluation a code can differ by +-1 only where u~ lies within fp32 rounding
 * of a half-integer. The fp32 summation order depends on the token's place in
 * the call (which 32-token block holds it), so such a code can also differ
 * between calls that place the same token differently; repeating a call gives
 * the same bits.
 * Errors: FSQ_ERR_NULL (x, E or codes NULL with n_tokens > 0),
 *         FSQ_ERR_SHAPE (n_tokens < 0, C < 1, G < 1), FSQ_ERR_UNSUPPORTED
 *         (C % 8 != 0, G > FSQ_MAX_G, x or E not 16-byte aligned), FSQ_ERR_HIP.
 */
int fsq_append(const uint16_t *x, const uint16_t *E, uint8_t *codes,
               int64_t n_tokens, int32_t C, int32_t G, void *stream);

/*
 * fsq_append_levels - fsq_append for L = levels per coordinate (4, 16 or 256;
 * the layout above); codes rows are ceil(G b / 8) bytes. fsq_append is
 * fsq_append_levels with levels = 16.
 * Errors: as fsq_append; FSQ_ERR_UNSUPPORTED for another number of levels.
 */
int fsq_append_levels(const uint16_t *x, const uint16_t *E, uint8_t *codes,
                      int64_t n_tokens, int32_t C, int32_t G, int32_t levels, void *stream);

/*
 * fsq_decode_workspace_bytes - device workspace that fsq_decode_attn needs for
 * these sizes (the absorbed queries and the split-K partial states).
 * Returns 0 for invalid sizes (batch < 1, n_q outside 1..FSQ_MAX_NQ, G outside
 * 1..FSQ_MAX_G, seq_cap < 0, or batch * seq_cap > 2^40). Depends only on its
 * arguments.
 */
size_t fsq_decode_workspace_bytes(int32_t batch, int32_t n_q, int32_t G, int64_t seq_cap);

/*
 * fsq_decode_plan_info - how fsq_decode_attn (4-bit codes) splits a call of
 * these sizes: *kernel = 0 for the round-synchronous split-K kernel (short
 * chunks), 1 for the streaming split-K kernel (long chunks), 2 for the
 * streaming kernel with the split chosen on the device from the actual
 * lengths (batches of up to 64 sequences); *splits = chunks per sequence (2: at
 * most); *chunk = tokens per chunk (2: at least). Host arithmetic only.
 * Errors: FSQ_ERR_SHAPE (invalid sizes), FSQ_ERR_NULL (an output pointer NULL).
 */
int fsq_decode_plan_info(int32_t batch, int32_t n_q, int32_t G, int64_t seq_cap, int32_t *kernel,
                         int32_t *splits, int64_t *chunk);

/*
 * fsq_decode_attn - one decode step of attention read from the packed cache.
 *
 * For each sequence b and query head h (kv head g = h / (n_q / n_kv)), over
 * the cached positions t < seq_lens[b]:
 *   q~   = (log2(e) / sqrt(d_h)) * W_k,g^T q[b,h]        (query absorbed into latent space)
 *   s_t  = q~ . z_t,  z_t = code_t - 8                   (scores, log2 domain)
 *   zbar = sum_t 2^(s_t - max s) z_t / sum_t 2^(s_t - max s)   (codes pooled, Eq. 6)
 *   out[b,h] = W_v,g zbar                                 (values decoded once, Eq. 6)
 * i.e. softmax(K q / sqrt(d_h))^T V with K = Z W_k,g^T and V = Z W_v,g^T (Eq. 5
 * without key norm and RoPE). Keys and values are never written to memory.
 *   q        [batch, n_q, d_h]              bf16.
 *   codes    [batch, seq_cap, ceil(G/2)]    u8 packed cache (layout above),
 *                                           16-byte aligned. The kernels read it
 *                                           in aligned 16-byte units, so the
 *                                           bytes from its end up to the next
 *                                           16-byte boundary must be readable
 *                                           memory (an allocation rounded up to
 *                                           16 bytes, as PyTorch's are, is
 *                                           enough); they never affect a result.
 *   W_kv     [2 * n_kv * d_h, G]            bf16; rows [0, n_kv d_h) are W_k and
 *                                           rows [n_kv d_h, 2 n_kv d_h) are W_v,
 *                                           each kv-head-major (d_h rows per head).
 *   seq_lens [batch]                        int32 on the device; values are
 *                                           clamped to [0, seq_cap]. A length of
 *                                           0 yields out[b] = 0.
 *   out      [batch, n_q, d_h]              bf16 (written).
 *   workspace, workspace_bytes              device scratch of at least
 *                                           fsq_decode_workspace_bytes(...) bytes,
 *                                           256-byte aligned; its content on entry
 *                                           is irrelevant and it is overwritten.
 * Sizes: batch >= 1, 1 <= n_q <= FSQ_MAX_NQ, n_kv >= 1, n_q % n_kv == 0,
 *        1 <= d_h <= FSQ_MAX_DH, 1 <= G <= FSQ_MAX_G, seq_cap >= 0,
 *        batch * seq_cap <= 2^40, batch <= 65535.
 * Arithmetic: fp16 MFMA operands (levels are exact in fp16; q~ rounded to
 * fp16 after scaling), fp32 accumulation and softmax, bf16 output.
 * Errors: FSQ_ERR_NULL, FSQ_ERR_SHAPE, FSQ_ERR_UNSUPPORTED (d_h, G, n_q limits,
 *         codes not 16-byte aligned),
 *         FSQ_ERR_WORKSPACE (NULL, too small or misaligned), FSQ_ERR_HIP.
 */
int fsq_decode_attn(const uint16_t *q, const uint8_t *codes, const uint16_t *W_kv,
                    const int32_t *seq_lens, uint16_t *out,
                    int32_t batch, int32_t n_q, int32_t n_kv, int32_t d_h, int32_t G,
                    int64_t seq_cap, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * fsq_decode_attn_noalloc - fsq_decode_attn for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).
 *
 * Same computation, kernels and results as fsq_decode_attn with the same
 * arguments (bit for bit); the workspace is instead a fixed scratch area inside
 * the library, FSQ_NOALLOC_SCRATCH_BYTES of device memory per GPU, held from
 * the library's loading until the process ends. No allocation, free or
 * allocating library routine is called. The scratch address of the current
 * device is looked up on the first call on that device.
 * Every call on one GPU shares that GPU's scratch area and leaves its last
 * contents there (nothing in it needs to start at zero): calls that may
 * overlap on one GPU (several streams, several host threads) race on it and
 * must be serialised by the caller.
 * Sizes and layouts: as fsq_decode_attn; the sizes must also satisfy
 * fsq_decode_workspace_bytes(batch, n_q, G, seq_cap) <= FSQ_NOALLOC_SCRATCH_BYTES
 * (e.g. batch 16 at seq_cap 65536 with n_q 16, G 256: 17.3 MB).
 * Errors: as fsq_decode_attn; FSQ_ERR_WORKSPACE when the sizes need more
 *         scratch than FSQ_NOALLOC_SCRATCH_BYTES (nothing is enqueued);
 *         FSQ_ERR_HIP when the device or its scratch address cannot be queried.
 */
#define FSQ_NOALLOC_SCRATCH_BYTES (32u << 20)
int fsq_decode_attn_noalloc(const uint16_t *q, const uint8_t *codes, const uint16_t *W_kv,
                            const int32_t *seq_lens, uint16_t *out,
                            int32_t batch, int32_t n_q, int32_t n_kv, int32_t d_h, int32_t G,
                            int64_t seq_cap, void *stream);

/*
 * fsq_decode_attn_levels - fsq_decode_attn over a cache of L = levels codes
 * per coordinate (4, 16 or 256; rows of ceil(G b / 8) bytes, the layout
 * above), z_t = code_t - L/2. Same workspace size as fsq_decode_attn for the
 * same sizes. fsq_decode_attn is this call with levels = 16.
 * Errors: as fsq_decode_attn; FSQ_ERR_UNSUPPORTED for another number of levels.
 */
int fsq_decode_attn_levels(const uint16_t *q, const uint8_t *codes, const uint16_t *W_kv,
                           const int32_t *seq_lens, uint16_t *out,
                           int32_t batch, int32_t n_q, int32_t n_kv, int32_t d_h, int32_t G,
                           int32_t levels, int64_t seq_cap, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * fsq_decode_attn_timed - fsq_decode_attn that also records two caller-created
 * hipEvent_t (passed as void *) around the split-K kernel, the call's dominant
 * kernel, using hipExtLaunchKernelGGL: split_start when that kernel starts and
 * split_stop when it completes. For measurement; the results are identical to
 * fsq_decode_attn. Not for use under stream capture.
 * Errors: as fsq_decode_attn; FSQ_ERR_NULL if an event is NULL.
 */
int fsq_decode_attn_timed(const uint16_t *q, const uint8_t *codes, const uint16_t *W_kv,
                          const int32_t *seq_lens, uint16_t *out,
                          int32_t batch, int32_t n_q, int32_t n_kv, int32_t d_h, int32_t G,
                          int64_t seq_cap, void *workspace, size_t workspace_bytes,
                          void *stream, void *split_start, void *split_stop);

/*
 * fsq_decode_attn_levels_timed - fsq_decode_attn_levels with the split-K kernel
 * bracketed by two caller-created events, as fsq_decode_attn_timed (same
 * results as fsq_decode_attn_levels; not for use under stream capture).
 * Errors: as fsq_decode_attn_levels; FSQ_ERR_NULL if an event is NULL.
 */
int fsq_decode_attn_levels_timed(const uint16_t *q, const uint8_t *codes, const uint16_t *W_kv,
                                 const int32_t *seq_lens, uint16_t *out,
                                 int32_t batch, int32_t n_q, int32_t n_kv, int32_t d_h, int32_t G,
                                 int32_t levels, int64_t seq_cap, void *workspace,
                                 size_t workspace_bytes, void *stream, void *split_start,
                                 void *split_stop);

/*
 * fsq_decode_step - one decode step of one layer: append each sequence's new
 * token to its cache, then attend over the cache including that token.
 *
 * The caller has already counted the new token in seq_lens. For every sequence
 * b with 1 <= seq_lens[b] <= seq_cap, row seq_lens[b] - 1 of codes[b] is set to
 * the packed codes of Q_FSQ(E x_new[b]) (Eq. 4 with the Eq. 2 forward value, as
 * fsq_append); sequences with seq_lens[b] outside that range get no append.
 * Then out is computed exactly as by fsq_decode_attn. The results are
 * bit-identical to fsq_append of each new row (one token per call) followed by
 * fsq_decode_attn with the same arguments; the difference is that the append
 * and the query absorption share one kernel launch.
 *   x_new    [batch, C]   bf16, 16-byte aligned: the new token of each sequence.
 *   E        [G, C]       bf16, 16-byte aligned.
 *   codes    [batch, seq_cap, ceil(G/2)] u8, 16-byte aligned; read, and row
 *                          seq_lens[b] - 1 of each sequence written (the bytes
 *                          up to the next 16-byte boundary after its end must be
 *                          readable, as for fsq_decode_attn).
 *   q, W_kv, seq_lens, out, workspace: as fsq_decode_attn (workspace size from
 *                          fsq_decode_workspace_bytes(batch, n_q, G, seq_cap)).
 * Sizes: as fsq_decode_attn, and C >= 1 with C % 8 == 0.
 * Errors: as fsq_decode_attn; also FSQ_ERR_SHAPE (C < 1), FSQ_ERR_NULL (x_new
 *         or E NULL), FSQ_ERR_UNSUPPORTED (C % 8 != 0, x_new or E not 16-byte
 *         aligned).
 */
int fsq_decode_step(const uint16_t *x_new, const uint16_t *E, const uint16_t *q, uint8_t *codes,
                    const uint16_t *W_kv, const int32_t *seq_lens, uint16_t *out,
                    int32_t batch, int32_t C, int32_t n_q, int32_t n_kv, int32_t d_h, int32_t G,
                    int64_t seq_cap, void *workspace, size_t workspace_bytes, void *stream);

/*
 * fsq_decode_step_levels - fsq_decode_step for L = levels per coordinate (4,
 * 16 or 256: 2-, 4- or 8-bit codes, rows of ceil(G b / 8) bytes; the slides'
 * backup frame "the grid size is an allocation choice"). The append of each
 * new token is fsq_append_levels' and the attention fsq_decode_attn_levels';
 * the results are bit-identical to those two calls. fsq_decode_step is
 * fsq_decode_step_levels with levels = 16.
 * Errors: as fsq_decode_step; FSQ_ERR_UNSUPPORTED for another number of levels.
 */
int fsq_decode_step_levels(const uint16_t *x_new, const uint16_t *E, const uint16_t *q, uint8_t *codes,
                           const uint16_t *W_kv, const int32_t *seq_lens, uint16_t *out, int32_t batch,
                           int32_t C, int32_t n_q, int32_t n_kv, int32_t d_h, int32_t G, int32_t levels,
                           int64_t seq_cap, void *workspace, size_t workspace_bytes, void *stream);

/*
 * fsq_decode_attn_recon - the same attention as fsq_decode_attn, computed the
 * way the pages' kernel does: keys are rebuilt per 32-token tile on chip,
 * K_tile = Z_tile W_k,g^T (Eq. 5 without key norm and RoPE), and scored against
 * q; values are still pooled in latent space and decoded once (Eq. 6). Kept as
 * a measured comparison of the absorbed path (about 2 n_kv d_h G flops per
 * token for the keys instead of 2 n_q G); nothing is written to memory but the
 * workspace and out. Same arguments, layouts and workspace size as
 * fsq_decode_attn; results agree with it to fp16 rounding, not bit for bit.
 * Sizes: as fsq_decode_attn, and d_h % 32 == 0, d_h <= 128, n_q / n_kv <= 32.
 * Errors: as fsq_decode_attn; FSQ_ERR_UNSUPPORTED for the further size limits.
 */
int fsq_decode_attn_recon(const uint16_t *q, const uint8_t *codes, const uint16_t *W_kv,
                          const int32_t *seq_lens, uint16_t *out,
                          int32_t batch, int32_t n_q, int32_t n_kv, int32_t d_h, int32_t G,
                          int64_t seq_cap, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * fsq_decode_attn_rope - one decode step with the keys of Eq. 5 in full,
 * k^_t = RoPE_t(N_k(W_k,g z_t)), rebuilt per 32-token tile on chip (absorbing
 * the query is not possible here: N_k is nonlinear and RoPE_t depends on t);
 * values are pooled in latent space and decoded once (Eq. 6):
 *   N_k(k)     = k * gamma / sqrt(mean_i k_i^2 + norm_eps)   (per key head)
 *   RoPE_t(k)  : for i < d_h/2, with a = t * rope_theta^(-2i/d_h),
 *                (k_i, k_{i+d_h/2}) -> (k_i cos a - k_{i+d_h/2} sin a,
 *                                        k_{i+d_h/2} cos a + k_i sin a),
 *                t = the key's 0-based position in the cache;
 *   s_t = q . k^_t / sqrt(d_h), softmax over t < seq_lens[b], out = W_v,g sum p z.
 * The pages fix neither gamma, eps nor theta, nor the RoPE pairing (these are
 * the conventions of the Qwen3 models the pages evaluate). q is taken as
 * already normalised and rotated at its own position.
 *   k_norm   [d_h]  bf16 (gamma, shared by the kv heads).
 *   the other arguments, layouts and the workspace as fsq_decode_attn.
 * Sizes: as fsq_decode_attn, and d_h in {64, 128}, n_q / n_kv <= 32,
 *        1 < rope_theta < 1e30, 0 <= norm_eps < 1.
 * Errors: as fsq_decode_attn; FSQ_ERR_NULL (k_norm NULL), FSQ_ERR_SHAPE
 *         (rope_theta or norm_eps out of range), FSQ_ERR_UNSUPPORTED (d_h).
 */
int fsq_decode_attn_rope(const uint16_t *q, const uint8_t *codes, const uint16_t *W_kv,
                         const uint16_t *k_norm, const int32_t *seq_lens, uint16_t *out,
                         int32_t batch, int32_t n_q, int32_t n_kv, int32_t d_h, int32_t G,
                         int64_t seq_cap, float rope_theta, float norm_eps, void *workspace,
                         size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FSQ_H */
