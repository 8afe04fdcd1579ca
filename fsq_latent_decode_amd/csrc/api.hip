// C ABI of the library (declared in include/fsq.h): validation, workspace
// sizing and launches on the caller's stream. No device memory is allocated here.
#include "../../include/fsq.h"
#include "common.h"
#include "decode_plan.h"

namespace fsq {
hipError_t launch_append(const uint16_t *x, const uint16_t *E, uint8_t *codes, int64_t n, int C,
                         int G, int levels, hipStream_t st);
hipError_t launch_decode(const DecodePlan &pl, const uint16_t *q, const uint8_t *codes,
                         const uint16_t *W_kv, const int32_t *seq_lens, uint16_t *out, int batch,
                         int n_q, int n_kv, int d_h, int G, int64_t seq_cap, void *workspace,
                         hipStream_t st, hipEvent_t ev0, hipEvent_t ev1, const uint16_t *x_new,
                         const uint16_t *E, int C, int levels);
hipError_t launch_decode_recon(const DecodePlan &pl, const uint16_t *q, const uint8_t *codes,
                               const uint16_t *W_kv, const int32_t *seq_lens, uint16_t *out,
                               int batch, int n_q, int n_kv, int d_h, int G, int64_t seq_cap,
                               void *workspace, hipStream_t st, const uint16_t *gamma, float eps,
                               float theta);
}  // namespace fsq

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
static bool levels_ok(int levels) { return levels == 4 || levels == 16 || levels == 256; }

extern "C" {

const char *fsq_status_string(int status) {
    switch (status) {
        case FSQ_OK: return "FSQ_OK";
        case FSQ_ERR_NULL: return "FSQ_ERR_NULL";
        case FSQ_ERR_SHAPE: return "FSQ_ERR_SHAPE";
        case FSQ_ERR_UNSUPPORTED: return "FSQ_ERR_UNSUPPORTED";
        case FSQ_ERR_WORKSPACE: return "FSQ_ERR_WORKSPACE";
        case FSQ_ERR_HIP: return "FSQ_ERR_HIP";
        default: return "FSQ_UNKNOWN";
    }
}

int fsq_append_levels(const uint16_t *x, const uint16_t *E, uint8_t *codes, int64_t n_tokens,
                      int32_t C, int32_t G, int32_t levels, void *stream) {
    if (n_tokens < 0 || C < 1 || G < 1) return FSQ_ERR_SHAPE;
    if (G > FSQ_MAX_G || C % 8 != 0 || !levels_ok(levels)) return FSQ_ERR_UNSUPPORTED;
    if (n_tokens == 0) return FSQ_OK;
    if (!x || !E || !codes) return FSQ_ERR_NULL;
    if (!aligned16(x) || !aligned16(E)) return FSQ_ERR_UNSUPPORTED;
    if (n_tokens > ((int64_t)1 << 31) * 32) return FSQ_ERR_UNSUPPORTED;
    hipError_t e = fsq::launch_append(x, E, codes, n_tokens, C, G, levels, (hipStream_t)stream);
    return e == hipSuccess ? FSQ_OK : FSQ_ERR_HIP;
}

int fsq_append(const uint16_t *x, const uint16_t *E, uint8_t *codes, int64_t n_tokens, int32_t C,
               int32_t G, void *stream) {
    return fsq_append_levels(x, E, codes, n_tokens, C, G, 16, stream);
}

int fsq_decode_plan_info(int32_t batch, int32_t n_q, int32_t G, int64_t seq_cap, int32_t *kernel,
                         int32_t *splits, int64_t *chunk) {
    if (batch < 1 || n_q < 1 || n_q > FSQ_MAX_NQ || G < 1 || G > FSQ_MAX_G || seq_cap < 0) return FSQ_ERR_SHAPE;
    if (!kernel || !splits || !chunk) return FSQ_ERR_NULL;
    const fsq::DecodePlan pl = fsq::make_decode_plan(batch, n_q, G, seq_cap);
    *kernel = pl.stream ? (pl.dyn ? 2 : 1) : 0;
    *splits = pl.S;
    *chunk = pl.chunk;
    return FSQ_OK;
}

size_t fsq_decode_workspace_bytes(int32_t batch, int32_t n_q, int32_t G, int64_t seq_cap) {
    if (batch < 1 || n_q < 1 || n_q > FSQ_MAX_NQ || G < 1 || G > FSQ_MAX_G || seq_cap < 0) return 0;
    return fsq::make_decode_plan(batch, n_q, G, seq_cap).total;
}

static int decode_common(const uint16_t *q, const uint8_t *codes, const uint16_t *W_kv,
                         const int32_t *seq_lens, uint16_t *out, int32_t batch, int32_t n_q,
                         int32_t n_kv, int32_t d_h, int32_t G, int64_t seq_cap, void *workspace,
                         size_t workspace_bytes, void *stream, void *ev0, void *ev1,
                         const uint16_t *x_new = nullptr, const uint16_t *E = nullptr, int32_t C = 0,
                         int32_t levels = 16) {
    if (batch < 1 || n_q < 1 || n_kv < 1 || d_h < 1 || G < 1 || seq_cap < 0) return FSQ_ERR_SHAPE;
    if (n_q % n_kv != 0) return FSQ_ERR_SHAPE;
    if (n_q > FSQ_MAX_NQ || G > FSQ_MAX_G || d_h > FSQ_MAX_DH || !levels_ok(levels))
        return FSQ_ERR_UNSUPPORTED;
    if (!q || !W_kv || !seq_lens || !out || (!codes && seq_cap > 0)) return FSQ_ERR_NULL;
    if (seq_cap > 0 && !aligned16(codes)) return FSQ_ERR_UNSUPPORTED;
    if ((int64_t)batch * seq_cap > ((int64_t)1 << 40)) return FSQ_ERR_UNSUPPORTED;
    const fsq::DecodePlan pl = fsq::make_decode_plan(batch, n_q, G, seq_cap, levels == 16);
    if (!workspace || workspace_bytes < fsq::make_decode_plan(batch, n_q, G, seq_cap).total ||
        ((uintptr_t)workspace & 255u))
        return FSQ_ERR_WORKSPACE;
    // the merge kernel reduces at most 1024 splits (the plan gives <= 512 / batch + 1)
    if (pl.S > 1024 || batch > 65535) return FSQ_ERR_UNSUPPORTED;
    hipError_t e = fsq::launch_decode(pl, q, codes, W_kv, seq_lens, out, batch, n_q, n_kv, d_h, G,
                                      seq_cap, workspace, (hipStream_t)stream, (hipEvent_t)ev0,
                                      (hipEvent_t)ev1, x_new, E, C, levels);
    return e == hipSuccess ? FSQ_OK : FSQ_ERR_HIP;
}

int fsq_decode_attn(const uint16_t *q, const uint8_t *codes, const uint16_t *W_kv,
                    const int32_t *seq_lens, uint16_t *out, int32_t batch, int32_t n_q,
                    int32_t n_kv, int32_t d_h, int32_t G, int64_t seq_cap, void *workspace,
                    size_t workspace_bytes, void *stream) {
    return decode_common(q, codes, W_kv, seq_lens, out, batch, n_q, n_kv, d_h, G, seq_cap,
                         workspace, workspace_bytes, stream, nullptr, nullptr);
}

int fsq_decode_attn_levels(const uint16_t *q, const uint8_t *codes, const uint16_t *W_kv,
                           const int32_t *seq_lens, uint16_t *out, int32_t batch, int32_t n_q,
                           int32_t n_kv, int32_t d_h, int32_t G, int32_t levels, int64_t seq_cap,
                           void *workspace, size_t workspace_bytes, void *stream) {
    return decode_common(q, codes, W_kv, seq_lens, out, batch, n_q, n_kv, d_h, G, seq_cap,
                         workspace, workspace_bytes, stream, nullptr, nullptr, nullptr, nullptr, 0,
                         levels);
}

int fsq_decode_attn_levels_timed(const uint16_t *q, const uint8_t *codes, const uint16_t *W_kv,
                                 const int32_t *seq_lens, uint16_t *out, int32_t batch, int32_t n_q,
                                 int32_t n_kv, int32_t d_h, int32_t G, int32_t levels, int64_t seq_cap,
                                 void *workspace, size_t workspace_bytes, void *stream, void *split_start,
                                 void *split_stop) {
    if (!split_start || !split_stop) return FSQ_ERR_NULL;
    return decode_common(q, codes, W_kv, seq_lens, out, batch, n_q, n_kv, d_h, G, seq_cap,
                         workspace, workspace_bytes, stream, split_start, split_stop, nullptr, nullptr, 0,
                         levels);
}

int fsq_decode_attn_timed(const uint16_t *q, const uint8_t *codes, const uint16_t *W_kv,
                          const int32_t *seq_lens, uint16_t *out, int32_t batch, int32_t n_q,
                          int32_t n_kv, int32_t d_h, int32_t G, int64_t seq_cap, void *workspace,
                          size_t workspace_bytes, void *stream, void *split_start,
                          void *split_stop) {
    if (!split_start || !split_stop) return FSQ_ERR_NULL;
    return decode_common(q, codes, W_kv, seq_lens, out, batch, n_q, n_kv, d_h, G, seq_cap,
                         workspace, workspace_bytes, stream, split_start, split_stop);
}

int fsq_decode_step(const uint16_t *x_new, const uint16_t *E, const uint16_t *q, uint8_t *codes,
                    const uint16_t *W_kv, const int32_t *seq_lens, uint16_t *out, int32_t batch,
                    int32_t C, int32_t n_q, int32_t n_kv, int32_t d_h, int32_t G, int64_t seq_cap,
                    void *workspace, size_t workspace_bytes, void *stream) {
    if (C < 1) return FSQ_ERR_SHAPE;
    if (batch >= 1 && n_q >= 1 && n_kv >= 1 && d_h >= 1 && G >= 1 && seq_cap >= 0) {
        if (C % 8 != 0) return FSQ_ERR_UNSUPPORTED;
        if (!x_new || !E) return FSQ_ERR_NULL;
        if (!aligned16(x_new) || !aligned16(E)) return FSQ_ERR_UNSUPPORTED;
    }
    return decode_common(q, codes, W_kv, seq_lens, out, batch, n_q, n_kv, d_h, G, seq_cap, workspace,
                         workspace_bytes, stream, nullptr, nullptr, x_new, E, C);
}

static int recon_common(const uint16_t *q, const uint8_t *codes, const uint16_t *W_kv,
                        const int32_t *seq_lens, uint16_t *out, int32_t batch, int32_t n_q,
                        int32_t n_kv, int32_t d_h, int32_t G, int64_t seq_cap, void *workspace,
                        size_t workspace_bytes, void *stream, const uint16_t *gamma, float eps,
                        float theta) {
    if (batch < 1 || n_q < 1 || n_kv < 1 || d_h < 1 || G < 1 || seq_cap < 0) return FSQ_ERR_SHAPE;
    if (n_q % n_kv != 0) return FSQ_ERR_SHAPE;
    if (n_q > FSQ_MAX_NQ || G > FSQ_MAX_G || d_h > 128 || d_h % 32 != 0 || n_q / n_kv > 32)
        return FSQ_ERR_UNSUPPORTED;
    if (!q || !W_kv || !seq_lens || !out || (!codes && seq_cap > 0)) return FSQ_ERR_NULL;
    if (seq_cap > 0 && !aligned16(codes)) return FSQ_ERR_UNSUPPORTED;
    if ((int64_t)batch * seq_cap > ((int64_t)1 << 40)) return FSQ_ERR_UNSUPPORTED;
    const fsq::DecodePlan pl = fsq::make_decode_plan(batch, n_q, G, seq_cap);
    if (!workspace || workspace_bytes < pl.total || ((uintptr_t)workspace & 255u))
        return FSQ_ERR_WORKSPACE;
    if (pl.S > 1024 || batch > 65535) return FSQ_ERR_UNSUPPORTED;
    hipError_t e = fsq::launch_decode_recon(pl, q, codes, W_kv, seq_lens, out, batch, n_q, n_kv, d_h,
                                            G, seq_cap, workspace, (hipStream_t)stream, gamma, eps,
                                            theta);
    return e == hipSuccess ? FSQ_OK : FSQ_ERR_HIP;
}

int fsq_decode_attn_recon(const uint16_t *q, const uint8_t *codes, const uint16_t *W_kv,
                          const int32_t *seq_lens, uint16_t *out, int32_t batch, int32_t n_q,
                          int32_t n_kv, int32_t d_h, int32_t G, int64_t seq_cap, void *workspace,
                          size_t workspace_bytes, void *stream) {
    return recon_common(q, codes, W_kv, seq_lens, out, batch, n_q, n_kv, d_h, G, seq_cap, workspace,
                        workspace_bytes, stream, nullptr, 0.0f, 0.0f);
}

int fsq_decode_attn_rope(const uint16_t *q, const uint8_t *codes, const uint16_t *W_kv,
                         const uint16_t *k_norm, const int32_t *seq_lens, uint16_t *out,
                         int32_t batch, int32_t n_q, int32_t n_kv, int32_t d_h, int32_t G,
                         int64_t seq_cap, float rope_theta, float norm_eps, void *workspace,
                         size_t workspace_bytes, void *stream) {
    if (batch < 1 || n_q < 1 || n_kv < 1 || d_h < 1 || G < 1 || seq_cap < 0) return FSQ_ERR_SHAPE;
    if (!(rope_theta > 1.0f) || !(norm_eps >= 0.0f) || !(rope_theta < 1e30f) || !(norm_eps < 1.0f))
        return FSQ_ERR_SHAPE;
    if (d_h != 64 && d_h != 128) return FSQ_ERR_UNSUPPORTED;
    if (!k_norm) return FSQ_ERR_NULL;
    return recon_common(q, codes, W_kv, seq_lens, out, batch, n_q, n_kv, d_h, G, seq_cap, workspace,
                        workspace_bytes, stream, k_norm, norm_eps, rope_theta);
}

}  // extern "C"
