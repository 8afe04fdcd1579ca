// Argument validation of the C ABI (include/fsq.h): pure host arithmetic on
// sizes, pointer values and alignment, with no HIP call, so that every check
// runs before anything is enqueued and the same code can be built and
// exercised on the CPU alone (under address and undefined-behaviour
// sanitizers) by the host test in tests/host/.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/fsq.h"
#include "decode_plan.h"

namespace fsq {

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline bool levels_ok(int levels) { return levels == 4 || levels == 16 || levels == 256; }

// fsq_append / fsq_append_levels. FSQ_OK with n_tokens == 0 means "nothing to
// enqueue" (the caller checks n_tokens).
inline int validate_append(const void *x, const void *E, const void *codes, int64_t n_tokens, int32_t C,
                           int32_t G, int32_t levels) {
    if (n_tokens < 0 || C < 1 || G < 1) return FSQ_ERR_SHAPE;
    if (G > FSQ_MAX_G || C % 8 != 0 || !levels_ok(levels)) return FSQ_ERR_UNSUPPORTED;
    if (n_tokens == 0) return FSQ_OK;
    if (!x || !E || !codes) return FSQ_ERR_NULL;
    if (!aligned16(x) || !aligned16(E)) return FSQ_ERR_UNSUPPORTED;
    if (n_tokens > ((int64_t)1 << 31) * 32) return FSQ_ERR_UNSUPPORTED;
    return FSQ_OK;
}

// batch x seq_cap tokens at most 2^40 (the kernels index a cache of up to 2^40
// rows); checked by division so that the product is never formed when it
// could overflow. Needs batch >= 1 and seq_cap >= 0.
constexpr int64_t kMaxCacheRows = (int64_t)1 << 40;
inline bool cache_rows_ok(int32_t batch, int64_t seq_cap) { return seq_cap <= kMaxCacheRows / batch; }

// Sizes shared by the workspace query, the plan query and the decode calls.
inline bool decode_sizes_ok(int32_t batch, int32_t n_q, int32_t G, int64_t seq_cap) {
    return batch >= 1 && n_q >= 1 && n_q <= FSQ_MAX_NQ && G >= 1 && G <= FSQ_MAX_G && seq_cap >= 0 &&
           cache_rows_ok(batch, seq_cap);
}

// Everything fsq_decode_attn checks except the workspace: on FSQ_OK *plan is
// the plan the launch uses and *ws_need the workspace bytes it needs.
inline int validate_decode_args(const void *q, const void *codes, const void *W_kv, const void *seq_lens,
                                const void *out, int32_t batch, int32_t n_q, int32_t n_kv, int32_t d_h,
                                int32_t G, int64_t seq_cap, int32_t levels, DecodePlan *plan, size_t *ws_need) {
    if (batch < 1 || n_q < 1 || n_kv < 1 || d_h < 1 || G < 1 || seq_cap < 0) return FSQ_ERR_SHAPE;
    if (n_q % n_kv != 0) return FSQ_ERR_SHAPE;
    if (n_q > FSQ_MAX_NQ || G > FSQ_MAX_G || d_h > FSQ_MAX_DH || !levels_ok(levels))
        return FSQ_ERR_UNSUPPORTED;
    if (!q || !W_kv || !seq_lens || !out || (!codes && seq_cap > 0)) return FSQ_ERR_NULL;
    if (seq_cap > 0 && !aligned16(codes)) return FSQ_ERR_UNSUPPORTED;
    if (!cache_rows_ok(batch, seq_cap)) return FSQ_ERR_UNSUPPORTED;
    const DecodePlan pl = make_decode_plan(batch, n_q, G, seq_cap, levels == 16);
    // the merge kernel reduces at most 1024 splits (the plan gives <= 512 / batch + 1)
    if (pl.S > 1024 || batch > 65535) return FSQ_ERR_UNSUPPORTED;
    if (plan) *plan = pl;
    // the workspace size does not depend on the code width (fsq_decode_workspace_bytes)
    if (ws_need) *ws_need = make_decode_plan(batch, n_q, G, seq_cap).total;
    return FSQ_OK;
}

// fsq_decode_attn, _levels, _timed and (with x_new, E, C) fsq_decode_step: on
// FSQ_OK *plan is the plan the launch uses.
inline int validate_decode(const void *q, const void *codes, const void *W_kv, const void *seq_lens,
                           const void *out, int32_t batch, int32_t n_q, int32_t n_kv, int32_t d_h,
                           int32_t G, int64_t seq_cap, const void *workspace, size_t workspace_bytes,
                           int32_t levels, DecodePlan *plan) {
    size_t need = 0;
    const int v = validate_decode_args(q, codes, W_kv, seq_lens, out, batch, n_q, n_kv, d_h, G, seq_cap, levels,
                                       plan, &need);
    if (v != FSQ_OK) return v;
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)) return FSQ_ERR_WORKSPACE;
    return FSQ_OK;
}

// The extra arguments of fsq_decode_step (checked first, as the call does).
inline int validate_step_append(const void *x_new, const void *E, int32_t batch, int32_t C, int32_t n_q,
                                int32_t n_kv, int32_t d_h, int32_t G, int64_t seq_cap) {
    if (C < 1) return FSQ_ERR_SHAPE;
    if (batch >= 1 && n_q >= 1 && n_kv >= 1 && d_h >= 1 && G >= 1 && seq_cap >= 0) {
        if (C % 8 != 0) return FSQ_ERR_UNSUPPORTED;
        if (!x_new || !E) return FSQ_ERR_NULL;
        if (!aligned16(x_new) || !aligned16(E)) return FSQ_ERR_UNSUPPORTED;
    }
    return FSQ_OK;
}

// fsq_decode_attn_recon and (after validate_rope_extra) fsq_decode_attn_rope.
inline int validate_recon(const void *q, const void *codes, const void *W_kv, const void *seq_lens,
                          const void *out, int32_t batch, int32_t n_q, int32_t n_kv, int32_t d_h, int32_t G,
                          int64_t seq_cap, const void *workspace, size_t workspace_bytes, DecodePlan *plan) {
    if (batch < 1 || n_q < 1 || n_kv < 1 || d_h < 1 || G < 1 || seq_cap < 0) return FSQ_ERR_SHAPE;
    if (n_q % n_kv != 0) return FSQ_ERR_SHAPE;
    if (n_q > FSQ_MAX_NQ || G > FSQ_MAX_G || d_h > 128 || d_h % 32 != 0 || n_q / n_kv > 32)
        return FSQ_ERR_UNSUPPORTED;
    if (!q || !W_kv || !seq_lens || !out || (!codes && seq_cap > 0)) return FSQ_ERR_NULL;
    if (seq_cap > 0 && !aligned16(codes)) return FSQ_ERR_UNSUPPORTED;
    if (!cache_rows_ok(batch, seq_cap)) return FSQ_ERR_UNSUPPORTED;
    const DecodePlan pl = make_decode_plan(batch, n_q, G, seq_cap);
    if (!workspace || workspace_bytes < pl.total || ((uintptr_t)workspace & 255u)) return FSQ_ERR_WORKSPACE;
    if (pl.S > 1024 || batch > 65535) return FSQ_ERR_UNSUPPORTED;
    if (plan) *plan = pl;
    return FSQ_OK;
}

inline int validate_rope_extra(const void *k_norm, int32_t batch, int32_t n_q, int32_t n_kv, int32_t d_h,
                               int32_t G, int64_t seq_cap, float rope_theta, float norm_eps) {
    if (batch < 1 || n_q < 1 || n_kv < 1 || d_h < 1 || G < 1 || seq_cap < 0) return FSQ_ERR_SHAPE;
    if (!(rope_theta > 1.0f) || !(norm_eps >= 0.0f) || !(rope_theta < 1e30f) || !(norm_eps < 1.0f))
        return FSQ_ERR_SHAPE;
    if (d_h != 64 && d_h != 128) return FSQ_ERR_UNSUPPORTED;
    if (!k_norm) return FSQ_ERR_NULL;
    return FSQ_OK;
}

}  // namespace fsq
