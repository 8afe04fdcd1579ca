// C ABI of the library (declared in include/fsq.h): validation (validate.h,
// host arithmetic only), workspace sizing and launches on the caller's stream.
// No device memory is allocated here.
#include "../../include/fsq.h"
#include "common.h"
#include "decode_plan.h"
#include "validate.h"

#include <mutex>

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

// Scratch memory of fsq_decode_attn_noalloc: the decode workspace (absorbed
// queries, split partials) of callers that cannot allocate. A file-scope
// device array, one copy per GPU the library is loaded on, kept until the
// process ends. Host code never uses the array's name as an address (on the
// host it names a stand-in, not device memory): the device address of each
// GPU's copy comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that pointer is passed to kernels.
static_assert(FSQ_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[FSQ_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on its first use); nullptr
// if the device cannot be queried or its copy not located.
void *device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}
}  // namespace

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
    const int v = fsq::validate_append(x, E, codes, n_tokens, C, G, levels);
    if (v != FSQ_OK || n_tokens == 0) return v;
    hipError_t e = fsq::launch_append(x, E, codes, n_tokens, C, G, levels, (hipStream_t)stream);
    return e == hipSuccess ? FSQ_OK : FSQ_ERR_HIP;
}

int fsq_append(const uint16_t *x, const uint16_t *E, uint8_t *codes, int64_t n_tokens, int32_t C,
               int32_t G, void *stream) {
    return fsq_append_levels(x, E, codes, n_tokens, C, G, 16, stream);
}

int fsq_decode_plan_info(int32_t batch, int32_t n_q, int32_t G, int64_t seq_cap, int32_t *kernel,
                         int32_t *splits, int64_t *chunk) {
    if (!fsq::decode_sizes_ok(batch, n_q, G, seq_cap)) return FSQ_ERR_SHAPE;
    if (!kernel || !splits || !chunk) return FSQ_ERR_NULL;
    const fsq::DecodePlan pl = fsq::make_decode_plan(batch, n_q, G, seq_cap);
    *kernel = pl.stream ? (pl.dyn ? 2 : 1) : 0;
    *splits = pl.S;
    *chunk = pl.chunk;
    return FSQ_OK;
}

size_t fsq_decode_workspace_bytes(int32_t batch, int32_t n_q, int32_t G, int64_t seq_cap) {
    if (!fsq::decode_sizes_ok(batch, n_q, G, seq_cap)) return 0;
    return fsq::make_decode_plan(batch, n_q, G, seq_cap).total;
}

static int decode_common(const uint16_t *q, const uint8_t *codes, const uint16_t *W_kv,
                         const int32_t *seq_lens, uint16_t *out, int32_t batch, int32_t n_q,
                         int32_t n_kv, int32_t d_h, int32_t G, int64_t seq_cap, void *workspace,
                         size_t workspace_bytes, void *stream, void *ev0, void *ev1,
                         const uint16_t *x_new = nullptr, const uint16_t *E = nullptr, int32_t C = 0,
                         int32_t levels = 16) {
    fsq::DecodePlan pl;
    const int v = fsq::validate_decode(q, codes, W_kv, seq_lens, out, batch, n_q, n_kv, d_h, G, seq_cap,
                                       workspace, workspace_bytes, levels, &pl);
    if (v != FSQ_OK) return v;
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

int fsq_decode_attn_noalloc(const uint16_t *q, const uint8_t *codes, const uint16_t *W_kv,
                            const int32_t *seq_lens, uint16_t *out, int32_t batch, int32_t n_q,
                            int32_t n_kv, int32_t d_h, int32_t G, int64_t seq_cap, void *stream) {
    // sizes first (as fsq_decode_attn would check them), then the scratch
    // capacity, and only then the device's scratch address: an invalid or
    // oversized call touches no HIP state
    size_t need = 0;
    const int v = fsq::validate_decode_args(q, codes, W_kv, seq_lens, out, batch, n_q, n_kv, d_h, G, seq_cap,
                                            16, nullptr, &need);
    if (v != FSQ_OK) return v;
    if (need > (size_t)FSQ_NOALLOC_SCRATCH_BYTES) return FSQ_ERR_WORKSPACE;
    void *ws = device_scratch();
    if (!ws) return FSQ_ERR_HIP;
    return decode_common(q, codes, W_kv, seq_lens, out, batch, n_q, n_kv, d_h, G, seq_cap, ws,
                         FSQ_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr);
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
    const int v = fsq::validate_step_append(x_new, E, batch, C, n_q, n_kv, d_h, G, seq_cap);
    if (v != FSQ_OK) return v;
    return decode_common(q, codes, W_kv, seq_lens, out, batch, n_q, n_kv, d_h, G, seq_cap, workspace,
                         workspace_bytes, stream, nullptr, nullptr, x_new, E, C);
}

int fsq_decode_step_levels(const uint16_t *x_new, const uint16_t *E, const uint16_t *q, uint8_t *codes,
                           const uint16_t *W_kv, const int32_t *seq_lens, uint16_t *out, int32_t batch,
                           int32_t C, int32_t n_q, int32_t n_kv, int32_t d_h, int32_t G, int32_t levels,
                           int64_t seq_cap, void *workspace, size_t workspace_bytes, void *stream) {
    const int v = fsq::validate_step_append(x_new, E, batch, C, n_q, n_kv, d_h, G, seq_cap);
    if (v != FSQ_OK) return v;
    return decode_common(q, codes, W_kv, seq_lens, out, batch, n_q, n_kv, d_h, G, seq_cap, workspace,
                         workspace_bytes, stream, nullptr, nullptr, x_new, E, C, levels);
}

static int recon_common(const uint16_t *q, const uint8_t *codes, const uint16_t *W_kv,
                        const int32_t *seq_lens, uint16_t *out, int32_t batch, int32_t n_q,
                        int32_t n_kv, int32_t d_h, int32_t G, int64_t seq_cap, void *workspace,
                        size_t workspace_bytes, void *stream, const uint16_t *gamma, float eps,
                        float theta) {
    fsq::DecodePlan pl;
    const int v = fsq::validate_recon(q, codes, W_kv, seq_lens, out, batch, n_q, n_kv, d_h, G, seq_cap,
                                      workspace, workspace_bytes, &pl);
    if (v != FSQ_OK) return v;
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
    const int v = fsq::validate_rope_extra(k_norm, batch, n_q, n_kv, d_h, G, seq_cap, rope_theta, norm_eps);
    if (v != FSQ_OK) return v;
    return recon_common(q, codes, W_kv, seq_lens, out, batch, n_q, n_kv, d_h, G, seq_cap, workspace,
                        workspace_bytes, stream, k_norm, norm_eps, rope_theta);
}

}  // extern "C"
