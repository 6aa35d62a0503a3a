// C ABI of the routed-attention library: host-side validation, error reporting, launches.
// Nothing here allocates memory or synchronises with the device.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "common.h"
#include "cold_kernels.h"
#include "decode_append.h"
#include "kernels.h"
#include "snapshot_kernels.h"

namespace {

thread_local char g_err[512] = "";

ra_status fail(ra_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

ra_status ok() {
    g_err[0] = 0;
    return RA_OK;
}

ra_status hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(RA_EHIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

constexpr int64_t kMaxGrid = 0x7fffffffLL;
constexpr int64_t kMaxItems = 1LL << 32;  // work-items (blocks x threads) per grid dimension

ra_status check_config(const ra_config *c) {
    if (!c) return fail(RA_EINVAL, "cfg is NULL");
    if (c->num_q_heads < 1 || c->num_kv_heads < 1) return fail(RA_EINVAL, "head counts must be >= 1");
    if (c->num_q_heads % c->num_kv_heads) return fail(RA_EINVAL, "num_q_heads must be a multiple of num_kv_heads");
    if (c->num_q_heads / c->num_kv_heads > 32) return fail(RA_EUNSUPPORTED, "more than 32 query heads per kv head");
    if (c->head_dim != 64 && c->head_dim != 128) return fail(RA_EUNSUPPORTED, "head_dim must be 64 or 128");
    if (c->dtype != RA_F32 && c->dtype != RA_BF16) return fail(RA_EUNSUPPORTED, "dtype must be RA_F32 or RA_BF16");
    if (c->span_size < 1) return fail(RA_EINVAL, "span_size must be >= 1");
    if (c->window < 1) return fail(RA_EINVAL, "window must be >= 1");
    if (c->top_k < 1) return fail(RA_EINVAL, "top_k must be >= 1");
    if (c->top_k > 64) return fail(RA_EUNSUPPORTED, "top_k must be <= 64");
    if (c->batch < 1) return fail(RA_EINVAL, "batch must be >= 1");
    if (c->capacity < 1) return fail(RA_EINVAL, "capacity must be >= 1");
    if (c->capacity >= (1LL << 40)) return fail(RA_EUNSUPPORTED, "capacity must be < 2^40 tokens");
    if (c->max_spans < c->capacity / c->span_size)
        return fail(RA_ECAPACITY, "max_spans (%lld) < capacity / span_size (%lld)", (long long)c->max_spans,
                    (long long)(c->capacity / c->span_size));
    return RA_OK;
}

ra_status check_rows(const ra_config *c, const ra_rows *r) {
    if (!r) return fail(RA_EINVAL, "rows is NULL");
    if (r->n_rows < 0) return fail(RA_EINVAL, "n_rows must be >= 0");
    if (r->n_rows > 0 && (!r->q || !r->row_seq || !r->row_pos)) return fail(RA_EINVAL, "rows has a NULL pointer");
    if (r->max_pos < 0 || r->max_pos >= c->capacity)
        return fail(RA_ECAPACITY, "max_pos (%lld) must be in [0, capacity=%lld)", (long long)r->max_pos,
                    (long long)c->capacity);
    if (r->n_rows * (int64_t)c->num_q_heads >= kMaxGrid) return fail(RA_EUNSUPPORTED, "too many rows");
    return RA_OK;
}

ra::RowArgs row_args(const ra_config *c, const ra_rows *r) {
    ra::RowArgs a;
    a.q = r->q;
    a.row_seq = r->row_seq;
    a.row_pos = r->row_pos;
    a.n_rows = r->n_rows;
    a.max_pos = r->max_pos;
    a.dtype = c->dtype;
    a.d = c->head_dim;
    a.Hq = c->num_q_heads;
    a.Hkv = c->num_kv_heads;
    a.G = c->num_q_heads / c->num_kv_heads;
    a.S = c->span_size;
    a.k = c->top_k;
    a.W = c->window;
    a.B = c->batch;
    a.cap = c->capacity;
    a.max_spans = c->max_spans;
    return a;
}

ra_status check_attn(const ra_config *c, const ra_rows *r, const void *k, const void *v, const int32_t *sel,
                     const float *out, const void *ws, size_t ws_bytes, int op, bool fp8 = false) {
    ra_status s = check_config(c);
    if (s) return s;
    if ((s = check_rows(c, r))) return s;
    if (r->n_rows > 0 && (!k || !v || !sel || !out)) return fail(RA_EINVAL, "NULL K, V, sel or out");
    const ra::RowArgs a = row_args(c, r);
    const int NW = ra::max_window_spans(a.S, a.W);
    if (op == RA_OP_DECODE) {
        // (a bound in double first, so that the exact count below stays far inside int64)
        if ((double)a.n_rows * a.Hkv * (double)(a.G * a.k + NW) * (double)a.S >= 0x1p52)
            return fail(RA_EUNSUPPORTED, "decode grid too large: use fewer rows per call");
        if (ra::decode_grid_items(a, fp8) >= kMaxItems)
            return fail(RA_EUNSUPPORTED, "decode grid of %lld work-items exceeds 2^32: use fewer rows per call",
                        (long long)ra::decode_grid_items(a, fp8));
    } else {
        if (a.n_rows * a.Hq * (int64_t)(a.k + NW) >= kMaxGrid)
            return fail(RA_EUNSUPPORTED, "prefill has more than 2^31 (row, head, span) entries: split the chunk");
        if ((int64_t)a.B * a.Hkv * ra::ceil_div(a.cap, a.S) >= kMaxGrid)
            return fail(RA_EUNSUPPORTED, "too many (sequence, kv head, span) buckets");
        if (ra::prefill_grid_items(a) >= kMaxItems)
            return fail(RA_EUNSUPPORTED, "prefill grid of %lld work-items exceeds 2^32: split the chunk",
                        (long long)ra::prefill_grid_items(a));
    }
    const size_t need = op == RA_OP_DECODE ? ra::decode_workspace_bytes(a) : ra::prefill_workspace_bytes(a);
    if (r->n_rows > 0 && (!ws || ws_bytes < need))
        return fail(RA_ECAPACITY, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, need);
    return RA_OK;
}

}  // namespace

extern "C" {

ra_status span_summary_update(const ra_config *cfg, const void *k_cache, float *span_mean, float *run_sum,
                              const int64_t *old_len, const int64_t *new_len, int64_t max_new_tokens, void *stream) {
    ra_status s = check_config(cfg);
    if (s) return s;
    if (!k_cache || !span_mean || !run_sum || !old_len || !new_len) return fail(RA_EINVAL, "NULL pointer argument");
    if (max_new_tokens < 0) return fail(RA_EINVAL, "max_new_tokens must be >= 0");
    if (max_new_tokens > cfg->capacity) return fail(RA_ECAPACITY, "max_new_tokens exceeds capacity");
    if (max_new_tokens == 0) return ok();
    const int64_t U = (max_new_tokens - 1 + cfg->span_size - 1) / cfg->span_size + 1;
    if ((int64_t)cfg->batch * cfg->num_kv_heads * U >= kMaxGrid) return fail(RA_EUNSUPPORTED, "grid too large");
    ra::SummaryArgs a;
    a.k = k_cache;
    a.kscale = nullptr;
    a.mean = span_mean;
    a.run_sum = run_sum;
    a.old_len = old_len;
    a.new_len = new_len;
    a.dtype = cfg->dtype;
    a.d = cfg->head_dim;
    a.B = cfg->batch;
    a.Hkv = cfg->num_kv_heads;
    a.S = cfg->span_size;
    a.cap = cfg->capacity;
    a.max_spans = cfg->max_spans;
    a.max_new = max_new_tokens;
    return hip_status(ra::launch_summary(a, (hipStream_t)stream), "span_summary_update launch");
}

ra_status route_scores(const ra_config *cfg, const ra_rows *rows, const float *span_mean, float *scores,
                       int64_t score_stride, void *stream) {
    ra_status s = check_config(cfg);
    if (s) return s;
    if ((s = check_rows(cfg, rows))) return s;
    if (rows->n_rows == 0) return ok();
    if (!span_mean || !scores) return fail(RA_EINVAL, "NULL span_mean or scores");
    const int64_t rmax = ra::num_routable(rows->max_pos, cfg->span_size, cfg->window);
    if (score_stride < 1 || score_stride < rmax)
        return fail(RA_ECAPACITY, "score_stride (%lld) < routable spans at max_pos (%lld)", (long long)score_stride,
                    (long long)rmax);
    return hip_status(ra::launch_route(row_args(cfg, rows), span_mean, scores, score_stride, (hipStream_t)stream),
                      "route_scores launch");
}

ra_status topk_spans(const ra_config *cfg, const ra_rows *rows, const float *scores, int64_t score_stride,
                     int32_t *sel, void *stream) {
    ra_status s = check_config(cfg);
    if (s) return s;
    if ((s = check_rows(cfg, rows))) return s;
    if (rows->n_rows == 0) return ok();
    if (!scores || !sel) return fail(RA_EINVAL, "NULL scores or sel");
    const int64_t rmax = ra::num_routable(rows->max_pos, cfg->span_size, cfg->window);
    if (score_stride < 1 || score_stride < rmax)
        return fail(RA_ECAPACITY, "score_stride (%lld) < routable spans at max_pos (%lld)", (long long)score_stride,
                    (long long)rmax);
    return hip_status(ra::launch_topk(row_args(cfg, rows), scores, score_stride, sel, (hipStream_t)stream),
                      "topk_spans launch");
}

ra_status route_topk_spans(const ra_config *cfg, const ra_rows *rows, const float *span_mean, int32_t *sel,
                           void *workspace, size_t workspace_bytes, void *stream) {
    ra_status s = check_config(cfg);
    if (s) return s;
    if ((s = check_rows(cfg, rows))) return s;
    if (rows->n_rows == 0) return ok();
    if (!span_mean || !sel) return fail(RA_EINVAL, "NULL span_mean or sel");
    const ra::RowArgs a = row_args(cfg, rows);
    if (a.n_rows * a.Hkv >= kMaxGrid) return fail(RA_EUNSUPPORTED, "too many rows for one launch");
    const size_t need = ra::route_topk_workspace_bytes(a);
    if (!workspace || workspace_bytes < need)
        return fail(RA_ECAPACITY, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
    return hip_status(ra::launch_route_topk(a, span_mean, sel, workspace, (hipStream_t)stream),
                      "route_topk_spans launch");
}

ra_status routed_attn_decode(const ra_config *cfg, const ra_rows *rows, const void *k_cache, const void *v_cache,
                             const int32_t *sel, float *out, void *workspace, size_t workspace_bytes, void *stream) {
    ra_status s = check_attn(cfg, rows, k_cache, v_cache, sel, out, workspace, workspace_bytes, RA_OP_DECODE);
    if (s) return s;
    if (rows->n_rows == 0) return ok();
    return hip_status(ra::launch_decode(row_args(cfg, rows), k_cache, v_cache, sel, out, workspace, (hipStream_t)stream),
                      "routed_attn_decode launch");
}

}  // extern "C"

namespace {

// The device scratch of routed_attn_decode_noalloc: one copy per GPU, held until the process
// ends.  In host code `scratch` names a host-side stand-in, not the device array: its device
// address comes from hipGetSymbolAddress, once per device (with that device current), and only
// that address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
std::vector<void *> g_scratch_ptr;  // per device ordinal; null until looked up

// The device address of this device's scratch (looked up on the first call on the device).
ra_status scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(RA_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(RA_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return RA_OK;
}

}  // namespace

extern "C" {

ra_status routed_attn_decode_noalloc(const ra_config *cfg, const ra_rows *rows, const void *k_cache,
                                     const void *v_cache, const int32_t *sel, float *out, void *stream) {
    ra_status s = check_config(cfg);
    if (s) return s;
    if ((s = check_rows(cfg, rows))) return s;
    const size_t need = ra::decode_workspace_bytes(row_args(cfg, rows));
    if (need > kNoAllocScratchBytes)
        return fail(RA_ECAPACITY,
                    "routed_attn_decode_noalloc needs %zu bytes of scratch, more than its fixed %zu: use fewer rows "
                    "per call, or routed_attn_decode with a workspace",
                    need, kNoAllocScratchBytes);
    // the full validation, with the scratch standing in for the workspace (nothing is launched
    // before it passes)
    s = check_attn(cfg, rows, k_cache, v_cache, sel, out, &kNoAllocScratchBytes, kNoAllocScratchBytes, RA_OP_DECODE);
    if (s) return s;
    if (rows->n_rows == 0) return ok();
    void *ws = nullptr;
    if ((s = scratch_address(&ws))) return s;
    return hip_status(ra::launch_decode(row_args(cfg, rows), k_cache, v_cache, sel, out, ws, (hipStream_t)stream),
                      "routed_attn_decode_noalloc launch");
}

ra_status routed_attn_prefill(const ra_config *cfg, const ra_rows *rows, const void *k_cache, const void *v_cache,
                              const int32_t *sel, float *out, void *workspace, size_t workspace_bytes, void *stream) {
    ra_status s = check_attn(cfg, rows, k_cache, v_cache, sel, out, workspace, workspace_bytes, RA_OP_PREFILL);
    if (s) return s;
    if (rows->n_rows == 0) return ok();
    return hip_status(
        ra::launch_prefill(row_args(cfg, rows), k_cache, v_cache, sel, out, workspace, (hipStream_t)stream),
        "routed_attn_prefill launch");
}

ra_status attn_dense_causal(const ra_config *cfg, const ra_rows *rows, const void *k_cache, const void *v_cache,
                            float *out, void *stream) {
    ra_status s = check_config(cfg);
    if (s) return s;
    if ((s = check_rows(cfg, rows))) return s;
    if (cfg->dtype != RA_BF16) return fail(RA_EUNSUPPORTED, "attn_dense_causal takes bf16 inputs only");
    if (cfg->capacity * (int64_t)cfg->head_dim >= kMaxGrid)
        return fail(RA_EUNSUPPORTED, "capacity * head_dim must be below 2^31 for attn_dense_causal");
    if (rows->n_rows == 0) return ok();
    if (!k_cache || !v_cache || !out) return fail(RA_EINVAL, "NULL K, V or out");
    const ra::RowArgs a = row_args(cfg, rows);
    const int RT = 128 / a.G;
    if (a.Hkv * ra::ceil_div(a.n_rows, RT) >= kMaxGrid) return fail(RA_EUNSUPPORTED, "too many rows");
    return hip_status(ra::launch_dense(a, k_cache, v_cache, out, (hipStream_t)stream), "attn_dense_causal launch");
}

// ------------------------------------------------------------------------- 8-bit K/V cache
ra_status kv_quantize_fp8(const ra_config *cfg, const void *src_cache, uint8_t *codes, float *scales,
                          const int64_t *old_len, const int64_t *new_len, int64_t max_new_tokens, void *stream) {
    ra_status s = check_config(cfg);
    if (s) return s;
    if (cfg->dtype != RA_BF16) return fail(RA_EUNSUPPORTED, "kv_quantize_fp8 takes a bf16 cache (cfg->dtype RA_BF16)");
    if (!src_cache || !codes || !scales || !old_len || !new_len) return fail(RA_EINVAL, "NULL pointer argument");
    if (max_new_tokens < 0) return fail(RA_EINVAL, "max_new_tokens must be >= 0");
    if (max_new_tokens > cfg->capacity) return fail(RA_ECAPACITY, "max_new_tokens exceeds capacity");
    if (max_new_tokens == 0) return ok();
    const int rpb = 256 / (cfg->head_dim / 8);
    if ((int64_t)cfg->batch * cfg->num_kv_heads * ra::ceil_div(max_new_tokens, rpb) >= kMaxGrid)
        return fail(RA_EUNSUPPORTED, "grid too large");
    ra::QuantArgs a;
    a.src = (const uint16_t *)src_cache;
    a.dst = codes;
    a.scale = scales;
    a.old_len = old_len;
    a.new_len = new_len;
    a.d = cfg->head_dim;
    a.B = cfg->batch;
    a.Hkv = cfg->num_kv_heads;
    a.cap = cfg->capacity;
    a.max_new = max_new_tokens;
    return hip_status(ra::launch_quantize_fp8(a, (hipStream_t)stream), "kv_quantize_fp8 launch");
}

ra_status span_summary_update_fp8(const ra_config *cfg, const uint8_t *k_codes, const float *k_scales,
                                  float *span_mean, float *run_sum, const int64_t *old_len, const int64_t *new_len,
                                  int64_t max_new_tokens, void *stream) {
    ra_status s = check_config(cfg);
    if (s) return s;
    if (cfg->dtype != RA_BF16) return fail(RA_EUNSUPPORTED, "8-bit caches go with bf16 queries (cfg->dtype RA_BF16)");
    if (!k_codes || !k_scales || !span_mean || !run_sum || !old_len || !new_len)
        return fail(RA_EINVAL, "NULL pointer argument");
    if (max_new_tokens < 0) return fail(RA_EINVAL, "max_new_tokens must be >= 0");
    if (max_new_tokens > cfg->capacity) return fail(RA_ECAPACITY, "max_new_tokens exceeds capacity");
    if (max_new_tokens == 0) return ok();
    const int64_t U = (max_new_tokens - 1 + cfg->span_size - 1) / cfg->span_size + 1;
    if ((int64_t)cfg->batch * cfg->num_kv_heads * U >= kMaxGrid) return fail(RA_EUNSUPPORTED, "grid too large");
    ra::SummaryArgs a;
    a.k = k_codes;
    a.kscale = k_scales;
    a.mean = span_mean;
    a.run_sum = run_sum;
    a.old_len = old_len;
    a.new_len = new_len;
    a.dtype = ra::kCacheFp8;
    a.d = cfg->head_dim;
    a.B = cfg->batch;
    a.Hkv = cfg->num_kv_heads;
    a.S = cfg->span_size;
    a.cap = cfg->capacity;
    a.max_spans = cfg->max_spans;
    a.max_new = max_new_tokens;
    return hip_status(ra::launch_summary(a, (hipStream_t)stream), "span_summary_update_fp8 launch");
}

ra_status routed_attn_decode_fp8(const ra_config *cfg, const ra_rows *rows, const uint8_t *k_codes,
                                 const uint8_t *v_codes, const float *k_scales, const float *v_scales,
                                 const int32_t *sel, float *out, void *workspace, size_t workspace_bytes,
                                 void *stream) {
    ra_status s = check_attn(cfg, rows, k_codes, v_codes, sel, out, workspace, workspace_bytes, RA_OP_DECODE, true);
    if (s) return s;
    if (cfg->dtype != RA_BF16) return fail(RA_EUNSUPPORTED, "8-bit caches go with bf16 queries (cfg->dtype RA_BF16)");
    if (rows->n_rows > 0 && (!k_scales || !v_scales)) return fail(RA_EINVAL, "NULL k_scales or v_scales");
    if (rows->n_rows == 0) return ok();
    return hip_status(ra::launch_decode_fp8(row_args(cfg, rows), k_codes, v_codes, k_scales, v_scales, sel, out,
                                            workspace, (hipStream_t)stream),
                      "routed_attn_decode_fp8 launch");
}

ra_status routed_attn_prefill_fp8(const ra_config *cfg, const ra_rows *rows, const uint8_t *k_codes,
                                  const uint8_t *v_codes, const float *k_scales, const float *v_scales,
                                  const int32_t *sel, float *out, void *workspace, size_t workspace_bytes,
                                  void *stream) {
    ra_status s = check_attn(cfg, rows, k_codes, v_codes, sel, out, workspace, workspace_bytes, RA_OP_PREFILL);
    if (s) return s;
    if (cfg->dtype != RA_BF16) return fail(RA_EUNSUPPORTED, "8-bit caches go with bf16 queries (cfg->dtype RA_BF16)");
    if (rows->n_rows > 0 && (!k_scales || !v_scales)) return fail(RA_EINVAL, "NULL k_scales or v_scales");
    if (rows->n_rows == 0) return ok();
    return hip_status(ra::launch_prefill_fp8(row_args(cfg, rows), k_codes, v_codes, k_scales, v_scales, sel, out,
                                             workspace, (hipStream_t)stream),
                      "routed_attn_prefill_fp8 launch");
}

// ------------------------------------------------------------------- token-level cold retrieval
}  // extern "C"

namespace {

ra_status check_cold(const ra_config *c, int32_t hot_window, int32_t top_k_cold) {
    if (hot_window < 1) return fail(RA_EINVAL, "hot_window must be >= 1");
    if (top_k_cold < 1 || top_k_cold > ra::kMaxCold)
        return fail(RA_EUNSUPPORTED, "top_k_cold must be in [1, %d]", ra::kMaxCold);
    if (c->capacity >= (1LL << 31)) return fail(RA_EUNSUPPORTED, "cold retrieval needs capacity < 2^31");
    return RA_OK;
}

}  // namespace

extern "C" {

ra_status kv_signature_update(const ra_config *cfg, const void *k_cache, uint8_t *sig, const int64_t *old_len,
                              const int64_t *new_len, int64_t max_new_tokens, void *stream) {
    ra_status s = check_config(cfg);
    if (s) return s;
    if (!k_cache || !sig || !old_len || !new_len) return fail(RA_EINVAL, "NULL pointer argument");
    if (max_new_tokens < 0) return fail(RA_EINVAL, "max_new_tokens must be >= 0");
    if (max_new_tokens > cfg->capacity) return fail(RA_ECAPACITY, "max_new_tokens exceeds capacity");
    if ((uintptr_t)sig & 15) return fail(RA_EINVAL, "sig must be 16-byte aligned");
    if (max_new_tokens == 0) return ok();
    const int rpb = 256 / (cfg->head_dim / 32);
    if ((int64_t)cfg->batch * cfg->num_kv_heads * ra::ceil_div(max_new_tokens, rpb) >= kMaxGrid)
        return fail(RA_EUNSUPPORTED, "grid too large");
    ra::SigArgs a;
    a.k = k_cache;
    a.sig = (uint32_t *)sig;
    a.old_len = old_len;
    a.new_len = new_len;
    a.dtype = cfg->dtype;
    a.d = cfg->head_dim;
    a.B = cfg->batch;
    a.Hkv = cfg->num_kv_heads;
    a.cap = cfg->capacity;
    a.max_new = max_new_tokens;
    return hip_status(ra::launch_signatures(a, (hipStream_t)stream), "kv_signature_update launch");
}

size_t ra_cold_workspace_bytes(const ra_config *cfg, int64_t n_rows, int64_t max_pos, int32_t hot_window,
                               int32_t top_k_cold) {
    if (check_config(cfg) || check_cold(cfg, hot_window, top_k_cold)) return 0;
    if (n_rows < 0 || max_pos < 0 || max_pos >= cfg->capacity) {
        fail(RA_EINVAL, "n_rows must be >= 0 and max_pos in [0, capacity)");
        return 0;
    }
    ra_rows r{nullptr, nullptr, nullptr, n_rows, max_pos};
    return ra::cold_workspace_bytes(row_args(cfg, &r), hot_window, top_k_cold);
}

ra_status cold_select(const ra_config *cfg, const ra_rows *rows, const uint8_t *sig, int32_t hot_window,
                      int32_t top_k_cold, int32_t *sel_cold, void *workspace, size_t workspace_bytes, void *stream) {
    ra_status s = check_config(cfg);
    if (s) return s;
    if ((s = check_rows(cfg, rows))) return s;
    if ((s = check_cold(cfg, hot_window, top_k_cold))) return s;
    if (rows->n_rows == 0) return ok();
    if (!sig || !sel_cold) return fail(RA_EINVAL, "NULL sig or sel_cold");
    if ((uintptr_t)sig & 15) return fail(RA_EINVAL, "sig must be 16-byte aligned");
    const ra::RowArgs a = row_args(cfg, rows);
    const int n_tiles = ra::cold_tiles(a.max_pos, hot_window, a.G);
    if (a.n_rows * a.Hkv * (int64_t)n_tiles >= kMaxGrid)
        return fail(RA_EUNSUPPORTED, "scan grid too large: use fewer rows per call");
    if (n_tiles > ra::kMergeTiles)
        return fail(RA_EUNSUPPORTED, "cold retrieval scans at most %d x %d cold positions per row", ra::kMergeTiles,
                    ra::cold_tile_positions(a.G));
    const size_t need = ra::cold_workspace_bytes(a, hot_window, top_k_cold);
    if (!workspace || workspace_bytes < need)
        return fail(RA_ECAPACITY, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
    return hip_status(ra::launch_cold_select(a, (const uint32_t *)sig, hot_window, top_k_cold, sel_cold, workspace,
                                             (hipStream_t)stream),
                      "cold_select launch");
}

ra_status cold_attn_decode(const ra_config *cfg, const ra_rows *rows, const void *k_cache, const void *v_cache,
                           const int32_t *sel_cold, int32_t hot_window, int32_t top_k_cold, float *out, void *stream) {
    ra_status s = check_config(cfg);
    if (s) return s;
    if ((s = check_rows(cfg, rows))) return s;
    if ((s = check_cold(cfg, hot_window, top_k_cold))) return s;
    if (rows->n_rows == 0) return ok();
    if (!k_cache || !v_cache || !sel_cold || !out) return fail(RA_EINVAL, "NULL K, V, sel_cold or out");
    return hip_status(ra::launch_cold_attn(row_args(cfg, rows), k_cache, v_cache, sel_cold, hot_window, top_k_cold,
                                           out, (hipStream_t)stream),
                      "cold_attn_decode launch");
}

// ------------------------------------------------------------------------- session snapshots
}  // extern "C"

namespace {

constexpr uint64_t kSnapMagic = 0x31504E5341535243ull;  // "CRSASNP1" read as a little-endian word
constexpr uint32_t kSnapVersion = 1, kSnapChunk = 4096, kSnapFanIn = 16;
constexpr int kMaxLevels = 16;  // 4096 * 16^15 bytes exceed any image
constexpr int kSnapE4M3 = RA_SNAPSHOT_E4M3;  // element type of the 8-bit cache's images

struct SnapLayout {
    int B, Hkv, d, S, dtype, esz;
    uint64_t H, P, data, image;
    int n_levels;
    uint64_t count[kMaxLevels], off[kMaxLevels];  // digests per level and where each level starts
    uint64_t root;
};

uint64_t snap_header_bytes(int B) { return (64 + 8 * (uint64_t)B + 15) / 16 * 16; }

// Image bytes of one run of L fp32 row scales (8-bit cache): 4 L, zero-padded to 16.
uint64_t snap_scale_run(int64_t L) { return (4 * (uint64_t)L + 15) / 16 * 16; }

// Layout of the image of B sequences with the given lengths (checked by the callers).
SnapLayout snap_layout(int B, int Hkv, int d, int S, int dtype, const int64_t *lengths) {
    SnapLayout L;
    L.B = B;
    L.Hkv = Hkv;
    L.d = d;
    L.S = S;
    L.dtype = dtype;
    L.esz = dtype == kSnapE4M3 ? 1 : (dtype == RA_BF16 ? 2 : 4);
    uint64_t rows = 0, spans = 0, runs = 0;
    for (int b = 0; b < B; ++b) {
        rows += (uint64_t)lengths[b];
        spans += (uint64_t)lengths[b] / (uint64_t)S;
        runs += snap_scale_run(lengths[b]);
    }
    L.H = snap_header_bytes(B);
    L.P = 2ull * Hkv * rows * d * L.esz + (dtype == kSnapE4M3 ? 2ull * Hkv * runs : 0ull) +
          (uint64_t)Hkv * (spans + B) * d * 4;
    L.data = L.H + L.P;
    uint64_t n = (L.data + kSnapChunk - 1) / kSnapChunk, at = L.data;
    L.n_levels = 0;
    while (true) {
        L.count[L.n_levels] = n;
        L.off[L.n_levels] = at;
        at += 32 * n;
        ++L.n_levels;
        if (n <= kSnapFanIn) break;
        n = (n + kSnapFanIn - 1) / kSnapFanIn;
    }
    L.root = at;
    L.image = at + 32;
    return L;
}

ra_status check_lengths(const ra_config *c, const int64_t *lengths, int B) {
    if (!lengths) return fail(RA_EINVAL, "lengths is NULL");
    for (int b = 0; b < B; ++b)
        if (lengths[b] < 0 || lengths[b] > c->capacity)
            return fail(RA_ECAPACITY, "lengths[%d] = %lld outside [0, capacity = %lld]", b, (long long)lengths[b],
                        (long long)c->capacity);
    return RA_OK;
}

// The payload's byte ranges in order, each paired with its place in the caches; `to_image`
// selects the copy direction.  ks / vs: the 8-bit cache's row scales (element type 2 only).
ra_status snap_copy(const SnapLayout &L, const ra_config *c, const int64_t *lengths, uint8_t *image,
                    const void *k, const void *v, const float *ks, const float *vs, const float *mean,
                    const float *run, bool to_image, const unsigned long long *guard, hipStream_t st) {
    ra::SegmentBatch sb;
    sb.n = 0;
    uint64_t at = L.H;
    auto flush = [&]() -> hipError_t {
        const hipError_t e = ra::launch_copy_segments(sb, guard, st);
        sb.n = 0;
        return e;
    };
    // `bytes` of the image at `at` <-> the cache at cache_ptr, in 16-byte units or (scales) 4-byte
    // words; `pad` zero bytes follow in the image (written when packing, skipped when restoring)
    auto add = [&](const void *cache_ptr, uint64_t bytes, bool words, uint64_t pad) -> hipError_t {
        hipError_t e = hipSuccess;
        if (bytes > 0) {
            ra::Segment &s = sb.seg[sb.n++];
            s.src = to_image ? cache_ptr : (const void *)(image + at);
            s.dst = to_image ? (void *)(image + at) : const_cast<void *>(cache_ptr);
            s.n = words ? bytes / 4 : bytes / 16;
            s.mode = words ? ra::kSegCopy4 : ra::kSegCopy16;
            at += bytes;
            if (sb.n == ra::kSegs) e = flush();
        }
        if (e == hipSuccess && pad > 0) {
            if (to_image) {
                ra::Segment &s = sb.seg[sb.n++];
                s.src = nullptr;
                s.dst = image + at;
                s.n = pad / 4;
                s.mode = ra::kSegZero4;
                if (sb.n == ra::kSegs) e = flush();
            }
            at += pad;
        }
        return e;
    };
    const uint64_t row = (uint64_t)L.d * L.esz;
    hipError_t e = hipSuccess;
    for (int b = 0; b < L.B && e == hipSuccess; ++b)
        for (int g = 0; g < L.Hkv && e == hipSuccess; ++g) {
            const uint64_t bg = (uint64_t)b * c->num_kv_heads + g;
            const uint64_t base = bg * (uint64_t)c->capacity * row;
            const uint64_t n = (uint64_t)lengths[b] * row;
            e = add((const uint8_t *)k + base, n, false, 0);
            if (e == hipSuccess) e = add((const uint8_t *)v + base, n, false, 0);
            if (L.dtype == kSnapE4M3) {
                const uint64_t sc = 4 * (uint64_t)lengths[b], pad = snap_scale_run(lengths[b]) - sc;
                if (e == hipSuccess) e = add(ks + bg * (uint64_t)c->capacity, sc, true, pad);
                if (e == hipSuccess) e = add(vs + bg * (uint64_t)c->capacity, sc, true, pad);
            }
        }
    for (int b = 0; b < L.B && e == hipSuccess; ++b)
        for (int g = 0; g < L.Hkv && e == hipSuccess; ++g) {
            const uint64_t bg = (uint64_t)b * c->num_kv_heads + g;
            e = add(mean + bg * (uint64_t)c->max_spans * L.d, (uint64_t)lengths[b] / L.S * L.d * 4, false, 0);
            if (e == hipSuccess) e = add(run + bg * L.d, (uint64_t)L.d * 4, false, 0);
        }
    if (e == hipSuccess) e = flush();
    if (e != hipSuccess) return hip_status(e, "snapshot copy launch");
    return RA_OK;
}

// Digest levels and root of an image: stored (compare = false) or checked against the stored
// ones (compare = true, mismatches reported in *bad).  Level 1 digests 4096-byte chunks of
// header | payload, the levels above groups of kSnapFanIn digests.
hipError_t snap_hash(const SnapLayout &L, uint8_t *image, bool compare, unsigned long long *bad, hipStream_t st) {
    uint64_t src = 0, len = L.data, chunk = kSnapChunk;
    for (int l = 0; l < L.n_levels; ++l) {
        const hipError_t e = ra::launch_sha_chunks(image + src, len, chunk, image + L.off[l], compare, bad, src, st);
        if (e != hipSuccess) return e;
        src = L.off[l];
        len = 32 * L.count[l];
        chunk = 32 * kSnapFanIn;
    }
    return ra::launch_sha_chunks(image + src, len, len, image + L.root, compare, bad, src, st);
}

// Header fields of a host header (any alignment); fills the layout and the lengths.
ra_status snap_parse(const void *header, size_t avail, SnapLayout *L, std::vector<int64_t> &lengths) {
    if (!header) return fail(RA_EINVAL, "header is NULL");
    if (avail < 64) return fail(RA_EFORMAT, "header needs at least 64 bytes, got %zu", avail);
    const uint8_t *h = (const uint8_t *)header;
    uint64_t magic, P, H, z;
    uint32_t version, dtype, B, Hkv, d, S, chunk, fan;
    memcpy(&magic, h, 8);
    memcpy(&version, h + 8, 4);
    memcpy(&dtype, h + 12, 4);
    memcpy(&B, h + 16, 4);
    memcpy(&Hkv, h + 20, 4);
    memcpy(&d, h + 24, 4);
    memcpy(&S, h + 28, 4);
    memcpy(&P, h + 32, 8);
    memcpy(&H, h + 40, 8);
    memcpy(&chunk, h + 48, 4);
    memcpy(&fan, h + 52, 4);
    memcpy(&z, h + 56, 8);
    if (magic != kSnapMagic) return fail(RA_EFORMAT, "not a snapshot image (magic)");
    if (version != kSnapVersion || chunk != kSnapChunk || fan != kSnapFanIn || z != 0)
        return fail(RA_EFORMAT, "unsupported snapshot version or digest parameters");
    if (dtype != RA_F32 && dtype != RA_BF16 && dtype != (uint32_t)kSnapE4M3)
        return fail(RA_EFORMAT, "unknown element type %u", dtype);
    if (B < 1 || B > (1u << 24) || Hkv < 1 || Hkv > 4096 || (d != 64 && d != 128) || S < 1 || S > (1u << 30))
        return fail(RA_EFORMAT, "header shape fields out of range");
    if (H != snap_header_bytes((int)B)) return fail(RA_EFORMAT, "header size field inconsistent with B");
    if (avail < H) return fail(RA_EFORMAT, "header of %llu bytes, %zu given", (unsigned long long)H, avail);
    lengths.resize(B);
    for (uint32_t b = 0; b < B; ++b) {
        int64_t x;
        memcpy(&x, h + 64 + 8 * (uint64_t)b, 8);
        if (x < 0 || x >= (1LL << 40)) return fail(RA_EFORMAT, "length %lld of sequence %u out of range", (long long)x, b);
        lengths[b] = x;
    }
    *L = snap_layout((int)B, (int)Hkv, (int)d, (int)S, (int)dtype, lengths.data());
    if (L->P != P) return fail(RA_EFORMAT, "payload size field inconsistent with the lengths");
    return RA_OK;
}

// Header words, payload copies and digest levels of an image of element type `elem` (cfg->dtype,
// or kSnapE4M3 with the scale arrays); cfg is checked by the caller.
ra_status snap_pack(const ra_config *cfg, int elem, const void *k_cache, const void *v_cache, const float *ks,
                    const float *vs, const float *span_mean, const float *run_sum, const int64_t *lengths,
                    void *image, size_t image_bytes, void *stream) {
    ra_status s = check_lengths(cfg, lengths, cfg->batch);
    if (s) return s;
    if (!k_cache || !v_cache || !span_mean || !run_sum || !image) return fail(RA_EINVAL, "NULL pointer argument");
    if (((uintptr_t)image | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)span_mean | (uintptr_t)run_sum) & 15)
        return fail(RA_EINVAL, "image and cache buffers must be 16-byte aligned");
    const SnapLayout L = snap_layout(cfg->batch, cfg->num_kv_heads, cfg->head_dim, cfg->span_size, elem, lengths);
    if (image_bytes < L.image)
        return fail(RA_ECAPACITY, "image buffer of %zu bytes, %llu needed", image_bytes, (unsigned long long)L.image);
    hipStream_t st = (hipStream_t)stream;
    uint8_t *img = (uint8_t *)image;
    // header words: 8 fixed, B lengths, one zero word when B is odd
    const uint64_t n_words = L.H / 8;
    ra::WordBatch wb;
    for (uint64_t w0 = 0; w0 < n_words; w0 += ra::kWords) {
        wb.n = (int)(n_words - w0 < (uint64_t)ra::kWords ? n_words - w0 : ra::kWords);
        for (int i = 0; i < wb.n; ++i) {
            const uint64_t w = w0 + i;
            uint64_t v = 0;
            switch (w) {
                case 0: v = kSnapMagic; break;
                case 1: v = kSnapVersion | ((uint64_t)(uint32_t)elem << 32); break;
                case 2: v = (uint64_t)(uint32_t)cfg->batch | ((uint64_t)(uint32_t)cfg->num_kv_heads << 32); break;
                case 3: v = (uint64_t)(uint32_t)cfg->head_dim | ((uint64_t)(uint32_t)cfg->span_size << 32); break;
                case 4: v = L.P; break;
                case 5: v = L.H; break;
                case 6: v = kSnapChunk | ((uint64_t)kSnapFanIn << 32); break;
                case 7: v = 0; break;
                default: v = w - 8 < (uint64_t)cfg->batch ? (uint64_t)lengths[w - 8] : 0; break;
            }
            wb.v[i] = v;
        }
        const hipError_t e = ra::launch_write_words((uint64_t *)(img + 8 * w0), wb, st);
        if (e != hipSuccess) return hip_status(e, "snapshot header launch");
    }
    if ((s = snap_copy(L, cfg, lengths, img, k_cache, v_cache, ks, vs, span_mean, run_sum, true, nullptr, st)))
        return s;
    return hip_status(snap_hash(L, img, false, nullptr, st), "snapshot digest launch");
}

// Restore of an image of element type `elem` (cfg is checked by the caller).
ra_status snap_unpack(const ra_config *cfg, int elem, const void *header, size_t header_avail, const void *image,
                      size_t image_bytes, const uint64_t *guard, void *k_cache, void *v_cache, float *ks, float *vs,
                      float *span_mean, float *run_sum, void *stream) {
    SnapLayout L;
    std::vector<int64_t> len;
    ra_status s = snap_parse(header, header_avail, &L, len);
    if (s) return s;
    if (L.dtype != elem || L.Hkv != cfg->num_kv_heads || L.d != cfg->head_dim || L.S != cfg->span_size)
        return fail(RA_EINVAL, "image (element type %d, Hkv %d, d %d, S %d) does not match (%d, %d, %d, %d)", L.dtype,
                    L.Hkv, L.d, L.S, elem, cfg->num_kv_heads, cfg->head_dim, cfg->span_size);
    if (L.B > cfg->batch) return fail(RA_ECAPACITY, "image holds %d sequences, cfg->batch is %d", L.B, cfg->batch);
    if ((s = check_lengths(cfg, len.data(), L.B))) return s;
    if (!image || !k_cache || !v_cache || !span_mean || !run_sum) return fail(RA_EINVAL, "NULL pointer argument");
    if (((uintptr_t)image | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)span_mean | (uintptr_t)run_sum) & 15)
        return fail(RA_EINVAL, "image and cache buffers must be 16-byte aligned");
    if (image_bytes < L.image)
        return fail(RA_EFORMAT, "image of %zu bytes, header describes %llu", image_bytes, (unsigned long long)L.image);
    return snap_copy(L, cfg, len.data(), (uint8_t *)const_cast<void *>(image), k_cache, v_cache, ks, vs, span_mean,
                     run_sum, false, (const unsigned long long *)guard, (hipStream_t)stream);
}

}  // namespace

extern "C" {

size_t kv_snapshot_bytes(const ra_config *cfg, const int64_t *lengths) {
    if (check_config(cfg) || check_lengths(cfg, lengths, cfg->batch)) return 0;
    return (size_t)snap_layout(cfg->batch, cfg->num_kv_heads, cfg->head_dim, cfg->span_size, cfg->dtype, lengths).image;
}

size_t kv_snapshot_bytes_fp8(const ra_config *cfg, const int64_t *lengths) {
    if (check_config(cfg) || check_lengths(cfg, lengths, cfg->batch)) return 0;
    return (size_t)snap_layout(cfg->batch, cfg->num_kv_heads, cfg->head_dim, cfg->span_size, kSnapE4M3, lengths).image;
}

ra_status kv_snapshot_pack(const ra_config *cfg, const void *k_cache, const void *v_cache, const float *span_mean,
                           const float *run_sum, const int64_t *lengths, void *image, size_t image_bytes,
                           void *stream) {
    ra_status s = check_config(cfg);
    if (s) return s;
    return snap_pack(cfg, cfg->dtype, k_cache, v_cache, nullptr, nullptr, span_mean, run_sum, lengths, image,
                     image_bytes, stream);
}

ra_status kv_snapshot_pack_fp8(const ra_config *cfg, const uint8_t *k_codes, const uint8_t *v_codes,
                               const float *k_scales, const float *v_scales, const float *span_mean,
                               const float *run_sum, const int64_t *lengths, void *image, size_t image_bytes,
                               void *stream) {
    ra_status s = check_config(cfg);
    if (s) return s;
    if (!k_scales || !v_scales) return fail(RA_EINVAL, "NULL scale array");
    if (((uintptr_t)k_scales | (uintptr_t)v_scales) & 3) return fail(RA_EINVAL, "scale arrays must be 4-byte aligned");
    return snap_pack(cfg, kSnapE4M3, k_codes, v_codes, k_scales, v_scales, span_mean, run_sum, lengths, image,
                     image_bytes, stream);
}

ra_status kv_snapshot_parse(const void *header, size_t header_avail, ra_snapshot_info *info, int64_t *lengths,
                            int32_t max_batch) {
    SnapLayout L;
    std::vector<int64_t> len;
    ra_status s = snap_parse(header, header_avail, &L, len);
    if (s) return s;
    if (lengths) {
        if (L.B > max_batch) return fail(RA_ECAPACITY, "image holds %d sequences, room for %d", L.B, max_batch);
        memcpy(lengths, len.data(), 8 * (size_t)L.B);
    }
    if (info) {
        info->dtype = L.dtype;
        info->batch = L.B;
        info->num_kv_heads = L.Hkv;
        info->head_dim = L.d;
        info->span_size = L.S;
        info->reserved = 0;
        info->header_bytes = L.H;
        info->payload_bytes = L.P;
        info->image_bytes = L.image;
    }
    return ok();
}

ra_status kv_snapshot_verify(const void *header, size_t header_avail, const void *image, size_t image_bytes,
                             uint64_t *bad_offset, void *stream) {
    SnapLayout L;
    std::vector<int64_t> len;
    ra_status s = snap_parse(header, header_avail, &L, len);
    if (s) return s;
    if (!image || !bad_offset) return fail(RA_EINVAL, "NULL image or bad_offset");
    if ((uintptr_t)image & 15) return fail(RA_EINVAL, "image must be 16-byte aligned");
    if (image_bytes < L.image)
        return fail(RA_EFORMAT, "image of %zu bytes, header describes %llu", image_bytes, (unsigned long long)L.image);
    hipStream_t st = (hipStream_t)stream;
    unsigned long long *bad = (unsigned long long *)bad_offset;
    hipError_t e = ra::launch_fill_u64(bad, ~0ull, st);
    if (e == hipSuccess) e = snap_hash(L, (uint8_t *)const_cast<void *>(image), true, bad, st);
    return hip_status(e, "snapshot verify launch");
}

ra_status kv_snapshot_unpack(const ra_config *cfg, const void *header, size_t header_avail, const void *image,
                             size_t image_bytes, const uint64_t *guard, void *k_cache, void *v_cache,
                             float *span_mean, float *run_sum, void *stream) {
    ra_status s = check_config(cfg);
    if (s) return s;
    return snap_unpack(cfg, cfg->dtype, header, header_avail, image, image_bytes, guard, k_cache, v_cache, nullptr,
                       nullptr, span_mean, run_sum, stream);
}

ra_status kv_snapshot_unpack_fp8(const ra_config *cfg, const void *header, size_t header_avail, const void *image,
                                 size_t image_bytes, const uint64_t *guard, uint8_t *k_codes, uint8_t *v_codes,
                                 float *k_scales, float *v_scales, float *span_mean, float *run_sum, void *stream) {
    ra_status s = check_config(cfg);
    if (s) return s;
    if (!k_scales || !v_scales) return fail(RA_EINVAL, "NULL scale array");
    if (((uintptr_t)k_scales | (uintptr_t)v_scales) & 3) return fail(RA_EINVAL, "scale arrays must be 4-byte aligned");
    return snap_unpack(cfg, kSnapE4M3, header, header_avail, image, image_bytes, guard, k_codes, v_codes, k_scales,
                       v_scales, span_mean, run_sum, stream);
}

ra_status kv_snapshot_write_file(const char *path, const void *data, size_t bytes) {
    if (!path || (!data && bytes)) return fail(RA_EINVAL, "NULL path or data");
    char tmp[4096];
    if (snprintf(tmp, sizeof(tmp), "%s.tmp", path) >= (int)sizeof(tmp)) return fail(RA_EINVAL, "path too long");
    FILE *f = fopen(tmp, "wb");
    if (!f) return fail(RA_EIO, "cannot open %s for writing", tmp);
    const size_t n = bytes ? fwrite(data, 1, bytes, f) : 0;
    const bool flushed = fflush(f) == 0;
    if (fclose(f) != 0 || n != bytes || !flushed) {
        remove(tmp);
        return fail(RA_EIO, "short write to %s", tmp);
    }
    if (rename(tmp, path) != 0) {
        remove(tmp);
        return fail(RA_EIO, "cannot rename %s to %s", tmp, path);
    }
    return ok();
}

ra_status kv_snapshot_read_file(const char *path, void *buf, size_t capacity, size_t *bytes) {
    if (!path || !bytes) return fail(RA_EINVAL, "NULL path or bytes");
    FILE *f = fopen(path, "rb");
    if (!f) return fail(RA_EIO, "cannot open %s", path);
    if (fseeko(f, 0, SEEK_END) != 0) {
        fclose(f);
        return fail(RA_EIO, "cannot seek in %s", path);
    }
    const off_t size = ftello(f);
    if (size < 0 || fseeko(f, 0, SEEK_SET) != 0) {
        fclose(f);
        return fail(RA_EIO, "cannot size %s", path);
    }
    *bytes = (size_t)size;
    if (!buf) {
        fclose(f);
        return ok();
    }
    if (capacity < (size_t)size) {
        fclose(f);
        return fail(RA_ECAPACITY, "%s has %lld bytes, buffer %zu", path, (long long)size, capacity);
    }
    const size_t n = size ? fread(buf, 1, (size_t)size, f) : 0;
    fclose(f);
    if (n != (size_t)size) return fail(RA_EIO, "short read from %s", path);
    return ok();
}

// ---------------------------------------------------- decode with the step's summary append
}  // extern "C"

namespace {

// Validates the summary-update half of the *_append entry points and fills its arguments.
ra_status append_args(const ra_config *cfg, const void *k, const float *kscale, float *span_mean, float *run_sum,
                      const int64_t *old_len, const int64_t *new_len, int64_t max_new, int dtype,
                      ra::SummaryArgs *a) {
    if (!k || !span_mean || !run_sum || !old_len || !new_len) return fail(RA_EINVAL, "NULL summary argument");
    if (max_new < 0) return fail(RA_EINVAL, "max_new_tokens must be >= 0");
    if (max_new > cfg->capacity) return fail(RA_ECAPACITY, "max_new_tokens exceeds capacity");
    const int64_t U = (max_new - 1 + cfg->span_size - 1) / cfg->span_size + 1;
    if ((int64_t)cfg->batch * cfg->num_kv_heads * U >= kMaxGrid) return fail(RA_EUNSUPPORTED, "grid too large");
    a->k = k;
    a->kscale = kscale;
    a->mean = span_mean;
    a->run_sum = run_sum;
    a->old_len = old_len;
    a->new_len = new_len;
    a->dtype = dtype;
    a->d = cfg->head_dim;
    a->B = cfg->batch;
    a->Hkv = cfg->num_kv_heads;
    a->S = cfg->span_size;
    a->cap = cfg->capacity;
    a->max_spans = cfg->max_spans;
    a->max_new = max_new;
    return RA_OK;
}

}  // namespace

extern "C" {

ra_status routed_attn_decode_append(const ra_config *cfg, const ra_rows *rows, const void *k_cache,
                                    const void *v_cache, const int32_t *sel, float *out, void *workspace,
                                    size_t workspace_bytes, float *span_mean, float *run_sum, const int64_t *old_len,
                                    const int64_t *new_len, int64_t max_new_tokens, void *stream) {
    ra_status s = check_attn(cfg, rows, k_cache, v_cache, sel, out, workspace, workspace_bytes, RA_OP_DECODE);
    if (s) return s;
    ra::SummaryArgs app;
    if ((s = append_args(cfg, k_cache, nullptr, span_mean, run_sum, old_len, new_len, max_new_tokens, cfg->dtype,
                         &app)))
        return s;
    return hip_status(ra::launch_decode_app(row_args(cfg, rows), k_cache, v_cache, sel, out, workspace,
                                            max_new_tokens > 0 ? &app : nullptr, (hipStream_t)stream),
                      "routed_attn_decode_append launch");
}

ra_status routed_attn_decode_fp8_append(const ra_config *cfg, const ra_rows *rows, const uint8_t *k_codes,
                                        const uint8_t *v_codes, const float *k_scales, const float *v_scales,
                                        const int32_t *sel, float *out, void *workspace, size_t workspace_bytes,
                                        float *span_mean, float *run_sum, const int64_t *old_len,
                                        const int64_t *new_len, int64_t max_new_tokens, void *stream) {
    ra_status s = check_attn(cfg, rows, k_codes, v_codes, sel, out, workspace, workspace_bytes, RA_OP_DECODE, true);
    if (s) return s;
    if (cfg->dtype != RA_BF16) return fail(RA_EUNSUPPORTED, "8-bit caches go with bf16 queries (cfg->dtype RA_BF16)");
    if (rows->n_rows > 0 && (!k_scales || !v_scales)) return fail(RA_EINVAL, "NULL k_scales or v_scales");
    ra::SummaryArgs app;
    if ((s = append_args(cfg, k_codes, k_scales, span_mean, run_sum, old_len, new_len, max_new_tokens, ra::kCacheFp8,
                         &app)))
        return s;
    if (!k_scales) return fail(RA_EINVAL, "NULL k_scales");
    return hip_status(ra::launch_decode_fp8_app(row_args(cfg, rows), k_codes, v_codes, k_scales, v_scales, sel, out,
                                                workspace, max_new_tokens > 0 ? &app : nullptr, (hipStream_t)stream),
                      "routed_attn_decode_fp8_append launch");
}

size_t ra_workspace_bytes(const ra_config *cfg, int32_t op, int64_t n_rows, int64_t max_pos) {
    if (check_config(cfg)) return 0;
    if (op != RA_OP_DECODE && op != RA_OP_PREFILL && op != RA_OP_ROUTE_TOPK) {
        fail(RA_EINVAL, "op must be RA_OP_DECODE, RA_OP_PREFILL or RA_OP_ROUTE_TOPK");
        return 0;
    }
    ra_rows r{nullptr, nullptr, nullptr, n_rows, max_pos};
    if (n_rows < 0 || max_pos < 0 || max_pos >= cfg->capacity) {
        fail(RA_EINVAL, "n_rows must be >= 0 and max_pos in [0, capacity)");
        return 0;
    }
    const ra::RowArgs a = row_args(cfg, &r);
    if (op == RA_OP_ROUTE_TOPK) return ra::route_topk_workspace_bytes(a);
    return op == RA_OP_DECODE ? ra::decode_workspace_bytes(a) : ra::prefill_workspace_bytes(a);
}

const char *ra_status_string(int32_t status) {
    switch (status) {
        case RA_OK: return "ok";
        case RA_EINVAL: return "invalid argument";
        case RA_EUNSUPPORTED: return "unsupported configuration";
        case RA_ECAPACITY: return "buffer too small";
        case RA_EHIP: return "HIP runtime error";
        case RA_EIO: return "file error";
        case RA_EFORMAT: return "not a readable snapshot";
        default: return "unknown status";
    }
}

const char *ra_last_error(void) { return g_err; }

}  // extern "C"
