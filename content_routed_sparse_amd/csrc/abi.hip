// C ABI of the routed-attention library: host-side validation, error reporting, launches.
// Nothing here allocates memory or synchronises with the device.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "common.h"
#include "kernels.h"

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
                     const float *out, const void *ws, size_t ws_bytes, int op) {
    ra_status s = check_config(c);
    if (s) return s;
    if ((s = check_rows(c, r))) return s;
    if (r->n_rows > 0 && (!k || !v || !sel || !out)) return fail(RA_EINVAL, "NULL K, V, sel or out");
    const ra::RowArgs a = row_args(c, r);
    const int NW = ra::max_window_spans(a.S, a.W);
    if (op == RA_OP_DECODE) {
        const int64_t nsub = ra::ceil_div(a.S, 64);  // upper bound on sub-tiles per span
        if (a.n_rows * a.Hkv * (int64_t)(a.G * a.k + NW) * nsub >= kMaxGrid)
            return fail(RA_EUNSUPPORTED, "decode grid too large: use fewer rows per call");
    } else {
        if (a.n_rows * a.Hq * (int64_t)(a.k + NW) >= kMaxGrid)
            return fail(RA_EUNSUPPORTED, "prefill has more than 2^31 (row, head, span) entries: split the chunk");
        if ((int64_t)a.B * a.Hkv * ra::ceil_div(a.cap, a.S) >= kMaxGrid)
            return fail(RA_EUNSUPPORTED, "too many (sequence, kv head, span) buckets");
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

ra_status routed_attn_decode(const ra_config *cfg, const ra_rows *rows, const void *k_cache, const void *v_cache,
                             const int32_t *sel, float *out, void *workspace, size_t workspace_bytes, void *stream) {
    ra_status s = check_attn(cfg, rows, k_cache, v_cache, sel, out, workspace, workspace_bytes, RA_OP_DECODE);
    if (s) return s;
    if (rows->n_rows == 0) return ok();
    return hip_status(ra::launch_decode(row_args(cfg, rows), k_cache, v_cache, sel, out, workspace, (hipStream_t)stream),
                      "routed_attn_decode launch");
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
    ra_status s = check_attn(cfg, rows, k_codes, v_codes, sel, out, workspace, workspace_bytes, RA_OP_DECODE);
    if (s) return s;
    if (cfg->dtype != RA_BF16) return fail(RA_EUNSUPPORTED, "8-bit caches go with bf16 queries (cfg->dtype RA_BF16)");
    if (rows->n_rows > 0 && (!k_scales || !v_scales)) return fail(RA_EINVAL, "NULL k_scales or v_scales");
    if (rows->n_rows == 0) return ok();
    return hip_status(ra::launch_decode_fp8(row_args(cfg, rows), k_codes, v_codes, k_scales, v_scales, sel, out,
                                            workspace, (hipStream_t)stream),
                      "routed_attn_decode_fp8 launch");
}

size_t ra_workspace_bytes(const ra_config *cfg, int32_t op, int64_t n_rows, int64_t max_pos) {
    if (check_config(cfg)) return 0;
    if (op != RA_OP_DECODE && op != RA_OP_PREFILL) {
        fail(RA_EINVAL, "op must be RA_OP_DECODE or RA_OP_PREFILL");
        return 0;
    }
    ra_rows r{nullptr, nullptr, nullptr, n_rows, max_pos};
    if (n_rows < 0 || max_pos < 0 || max_pos >= cfg->capacity) {
        fail(RA_EINVAL, "n_rows must be >= 0 and max_pos in [0, capacity)");
        return 0;
    }
    const ra::RowArgs a = row_args(cfg, &r);
    return op == RA_OP_DECODE ? ra::decode_workspace_bytes(a) : ra::prefill_workspace_bytes(a);
}

const char *ra_status_string(int32_t status) {
    switch (status) {
        case RA_OK: return "ok";
        case RA_EINVAL: return "invalid argument";
        case RA_EUNSUPPORTED: return "unsupported configuration";
        case RA_ECAPACITY: return "buffer too small";
        case RA_EHIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char *ra_last_error(void) { return g_err; }

}  // extern "C"
