// Internal launch interface between the C ABI layer (abi.hip) and the kernel files.
// Arguments arrive here already validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

// Element types of a K/V cache (internal): the config's dtype, or 8-bit codes with row scales.
constexpr int kCacheFp8 = 2;

struct SummaryArgs {
    const void *k;
    const float *kscale;  // per (sequence, kv head, token) scales of an 8-bit cache, else unused
    float *mean, *run_sum;
    const int64_t *old_len, *new_len;
    int dtype, d, B, Hkv, S;
    int64_t cap, max_spans, max_new;
};

struct RowArgs {  // query rows and shapes shared by routing, selection and attention
    const void *q;
    const int32_t *row_seq;
    const int64_t *row_pos;
    int64_t n_rows, max_pos;
    int dtype, d, Hq, Hkv, G, S, k, W, B;
    int64_t cap, max_spans;
};

hipError_t launch_summary(const SummaryArgs &a, hipStream_t st);

// 8-bit cache: quantise rows [old_len[b], new_len[b]) of a bf16 cache into codes and scales.
struct QuantArgs {
    const uint16_t *src;
    uint8_t *dst;
    float *scale;
    const int64_t *old_len, *new_len;
    int d, B, Hkv;
    int64_t cap, max_new;
};
hipError_t launch_quantize_fp8(const QuantArgs &a, hipStream_t st);
hipError_t launch_route(const RowArgs &a, const float *mean, float *scores, int64_t stride, hipStream_t st);
hipError_t launch_topk(const RowArgs &a, const float *scores, int64_t stride, int32_t *sel, hipStream_t st);
// Routing and selection in one launch (few rows): the workspace holds one counter per (row, kv
// head) -- zero before the first call, zero again after each -- and the scores.
size_t route_topk_workspace_bytes(const RowArgs &a);
hipError_t launch_route_topk(const RowArgs &a, const float *mean, int32_t *sel, void *ws, hipStream_t st);

// Decode: workspace holds partial records [n_rows][Hq][k + max_window_spans][n_sub].
size_t decode_workspace_bytes(const RowArgs &a);
// Work-items (blocks x threads) of the largest launch of a decode call (bf16/fp32 cache, or the
// 8-bit cache with fp8 = true); a launch needs fewer than 2^32 per grid dimension.
int64_t decode_grid_items(const RowArgs &a, bool fp8);
hipError_t launch_decode(const RowArgs &a, const void *K, const void *V, const int32_t *sel, float *out,
                         void *ws, hipStream_t st);
// Decode over an 8-bit cache (bf16 queries): codes K8/V8 with row scales ks/vs.
hipError_t launch_decode_fp8(const RowArgs &a, const uint8_t *K8, const uint8_t *V8, const float *ks,
                             const float *vs, const int32_t *sel, float *out, void *ws, hipStream_t st);

// Prefill: span-major dispatch + tiles + merge.
size_t prefill_workspace_bytes(const RowArgs &a);
int64_t prefill_grid_items(const RowArgs &a);  // as decode_grid_items
hipError_t launch_prefill(const RowArgs &a, const void *K, const void *V, const int32_t *sel, float *out,
                          void *ws, hipStream_t st);
// Prefill over an 8-bit cache (bf16 queries): codes K8/V8 with row scales ks/vs; the same
// workspace as bf16.
hipError_t launch_prefill_fp8(const RowArgs &a, const uint8_t *K8, const uint8_t *V8, const float *ks,
                              const float *vs, const int32_t *sel, float *out, void *ws, hipStream_t st);

// Dense causal attention (bf16): every key at or before each row's position; no workspace.
hipError_t launch_dense(const RowArgs &a, const void *K, const void *V, float *out, hipStream_t st);

}  // namespace ra
