/*
 * routed_attn.h -- C ABI of the MI355X (gfx950) content-routed sparse attention library.
 *
 * The method (release post "Experimental model with subquadratic attention: 100 tok/s @ 1M
 * context, 76 tok/s @ 10M context (30B model, single GPU)", section "Key idea"): the key/value
 * cache of a sequence is cut into spans of S consecutive tokens (about sqrt(L) of them); each
 * query scores every span, keeps the top-k spans, and runs token-level softmax attention over
 * the tokens of those spans plus a local window, for O(L^(3/2)) total work.  The post does not
 * fix the details; this library computes the following, step by step:
 *
 *   span summary      mean_j = (fp32 running sum of keys jS .. jS+S-1, in token order) / S
 *   window            w0(t) = S * floor(max(0, t-W+1) / S);  window = [w0(t), t]
 *   routable spans    j < r(t) = w0(t) / S   (complete spans wholly before the window)
 *   score             s_j = q . kappa(mean_j)   (kappa = round-to-nearest-even to bf16 for bf16
 *                     inputs, identity for fp32; no 1/sqrt(d) factor)
 *   selection         m = min(k, r(t)) spans by (score descending, span index ascending)
 *   attention         softmax(q . k_p / sqrt(d)) over p in window U selected spans; O = sum w_p v_p
 *
 * Each (token, query head) row routes on its own; query head h uses kv head h / (Hq / Hkv).
 *
 * Conventions shared by every entry point
 *  - Every pointer argument except `cfg`/`rows` (host structs) is DEVICE memory owned by the
 *    caller.  The library allocates nothing and keeps no state between calls.
 *  - All work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null stream).
 *    No call synchronises with the host.
 *  - Arguments are validated on the host before anything is launched.  On error the call
 *    returns a non-zero ra_status, records a message (ra_last_error, per thread) and launches
 *    nothing.  RA_EHIP reports a launch failure; outputs are then undefined.
 *  - Values that live in device memory (row positions, sequence ids, lengths, selections) are
 *    trusted but clamped before use, so a wrong value gives a wrong result, never an access
 *    outside the buffers described here.
 *
 * Layouts (all dense, row-major, innermost dimension contiguous)
 *  - K cache, V cache : [batch][Hkv][capacity][d], dtype of cfg (fp32, or bf16 bit patterns).
 *  - span_mean        : [batch][Hkv][max_spans][d] float.  Slot j holds the mean of span j once
 *                       that span is complete; other slots are not read.
 *  - run_sum          : [batch][Hkv][d] float, fp32 sum of the open span's keys; zero it before
 *                       the first update of a sequence.
 *  - q                : [n_rows][Hq][d], dtype of cfg.
 *  - scores           : [n_rows][Hq][score_stride] float; entry j < r(t) holds s_j.
 *  - sel              : [n_rows][Hq][k] int32; the m selected span ids ascending, then -1.
 *  - out              : [n_rows][Hq][d] float.
 */
#ifndef ROUTED_ATTN_H
#define ROUTED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RA_OK = 0,
    RA_EINVAL = 1,       /* null pointer, inconsistent sizes, out-of-range parameter */
    RA_EUNSUPPORTED = 2, /* valid but not implemented: head_dim, dtype, top_k, group size */
    RA_ECAPACITY = 3,    /* a buffer is too small (capacity, max_spans, score_stride, workspace) */
    RA_EHIP = 4,         /* the HIP runtime reported an error when launching */
    RA_EIO = 5,          /* a file could not be opened, read or written */
    RA_EFORMAT = 6       /* bytes that are not a snapshot this library can read */
} ra_status;

typedef enum { RA_F32 = 0, RA_BF16 = 1 } ra_dtype;

typedef enum { RA_OP_DECODE = 0, RA_OP_PREFILL = 1, RA_OP_ROUTE_TOPK = 2 } ra_op;

/* Shapes and method parameters.  Supported: head_dim in {64, 128}; num_q_heads a multiple of
 * num_kv_heads with Hq/Hkv <= 32; 1 <= top_k <= 64; span_size >= 1; window >= 1;
 * max_spans >= floor(capacity / span_size). */
typedef struct {
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t span_size;
    int32_t top_k;
    int32_t window;
    int32_t dtype;     /* ra_dtype of q, K and V */
    int32_t batch;     /* sequences in the cache */
    int64_t capacity;  /* token slots per (sequence, kv head) */
    int64_t max_spans; /* summary slots per (sequence, kv head) */
} ra_config;

/* Query rows.  Row i belongs to sequence row_seq[i] and sits at position row_pos[i]; its own
 * K/V must already be in the cache (decode: the new token; prefill: the whole chunk). */
typedef struct {
    const void *q;          /* device [n_rows][Hq][d] */
    const int32_t *row_seq; /* device [n_rows], each in [0, batch) */
    const int64_t *row_pos; /* device [n_rows], each in [0, max_pos] */
    int64_t n_rows;
    int64_t max_pos; /* host-side upper bound on row_pos (< capacity), sizes grids and checks */
} ra_rows;

/*
 * span_summary_update -- append tokens [old_len[b], new_len[b]) of every sequence b to its
 * span summaries (the span summary of the method; release post, "Key idea").  Keys are added
 * to the open span's fp32 running sum one token at a time in position order; when a span
 * completes its mean (sum / S, IEEE division) is written to span_mean and the sum restarts at
 * zero.  Incremental updates are bit-identical to a single update over the whole range.
 *   k_cache        device K cache (layout above)
 *   span_mean      device [batch][Hkv][max_spans][d] float (written)
 *   run_sum        device [batch][Hkv][d] float (read and written)
 *   old_len/new_len device int64 [batch]; new_len <= capacity; equal values = no-op
 *   max_new_tokens host bound on new_len[b] - old_len[b] (used to size the grid; a larger
 *                  device value leaves the excess spans unprocessed)
 */
ra_status span_summary_update(const ra_config *cfg, const void *k_cache, float *span_mean, float *run_sum,
                              const int64_t *old_len, const int64_t *new_len, int64_t max_new_tokens,
                              void *stream);

/*
 * route_scores -- every row scores every routable span of its sequence (release post, "Key
 * idea": score the O(L^0.5) candidate spans):  scores[row][h][j] = q[row][h] . kappa(mean_j)
 * for j < r(row_pos[row]); other entries are not written.  bf16 inputs run on bf16 MFMA with
 * fp32 accumulation; fp32 inputs use fp32 FMA.
 *   score_stride   floats per (row, head) in `scores`; must be >= r(max_pos).  A multiple of 32
 *                  (rows starting on 128-byte cache lines) lets the bf16 kernel write whole
 *                  lines, which is much faster when many rows are scored.
 */
ra_status route_scores(const ra_config *cfg, const ra_rows *rows, const float *span_mean, float *scores,
                       int64_t score_stride, void *stream);

/*
 * topk_spans -- per (row, head): keep the m = min(k, r) best routable spans by (score
 * descending, index ascending), written ascending and padded with -1 (release post, "Key
 * idea": select the top k).  One 64-lane wavefront per row.
 */
ra_status topk_spans(const ra_config *cfg, const ra_rows *rows, const float *scores, int64_t score_stride,
                     int32_t *sel, void *stream);

/*
 * route_topk_spans -- route_scores then topk_spans in one call: the same selection, bit for bit
 * (both paths compute route_scores' scores with route_scores' own arithmetic).
 *   - few rows (decode), r(max_pos) <= 1088: one launch; the blocks score the spans into the
 *     workspace and the last block of each (row, kv head) to finish selects for its query heads;
 *   - otherwise (many bf16 rows, as in a prefill chunk, or more spans): route_scores, then
 *     topk_spans, through the workspace.
 *   workspace      device memory of at least ra_workspace_bytes(cfg, RA_OP_ROUTE_TOPK, n_rows,
 *                  max_pos) bytes: n_rows x Hkv counters, then room for the scores.  The counters
 *                  must be zero before the first call (clear a new workspace once); every call
 *                  leaves them zero.  Calls that share a workspace must not overlap.
 */
ra_status route_topk_spans(const ra_config *cfg, const ra_rows *rows, const float *span_mean, int32_t *sel,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * routed_attn_decode -- exact softmax attention of each row over its window and its selected
 * spans (release post, "Key idea": token-level attention inside the chosen spans), tuned for
 * few rows per sequence: the spans chosen by the query heads that share a kv head are read
 * once and split into sub-tiles across the GPU, and the partial softmax states are merged in
 * a second kernel (log-sum-exp, fixed order: results do not depend on scheduling).
 * Entries of `sel` outside [0, r(t)) are ignored, and so is an entry that repeats an earlier
 * entry of the same (row, head).
 *   workspace      device scratch of at least ra_workspace_bytes(cfg, RA_OP_DECODE, n_rows,
 *                  max_pos) bytes; contents on entry do not matter.
 */
ra_status routed_attn_decode(const ra_config *cfg, const ra_rows *rows, const void *k_cache, const void *v_cache,
                             const int32_t *sel, float *out, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * routed_attn_decode_noalloc -- routed_attn_decode for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  The same kernels and the same results, bit for bit; the partial records
 * go to a device array inside the library, fixed at 32 MiB per GPU and held until the process
 * ends (its address is looked up on the first call on each device).  No allocation, no
 * host synchronisation.
 *   Limit: ra_workspace_bytes(cfg, RA_OP_DECODE, n_rows, max_pos) <= 32 MiB, else RA_ECAPACITY
 *   (32 query heads, d 128, top-16, window = span: about 1.16 MiB per row at spans of 1024,
 *   0.58 MiB per row at spans of 512, 4.6 MiB per row at spans of 4096).
 *   Calls that overlap on one GPU (other streams, other threads) share the array and race:
 *   serialise them.  Every call writes every record it reads, so nothing needs clearing.
 */
ra_status routed_attn_decode_noalloc(const ra_config *cfg, const ra_rows *rows, const void *k_cache,
                                     const void *v_cache, const int32_t *sel, float *out, void *stream);

/*
 * routed_attn_prefill -- the same result for many rows (a chunk of new tokens, causal in the
 * chunk).  Rows are grouped span by span (every (sequence, kv head, span) gathers the rows
 * that attend to it, as selected span or as window span), each group runs as dense tiles over
 * the span's keys, and the per-span partial states are merged per row in entry order.  A row's
 * result does not depend on the other rows of the call.  Entries of `sel` outside [0, r(t))
 * are ignored, and so is an entry that repeats an earlier entry of the same (row, head).
 *   workspace      at least ra_workspace_bytes(cfg, RA_OP_PREFILL, n_rows, max_pos) bytes.
 */
ra_status routed_attn_prefill(const ra_config *cfg, const ra_rows *rows, const void *k_cache, const void *v_cache,
                              const int32_t *sel, float *out, void *workspace, size_t workspace_bytes,
                              void *stream);

/*
 * attn_dense_causal -- exact softmax attention of each row over every key of its sequence at or
 * before its position: the brute-force scan that routing replaces (release post, "Key idea"),
 * and the "k = all spans" case of the method (with k >= r(t) the routed result equals it).  It
 * is the reference the routed path is measured against.  Rows are taken in tiles of 128 / G
 * consecutive rows x the G query heads of a kv head; rows of several sequences in one tile are
 * handled in successive passes, so a call is fastest when rows come grouped by sequence (as a
 * prefill chunk does).
 *   Supported: bf16 inputs (RA_EUNSUPPORTED otherwise), capacity * head_dim < 2^31.
 *   k_cache, v_cache  [batch][Hkv][capacity][d]; out [n_rows][Hq][d] float.  No workspace.
 */
ra_status attn_dense_causal(const ra_config *cfg, const ra_rows *rows, const void *k_cache, const void *v_cache,
                            float *out, void *stream);

/*
 * 8-bit K/V cache.  The release post ("Limitations and next steps") plans 8-bit quantisation
 * without a format; this library's: every (sequence, kv head, token) row of d values is stored
 * as FP8 E4M3 codes (finite variant: bias 7, subnormals, largest value 448, no infinity) with
 * one fp32 scale s = max|x| / 448 (1 for an all-zero row); code = E4M3(x / s) rounded to nearest
 * even after clamping to +-448.  The cache then holds fl32(E4M3^-1(code) * s), and summaries,
 * routing and attention read those values; queries stay bf16 (cfg->dtype = RA_BF16) and routing
 * rounds the means to bf16 as for a bf16 cache.
 * Layouts: codes [batch][Hkv][capacity][d] uint8, scales [batch][Hkv][capacity] float.
 */

/* kv_quantize_fp8 -- quantise rows [old_len[b], new_len[b]) of every (sequence b, kv head) of a
 * bf16 cache (layout above) into codes and scales; other rows are not touched.  Call it once for
 * K and once for V.  max_new_tokens: host bound on new_len[b] - old_len[b] (sizes the grid). */
ra_status kv_quantize_fp8(const ra_config *cfg, const void *src_cache, uint8_t *codes, float *scales,
                          const int64_t *old_len, const int64_t *new_len, int64_t max_new_tokens, void *stream);

/* span_summary_update_fp8 -- span_summary_update over an 8-bit K cache: the running sums add the
 * cache's values fl32(E4M3^-1(code) * s) in token order (same contract otherwise). */
ra_status span_summary_update_fp8(const ra_config *cfg, const uint8_t *k_codes, const float *k_scales,
                                  float *span_mean, float *run_sum, const int64_t *old_len, const int64_t *new_len,
                                  int64_t max_new_tokens, void *stream);

/* routed_attn_decode_fp8 -- routed_attn_decode over an 8-bit K/V cache (bf16 queries): half the
 * K/V bytes of a bf16 cache per step.  Scores are s_k * (q . codes) and the weights carry s_v;
 * same workspace size and contract as routed_attn_decode. */
ra_status routed_attn_decode_fp8(const ra_config *cfg, const ra_rows *rows, const uint8_t *k_codes,
                                 const uint8_t *v_codes, const float *k_scales, const float *v_scales,
                                 const int32_t *sel, float *out, void *workspace, size_t workspace_bytes,
                                 void *stream);

/* routed_attn_prefill_fp8 -- routed_attn_prefill over an 8-bit K/V cache (bf16 queries), the
 * path a chunk of new tokens takes when the cache is stored in 8 bits (the release post's
 * "Limitations and next steps" plan 8-bit quantisation so that long contexts fit).  The same
 * grouping, tiles and merge as routed_attn_prefill: each tile converts a staged chunk of codes
 * exactly to bf16 for the MFMAs and applies the rows' scales to the scores (keys) and to the P.V
 * weights (values), with fp32 softmax state.  Same workspace size as routed_attn_prefill; the
 * same handling of repeated and unroutable selection entries. */
ra_status routed_attn_prefill_fp8(const ra_config *cfg, const ra_rows *rows, const uint8_t *k_codes,
                                  const uint8_t *v_codes, const float *k_scales, const float *v_scales,
                                  const int32_t *sel, float *out, void *workspace, size_t workspace_bytes,
                                  void *stream);

/* routed_attn_decode_append / routed_attn_decode_fp8_append -- the decode call together with
 * the step's summary update: the same as routed_attn_decode (resp. _fp8) followed by
 * span_summary_update (resp. _fp8) of tokens [old_len[b], new_len[b]) into span_mean / run_sum.
 * The update reads only K and writes only the summaries, which the attention does not read, so
 * with one new token per sequence (max_new_tokens = 1) it runs inside the attention's merge
 * launch (one launch less per decode step); otherwise it runs as its own launches after the
 * merge.  A decode step can call route_scores and topk_spans first and this last: the span that
 * the token at position t completes is never routable at t (it lies in the window), and the
 * running sum is not read by routing, so routing before the update selects what it would
 * select after it. */
ra_status routed_attn_decode_append(const ra_config *cfg, const ra_rows *rows, const void *k_cache,
                                    const void *v_cache, const int32_t *sel, float *out, void *workspace,
                                    size_t workspace_bytes, float *span_mean, float *run_sum, const int64_t *old_len,
                                    const int64_t *new_len, int64_t max_new_tokens, void *stream);
ra_status routed_attn_decode_fp8_append(const ra_config *cfg, const ra_rows *rows, const uint8_t *k_codes,
                                        const uint8_t *v_codes, const float *k_scales, const float *v_scales,
                                        const int32_t *sel, float *out, void *workspace, size_t workspace_bytes,
                                        float *span_mean, float *run_sum, const int64_t *old_len,
                                        const int64_t *new_len, int64_t max_new_tokens, void *stream);

/* ------------------------------------------------------- token-level cold retrieval
 * A second way to reach old context (InfiniteKV post): the last H positions (the hot window)
 * are attended exactly; every older ("cold") position is found by a Hamming scan over compact
 * signatures, and the top_k_cold nearest are attended together with the hot window.  The post
 * fixes no signature format; this library computes, for a row at position t with query q:
 *
 *   signature     sig(x) = the d sign bits of x (bit e set iff element e has its sign bit set,
 *                 -0 included), packed little-endian: bit e is bit e % 8 of byte e / 8
 *   cold set      positions [0, t-H+1);  hot window [max(0, t-H+1), t]
 *   distance      popcount(sig(q) xor sig(k_p)) (integers: the selection is exact)
 *   selection     m = min(top_k_cold, |cold set|) positions by (distance ascending, position
 *                 ascending), listed ascending and padded with -1
 *   attention     softmax(q . k_p / sqrt(d)) over selection U hot window; O = sum w_p v_p
 *
 * Query head h reads kv head h / (Hq / Hkv).  Layouts: sig [batch][Hkv][capacity][d/8] uint8
 * (16-byte aligned), sel_cold [n_rows][Hq][top_k_cold] int32, out [n_rows][Hq][d] float; K, V, q
 * as above.  Supported: 1 <= top_k_cold <= 128, hot_window >= 1, capacity < 2^31, at most
 * 4096 scan tiles of cold positions per row (tiles of 16384 positions when a kv head serves at
 * most 8 query heads, else 8192; cold_select returns RA_EUNSUPPORTED beyond).  The span
 * fields of cfg (span_size, top_k, window) are validated but not used by these calls. */

/* kv_signature_update -- signatures of K rows [old_len[b], new_len[b]) of every (sequence b, kv
 * head); other rows are not touched.  max_new_tokens: host bound on new_len[b] - old_len[b]. */
ra_status kv_signature_update(const ra_config *cfg, const void *k_cache, uint8_t *sig, const int64_t *old_len,
                              const int64_t *new_len, int64_t max_new_tokens, void *stream);

/* Workspace bytes of cold_select (per-tile candidate lists); 0 if the arguments are invalid. */
size_t ra_cold_workspace_bytes(const ra_config *cfg, int64_t n_rows, int64_t max_pos, int32_t hot_window,
                               int32_t top_k_cold);

/* cold_select -- the Hamming scan and selection of every (row, query head): sel_cold as above.
 * Reads each signature of a row's cold set once per kv head (scored against all its query
 * heads); workspace of at least ra_cold_workspace_bytes bytes. */
ra_status cold_select(const ra_config *cfg, const ra_rows *rows, const uint8_t *sig, int32_t hot_window,
                      int32_t top_k_cold, int32_t *sel_cold, void *workspace, size_t workspace_bytes, void *stream);

/* cold_attn_decode -- exact attention of each row over its selected cold positions and its hot
 * window; out as above.  Entries outside the row's cold set [0, t-H+1) (the -1 padding among
 * them) are ignored, and so is an entry that repeats an earlier entry of the same row-head, so
 * no position is counted twice. */
ra_status cold_attn_decode(const ra_config *cfg, const ra_rows *rows, const void *k_cache, const void *v_cache,
                           const int32_t *sel_cold, int32_t hot_window, int32_t top_k_cold, float *out, void *stream);

/* ---------------------------------------------------------------- session snapshots
 * Keeping the cache instead of reprocessing it, with sessions saved to and restored from disk
 * (release post, on why fast long context matters; its stack lists session snapshots), with
 * every saved byte covered by SHA-256 digests in the spirit of the InfiniteKV post's hashed
 * receipts.  The image format is the library's own; all integers little-endian:
 *
 *   header   64 bytes of fields, then int64 lengths[B], zero-padded to a multiple of 16 bytes:
 *              0 magic "CRSASNP1" | 8 u32 version 1 | 12 u32 element type (0 fp32, 1 bf16,
 *                2 the 8-bit cache: E4M3 codes + fp32 row scales)
 *             16 u32 B | 20 u32 Hkv | 24 u32 d | 28 u32 S | 32 u64 payload bytes
 *             40 u64 header bytes | 48 u32 chunk bytes 4096 | 52 u32 fan-in 16 | 56 u64 0
 *   payload  for b, for g: K[b][g][0:L_b][:] then V[b][g][0:L_b][:] (cache element bytes; for
 *            element type 2 the codes, then k_scale[b][g][0:L_b] and v_scale[b][g][0:L_b] (fp32),
 *            each run zero-padded to a multiple of 16 bytes);
 *            then for b, for g: span_mean[b][g][0:floor(L_b/S)][:] then run_sum[b][g][:] (fp32)
 *   levels   D_1 = SHA-256 (FIPS 180-4) of each 4096-byte chunk of header|payload (the last one
 *            may be short); D_(l+1) = SHA-256 of each group of 16 digests (512 bytes) of D_l while
 *            |D_l| > 16; root = SHA-256 of the last level.
 *   image    header | payload | D_1 | ... | D_m | root
 *
 * Only live state is saved (rows [0, L_b), complete span means, the running sums); restoring
 * writes exactly those and leaves every other row and slot of the destination untouched.
 * `lengths` arguments are HOST arrays of cfg->batch int64 token counts; `header` arguments are
 * HOST copies of the first bytes of an image (at least the header); `image` is DEVICE memory.
 * The 8-bit cache (the release post's planned quantised cache, "Limitations and next steps")
 * has its own pack / unpack / size calls (element type 2); parse and verify read every type. */

#define RA_SNAPSHOT_E4M3 2 /* element type of images of the 8-bit cache */

typedef struct {
    int32_t dtype;         /* element type of the saved K/V rows: ra_dtype, or RA_SNAPSHOT_E4M3 */
    int32_t batch;         /* B */
    int32_t num_kv_heads;  /* Hkv */
    int32_t head_dim;      /* d */
    int32_t span_size;     /* S */
    int32_t reserved;
    uint64_t header_bytes;
    uint64_t payload_bytes;
    uint64_t image_bytes;  /* whole image including digest levels and root */
} ra_snapshot_info;

/* Image bytes for the given host lengths[cfg->batch]; 0 if cfg or a length is invalid. */
size_t kv_snapshot_bytes(const ra_config *cfg, const int64_t *lengths);

/* kv_snapshot_pack -- write the image of the cache state (K/V caches, span_mean, run_sum in the
 * layouts above; lengths: host) into the device buffer `image` of at least kv_snapshot_bytes
 * bytes: header, payload copies and every digest level, all enqueued on `stream`. */
ra_status kv_snapshot_pack(const ra_config *cfg, const void *k_cache, const void *v_cache, const float *span_mean,
                           const float *run_sum, const int64_t *lengths, void *image, size_t image_bytes,
                           void *stream);

/* kv_snapshot_parse -- read a header (host bytes, `header_avail` of them) into `info` and, when
 * `lengths` is not NULL, its B lengths (B <= max_batch).  RA_EFORMAT for anything but a header
 * written by kv_snapshot_pack (magic, version, chunk size, fan-in, sizes consistent). */
ra_status kv_snapshot_parse(const void *header, size_t header_avail, ra_snapshot_info *info, int64_t *lengths,
                            int32_t max_batch);

/* kv_snapshot_verify -- recompute every digest of a device image and compare it with the stored
 * one.  Writes to the device word *bad_offset: UINT64_MAX if all match, else the smallest image
 * offset of a chunk whose digest differs (the root's chunk is the whole last level). */
ra_status kv_snapshot_verify(const void *header, size_t header_avail, const void *image, size_t image_bytes,
                             uint64_t *bad_offset, void *stream);

/* kv_snapshot_unpack -- copy the saved state of a device image into K/V caches, span_mean and
 * run_sum laid out per cfg (same dtype, Hkv, d and S as the image; image B <= cfg->batch; each
 * length <= capacity).  If `guard` (device) is not NULL the copies run only when *guard reads
 * UINT64_MAX, so unpack after verify on one stream restores nothing from a damaged image. */
ra_status kv_snapshot_unpack(const ra_config *cfg, const void *header, size_t header_avail, const void *image,
                             size_t image_bytes, const uint64_t *guard, void *k_cache, void *v_cache,
                             float *span_mean, float *run_sum, void *stream);

/* kv_snapshot_bytes, _pack and _unpack for the 8-bit cache (image element type 2): codes
 * [B][Hkv][capacity][d] (uint8, 16-byte aligned) and one fp32 scale per row [B][Hkv][capacity]
 * (4-byte aligned) for K and V, as kv_quantize_fp8 writes them; cfg->dtype plays no part.
 * Unpack restores codes, scales and summaries of the live rows only, as above. */
size_t kv_snapshot_bytes_fp8(const ra_config *cfg, const int64_t *lengths);
ra_status kv_snapshot_pack_fp8(const ra_config *cfg, const uint8_t *k_codes, const uint8_t *v_codes,
                               const float *k_scales, const float *v_scales, const float *span_mean,
                               const float *run_sum, const int64_t *lengths, void *image, size_t image_bytes,
                               void *stream);
ra_status kv_snapshot_unpack_fp8(const ra_config *cfg, const void *header, size_t header_avail, const void *image,
                                 size_t image_bytes, const uint64_t *guard, uint8_t *k_codes, uint8_t *v_codes,
                                 float *k_scales, float *v_scales, float *span_mean, float *run_sum, void *stream);

/* Host file helpers: write `bytes` bytes (through a temporary file renamed into place), or read
 * a whole file into `buf` (capacity bytes); with buf NULL only *bytes (the file size) is set. */
ra_status kv_snapshot_write_file(const char *path, const void *data, size_t bytes);
ra_status kv_snapshot_read_file(const char *path, void *buf, size_t capacity, size_t *bytes);

/* Workspace bytes needed by routed_attn_decode / routed_attn_prefill / route_topk_spans (op =
 * ra_op); 0 if the
 * configuration is invalid (ra_last_error then says why). */
size_t ra_workspace_bytes(const ra_config *cfg, int32_t op, int64_t n_rows, int64_t max_pos);

/* Static description of a status code. */
const char *ra_status_string(int32_t status);

/* Message of the last non-OK return on the calling thread ("" if none). */
const char *ra_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ROUTED_ATTN_H */
