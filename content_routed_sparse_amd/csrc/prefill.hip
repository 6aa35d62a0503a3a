// Prefill attention: the same exact attention for a chunk of many rows (release post, "Key
// idea"; the post's stack processes long prompts by chunked prefill).
//
// Rows that attend to the same span share its keys, so the work is regrouped span by span, the
// way tokens are dispatched to experts: every (row-head, entry) pair -- entries are the k
// selected spans and the window spans of the row -- is appended to the bucket of its
// (sequence, kv head, span).  Buckets are cut into tiles of at most MT entries, a tile runs as
// one block over the span's keys (a dense Q.K^T / softmax / P.V on MFMA for bf16), and the
// per-span partial softmax states are merged per row in fixed order by the combine kernel.
// Keys after a row's own position are masked (only window spans can contain them).  Slots in a
// bucket are handed out by atomics, so which entries share a tile varies from run to run; the
// results do not: every entry's partial state is computed from its own query and the span's
// keys alone (the tile kernels decide a second pass per entry, not per tile), and the merge
// adds a row's records in entry order.
//
// Workspace (all offsets 256-byte aligned):
//   counts[n_exp+1], offsets[n_exp+1], tile_off[n_exp+1]   int32
//   local[n_ent], list[n_ent]                               int32   (n_ent = n_rowheads * NE)
//   list_t[n_ent]                                           int64   (position of the entry's row)
//   tiles[max_tiles]                                        int4    (expert, first entry, entries),
//                                                                   tile t at slot 8 (t mod Q) + t / Q
//   records[n_ent]                                          prefill_record_words(d, bf16) x 4 bytes
#include "common.h"
#include "kernels.h"
#include "prefill_tiles.h"
#include "wave_ops.h"

namespace ra {
namespace {

struct PrefillLayout {
    int64_t n_exp, n_ent, max_tiles, span_slots;
    size_t off_counts, off_offsets, off_tile_off, off_local, off_list, off_list_t, off_tiles, off_records, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

PrefillLayout prefill_layout(const RowArgs &a) {
    PrefillLayout L;
    const int NE = a.k + max_window_spans(a.S, a.W);
    L.span_slots = ceil_div(a.cap, a.S);
    L.n_exp = (int64_t)a.B * a.Hkv * L.span_slots;
    L.n_ent = a.n_rows * a.Hq * NE;
    const int MT = prefill_tile_rows(a);
    // an upper bound on the tile count (every bucket's last tile may be partial), rounded up to a
    // multiple of 8 so that the XCD-ordered descriptor slots of any tile count fit
    L.max_tiles = 8 * ceil_div(ceil_div(L.n_ent, MT) + (L.n_exp < L.n_ent ? L.n_exp : L.n_ent), 8);
    size_t o = 0;
    L.off_counts = o;   o = align256(o + (L.n_exp + 1) * 4);
    L.off_offsets = o;  o = align256(o + (L.n_exp + 1) * 4);
    L.off_tile_off = o; o = align256(o + (L.n_exp + 1) * 4);
    L.off_local = o;    o = align256(o + L.n_ent * 4);
    L.off_list = o;     o = align256(o + L.n_ent * 4);
    L.off_list_t = o;   o = align256(o + L.n_ent * 8);
    L.off_tiles = o;    o = align256(o + L.max_tiles * 16);
    L.off_records = o;  o = align256(o + (size_t)L.n_ent * prefill_record_words(a.d, a.dtype == RA_BF16) * 4);
    L.total = o;
    return L;
}

__global__ void fill_i32(int32_t *p, int64_t n, int32_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// span id of entry e of a row-head; false if the entry attends to nothing: a selected span
// (e < k) outside [0, r(t)) or equal to an earlier entry of the same row-head, or a window span
// (e >= k) that starts after t.  (Selections from topk_spans are ascending and distinct; the
// repeat check serves caller-made selections, whose first occurrence counts, as in decode.)
__device__ __forceinline__ bool entry_span(const int32_t *sel, int64_t rh, int e, int k, int64_t t, int S, int W,
                                           int64_t &j) {
    const int64_t w0 = window_start(t, S, W);
    if (e < k) {
        const int32_t *row = sel + rh * k;
        j = row[e];
        // an entry that repeats an earlier entry of its row-head is not attended again; the
        // earlier entries are compared without early exit, so their loads go out together
        int rep = 0;
#pragma unroll 8
        for (int x = 0; x < e; ++x) rep |= row[x] == (int32_t)j;
        return j >= 0 && j < div_nonneg(w0, S) && rep == 0;
    }
    j = div_nonneg(w0, S) + (e - k);
    return j * S <= t;
}

// span id of an entry that entry_span accepted (no checks)
__device__ __forceinline__ int64_t valid_entry_span(const int32_t *sel, int64_t rh, int e, int k, int64_t t, int S,
                                                    int W) {
    return e < k ? (int64_t)sel[rh * k + e] : div_nonneg(window_start(t, S, W), S) + (e - k);
}

__global__ void count_kernel(const int32_t *__restrict__ sel, const int32_t *__restrict__ row_seq,
                             const int64_t *__restrict__ row_pos, int32_t *__restrict__ counts,
                             int32_t *__restrict__ local, int64_t n_ent, int NE, int Hq, int Hkv, int G, int S, int k,
                             int W, int B, int64_t max_pos, int64_t span_slots) {
    const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= n_ent) return;
    const int64_t rh = x / NE;
    const int e = (int)(x % NE);
    const int64_t row = rh / Hq;
    const int g = (int)(rh % Hq) / G;
    int64_t t = row_pos[row];
    t = t < 0 ? 0 : (t > max_pos ? max_pos : t);
    int seq = row_seq[row];
    seq = seq < 0 ? 0 : (seq >= B ? B - 1 : seq);
    int64_t j;
    int32_t slot = -1;
    if (entry_span(sel, rh, e, k, t, S, W, j)) {
        const int64_t expert = ((int64_t)seq * Hkv + g) * span_slots + j;
        slot = atomicAdd(&counts[expert], 1);
    }
    local[x] = slot;
}

// Same counts with far fewer global atomics: a block takes kCountRows rows x the G heads of one
// kv head, counts their entries per span in an LDS histogram (entries of other sequences than
// the block's first row go straight to the global counters), then adds each non-empty bin to
// the global counter once and hands the entries their final slots.
constexpr int kCountRows = 32;
constexpr int kCountMaxSpans = 8192;

__global__ void __launch_bounds__(256) count_kernel_lds(const int32_t *__restrict__ sel,
                                                        const int32_t *__restrict__ row_seq,
                                                        const int64_t *__restrict__ row_pos,
                                                        int32_t *__restrict__ counts, int32_t *__restrict__ local,
                                                        int64_t n_rows, int NE, int Hq, int Hkv, int G, int S, int k,
                                                        int W, int B, int64_t max_pos, int64_t span_slots) {
    __shared__ int32_t hist[kCountMaxSpans];
    const int tid = threadIdx.x;
    const int g = blockIdx.y;
    const int64_t r0 = (int64_t)blockIdx.x * kCountRows;
    const int64_t r1 = r0 + kCountRows < n_rows ? r0 + kCountRows : n_rows;
    int ref = row_seq[r0];
    ref = ref < 0 ? 0 : (ref >= B ? B - 1 : ref);
    for (int64_t j = tid; j < span_slots; j += 256) hist[j] = 0;
    __syncthreads();
    const int64_t per_row = (int64_t)G * NE;
    const int64_t n_ent = (r1 - r0) * per_row;
    for (int64_t y = tid; y < n_ent; y += 256) {
        const int64_t row = r0 + y / per_row;
        const int h = (int)((y % per_row) / NE), e = (int)(y % NE);
        const int64_t rh = row * Hq + (int64_t)g * G + h;
        const int64_t x = rh * NE + e;
        int64_t t = row_pos[row];
        t = t < 0 ? 0 : (t > max_pos ? max_pos : t);
        int seq = row_seq[row];
        seq = seq < 0 ? 0 : (seq >= B ? B - 1 : seq);
        int64_t j;
        int32_t slot = -1;
        if (entry_span(sel, rh, e, k, t, S, W, j)) {
            if (seq == ref) slot = atomicAdd(&hist[j], 1);  // rank within this block's bin
            else slot = -2 - atomicAdd(&counts[((int64_t)seq * Hkv + g) * span_slots + j], 1);
        }
        local[x] = slot;
    }
    __syncthreads();
    for (int64_t j = tid; j < span_slots; j += 256) {
        const int32_t c = hist[j];
        hist[j] = c > 0 ? atomicAdd(&counts[((int64_t)ref * Hkv + g) * span_slots + j], c) : 0;
    }
    __syncthreads();
    for (int64_t y = tid; y < n_ent; y += 256) {
        const int64_t row = r0 + y / per_row;
        const int h = (int)((y % per_row) / NE), e = (int)(y % NE);
        const int64_t rh = row * Hq + (int64_t)g * G + h;
        const int64_t x = rh * NE + e;
        const int32_t v = local[x];
        if (v >= 0) {
            int64_t t = row_pos[row];
            t = t < 0 ? 0 : (t > max_pos ? max_pos : t);
            local[x] = hist[valid_entry_span(sel, rh, e, k, t, S, W)] + v;
        } else if (v <= -2) {
            local[x] = -2 - v;  // slot taken directly in the global counter
        }
    }
}

// Exclusive scans of counts and of tiles per expert, in one block.
__global__ void __launch_bounds__(1024) scan_kernel(const int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                    int32_t *__restrict__ tile_off, int64_t n_exp, int MT) {
    __shared__ int32_t sa[1024], sb[1024];
    __shared__ int32_t carry_a, carry_b;
    const int tid = threadIdx.x;
    if (tid == 0) {
        carry_a = 0;
        carry_b = 0;
    }
    __syncthreads();
    for (int64_t base = 0; base < n_exp; base += 1024) {
        const int64_t i = base + tid;
        const int32_t c = i < n_exp ? counts[i] : 0;
        int32_t va = c, vb = (c + MT - 1) / MT;
        sa[tid] = va;
        sb[tid] = vb;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {  // Hillis-Steele inclusive scan
            const int32_t ta = tid >= off ? sa[tid - off] : 0;
            const int32_t tb = tid >= off ? sb[tid - off] : 0;
            __syncthreads();
            sa[tid] += ta;
            sb[tid] += tb;
            __syncthreads();
        }
        if (i < n_exp) {
            offsets[i] = carry_a + sa[tid] - va;
            tile_off[i] = carry_b + sb[tid] - vb;
        }
        __syncthreads();
        if (tid == 1023) {
            carry_a += sa[1023];
            carry_b += sb[1023];
        }
        __syncthreads();
    }
    if (tid == 0) {
        offsets[n_exp] = carry_a;
        tile_off[n_exp] = carry_b;
    }
}

__global__ void scatter_kernel(const int32_t *__restrict__ sel, const int32_t *__restrict__ row_seq,
                               const int64_t *__restrict__ row_pos, const int32_t *__restrict__ offsets,
                               const int32_t *__restrict__ local, int32_t *__restrict__ list,
                               int64_t *__restrict__ list_t, int64_t n_ent, int NE,
                               int Hq, int Hkv, int G, int S, int k, int W, int B, int64_t max_pos,
                               int64_t span_slots) {
    const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= n_ent) return;
    const int32_t slot = local[x];
    if (slot < 0) return;
    const int64_t rh = x / NE;
    const int e = (int)(x % NE);
    const int64_t row = rh / Hq;
    const int g = (int)(rh % Hq) / G;
    int64_t t = row_pos[row];
    t = t < 0 ? 0 : (t > max_pos ? max_pos : t);
    int seq = row_seq[row];
    seq = seq < 0 ? 0 : (seq >= B ? B - 1 : seq);
    const int64_t j = valid_entry_span(sel, rh, e, k, t, S, W);
    const int64_t expert = ((int64_t)seq * Hkv + g) * span_slots + j;
    list[offsets[expert] + slot] = (int32_t)x;
    list_t[offsets[expert] + slot] = t;
}

// Tile descriptors: (expert, first entry in the list, entries in the tile).  One wave per expert,
// its lanes taking the bucket's tiles in turn: the buckets of the spans inside a chunk's windows
// hold many times the entries of a routed span's bucket (one thread per expert left those few
// threads with a long serial loop of stores).
constexpr int kTilesWaves = 4;  // experts per block

__global__ void __launch_bounds__(kTilesWaves * 64) tiles_kernel(const int32_t *__restrict__ counts,
                                                                 const int32_t *__restrict__ offsets,
                                                                 const int32_t *__restrict__ tile_off,
                                                                 int4 *__restrict__ tiles, int64_t n_exp, int MT) {
    const int64_t x = (int64_t)blockIdx.x * kTilesWaves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (x >= n_exp) return;
    const int32_t c = counts[x];
    const int32_t base = tile_off[x];
    const int32_t first = offsets[x];
    const int32_t Q = (tile_off[n_exp] + 7) / 8;  // tiles per XCD
    for (int32_t i = lane; i * MT < c; i += 64) {
        const int32_t t = base + i;
        tiles[tile_slot(t, Q)] = make_int4((int32_t)x, first + i * MT, c - i * MT < MT ? c - i * MT : MT, 0);
    }
}


// A record exists for entry x of a row-head iff the dispatch gave the entry a slot (local >= 0):
// the same test as entry_span, taken once by the count kernel.

constexpr int kRecBatch = 8;

// This lane's slice of the output-sized part of a record: the values of elements
// lane + 64 i (fp32 records), or of elements 2 lane, 2 lane + 1 (fp16 records, d = 128) or
// lane (fp16 records, d = 64).
template <int D, bool HALF>
__device__ __forceinline__ void load_slice(const float *rec, int lane, float (&v)[D / 64]) {
    if constexpr (!HALF) {
#pragma unroll
        for (int i = 0; i < D / 64; ++i) v[i] = rec[4 + lane + 64 * i];
    } else if constexpr (D == 128) {
        typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
        const half2_t h = __builtin_bit_cast(half2_t, reinterpret_cast<const uint32_t *>(rec + 4)[lane]);
        v[0] = (float)h.x;
        v[1] = (float)h.y;
    } else {
        v[0] = (float)reinterpret_cast<const _Float16 *>(rec + 4)[lane];
    }
}

// Merge: one wave per row-head; lane x reads the header of record x, then the records are summed
// in entry order with their weights.  Each batch of kRecBatch records is loaded (indices
// clamped into range) and pinned before its first use: one memory round trip per batch.
//   fp32 records (m, l, -, -, o[d]):       out = sum 2^(m - M) o / sum 2^(m - M) l
//   fp16 records (m, l, s, -, h[d]), h = o / (l s):  o = 2^(m - M) l s h in the same sums
template <int D, bool HALF>
__global__ void __launch_bounds__(256) combine_wave(const float *__restrict__ part, const int32_t *__restrict__ local,
                                                    float *__restrict__ out, int64_t n_rowheads, int k, int NW) {
    constexpr int PER = D / 64;
    constexpr int RW = prefill_record_words(D, HALF);
    constexpr float kNegInf = -__builtin_huge_valf();
    const int lane = threadIdx.x & 63;
    const int64_t rh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (rh >= n_rowheads) return;
    const int nrec = k + NW;
    const int32_t *valid_rh = local + rh * (int64_t)nrec;  // slot of each entry, -1: no record
    const float *base = part + rh * (int64_t)nrec * RW;

    // lane x holds record x's (m, l, s) (one round trip for up to 64 records); invalid: m = -inf
    float M = kNegInf;
    float mine_m = kNegInf, mine_l = 0.f, mine_s = 0.f;
    for (int x0 = 0; x0 < nrec; x0 += 64) {
        const int x = x0 + lane;
        const int xc = x < nrec ? x : nrec - 1;
        const float4 h = *reinterpret_cast<const float4 *>(base + (int64_t)xc * RW);
        const bool ok = x < nrec && valid_rh[xc] >= 0;
        const float m = ok ? h.x : kNegInf;
        if (x0 == 0) {
            mine_m = m;
            mine_l = ok ? h.y : 0.f;
            mine_s = ok ? h.z : 0.f;
        }
        M = fmaxf(M, wave_max(m));
    }
    float l = 0.f, o[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = 0.f;
    for (int x0 = 0; x0 < nrec; x0 += kRecBatch) {
        float v[kRecBatch][PER];
#pragma unroll
        for (int b = 0; b < kRecBatch; ++b) {
            const int x = x0 + b < nrec ? x0 + b : nrec - 1;
            load_slice<D, HALF>(base + (int64_t)x * RW, lane, v[b]);
        }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int b = 0; b < kRecBatch; ++b)
#pragma unroll
            for (int i = 0; i < PER; ++i) asm volatile("" : "+v"(v[b][i]));
#pragma unroll
        for (int b = 0; b < kRecBatch; ++b) {
            const int x = x0 + b;
            if (x >= nrec) break;
            float m, lx, sx;
            if (x < 64) {
                m = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mine_m), x));
                lx = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mine_l), x));
                sx = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mine_s), x));
            } else {
                const float4 h = *reinterpret_cast<const float4 *>(base + (int64_t)x * RW);
                m = valid_rh[x] >= 0 ? h.x : kNegInf;
                lx = h.y;
                sx = h.z;
            }
            const bool ok = m != kNegInf;
            const float f = ok ? exp2f(m - M) : 0.f;
            l = ok ? fmaf(lx, f, l) : l;
            const float c = HALF ? f * lx * sx : f;
#pragma unroll
            for (int i = 0; i < PER; ++i) o[i] = ok ? fmaf(v[b][i], c, o[i]) : o[i];
        }
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if constexpr (HALF && D == 128) {
        *reinterpret_cast<float2 *>(out + rh * D + 2 * lane) = make_float2(o[0] * inv, o[1] * inv);
    } else {
#pragma unroll
        for (int i = 0; i < PER; ++i) out[rh * D + lane + 64 * i] = o[i] * inv;
    }
}

template <int D, bool HALF>
hipError_t launch_combine_t(const RowArgs &a, const float *part, const int32_t *local, float *out, hipStream_t st) {
    const int64_t n = a.n_rows * a.Hq;
    hipLaunchKernelGGL((combine_wave<D, HALF>), dim3((unsigned)ceil_div(n, 4)), dim3(256), 0, st, part, local, out, n,
                       a.k, max_window_spans(a.S, a.W));
    return hipGetLastError();
}

// Records of entries that attend to nothing are never written, so the merge checks validity.
hipError_t launch_combine(const RowArgs &a, const float *part, const int32_t *local, float *out, hipStream_t st) {
    if (a.dtype == RA_BF16)
        return a.d == 64 ? launch_combine_t<64, true>(a, part, local, out, st)
                         : launch_combine_t<128, true>(a, part, local, out, st);
    return a.d == 64 ? launch_combine_t<64, false>(a, part, local, out, st)
                     : launch_combine_t<128, false>(a, part, local, out, st);
}

}  // namespace

size_t prefill_workspace_bytes(const RowArgs &a) { return prefill_layout(a).total; }

int64_t prefill_entry_count(const RowArgs &a) { return prefill_layout(a).n_ent; }

int64_t prefill_grid_items(const RowArgs &a) {
    const PrefillLayout L = prefill_layout(a);
    const int64_t tiles = L.max_tiles * 256;                         // tile kernels: 256 threads
    const int64_t merge = ceil_div(a.n_rows * a.Hq, 4) * 256;        // combine_wave: 4 row-heads per block
    const int64_t count = ceil_div(L.n_ent, 256) * 256;              // count / scatter: one thread per entry
    const int64_t descs = L.n_exp * 64;                               // tiles_kernel: one wave per expert
    int64_t m = tiles > merge ? tiles : merge;
    m = m > descs ? m : descs;
    return m > count ? m : count;
}

namespace {

// The dispatch, the tiles and the merge; ks, vs: row scales of an 8-bit cache (null for bf16/fp32).
hipError_t prefill_impl(const RowArgs &a, const void *K, const void *V, const float *ks, const float *vs,
                        const int32_t *sel, float *out, void *ws, hipStream_t st) {
    if (a.n_rows == 0) return hipSuccess;
    const PrefillLayout L = prefill_layout(a);
    char *w = (char *)ws;
    int32_t *counts = (int32_t *)(w + L.off_counts);
    int32_t *offsets = (int32_t *)(w + L.off_offsets);
    int32_t *tile_off = (int32_t *)(w + L.off_tile_off);
    int32_t *local = (int32_t *)(w + L.off_local);
    int32_t *list = (int32_t *)(w + L.off_list);
    int64_t *list_t = (int64_t *)(w + L.off_list_t);
    int4 *tiles = (int4 *)(w + L.off_tiles);
    float *records = (float *)(w + L.off_records);
    const int NE = a.k + max_window_spans(a.S, a.W);
    const int MT = prefill_tile_rows(a);

    hipLaunchKernelGGL(fill_i32, dim3((unsigned)ceil_div(L.n_exp + 1, 256)), dim3(256), 0, st, counts, L.n_exp + 1, 0);
    if (L.span_slots <= kCountMaxSpans) {
        hipLaunchKernelGGL(count_kernel_lds, dim3((unsigned)ceil_div(a.n_rows, kCountRows), (unsigned)a.Hkv), dim3(256),
                           0, st, sel, a.row_seq, a.row_pos, counts, local, a.n_rows, NE, a.Hq, a.Hkv, a.G, a.S, a.k,
                           a.W, a.B, a.max_pos, L.span_slots);
    } else {
        hipLaunchKernelGGL(count_kernel, dim3((unsigned)ceil_div(L.n_ent, 256)), dim3(256), 0, st, sel, a.row_seq,
                           a.row_pos, counts, local, L.n_ent, NE, a.Hq, a.Hkv, a.G, a.S, a.k, a.W, a.B, a.max_pos,
                           L.span_slots);
    }
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, counts, offsets, tile_off, L.n_exp, MT);
    hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)ceil_div(L.n_ent, 256)), dim3(256), 0, st, sel, a.row_seq,
                       a.row_pos, offsets, local, list, list_t, L.n_ent, NE, a.Hq, a.Hkv, a.G, a.S, a.k, a.W, a.B,
                       a.max_pos,
                       L.span_slots);
    hipLaunchKernelGGL(tiles_kernel, dim3((unsigned)ceil_div(L.n_exp, kTilesWaves)), dim3(kTilesWaves * 64), 0, st,
                       counts, offsets, tile_off, tiles, L.n_exp, MT);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    TileArgs ta{a, K, V, ks, vs, tile_off, list, list_t, tiles, records, L.n_exp, L.max_tiles, L.span_slots, NE};
    e = launch_prefill_tiles(ta, st);
    if (e != hipSuccess) return e;
    return launch_combine(a, records, local, out, st);
}

}  // namespace

hipError_t launch_prefill(const RowArgs &a, const void *K, const void *V, const int32_t *sel, float *out, void *ws,
                          hipStream_t st) {
    return prefill_impl(a, K, V, nullptr, nullptr, sel, out, ws, st);
}

hipError_t launch_prefill_fp8(const RowArgs &a, const uint8_t *K8, const uint8_t *V8, const float *ks,
                              const float *vs, const int32_t *sel, float *out, void *ws, hipStream_t st) {
    return prefill_impl(a, K8, V8, ks, vs, sel, out, ws, st);
}

}  // namespace ra
