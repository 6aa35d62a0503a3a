// Routing scores: every (row, query head) scores every routable span summary of its sequence
// (release post, "Key idea": score the O(L^0.5) candidate spans).  s_j = q . kappa(mean_j).
//
// Two kernels:
//  * route_mfma (bf16 inputs, many rows): a dense [row-heads x spans] contraction on bf16 MFMA
//    (v_mfma_f32_16x16x32_bf16), fp32 accumulation.  A block owns 128 row-heads of one kv head
//    (4 waves x 2 groups of 16) and a range of spans; span summaries are rounded to bf16 once per
//    block and staged in LDS, shared by the 4 waves and the 2 groups of each.  The kernel is
//    bound by its score stores (1.08 GB for an 8192-row chunk on 1M tokens): 16-byte stores,
//    which run fastest when score rows start on 128-byte cache lines (a score stride that is a
//    multiple of 32 floats).  Rows of different sequences in one tile are handled
//    in successive passes (one pass in the usual single-sequence chunk).
//  * route_valu (fp32 inputs, or few rows as in decode): fp32 FMA; lanes split each summary
//    row, 8 query heads per pass, butterfly reduction over the lanes of a row.
#include "common.h"
#include "kernels.h"
#include "route_body.h"
#include "topk_body.h"
#include "wave_ops.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// A block scores 64 spans of one (row, kv head) for all the kv head's query heads (4 waves of 16).
template <typename T, int D>
__global__ void __launch_bounds__(256) route_valu(const T *__restrict__ q, const int32_t *__restrict__ row_seq,
                                                  const int64_t *__restrict__ row_pos,
                                                  const float *__restrict__ mean, float *__restrict__ scores,
                                                  int64_t stride, int Hq, int Hkv, int G, int S, int W, int B,
                                                  int64_t max_spans, int64_t max_pos) {
    using VS = ValuScore<T, D>;
    // all kernel arguments in one round trip (otherwise some are fetched only where first used)
    asm volatile("" ::"s"(q), "s"(row_seq), "s"(row_pos), "s"(mean), "s"(scores), "s"(stride), "s"(Hq), "s"(Hkv),
                 "s"(G), "s"(S), "s"(W), "s"(B), "s"(max_spans), "s"(max_pos));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane % VS::LPR, rr = lane / VS::LPR;
    const int rg = blockIdx.x;
    const int64_t row = rg / Hkv;
    const int g = rg % Hkv;
    uint4 qraw[8][VS::QV];
    // the row's position and sequence together with the first 8 heads' queries (which do not
    // depend on them): one round trip
    const int64_t t_raw = row_pos[row];
    const int seq_raw = row_seq[row];
    VS::load_q(qraw, q, row, Hq, g, G, 0, c);
    asm volatile("" ::"s"(t_raw), "s"(seq_raw));
    const int64_t t = t_raw < 0 ? 0 : (t_raw > max_pos ? max_pos : t_raw);
    const int seq = seq_raw < 0 ? 0 : (seq_raw >= B ? B - 1 : seq_raw);
    const int64_t r = num_routable(t, S, W);
    const int64_t jw = (int64_t)blockIdx.y * 64 + wave * 16;  // this wave's first span
    if (jw >= r) return;
    const float *mbase = mean + ((int64_t)seq * Hkv + g) * max_spans * D;
    float mv[VS::STEPS][8];
    VS::load_means(mv, mbase, jw, r, c, rr);
    float *srow = scores + (row * Hq + g * G) * stride;
    for (int hc = 0; hc < G; hc += 8) {
        if (hc > 0) VS::load_q(qraw, q, row, Hq, g, G, hc, c);
        VS::score(qraw, mv, hc, G, lane, jw, r, [&](int h, int64_t n, float v) { srow[h * stride + n] = v; });
    }
}

// Decode routing and selection in one launch: one block of route_select_block per (row, kv head,
// span block of 16 kRtWaves spans); each block selects its own candidates, the last block of each
// (row, kv head) to finish selects among them.
constexpr int kRtWaves = 8;  // waves per block: 16 spans each; in the selections, one query head each
constexpr int kRtSpans = 16 * kRtWaves;

template <typename T, int D, int PER_LANE>
__global__ void __launch_bounds__(kRtWaves * 64) route_topk(const T *__restrict__ q,
                                                            const int32_t *__restrict__ row_seq,
                                                            const int64_t *__restrict__ row_pos,
                                                            const float *__restrict__ mean, uint64_t *cands,
                                                            int32_t *__restrict__ sel, uint32_t *__restrict__ counters,
                                                            int Hq, int Hkv, int G, int S, int k, int W, int B,
                                                            int64_t max_spans, int64_t max_pos) {
    __shared__ uint64_t cand[kRtWaves][64];
    __shared__ __align__(16) float stile[32 * kRtSpans];
    __shared__ int32_t lsel[kRtWaves][64];
    __shared__ int is_last;
    asm volatile("" ::"s"(q), "s"(row_seq), "s"(row_pos), "s"(mean), "s"(cands), "s"(sel), "s"(counters), "s"(Hq),
                 "s"(Hkv), "s"(G), "s"(S), "s"(k), "s"(W), "s"(B), "s"(max_spans), "s"(max_pos));
    route_select_block<T, D, PER_LANE, kRtWaves>(q, row_seq, row_pos, mean, cands, sel, counters, Hq, Hkv, G, S, k, W,
                                                  B, max_spans, max_pos, (int)blockIdx.x, (int)blockIdx.y,
                                                  (int)gridDim.y, cand, stile, lsel, &is_last);
}

constexpr int kRouteGroups = 2;                // 16-row MFMA groups per wave (measured: 2 beats 1, 4 and 8)
constexpr int kRowTile = 64 * kRouteGroups;     // row-heads per block (4 waves)
constexpr int kSpanBlock = 64;                  // spans staged per LDS step
constexpr int kRouteBlocks = 1024;              // blocks wanted before a tile's spans are split

// A block owns kRowTile row-heads of one kv head and the spans [jc0, jc0 + span_chunk).  Each
// LDS step stages kappa(mean) of 64 spans as bf16 (double-buffered: the next step's summaries
// are loaded into registers while the current step's products run, one barrier per step); every
// staged span fragment feeds the MFMAs of all RG row groups of the wave.  The product is formed
// as spans x row-heads, so a lane ends with 4 consecutive spans of one row-head and stores them
// with one 16-byte store.  Each score is one chain of D/32 MFMAs over the same operands whatever
// the tiling, so the values do not depend on it.
template <int D, int RG>
__global__ void __launch_bounds__(256) route_mfma(const uint16_t *__restrict__ q, const int32_t *__restrict__ row_seq,
                                                  const int64_t *__restrict__ row_pos,
                                                  const float *__restrict__ mean, float *__restrict__ scores,
                                                  int64_t stride, int64_t n_rows, int Hq, int Hkv, int G, int S,
                                                  int W, int B, int64_t max_spans, int64_t max_pos,
                                                  int64_t tiles_per_head, int64_t span_chunk) {
    constexpr int KS = D / 32;          // k-steps of 32
    constexpr int LDS_ROW = D + 8;      // bf16 elements per staged span row (padding vs bank conflicts)
    constexpr int TILE = 64 * RG;
    constexpr int PER = kSpanBlock * (D / 4) / 256;  // float4 summary loads per thread per step
    typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));  // score rows need not be 16-byte aligned
    __shared__ uint16_t bstage[2][kSpanBlock * LDS_ROW];
    __shared__ int tile_seq[TILE];
    __shared__ int pass_seq;
    __shared__ int64_t rmax_w[4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = (int)(blockIdx.x / tiles_per_head);
    const int64_t rh0 = (blockIdx.x % tiles_per_head) * TILE;
    const int64_t jc0 = (int64_t)blockIdx.y * span_chunk;
    const int64_t n_rh = n_rows * G;

    // sequence of each row-head of the tile (-1 when past the last row)
    for (int x = tid; x < TILE; x += 256) {
        const int64_t rh = rh0 + x;
        int s = -1;
        if (rh < n_rh) {
            s = row_seq[rh / G];
            s = s < 0 ? 0 : (s >= B ? B - 1 : s);
        }
        tile_seq[x] = s;
    }
    // row group gr of this wave: row-heads rh0 + (wave * RG + gr) * 16 + [0, 16); the lane's
    // row-head (lane % 16) is both its query fragment's row and its outputs' column.  Per group:
    // the score row offset and the routable count relative to the block's span range.
    int64_t out_off[RG];
    int out_r[RG];
    int64_t rmax = 0;
#pragma unroll
    for (int gr = 0; gr < RG; ++gr) {
        const int64_t rh = rh0 + (wave * RG + gr) * 16 + (lane & 15);
        int64_t r = 0;
        out_off[gr] = 0;
        if (rh < n_rh) {
            const int64_t row = rh / G;
            int64_t t = row_pos[row];
            t = t < 0 ? 0 : (t > max_pos ? max_pos : t);
            r = num_routable(t, S, W);
            out_off[gr] = (row * Hq + g * G + (int)(rh % G)) * stride + jc0;
        }
        rmax = r > rmax ? r : rmax;
        int64_t rel = r - jc0;
        rel = rel < 0 ? 0 : (rel > span_chunk ? span_chunk : rel);
        out_r[gr] = (int)rel;
    }
    // largest routable count in the tile bounds the span loop
    for (int off = 32; off > 0; off >>= 1) {
        const int64_t o = __shfl_xor(rmax, off);
        rmax = o > rmax ? o : rmax;
    }
    if (lane == 0) rmax_w[wave] = rmax;
    __syncthreads();
    rmax = rmax_w[0];
    for (int w = 1; w < 4; ++w) rmax = rmax_w[w] > rmax ? rmax_w[w] : rmax;
    int64_t jend = jc0 + span_chunk;
    if (jend > rmax) jend = rmax;
    if (jc0 >= jend) return;

    int done_below = -1;  // passes go over the distinct sequences of the tile in increasing order
    while (true) {
        __syncthreads();
        if (tid == 0) {
            int nxt = 0x7fffffff;
            for (int x = 0; x < TILE; ++x)
                if (tile_seq[x] > done_below && tile_seq[x] < nxt) nxt = tile_seq[x];
            pass_seq = nxt;
        }
        __syncthreads();
        const int seq = pass_seq;
        if (seq == 0x7fffffff) break;
        done_below = seq;
        // query fragments of the pass's rows (zero for rows of other sequences or past the end)
        bf16x8 qf[RG][KS];
        int lim[RG];  // spans of the pass's rows (0 for rows of other sequences)
#pragma unroll
        for (int gr = 0; gr < RG; ++gr) {
            const int x = (wave * RG + gr) * 16 + (lane & 15);
            const bool ok = tile_seq[x] == seq;  // -1 past the last row
            const int64_t rh = ok ? rh0 + x : 0;
            const uint16_t *qp = q + ((rh / G) * Hq + g * G + (int)(rh % G)) * D + 8 * (lane >> 4);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const uint4 raw = ok ? *reinterpret_cast<const uint4 *>(qp + 32 * ks) : make_uint4(0, 0, 0, 0);
                qf[gr][ks] = __builtin_bit_cast(bf16x8, raw);
            }
            lim[gr] = ok ? out_r[gr] : 0;
        }
        const float *mseq = mean + ((int64_t)seq * Hkv + g) * max_spans * D;
        float4 pre[PER];
        auto fetch = [&](int64_t jb) {
#pragma unroll
            for (int p = 0; p < PER; ++p) {
                const int x = tid + 256 * p;
                const int64_t j = jb + x / (D / 4);
                pre[p] = j < jend ? *reinterpret_cast<const float4 *>(mseq + j * D + (x % (D / 4)) * 4)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        };
        fetch(jc0);
        int buf = 0;
        for (int64_t jb = jc0; jb < jend; jb += kSpanBlock, buf ^= 1) {
            // stage kappa(mean) of spans [jb, jb+64) as bf16, then start loading the next 64
#pragma unroll
            for (int p = 0; p < PER; ++p) {
                const int x = tid + 256 * p;
                const uint32_t lo = f32_to_bf16_bits(pre[p].x) | (f32_to_bf16_bits(pre[p].y) << 16);
                const uint32_t hi = f32_to_bf16_bits(pre[p].z) | (f32_to_bf16_bits(pre[p].w) << 16);
                *reinterpret_cast<uint2 *>(&bstage[buf][(x / (D / 4)) * LDS_ROW + (x % (D / 4)) * 4]) =
                    make_uint2(lo, hi);
            }
            if (jb + kSpanBlock < jend) fetch(jb + kSpanBlock);
            __syncthreads();
#pragma unroll
            for (int nb = 0; nb < kSpanBlock / 16; ++nb) {
                const uint16_t *bp = &bstage[buf][(nb * 16 + (lane & 15)) * LDS_ROW + 8 * (lane >> 4)];
                bf16x8 sf[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    sf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(bp + 32 * ks));
                // this lane's outputs: spans j0 .. j0+3 (relative to jc0) of its row-head
                const int j0 = (int)(jb - jc0) + nb * 16 + 4 * (lane >> 4);
#pragma unroll
                for (int gr = 0; gr < RG; ++gr) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf[ks], qf[gr][ks], acc, 0, 0, 0);
                    float *dst = scores + out_off[gr] + j0;
                    if (j0 + 3 < lim[gr]) {
                        *reinterpret_cast<f32x4u *>(dst) = f32x4u{acc[0], acc[1], acc[2], acc[3]};
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (j0 + i < lim[gr]) dst[i] = acc[i];
                    }
                }
            }
        }
        __syncthreads();
    }
}

template <typename T, int D>
hipError_t route_valu_launch(const RowArgs &a, const float *mean, float *scores, int64_t stride, hipStream_t st) {
    const int64_t rmax = num_routable(a.max_pos, a.S, a.W);
    if (rmax == 0 || a.n_rows == 0) return hipSuccess;
    dim3 grid((unsigned)(a.n_rows * a.Hkv), (unsigned)ceil_div(rmax, 64));
    hipLaunchKernelGGL((route_valu<T, D>), grid, dim3(256), 0, st, (const T *)a.q, a.row_seq, a.row_pos, mean, scores,
                       stride, a.Hq, a.Hkv, a.G, a.S, a.W, a.B, a.max_spans, a.max_pos);
    return hipGetLastError();
}

template <int D>
hipError_t route_mfma_launch(const RowArgs &a, const float *mean, float *scores, int64_t stride, hipStream_t st) {
    const int64_t rmax = num_routable(a.max_pos, a.S, a.W);
    if (rmax == 0 || a.n_rows == 0) return hipSuccess;
    const int64_t tiles = ceil_div(a.n_rows * a.G, kRowTile);
    // split the spans only as far as needed for kRouteBlocks blocks
    int64_t parts = ceil_div(kRouteBlocks, tiles * a.Hkv);
    const int64_t max_parts = ceil_div(rmax, kSpanBlock);
    parts = parts < 1 ? 1 : (parts > max_parts ? max_parts : parts);
    const int64_t min_parts = ceil_div(rmax, (int64_t)1 << 30);  // span offsets inside a block fit in int
    parts = parts < min_parts ? min_parts : parts;
    const int64_t chunk = ceil_div(ceil_div(rmax, parts), kSpanBlock) * kSpanBlock;
    dim3 grid((unsigned)(tiles * a.Hkv), (unsigned)ceil_div(rmax, chunk));
    hipLaunchKernelGGL((route_mfma<D, kRouteGroups>), grid, dim3(256), 0, st, (const uint16_t *)a.q, a.row_seq,
                       a.row_pos, mean, scores, stride, a.n_rows, a.Hq, a.Hkv, a.G, a.S, a.W, a.B, a.max_spans,
                       a.max_pos, tiles, chunk);
    return hipGetLastError();
}

// span blocks of the one-launch routing (at least one per (row, kv head): with no routable span it
// writes the -1 padding)
int64_t route_topk_blocks(int64_t rmax) { return rmax > 0 ? ceil_div(rmax, kRtSpans) : 1; }

template <typename T, int D, int PL>
hipError_t route_topk_launch(const RowArgs &a, const float *mean, uint64_t *cands, int32_t *sel,
                             uint32_t *counters, int64_t rmax, hipStream_t st) {
    dim3 grid((unsigned)(a.n_rows * a.Hkv), (unsigned)route_topk_blocks(rmax));
    hipLaunchKernelGGL((route_topk<T, D, PL>), grid, dim3(kRtWaves * 64), 0, st, (const T *)a.q, a.row_seq, a.row_pos, mean,
                       cands, sel, counters, a.Hq, a.Hkv, a.G, a.S, a.k, a.W, a.B, a.max_spans, a.max_pos);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t route_topk_dispatch(const RowArgs &a, const float *mean, uint64_t *cands, int32_t *sel,
                               uint32_t *counters, int64_t rmax, hipStream_t st) {
    if (rmax <= 64 * 2) return route_topk_launch<T, D, 2>(a, mean, cands, sel, counters, rmax, st);
    if (rmax <= 64 * 8) return route_topk_launch<T, D, 8>(a, mean, cands, sel, counters, rmax, st);
    return route_topk_launch<T, D, 17>(a, mean, cands, sel, counters, rmax, st);
}

// Workspace of route_topk_spans: n_rows x Hkv counters (256-byte aligned), then room for either the
// one-launch path's candidates (n_rows x Hq x blocks x k words of 8 bytes) or the two launches'
// score rows.
int64_t route_topk_stride(const RowArgs &a) {
    const int64_t r = num_routable(a.max_pos, a.S, a.W);
    return r > 0 ? ceil_div(r, 32) * 32 : 32;
}
size_t route_topk_counter_bytes(const RowArgs &a) { return (size_t)ceil_div(a.n_rows * a.Hkv * 4, 256) * 256; }

}  // namespace

size_t route_topk_workspace_bytes(const RowArgs &a) {
    const int64_t scores = a.n_rows * a.Hq * route_topk_stride(a) * 4;
    const int64_t cands = a.n_rows * a.Hq * route_topk_blocks(num_routable(a.max_pos, a.S, a.W)) * a.k * 8;
    return route_topk_counter_bytes(a) + (size_t)(scores > cands ? scores : cands);
}

// Routing and selection in one call; the path depends on the shape, the result does not (both
// compute route_scores' scores and topk_spans' selection):
//  * few rows (decode), r <= 64 * 17: route_topk (the last block of each (row, kv head) selects);
//  * many bf16 rows (route_scores' MFMA regime) or more spans: route_scores then topk_spans through
//    the workspace's score rows (for few rows and 2559 spans the two launches were measured
//    faster than one; for a prefill chunk see the design notes on the fused sweep).
hipError_t launch_route_topk(const RowArgs &a, const float *mean, int32_t *sel, void *ws, hipStream_t st) {
    const int64_t rmax = num_routable(a.max_pos, a.S, a.W);
    if (a.n_rows == 0) return hipSuccess;
    uint32_t *counters = (uint32_t *)ws;
    float *scores = (float *)((char *)ws + route_topk_counter_bytes(a));
    uint64_t *cands = (uint64_t *)scores;
    const int64_t stride = route_topk_stride(a);
    const bool many = a.dtype == RA_BF16 && a.n_rows * a.G >= 256;
    if (!many && rmax <= 64 * 17) {
        if (a.dtype == RA_BF16)
            return a.d == 64 ? route_topk_dispatch<uint16_t, 64>(a, mean, cands, sel, counters, rmax, st)
                             : route_topk_dispatch<uint16_t, 128>(a, mean, cands, sel, counters, rmax, st);
        return a.d == 64 ? route_topk_dispatch<float, 64>(a, mean, cands, sel, counters, rmax, st)
                         : route_topk_dispatch<float, 128>(a, mean, cands, sel, counters, rmax, st);
    }
    const hipError_t e = launch_route(a, mean, scores, stride, st);
    return e != hipSuccess ? e : launch_topk(a, scores, stride, sel, st);
}

hipError_t launch_route(const RowArgs &a, const float *mean, float *scores, int64_t stride, hipStream_t st) {
    if (a.dtype == RA_BF16) {
        if (a.n_rows * a.G >= 256) return a.d == 64 ? route_mfma_launch<64>(a, mean, scores, stride, st)
                                                    : route_mfma_launch<128>(a, mean, scores, stride, st);
        return a.d == 64 ? route_valu_launch<uint16_t, 64>(a, mean, scores, stride, st)
                         : route_valu_launch<uint16_t, 128>(a, mean, scores, stride, st);
    }
    return a.d == 64 ? route_valu_launch<float, 64>(a, mean, scores, stride, st)
                     : route_valu_launch<float, 128>(a, mean, scores, stride, st);
}

}  // namespace ra
