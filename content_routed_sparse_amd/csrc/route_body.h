// Few-row routing (decode) shared by route_valu, route_topk and the one-launch decode step:
// the fp32 scores s_j = q . kappa(mean_j) of a (row, kv head)'s query heads against 16 spans per
// wave, and one block of the routing + selection of few rows (release post, "Key idea": score the
// candidate spans, keep the top k).
#pragma once

#include "common.h"
#include "topk_body.h"
#include "wave_ops.h"

namespace ra {

// Few rows (decode) or fp32 inputs: lanes split each fp32 summary row (8 elements per lane, LPR
// lanes per row, coalesced 32-byte loads); a wave takes 16 spans, each lane forms partial dot
// products for 8 query heads at once, and a butterfly reduce-scatter over the LPR lanes leaves
// KEEP finished scores per lane.  The same steps serve route_valu and the routing + selection
// blocks (route_select_block), so both give the same fp32 scores.
template <typename T, int D>
struct ValuScore {
    static constexpr int LPR = D / 8, RPI = 64 / LPR, STEPS = 16 / RPI, N = STEPS * 8, KEEP = N / LPR;
    static constexpr int QV = sizeof(T) == 2 ? 1 : 2;  // 16-byte pieces per head slice of 8 elements

    // q slices of query heads hc..hc+7 of kv head g (a head past G loads head G-1; score() zeroes it)
    __device__ static __forceinline__ void load_q(uint4 (&qraw)[8][QV], const T *q, int64_t row, int Hq, int g,
                                                  int G, int hc, int c) {
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            const int hh = hc + h < G ? hc + h : G - 1;
            const uint4 *qp = reinterpret_cast<const uint4 *>(q + (row * Hq + g * G + hh) * D + c * 8);
#pragma unroll
            for (int v = 0; v < QV; ++v) qraw[h][v] = qp[v];
        }
    }

    // kappa of the summaries of spans jw + s RPI + rr (clamped to r - 1): every load of the wave
    // issued before any use and pinned there
    __device__ static __forceinline__ void load_means(float (&mv)[STEPS][8], const float *mbase, int64_t jw,
                                                      int64_t r, int c, int rr) {
        float4 mraw[STEPS][2];
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            int64_t n = jw + s * RPI + rr;
            n = n < r ? n : r - 1;
            mraw[s][0] = *reinterpret_cast<const float4 *>(mbase + n * D + c * 8);
            mraw[s][1] = *reinterpret_cast<const float4 *>(mbase + n * D + c * 8 + 4);
        }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int s = 0; s < STEPS; ++s)
#pragma unroll
            for (int v = 0; v < 2; ++v)
                asm volatile("" : "+v"(mraw[s][v].x), "+v"(mraw[s][v].y), "+v"(mraw[s][v].z), "+v"(mraw[s][v].w));
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            const float f[8] = {mraw[s][0].x, mraw[s][0].y, mraw[s][0].z, mraw[s][0].w,
                                mraw[s][1].x, mraw[s][1].y, mraw[s][1].z, mraw[s][1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) mv[s][e] = sizeof(T) == 2 ? round_bf16(f[e]) : f[e];
        }
    }

    // scores of spans jw.. (16) for query heads hc..hc+7: store(head, span, score) for every
    // finished score with span < r and head < G
    template <typename F>
    __device__ static __forceinline__ void score(const uint4 (&qraw)[8][QV], const float (&mv)[STEPS][8], int hc,
                                                 int G, int lane, int64_t jw, int64_t r, F &&store) {
        const int c = lane % LPR, rr = lane / LPR;
        float acc[N];
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            float qf[8];
            if constexpr (sizeof(T) == 2) {
                const uint32_t w[4] = {qraw[h][0].x, qraw[h][0].y, qraw[h][0].z, qraw[h][0].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    qf[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
                    qf[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
                }
            } else {
                const uint32_t w[8] = {qraw[h][0].x, qraw[h][0].y, qraw[h][0].z, qraw[h][0].w,
                                       qraw[h][1].x, qraw[h][1].y, qraw[h][1].z, qraw[h][1].w};
#pragma unroll
                for (int i = 0; i < 8; ++i) qf[i] = __uint_as_float(w[i]);
            }
            if (hc + h >= G) {
#pragma unroll
                for (int e = 0; e < 8; ++e) qf[e] = 0.f;
            }
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) d = fmaf(qf[e], mv[s][e], d);
                acc[s * 8 + h] = d;
            }
        }
        ReduceScatter<N, ilog2(LPR), LPR / 2>::run(acc, lane);
#pragma unroll
        for (int i = 0; i < KEEP; ++i) {
            const int v = c * KEEP + i;
            const int s = v / 8, h = v % 8;
            const int64_t n = jw + s * RPI + rr;
            if (n < r && hc + h < G) store(hc + h, n, acc[i]);
        }
    }
};

// One block of routing + selection for few rows: NWR waves score 16 spans each (span block yb of
// nyb, SPB = 16 NWR spans) of (row, kv head) rg for all the kv head's query heads (ValuScore: the
// scores route_valu writes, bit for bit), into LDS (stile: 32 rows of SPB floats).  Each wave then
// selects, for its query heads, the block's own top min(k, r_b) spans (wave_topk over the block's
// r_b routable spans) and writes them as candidates -- (score image, span index), k slots per
// (row, head, block), unused slots (0, -1) -- with system-coherent stores (they reach memory, past
// every XCD's L2).  The block counts itself in counters[rg]; the block that arrives last (all the
// others' candidates are in memory by then) reads the nyb k candidates of each head back with
// system-coherent loads and selects again among them.  The union of the blocks' top-k holds the
// global top-k, and the candidates sit in span order (blocks in span order, each block's slots
// ascending), so the second selection, by (image desc, position asc), is exactly topk_spans'
// selection; its output positions become span indices.  Block 0's first min(k, r) slots are
// valid, so at least m of the 64 lanes hold a valid image, as wave_topk needs.  Both selections
// run the same wave_topk code (the final one, run by a single block, finds it warm in the
// instruction cache: with every block reading back all the scores, the cold selection code of
// that one block cost several microseconds).  The last block resets the counter, so counters that
// start at zero are at zero again after every call.  Returns true in the block that selected (the
// same value in every thread).  cand: NWR x 64 words of LDS; lsel: NWR x 64 ints of LDS.
template <typename T, int D, int PER_LANE, int NWR>
__device__ __forceinline__ bool route_select_block(const T *__restrict__ q, const int32_t *__restrict__ row_seq,
                                                   const int64_t *__restrict__ row_pos, const float *__restrict__ mean,
                                                   uint64_t *cands, int32_t *sel, uint32_t *counters, int Hq,
                                                   int Hkv, int G, int S, int k, int W, int B, int64_t max_spans,
                                                   int64_t max_pos, int rg, int yb, int nyb, uint64_t (*cand)[64],
                                                   float *stile, int32_t (*lsel)[64], int *is_last) {
    using VS = ValuScore<T, D>;
    constexpr int SPB = 16 * NWR;            // spans per block
    constexpr int PLL = SPB / 64;            // local selection: spans per lane
    constexpr int PLF = (PER_LANE + 1) / 2;  // final selection: candidates per lane (nyb k <= 64 PLF)
    static_assert(SPB % 64 == 0 && SPB >= 64, "whole spans per lane; k <= 64 <= SPB");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane % VS::LPR, rr = lane / VS::LPR;
    const int64_t row = rg / Hkv;
    const int g = rg % Hkv;
    uint4 qraw[8][VS::QV];
    const int64_t t_raw = row_pos[row];
    const int seq_raw = row_seq[row];
    VS::load_q(qraw, q, row, Hq, g, G, 0, c);
    asm volatile("" ::"s"(t_raw), "s"(seq_raw));
    const int64_t t = t_raw < 0 ? 0 : (t_raw > max_pos ? max_pos : t_raw);
    const int seq = seq_raw < 0 ? 0 : (seq_raw >= B ? B - 1 : seq_raw);
    const int64_t r = num_routable(t, S, W);
    const int64_t jb = (int64_t)yb * SPB;  // this block's first span
    const int64_t jw = jb + wave * 16;     // this wave's first span
    if (jw < r) {
        const float *mbase = mean + ((int64_t)seq * Hkv + g) * max_spans * D;
        float mv[VS::STEPS][8];
        VS::load_means(mv, mbase, jw, r, c, rr);
        for (int hc = 0; hc < G; hc += 8) {
            if (hc > 0) VS::load_q(qraw, q, row, Hq, g, G, hc, c);
            VS::score(qraw, mv, hc, G, lane, jw, r,
                      [&](int h, int64_t n, float v) { stile[h * SPB + (int)(n - jb)] = v; });
        }
    }
    __syncthreads();
    // the block's candidates: wave w takes query heads w, w + NWR, ...
    const int rb = (int)(r - jb < 0 ? 0 : (r - jb > SPB ? SPB : r - jb));  // the block's routable spans
    const int mb = rb < k ? rb : k;
    uint64_t *crow = cands + ((row * Hq + g * G) * nyb + yb) * k;  // + h nyb k: head h's slots
    for (int h = wave; h < G; h += NWR) {
        uint32_t img[PLL];
#pragma unroll
        for (int i = 0; i < PLL; ++i) {
            const int p = lane + 64 * i;
            img[i] = p < rb ? score_image(stile[h * SPB + p]) : 0u;
        }
        wave_topk<PLL>(img, mb, k, lane, cand[wave], lsel[wave]);
        __builtin_amdgcn_wave_barrier();
        if (lane < k) {
            const int p = lsel[wave][lane];
            const uint64_t v = p >= 0 ? ((uint64_t)(uint32_t)(jb + p) << 32) | score_image(stile[h * SPB + p])
                                      : 0xFFFFFFFF00000000ull;
            __hip_atomic_store(crow + (int64_t)h * nyb * k + lane, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
        __builtin_amdgcn_wave_barrier();
    }
    // this block's candidates have reached memory (stores are counted by vmcnt) before it counts itself
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t before = __hip_atomic_fetch_add(counters + rg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *is_last = before == (uint32_t)nyb - 1;
        if (*is_last) __hip_atomic_store(counters + rg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!*is_last) return false;
    const int m = (int)(r < k ? r : k);
    const int nc = nyb * k;  // candidates per head, position p = block * k + slot
    for (int h = wave; h < G; h += NWR) {
        const uint64_t *hrow = cands + ((row * Hq + g * G + h) * nyb) * k;
        uint32_t img[PLF], ids[PLF];
#pragma unroll
        for (int i = 0; i < PLF; ++i) {
            const int p = lane + 64 * i;
            const uint64_t v = __hip_atomic_load(hrow + (p < nc ? p : 0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            img[i] = p < nc ? (uint32_t)v : 0u;
            ids[i] = (uint32_t)(v >> 32);
        }
        wave_topk<PLF>(img, m, k, lane, cand[wave], lsel[wave]);
        __builtin_amdgcn_wave_barrier();
        // winners' positions -> span indices (position p is held by lane p % 64 in ids[p / 64])
        const int p = lane < k ? lsel[wave][lane] : -1;
        const int src = (p < 0 ? 0 : p) & 63, reg = (p < 0 ? 0 : p) >> 6;
        int32_t span = -1;
#pragma unroll
        for (int i = 0; i < PLF; ++i) {
            const int32_t v = __shfl((int32_t)ids[i], src);
            span = (p >= 0 && reg == i) ? v : span;
        }
        if (lane < k) sel[(row * Hq + g * G + h) * k + lane] = span;
        __builtin_amdgcn_wave_barrier();
    }
    return true;
}

}  // namespace ra
