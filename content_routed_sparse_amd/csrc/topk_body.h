// Wave-level top-k selection shared by topk_spans and the fused decode routing + selection
// (release post, "Key idea": keep the top k of the scored spans).
//
// Each routable span j < r(t) becomes a 64-bit key  (order-preserving image of the fp32 score)
// << 32 | (0xFFFFFFFF - j),  so a larger key means a higher score and, on equal scores, a lower
// span index: the selection order is a strict total order.  Lane l of a wave holds the keys of
// spans j = l + 64 i in registers.  The m winners are written in ascending span order, and the
// entries m..k-1 as -1.
#pragma once

#include "common.h"
#include "wave_ops.h"

namespace ra {

__device__ __forceinline__ uint64_t score_key(float s, int64_t j) {
    uint32_t u = __float_as_uint(s);
    if (s == 0.f) u = 0u;  // -0 and +0 are the same score: the lower index must win
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

// One wave selects from key[] (lane l holds spans l + 64 i; 0 for j >= r) the m = min(k, r) largest
// keys and writes their span indices to out[0..k) (ascending, -1 padded).  cand: 64 words of LDS
// owned by the wave.
//
// Threshold first: v = the m-th largest of the 64 per-lane maximum scores (the keys' upper
// halves), found bit by bit from the top: a bit is kept when at least m lanes still reach the
// value (one ballot per bit).  At least m lanes then hold a key >= T0 = v * 2^32, so every one of
// the m winners is >= T0.  The keys >= T0 (usually little more than m; more only where scores
// tie) are compacted into LDS in span order and each is ranked against the others; if more than
// 64 pass, the selection falls back to m rounds of "largest key below the previous winner".
template <int PER_LANE>
__device__ __forceinline__ void wave_topk(const uint64_t (&key)[PER_LANE], int m, int k, int lane, uint64_t *cand,
                                          int32_t *out) {
    if (m == 0) {
        if (lane < k) out[lane] = -1;
        return;
    }
    // per-lane maximum (balanced tree)
    uint64_t f[PER_LANE];
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) f[i] = key[i];
#pragma unroll
    for (int width = 1; width < PER_LANE; width *= 2) {
#pragma unroll
        for (int i = 0; i + width < PER_LANE; i += 2 * width) f[i] = f[i + width] > f[i] ? f[i + width] : f[i];
    }
    // at least m lanes hold a valid key (candidates are dealt round-robin and m <= r), so the
    // search ends on the upper half of a valid key
    const uint32_t lhi = (uint32_t)(f[0] >> 32);
    uint32_t v = 0;
#pragma unroll
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t test = v | (1u << bit);
        if ((int)__builtin_popcountll(__ballot(lhi >= test)) >= m) v = test;
    }
    const uint64_t T0 = (uint64_t)v << 32;

    int C = 0;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
        const bool c = key[i] >= T0;
        const uint64_t b = __ballot(c);
        const int pos = C + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
        if (c && pos < 64) cand[pos] = key[i];
        C += (int)__builtin_popcountll(b);
    }
    if (C <= 64) {
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const uint64_t mine = lane < C ? cand[lane] : 0ull;
        int rank = 0;
        for (int j2 = 0; j2 < C; ++j2) rank += cand[j2] > mine ? 1 : 0;
        const bool chosen = lane < C && rank < m;
        const uint32_t idx = 0xFFFFFFFFu - (uint32_t)(mine & 0xFFFFFFFFull);
        // the list is in increasing span order (compacted register by register, lane by lane,
        // and lane l of register i holds span l + 64 i), so a winner's output slot is the number
        // of winners before it in the list
        const uint64_t cb = __ballot(chosen);
        const int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(cb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)cb, 0u));
        if (chosen) out[pos] = (int32_t)idx;
        if (lane >= m && lane < k) out[lane] = -1;
        return;
    }

    // fallback: m rounds, each taking the wave maximum among keys below the previous winner
    uint64_t last = ~0ull;
    uint32_t win = 0xFFFFFFFFu;  // lane w keeps the w-th winner's span index
    for (int w = 0; w < m; ++w) {
        uint64_t g[PER_LANE];
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) g[i] = key[i] < last ? key[i] : 0ull;
#pragma unroll
        for (int width = 1; width < PER_LANE; width *= 2) {
#pragma unroll
            for (int i = 0; i + width < PER_LANE; i += 2 * width) g[i] = g[i + width] > g[i] ? g[i + width] : g[i];
        }
        const uint64_t best = wave_max_u64(g[0]);
        last = best;
        if (lane == w) win = 0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull);
    }
    int rank = 0;
    for (int w = 0; w < m; ++w) {
        const uint32_t o = __shfl(win, w);
        rank += (o < win) ? 1 : 0;
    }
    if (lane < m) out[rank] = (int32_t)win;
    else if (lane < k) out[lane] = -1;
}

}  // namespace ra
