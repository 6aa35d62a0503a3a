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

// The order-preserving 32-bit image of a score (the upper half of its key); valid images are >= 1.
// s + 0 is +0 for both zeros (round to nearest), so -0 and +0 share one image and the lower index
// wins; then negative scores flip every bit and the others set the sign bit (4 VALU instructions).
__device__ __forceinline__ uint32_t score_image(float s) {
    const uint32_t u = __float_as_uint(s + 0.f);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ uint64_t score_key(float s, int64_t j) {
    return ((uint64_t)score_image(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

// One wave selects among the spans j = lane + 64 i (i < PER_LANE) whose score images img[i] are
// given (0 for j >= r) the m = min(k, r) largest keys  img << 32 | (0xFFFFFFFF - j)  and writes
// their span indices to out[0..k) (ascending, -1 padded).  cand: 64 words of LDS owned by the wave.
//
// Threshold first: v = the m-th largest of the 64 per-lane maximum images with its low 16 bits
// cleared, found bit by bit from the top: a bit is kept when at least m lanes still reach the
// value (one ballot per bit, 16 bits: sign, exponent and 7 significand bits of the score).  At
// least m lanes then hold an image >= v, so every one of the m winners has an image >= v (the
// cleared bits only lower v: the extra candidates are scores within 2^-7 of the threshold).  The
// spans with images >= v (usually little more than m; more only where scores tie) are compacted
// into LDS in span order as 64-bit keys and each is ranked against the others; if more than 64
// pass, the selection falls back to m rounds of "largest key below the previous winner".  Only
// the candidates become 64-bit keys: the rest of the work is on 32-bit images.
template <int PER_LANE>
__device__ __forceinline__ void wave_topk(const uint32_t (&img)[PER_LANE], int m, int k, int lane, uint64_t *cand,
                                          int32_t *out) {
    if (m == 0) {
        if (lane < k) out[lane] = -1;
        return;
    }
    // per-lane maximum image
    uint32_t lmax = img[0];
#pragma unroll
    for (int i = 1; i < PER_LANE; ++i) lmax = img[i] > lmax ? img[i] : lmax;
    // at least m lanes hold a valid image (candidates are dealt round-robin and m <= r), so the
    // search ends on a valid image
    uint32_t v = 0;
#pragma unroll
    for (int bit = 31; bit >= 16; --bit) {
        const uint32_t test = v | (1u << bit);
        if ((int)__builtin_popcountll(__ballot(lmax >= test)) >= m) v = test;
    }

    int C = 0;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
        const bool c = img[i] >= v;
        const uint64_t b = __ballot(c);
        if (b == 0ull) continue;  // (most registers hold no candidate)
        const int pos = C + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
        if (c && pos < 64) cand[pos] = ((uint64_t)img[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(lane + 64 * i));
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
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) {
            const uint64_t key = img[i] ? ((uint64_t)img[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(lane + 64 * i))
                                        : 0ull;
            best = (key < last && key > best) ? key : best;
        }
        best = wave_max_u64(best);
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
