// Top-k span selection (release post, "Key idea": keep the top k of the scored spans).
//
// One 64-lane wavefront per (row, query head).  Each routable span j < r(t) becomes a 64-bit
// key  (order-preserving image of the fp32 score) << 32 | (0xFFFFFFFF - j),  so a larger key
// means a higher score and, on equal scores, a lower span index: the selection order is a
// strict total order.  Lanes hold their candidates in registers (lane l owns j = l + 64 i).
// The winners are written in ascending span order and padded with -1.
#include "common.h"
#include "kernels.h"
#include "wave_ops.h"

namespace ra {
namespace {

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

// PER_LANE candidates per lane kept in registers (r <= 64 * PER_LANE).
//
// Threshold first: v = the m-th largest of the 64 per-lane maximum scores (the keys' upper
// halves), found bit by bit from the top: a bit is kept when at least m lanes still reach the
// value (one ballot per bit).  At least m lanes then hold a key >= T0 = v * 2^32, so every one of
// the m winners is >= T0.  The keys >= T0 (usually little more than m; more only where scores
// tie) are compacted into LDS in span order and each is ranked against the others; if more than
// 64 pass, the selection falls back to m rounds of "largest key below the previous winner".
template <int PER_LANE>
__global__ void __launch_bounds__(256) topk_kernel(const float *__restrict__ scores, int64_t stride,
                                                   const int64_t *__restrict__ row_pos, int32_t *__restrict__ sel,
                                                   int64_t n_rowheads, int Hq, int k, int S, int W, int64_t max_pos) {
    __shared__ uint64_t cand[4][64];
    // all kernel arguments in one round trip (otherwise some are fetched only where first used)
    asm volatile("" ::"s"(scores), "s"(stride), "s"(row_pos), "s"(sel), "s"(n_rowheads), "s"(Hq), "s"(k), "s"(S),
                 "s"(W), "s"(max_pos));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t rh = (int64_t)blockIdx.x * (blockDim.x / 64) + wave;
    if (rh >= n_rowheads) return;
    const float *srow = scores + rh * stride;
    int32_t *out = sel + rh * k;

    // The row's position and its scores in one round trip: the score loads do not wait for r
    // (indices are clamped to the row's stride, which bounds r; entries j >= r are masked
    // below).  Unconditional loads: a conditional load would be issued and waited for alone.
    const int64_t t_raw = row_pos[rh / Hq];
    uint64_t key[PER_LANE];
    float sv[PER_LANE];
    const int64_t jmax = stride - 1;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
        const int64_t j = lane + 64 * i;
        sv[i] = srow[j < jmax ? j : jmax];
    }
    asm volatile("" ::: "memory");
    const int64_t t = t_raw < 0 ? 0 : (t_raw > max_pos ? max_pos : t_raw);
    const int64_t r = num_routable(t, S, W);
    const int m = (int)(r < k ? r : k);
    // every valid key is > 0, invalid candidates get key 0
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
        const int64_t j = lane + 64 * i;
        key[i] = j < r ? score_key(sv[i], j) : 0ull;
    }
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
        if (c && pos < 64) cand[wave][pos] = key[i];
        C += (int)__builtin_popcountll(b);
    }
    if (C <= 64) {
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const uint64_t mine = lane < C ? cand[wave][lane] : 0ull;
        int rank = 0;
        for (int j2 = 0; j2 < C; ++j2) rank += cand[wave][j2] > mine ? 1 : 0;
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

// Candidates re-read from memory each round (any r).
__global__ void __launch_bounds__(256) topk_kernel_any(const float *__restrict__ scores, int64_t stride,
                                                       const int64_t *__restrict__ row_pos, int32_t *__restrict__ sel,
                                                       int64_t n_rowheads, int Hq, int k, int S, int W,
                                                       int64_t max_pos) {
    const int lane = threadIdx.x & 63;
    const int64_t rh = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    if (rh >= n_rowheads) return;
    int64_t t = row_pos[rh / Hq];
    t = t < 0 ? 0 : (t > max_pos ? max_pos : t);
    const int64_t r = num_routable(t, S, W);
    const float *srow = scores + rh * stride;
    const int m = (int)(r < k ? r : k);
    uint64_t last = ~0ull;
    uint32_t mine = 0xFFFFFFFFu;
    for (int w = 0; w < m; ++w) {
        uint64_t best = 0;
        for (int64_t j = lane; j < r; j += 64) {
            const uint64_t kk = score_key(srow[j], j);
            best = (kk < last && kk > best) ? kk : best;
        }
        best = wave_max_u64(best);
        last = best;
        if (lane == w) mine = 0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull);
    }
    int rank = 0;
    for (int w = 0; w < m; ++w) {
        const uint32_t o = __shfl(mine, w);
        rank += (o < mine) ? 1 : 0;
    }
    int32_t *out = sel + rh * k;
    if (lane < m) out[rank] = (int32_t)mine;
    else if (lane < k) out[lane] = -1;
}

template <int PL>
hipError_t topk_launch(const RowArgs &a, const float *scores, int64_t stride, int32_t *sel, hipStream_t st) {
    const int64_t n = a.n_rows * a.Hq;
    hipLaunchKernelGGL((topk_kernel<PL>), dim3((unsigned)ceil_div(n, 4)), dim3(256), 0, st, scores, stride, a.row_pos,
                       sel, n, a.Hq, a.k, a.S, a.W, a.max_pos);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const RowArgs &a, const float *scores, int64_t stride, int32_t *sel, hipStream_t st) {
    const int64_t n = a.n_rows * a.Hq;
    if (n == 0) return hipSuccess;
    const int64_t rmax = num_routable(a.max_pos, a.S, a.W);
    if (rmax <= 64 * 2) return topk_launch<2>(a, scores, stride, sel, st);
    if (rmax <= 64 * 8) return topk_launch<8>(a, scores, stride, sel, st);
    if (rmax <= 64 * 17) return topk_launch<17>(a, scores, stride, sel, st);
    if (rmax <= 64 * 40) return topk_launch<40>(a, scores, stride, sel, st);
    hipLaunchKernelGGL(topk_kernel_any, dim3((unsigned)ceil_div(n, 4)), dim3(256), 0, st, scores, stride, a.row_pos,
                       sel, n, a.Hq, a.k, a.S, a.W, a.max_pos);
    return hipGetLastError();
}

}  // namespace ra
