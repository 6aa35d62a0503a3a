// Top-k span selection (release post, "Key idea": keep the top k of the scored spans).
//
// One 64-lane wavefront per (row, query head).  Each routable span j < r(t) becomes a 64-bit
// key  (order-preserving image of the fp32 score) << 32 | (0xFFFFFFFF - j),  so a larger key
// means a higher score and, on equal scores, a lower span index: the selection order is a
// strict total order.  Lanes hold their candidates in registers (lane l owns j = l + 64 i);
// m = min(k, r) rounds each take the wave maximum among keys below the previous winner.  The
// winners are then written in ascending span order and padded with -1.
#include "common.h"
#include "kernels.h"
#include "wave_ops.h"

namespace ra {
namespace {

__device__ __forceinline__ uint64_t score_key(float s, int64_t j) {
    uint32_t u = __float_as_uint(s);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}

// PER_LANE candidates per lane kept in registers (r <= 64 * PER_LANE).
template <int PER_LANE>
__global__ void __launch_bounds__(256) topk_kernel(const float *__restrict__ scores, int64_t stride,
                                                   const int64_t *__restrict__ row_pos, int32_t *__restrict__ sel,
                                                   int64_t n_rowheads, int Hq, int k, int S, int W, int64_t max_pos) {
    const int lane = threadIdx.x & 63;
    const int64_t rh = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    if (rh >= n_rowheads) return;
    int64_t t = row_pos[rh / Hq];
    t = t < 0 ? 0 : (t > max_pos ? max_pos : t);
    const int64_t r = num_routable(t, S, W);
    const float *srow = scores + rh * stride;

    // unconditional loads from clamped indices (a conditional load would be issued and waited
    // for one at a time); every valid key is > 0, invalid candidates get key 0
    uint64_t key[PER_LANE];
    float sv[PER_LANE];
    const int64_t jmax = r > 0 ? r - 1 : 0;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
        const int64_t j = lane + 64 * i;
        sv[i] = srow[j < jmax ? j : jmax];
    }
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
        const int64_t j = lane + 64 * i;
        key[i] = j < r ? score_key(sv[i], j) : 0ull;
    }
    const int m = (int)(r < k ? r : k);
    uint64_t last = ~0ull;
    uint32_t mine = 0xFFFFFFFFu;  // lane w keeps the w-th winner's span index
    for (int w = 0; w < m; ++w) {
        // candidates below the previous winner, maximum by a balanced tree (short dependency chain)
        uint64_t f[PER_LANE];
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) f[i] = key[i] < last ? key[i] : 0ull;
#pragma unroll
        for (int width = 1; width < PER_LANE; width *= 2) {
#pragma unroll
            for (int i = 0; i + width < PER_LANE; i += 2 * width) f[i] = f[i + width] > f[i] ? f[i + width] : f[i];
        }
        const uint64_t best = wave_max_u64(f[0]);
        last = best;
        if (lane == w) mine = 0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull);
    }
    // ascending order: rank of each winner among the winners
    int rank = 0;
    for (int w = 0; w < m; ++w) {
        const uint32_t o = __shfl(mine, w);
        rank += (o < mine) ? 1 : 0;
    }
    int32_t *out = sel + rh * k;
    if (lane < m) out[rank] = (int32_t)mine;
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
