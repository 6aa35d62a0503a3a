// Top-k span selection (release post, "Key idea": keep the top k of the scored spans).
//
// One 64-lane wavefront per (row, query head).  Each routable span j < r(t) becomes a 64-bit
// key  (order-preserving image of the fp32 score) << 32 | (0xFFFFFFFF - j),  so a larger key
// means a higher score and, on equal scores, a lower span index: the selection order is a
// strict total order.  Lanes hold their candidates in registers (lane l owns j = l + 64 i).
// The winners are written in ascending span order and padded with -1.
#include "common.h"
#include "kernels.h"
#include "topk_body.h"
#include "wave_ops.h"

namespace ra {
namespace {

// One 64-lane wavefront per (row, query head): the row's scores are loaded into the lanes'
// registers as keys, then wave_topk selects (topk_body.h).
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

    // The row's position and its scores in one round trip: the score loads do not wait for r
    // (indices are clamped to the row's stride, which bounds r; entries j >= r are masked
    // below).  Unconditional loads: a conditional load would be issued and waited for alone.
    const int64_t t_raw = row_pos[rh / Hq];
    uint32_t img[PER_LANE];
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
    // every valid image is > 0, spans past r get 0
    const int rl = (int)(r < 64 * PER_LANE ? r : 64 * PER_LANE);
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) img[i] = lane + 64 * i < rl ? score_image(sv[i]) : 0u;
    wave_topk<PER_LANE>(img, m, k, lane, cand[wave], sel + rh * k);
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
