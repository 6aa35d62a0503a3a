// Span summaries: fp32 running sum of each span's keys in token order, mean on completion
// (the span summary that queries score; release post, "Key idea").
//
// Work unit = (sequence, kv head, touched span).  Units are independent except through the
// open span's running sum: the first touched span continues it, the last touched span leaves
// the new value.  The first span's units run in one launch and the others in a second launch
// on the same stream, so the read of the old running sum never races with the write of the
// new one.  Within a unit, block threads own one element each and add the span's keys
// sequentially (exactly the token-order fp32 additions of the definition), with the keys
// staged through LDS in coalesced 16-byte loads.
#include "common.h"
#include "kernels.h"

namespace ra {
namespace {

constexpr int kStageTokens = 64;  // tokens staged through LDS per step

template <typename T, int D>
__global__ void __launch_bounds__(256) summary_kernel(const T *__restrict__ K, const float *__restrict__ kscale,
                                                      float *__restrict__ mean,
                                                      float *__restrict__ run_sum,
                                                      const int64_t *__restrict__ old_len,
                                                      const int64_t *__restrict__ new_len, int Hkv, int S,
                                                      int64_t cap, int64_t max_spans, int u_base, int U) {
    __shared__ float stage[kStageTokens][D];
    // all kernel arguments in one round trip (otherwise some are fetched only where first used)
    asm volatile("" ::"s"(K), "s"(kscale), "s"(mean), "s"(run_sum), "s"(old_len), "s"(new_len), "s"(Hkv), "s"(S), "s"(cap),
                 "s"(max_spans), "s"(u_base), "s"(U));
    const int unit = blockIdx.x;
    const int u = u_base + unit % U;
    const int bg = unit / U;  // sequence * Hkv + kv head
    const int b = bg / Hkv;
    int64_t lo = old_len[b], hi = new_len[b];
    if (hi > cap) hi = cap;
    if (lo < 0) lo = 0;
    if (lo >= hi) return;
    const int64_t j = div_nonneg(lo, S) + u;
    const int64_t p0 = j * S > lo ? j * S : lo;
    int64_t p1 = j * S + S;
    if (p1 > hi) p1 = hi;
    if (p0 >= p1) return;

    const int tid = threadIdx.x;
    const int e = tid;  // element owned by this thread (tid < D)
    float acc = 0.f;
    if (u == 0 && e < D) acc = run_sum[(int64_t)bg * D + e];
    const T *base = K + (int64_t)bg * cap * D;

    constexpr int kVec = 16 / sizeof(T);            // elements per 16-byte load
    constexpr int kVecPerTok = D / kVec;            // 16-byte loads per token
    for (int64_t p = p0; p < p1; p += kStageTokens) {
        const int n = (int)((p1 - p) < kStageTokens ? (p1 - p) : kStageTokens);
        // stage n tokens: every thread loads 16-byte pieces, coalesced over the token rows
        for (int v = tid; v < n * kVecPerTok; v += blockDim.x) {
            const int tok = v / kVecPerTok, piece = v % kVecPerTok;
            const uint4 raw = *reinterpret_cast<const uint4 *>(base + (p + tok) * D + piece * kVec);
            if constexpr (sizeof(T) == 1) {
                // 8-bit codes: the cache's value is fl32(E4M3^-1(c) * s), s the token's scale
                const float sc = kscale[(int64_t)bg * cap + p + tok];
                const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float *dst = &stage[tok][piece * 16 + 4 * i];
                    dst[0] = __builtin_amdgcn_cvt_f32_fp8((int)w[i], 0) * sc;
                    dst[1] = __builtin_amdgcn_cvt_f32_fp8((int)w[i], 1) * sc;
                    dst[2] = __builtin_amdgcn_cvt_f32_fp8((int)w[i], 2) * sc;
                    dst[3] = __builtin_amdgcn_cvt_f32_fp8((int)w[i], 3) * sc;
                }
            } else if constexpr (sizeof(T) == 2) {
                const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    stage[tok][piece * 8 + 2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
                    stage[tok][piece * 8 + 2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
                }
            } else {
                stage[tok][piece * 4 + 0] = __uint_as_float(raw.x);
                stage[tok][piece * 4 + 1] = __uint_as_float(raw.y);
                stage[tok][piece * 4 + 2] = __uint_as_float(raw.z);
                stage[tok][piece * 4 + 3] = __uint_as_float(raw.w);
            }
        }
        __syncthreads();
        if (e < D) {
            for (int tok = 0; tok < n; ++tok) acc = acc + stage[tok][e];  // token order, fp32
        }
        __syncthreads();
    }
    if (e >= D) return;
    const bool complete = (p1 == j * S + S);
    if (complete && j < max_spans) mean[((int64_t)bg * max_spans + j) * D + e] = acc / (float)S;
    if (p1 == hi) run_sum[(int64_t)bg * D + e] = complete ? 0.f : acc;
}

template <typename T, int D>
hipError_t launch_summary_t(const SummaryArgs &a, hipStream_t st) {
    // spans touched by at most max_new consecutive tokens starting anywhere in a span
    const int64_t max_new = a.max_new < 1 ? 1 : a.max_new;
    const int64_t U = (max_new - 1 + a.S - 1) / a.S + 1;
    const int64_t units0 = (int64_t)a.B * a.Hkv;
    const int threads = D < 128 ? 128 : D;
    hipLaunchKernelGGL((summary_kernel<T, D>), dim3((unsigned)units0), dim3(threads), 0, st,
                       (const T *)a.k, a.kscale, a.mean, a.run_sum, a.old_len, a.new_len, a.Hkv, a.S, a.cap, a.max_spans,
                       0, 1);
    if (U > 1) {
        const int64_t rest = U - 1;
        hipLaunchKernelGGL((summary_kernel<T, D>), dim3((unsigned)(units0 * rest)), dim3(threads), 0, st,
                           (const T *)a.k, a.kscale, a.mean, a.run_sum, a.old_len, a.new_len, a.Hkv, a.S, a.cap,
                           a.max_spans, 1, (int)rest);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_summary(const SummaryArgs &a, hipStream_t st) {
    if (a.dtype == kCacheFp8) return a.d == 64 ? launch_summary_t<uint8_t, 64>(a, st) : launch_summary_t<uint8_t, 128>(a, st);
    if (a.dtype == RA_BF16) return a.d == 64 ? launch_summary_t<uint16_t, 64>(a, st) : launch_summary_t<uint16_t, 128>(a, st);
    return a.d == 64 ? launch_summary_t<float, 64>(a, st) : launch_summary_t<float, 128>(a, st);
}

}  // namespace ra
