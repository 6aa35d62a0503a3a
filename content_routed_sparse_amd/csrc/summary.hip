// Span summaries: fp32 running sum of each span's keys in token order, mean on completion
// (the span summary that queries score; release post, "Key idea").
//
// Work unit = (sequence, kv head, touched span).  Units are independent except through the
// open span's running sum: the first touched span continues it, the last touched span leaves
// the new value.  The first span's units run in one launch and the others in a second launch
// on the same stream, so the read of the old running sum never races with the write of the
// new one.  Within a unit, block threads own one element each and add the span's keys
// sequentially (exactly the token-order fp32 additions of the definition), with the keys
// staged through LDS in coalesced 16-byte loads.  Few new tokens (decode): summary_kernel, one
// 64-token stage at a time.  Many (prefill, setup): summary_stream, whose 1024 threads keep the
// loads of the next kPipeDepth stages in flight in registers while the current stage is added,
// so a unit streams its span instead of waiting for one stage at a time.  Both add the same
// values in the same order.
#include "common.h"
#include "kernels.h"
#include "summary_body.h"

namespace ra {
namespace {

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
    summary_unit<T, D>(K, kscale, mean, run_sum, old_len, new_len, Hkv, S, cap, max_spans, u_base, U, blockIdx.x, stage);
}

constexpr int kPipeThreads = 1024;
constexpr int kPipeDepth = 8;  // stages whose loads are in flight ahead of the one being added

template <typename T, int D>
__global__ void __launch_bounds__(kPipeThreads) summary_stream(const T *__restrict__ K, const float *__restrict__ kscale,
                                                               float *__restrict__ mean, float *__restrict__ run_sum,
                                                               const int64_t *__restrict__ old_len,
                                                               const int64_t *__restrict__ new_len, int Hkv, int S,
                                                               int64_t cap, int64_t max_spans, int u_base, int U) {
    constexpr int kVec = 16 / sizeof(T);                 // elements per 16-byte load
    constexpr int kVecPerTok = D / kVec;                 // 16-byte loads per token
    constexpr int PIECES = kStageTokens * kVecPerTok;    // 16-byte loads per stage
    constexpr int PPT = (PIECES + kPipeThreads - 1) / kPipeThreads;
    __shared__ float stage[2][kStageTokens][D];

    const int u = u_base + (int)(blockIdx.x % U);
    const int bg = (int)(blockIdx.x / U);  // sequence * Hkv + kv head
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
    const int nst = (int)((p1 - p0 + kStageTokens - 1) / kStageTokens);

    const int tid = threadIdx.x;
    const T *base = K + (int64_t)bg * cap * D;
    const float *sbase = kscale + (int64_t)bg * cap;
    uint4 pf[kPipeDepth][PPT];
    float pfs[kPipeDepth][PPT];
    // this thread's pieces of stage st (tokens past the span's new end are not loaded)
    auto fetch = [&](int st, uint4 (&dst)[PPT], float (&dsc)[PPT]) {
#pragma unroll
        for (int q = 0; q < PPT; ++q) {
            const int v = tid + q * kPipeThreads;
            const int64_t p = p0 + (int64_t)st * kStageTokens + v / kVecPerTok;
            if (v < PIECES && st < nst && p < p1) {
                dst[q] = *reinterpret_cast<const uint4 *>(base + p * D + (v % kVecPerTok) * kVec);
                if constexpr (sizeof(T) == 1) dsc[q] = sbase[p];
            }
        }
    };
#pragma unroll
    for (int i = 0; i < kPipeDepth; ++i) fetch(i, pf[i], pfs[i]);

    float acc = 0.f;
    if (u == 0 && tid < D) acc = run_sum[(int64_t)bg * D + tid];
    for (int s0 = 0; s0 < nst; s0 += kPipeDepth) {
#pragma unroll
        for (int i = 0; i < kPipeDepth; ++i) {
            const int st = s0 + i;
            if (st >= nst) break;
            const int64_t pst = p0 + (int64_t)st * kStageTokens;
            const int n = (int)((p1 - pst) < kStageTokens ? (p1 - pst) : kStageTokens);
            float (*buf)[D] = stage[st & 1];
            // the cache's values of this thread's pieces (the conversions of summary_unit)
#pragma unroll
            for (int q = 0; q < PPT; ++q) {
                const int v = tid + q * kPipeThreads;
                const int tok = v / kVecPerTok, piece = v % kVecPerTok;
                if (v < PIECES && tok < n) {
                    const uint4 raw = pf[i][q];
                    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
                    if constexpr (sizeof(T) == 1) {
                        const float sc = pfs[i][q];
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
                            float *dst = &buf[tok][piece * 16 + 4 * x];
                            dst[0] = __builtin_amdgcn_cvt_f32_fp8((int)w[x], 0) * sc;
                            dst[1] = __builtin_amdgcn_cvt_f32_fp8((int)w[x], 1) * sc;
                            dst[2] = __builtin_amdgcn_cvt_f32_fp8((int)w[x], 2) * sc;
                            dst[3] = __builtin_amdgcn_cvt_f32_fp8((int)w[x], 3) * sc;
                        }
                    } else if constexpr (sizeof(T) == 2) {
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
                            buf[tok][piece * 8 + 2 * x] = bf16_bits_to_f32(w[x] & 0xFFFFu);
                            buf[tok][piece * 8 + 2 * x + 1] = bf16_bits_to_f32(w[x] >> 16);
                        }
                    } else {
#pragma unroll
                        for (int x = 0; x < 4; ++x) buf[tok][piece * 4 + x] = __uint_as_float(w[x]);
                    }
                }
            }
            fetch(st + kPipeDepth, pf[i], pfs[i]);
            __syncthreads();
            if (tid < D) {
                for (int tok = 0; tok < n; ++tok) acc = acc + buf[tok][tid];  // token order, fp32
            }
        }
    }
    if (tid >= D) return;
    const bool complete = (p1 == j * S + S);
    if (complete && j < max_spans) mean[((int64_t)bg * max_spans + j) * D + tid] = acc / (float)S;
    if (p1 == hi) run_sum[(int64_t)bg * D + tid] = complete ? 0.f : acc;
}

template <typename T, int D>
hipError_t launch_summary_t(const SummaryArgs &a, hipStream_t st) {
    // spans touched by at most max_new consecutive tokens starting anywhere in a span
    const int64_t max_new = a.max_new < 1 ? 1 : a.max_new;
    const int64_t U = (max_new - 1 + a.S - 1) / a.S + 1;
    const int64_t units0 = (int64_t)a.B * a.Hkv;
    const int threads = D < 128 ? 128 : D;
    // a unit adds at most min(S, max_new) tokens: stream them when that is more than one stage
    const bool stream = (max_new < a.S ? max_new : a.S) > kStageTokens;
    auto kern = stream ? summary_stream<T, D> : summary_kernel<T, D>;
    const int nthr = stream ? kPipeThreads : threads;
    hipLaunchKernelGGL(kern, dim3((unsigned)units0), dim3(nthr), 0, st, (const T *)a.k, a.kscale, a.mean, a.run_sum,
                       a.old_len, a.new_len, a.Hkv, a.S, a.cap, a.max_spans, 0, 1);
    if (U > 1) {
        const int64_t rest = U - 1;
        hipLaunchKernelGGL(kern, dim3((unsigned)(units0 * rest)), dim3(nthr), 0, st, (const T *)a.k, a.kscale, a.mean,
                           a.run_sum, a.old_len, a.new_len, a.Hkv, a.S, a.cap, a.max_spans, 1, (int)rest);
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
