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
