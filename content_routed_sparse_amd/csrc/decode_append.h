// Decode with a span-summary append (internal launch interface for the C ABI layer): the
// attention of launch_decode / launch_decode_fp8 plus the summary update `app` (its tokens join
// the summaries; run in the merge launch when it adds one token per sequence, else as its own
// launches after it).  The update reads K and writes span_mean / run_sum, which the attention
// does not read.
#pragma once

#include "kernels.h"

namespace ra {

hipError_t launch_decode_app(const RowArgs &a, const void *K, const void *V, const int32_t *sel, float *out,
                             void *ws, const SummaryArgs *app, hipStream_t st);
hipError_t launch_decode_fp8_app(const RowArgs &a, const uint8_t *K8, const uint8_t *V8, const float *ks,
                                 const float *vs, const int32_t *sel, float *out, void *ws, const SummaryArgs *app,
                                 hipStream_t st);

}  // namespace ra
