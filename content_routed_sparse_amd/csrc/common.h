// Internal device/host helpers shared by the gfx950 kernels of the routed-attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/routed_attn.h"

namespace ra {

constexpr int kWave = 64;

// ------------------------------------------------------------------------------------ numbers
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Round-to-nearest-even fp32 -> bf16 bit pattern (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// kappa of the routing score: the fp32 mean rounded to bf16 and widened back.
__device__ __forceinline__ float round_bf16(float f) { return __uint_as_float(f32_to_bf16_bits(f) << 16); }

// ------------------------------------------------------------------------- span / window rules
// a / b for a >= 0, b > 0, in 32-bit arithmetic whenever a fits (a 64-bit division is a long
// instruction sequence on the GPU).
__device__ __host__ __forceinline__ int64_t div_nonneg(int64_t a, int b) {
    return (uint64_t)a <= 0x7FFFFFFFull ? (int64_t)((uint32_t)a / (uint32_t)b) : a / b;
}
// Number of routable spans: complete spans that end before the window, floor(max(0, t-W+1) / S).
__device__ __host__ __forceinline__ int64_t num_routable(int64_t t, int S, int W) {
    const int64_t a = t - W + 1;
    return a > 0 ? div_nonneg(a, S) : 0;
}
// Window start: span boundary at or below t - W + 1 (never below 0).
__device__ __host__ __forceinline__ int64_t window_start(int64_t t, int S, int W) { return num_routable(t, S, W) * S; }

// Largest number of spans a window can touch: the window has at most W + S - 1 tokens and
// starts on a span boundary.
__host__ __device__ __forceinline__ int max_window_spans(int S, int W) { return (W + S - 2) / S + 1; }

// --------------------------------------------------------------------- partial softmax records
// A partial softmax state over a set of keys: running max m (log2 domain: scores are scaled by
// log2(e)/sqrt(d)), sum l of 2^(z - m), and unnormalised output o[d] = sum 2^(z - m) v.
// Layout of one record: {m, l, 0, 0, o[0..d)} floats (16-byte aligned).
__host__ __device__ __forceinline__ int64_t record_floats(int d) { return 4 + d; }

// Stores of partial records are plain vector stores; the combine kernel reads them after the
// producing kernel finished (stream order).

// ------------------------------------------------------------------------------ launch sizes
__host__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace ra
