// Span-summary work unit shared by the summary kernel and the decode merge kernel that can append
// new tokens in the same launch (the update never touches what the attention reads).
#pragma once

#include "common.h"

namespace ra {

constexpr int kStageTokens = 64;  // tokens staged through LDS per step

// One work unit (sequence * Hkv + kv head, touched span u_base + unit % U); `stage` is the
// block's LDS staging area.  Every thread of the block calls it (it synchronises the block).
template <typename T, int D>
__device__ __forceinline__ void summary_unit(const T *__restrict__ K, const float *__restrict__ kscale,
                                             float *__restrict__ mean, float *__restrict__ run_sum,
                                             const int64_t *__restrict__ old_len, const int64_t *__restrict__ new_len,
                                             int Hkv, int S, int64_t cap, int64_t max_spans, int u_base, int U,
                                             int unit, float (*stage)[D]) {
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

}  // namespace ra
