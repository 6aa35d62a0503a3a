// 8-bit key/value cache: rows of d bf16 values stored as FP8 E4M3 codes with one fp32 scale
// per (sequence, kv head, token) row (the release post, "Limitations and next steps", plans
// 8-bit quantisation without a format; this is the library's own).  Scale s = max|x| / 448 (1 for
// an all-zero row), codes = E4M3(x / s) rounded to nearest even after clamping to +-448; the
// cache then holds fl32(E4M3^-1(c) * s), which every later step reads.
//
// One wave quantises 64 / (d / 8) rows: each lane takes 8 consecutive values of a row (one
// 16-byte load), the row maximum comes from a butterfly over the row's lanes, and the lane
// writes its 8 codes with one 8-byte store.
#include "common.h"
#include "kernels.h"

namespace ra {
namespace {

template <int D>
__global__ void __launch_bounds__(256) quantize_kernel(const uint16_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                       float *__restrict__ scale, const int64_t *__restrict__ old_len,
                                                       const int64_t *__restrict__ new_len, int B, int Hkv,
                                                       int64_t cap, int64_t max_new) {
    constexpr int LPR = D / 8;        // lanes per row
    constexpr int RPB = 256 / LPR;    // rows per block
    asm volatile("" ::"s"(src), "s"(dst), "s"(scale), "s"(old_len), "s"(new_len), "s"(B), "s"(Hkv), "s"(cap),
                 "s"(max_new));
    const int tid = threadIdx.x, c = tid % LPR;
    // block = (sequence * Hkv + kv head, group of RPB new tokens)
    const int64_t per_bg = (max_new + RPB - 1) / RPB;
    const int64_t bg = blockIdx.x / per_bg;
    const int64_t i = (blockIdx.x % per_bg) * RPB + tid / LPR;  // new-token index of this lane's row
    const int b = (int)(bg / Hkv);
    int64_t lo = old_len[b], hi = new_len[b];
    if (lo < 0) lo = 0;
    if (hi > cap) hi = cap;
    const int64_t p = lo + i;
    const bool live = i < max_new && p < hi;
    const int64_t row = bg * cap + (live ? p : 0);
    const uint4 raw = *reinterpret_cast<const uint4 *>(src + row * D + c * 8);
    float x[8];
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        x[2 * k] = bf16_bits_to_f32(w[k] & 0xFFFFu);
        x[2 * k + 1] = bf16_bits_to_f32(w[k] >> 16);
    }
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float s = amax > 0.f ? amax / 448.f : 1.f;  // (IEEE division)
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = fminf(fmaxf(x[k] / s, -448.f), 448.f);
    // two codes into the low, then the high half of each word (round to nearest even)
    int lo4 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    lo4 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo4, true);
    int hi4 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
    hi4 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi4, true);
    if (!live) return;
    *reinterpret_cast<uint2 *>(dst + row * D + c * 8) = make_uint2((uint32_t)lo4, (uint32_t)hi4);
    if (c == 0) scale[row] = s;
}

}  // namespace

hipError_t launch_quantize_fp8(const QuantArgs &a, hipStream_t st) {
    if (a.max_new <= 0) return hipSuccess;
    const int lpr = a.d / 8, rpb = 256 / lpr;
    const int64_t blocks = (int64_t)a.B * a.Hkv * ((a.max_new + rpb - 1) / rpb);
    if (a.d == 64)
        hipLaunchKernelGGL((quantize_kernel<64>), dim3((unsigned)blocks), dim3(256), 0, st, a.src, a.dst, a.scale,
                           a.old_len, a.new_len, a.B, a.Hkv, a.cap, a.max_new);
    else
        hipLaunchKernelGGL((quantize_kernel<128>), dim3((unsigned)blocks), dim3(256), 0, st, a.src, a.dst, a.scale,
                           a.old_len, a.new_len, a.B, a.Hkv, a.cap, a.max_new);
    return hipGetLastError();
}

}  // namespace ra
