// Wave64 exchange and reduction helpers for gfx950.
//
// Inside a row of 16 lanes the exchanges use DPP (no LDS traffic, a few cycles each):
//   partner of bit 0 / bit 1: quad_perm xor 1 / xor 2;  bit 2: row_half_mirror (lane i <-> 7-i
//   within 8, which flips bit 2); bit 3: row_ror:8 (lane i <-> i^8 within 16).
// Bits 4 and 5 (across rows) use ds_bpermute (__shfl_xor).  Every partner map is an
// involution that flips the named bit and keeps all higher bits, which is what butterfly
// reduce-scatter and all-reduce need.  Wave-uniform results combine the four rows with
// v_readlane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

constexpr int kDppXor1 = 0xB1;        // quad_perm(1,0,3,2)
constexpr int kDppXor2 = 0x4E;        // quad_perm(2,3,0,1)
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppRor8 = 0x128;       // row_ror:8

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

// Value of the lane that differs in bit log2(OFF) (see partner maps above).
template <int OFF>
__device__ __forceinline__ float partner(float v) {
    if constexpr (OFF == 1) return dpp_f<kDppXor1>(v);
    else if constexpr (OFF == 2) return dpp_f<kDppXor2>(v);
    else if constexpr (OFF == 4) return dpp_f<kDppHalfMirror>(v);
    else if constexpr (OFF == 8) return dpp_f<kDppRor8>(v);
    else return __shfl_xor(v, OFF);
}
template <int OFF>
__device__ __forceinline__ uint32_t partner_u(uint32_t v) {
    if constexpr (OFF == 1) return dpp_u<kDppXor1>(v);
    else if constexpr (OFF == 2) return dpp_u<kDppXor2>(v);
    else if constexpr (OFF == 4) return dpp_u<kDppHalfMirror>(v);
    else if constexpr (OFF == 8) return dpp_u<kDppRor8>(v);
    else return (uint32_t)__shfl_xor((int)v, OFF);
}

// The lane lane ^ OFF exactly (row_half_mirror, used by partner<4>, also flips bits 0 and 1):
// for exchanges between lanes that must agree in every other bit.
template <int OFF>
__device__ __forceinline__ float partner_xor(float v) {
    if constexpr (OFF == 4) return __shfl_xor(v, 4);
    else return partner<OFF>(v);
}

// Sum over the lanes that share all bits above log2(OFF): stages OFF, OFF/2, ..., 1.
template <int OFF>
__device__ __forceinline__ float allreduce_sum(float v) {
    if constexpr (OFF >= 1) {
        v += partner<OFF>(v);
        return allreduce_sum<OFF / 2>(v);
    } else {
        return v;
    }
}
template <int OFF>
__device__ __forceinline__ float allreduce_max(float v) {
    if constexpr (OFF >= 1) {
        v = fmaxf(v, partner<OFF>(v));
        return allreduce_max<OFF / 2>(v);
    } else {
        return v;
    }
}

// Wave-uniform max / sum of one float per lane.
__device__ __forceinline__ float wave_max(float v) {
    v = allreduce_max<8>(v);
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}
__device__ __forceinline__ float wave_sum(float v) {
    v = allreduce_sum<8>(v);
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (a + b) + (c + d);
}

// Wave-uniform maximum of a 64-bit key per lane.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    uint32_t hi = (uint32_t)(v >> 32), lo = (uint32_t)v;
#define RA_STEP(OFF)                                                              \
    {                                                                             \
        const uint32_t ph = partner_u<OFF>(hi), pl = partner_u<OFF>(lo);          \
        const bool take = ph > hi || (ph == hi && pl > lo);                       \
        hi = take ? ph : hi;                                                      \
        lo = take ? pl : lo;                                                      \
    }
    RA_STEP(8) RA_STEP(4) RA_STEP(2) RA_STEP(1)
#undef RA_STEP
    uint64_t best = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint64_t h = (uint32_t)__builtin_amdgcn_readlane((int)hi, 16 * r);
        const uint64_t l = (uint32_t)__builtin_amdgcn_readlane((int)lo, 16 * r);
        const uint64_t x = (h << 32) | l;
        best = x > best ? x : best;
    }
    return best;
}

// One butterfly stage of a reduce-scatter: lanes that differ in bit log2(OFF) exchange halves
// of their N values and add; the lane whose bit is set keeps the upper half.  EXACT: the
// partner is lane ^ OFF (needed when the lanes below bit log2(OFF) hold different data).
template <int N, int OFF, bool EXACT>
__device__ __forceinline__ void rs_stage(float *v, int lane) {
    const bool hi = (lane & OFF) != 0;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
        const float keep = hi ? v[i + N / 2] : v[i];
        const float send = hi ? v[i] : v[i + N / 2];
        v[i] = keep + (EXACT ? partner_xor<OFF>(send) : partner<OFF>(send));
    }
}

// STAGES stages over N values at offsets OFF, OFF/2, ...: N -> N / 2^STAGES values per lane,
// each summed over 2^STAGES lanes.  With all stages, lane bits (high to low) index the value.
template <int N, int STAGES, int OFF, bool EXACT = false>
struct ReduceScatter {
    __device__ __forceinline__ static void run(float *v, int lane) {
        if constexpr (STAGES > 0) {
            rs_stage<N, OFF, EXACT>(v, lane);
            ReduceScatter<N / 2, STAGES - 1, OFF / 2, EXACT>::run(v, lane);
        }
    }
};

constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n / 2); }

}  // namespace ra
