// Prefill tiles: each tile is up to MT (row-head, entry) pairs that attend to the same span of
// one (sequence, kv head); the tile produces each pair's partial softmax state over the span's
// keys (masked to keys <= the row's position).
//
// tile_valu: one wave per entry, keys streamed in chunks of KPW rows with an online softmax
// (fp32 inputs, and the generic path).  The span's rows are shared by the tile's entries
// through the caches.
#include "common.h"
#include "prefill_tiles.h"

namespace ra {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

template <typename T, int D>
struct WaveLayout {
    static constexpr int EPL = 16 / sizeof(T);
    static constexpr int LPR = D / EPL;
    static constexpr int RPI = 64 / LPR;
    static constexpr int KPW = (sizeof(T) == 4 && D == 128) ? 32 : 64;
    static constexpr int STEPS = KPW / RPI;
};

__device__ __forceinline__ void to_f32(const uint4 &raw, float *f, uint16_t) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
        f[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
}
__device__ __forceinline__ void to_f32(const uint4 &raw, float *f, float) {
    f[0] = __uint_as_float(raw.x);
    f[1] = __uint_as_float(raw.y);
    f[2] = __uint_as_float(raw.z);
    f[3] = __uint_as_float(raw.w);
}

constexpr int kValuTile = 16;

template <typename T, int D>
__global__ void __launch_bounds__(256) tile_valu(const T *__restrict__ q, const int64_t *__restrict__ row_pos,
                                                 const T *__restrict__ K, const T *__restrict__ V,
                                                 const int32_t *__restrict__ counts,
                                                 const int32_t *__restrict__ offsets,
                                                 const int32_t *__restrict__ tile_off,
                                                 const int32_t *__restrict__ list, const int2 *__restrict__ tiles,
                                                 float *__restrict__ records, int64_t n_exp, int64_t span_slots,
                                                 int NE, int Hq, int Hkv, int S, int64_t cap, int64_t max_pos,
                                                 float scale_log2) {
    using L = WaveLayout<T, D>;
    constexpr int EPL = L::EPL, LPR = L::LPR, RPI = L::RPI, KPW = L::KPW, STEPS = L::STEPS;
    const int64_t tile = blockIdx.x;
    if (tile >= tile_off[n_exp]) return;
    const int2 tl = tiles[tile];
    const int64_t expert = tl.x;
    const int count = counts[expert];
    const int n = count - tl.y < kValuTile ? count - tl.y : kValuTile;
    const int64_t j = expert % span_slots;
    const int64_t sg = expert / span_slots;  // sequence * Hkv + kv head
    const int32_t *entries = list + offsets[expert] + tl.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane % LPR, rr = lane / LPR;
    const T *Kb = K + sg * cap * D;
    const T *Vb = V + sg * cap * D;

    for (int i = wave; i < n; i += 4) {
        const int64_t x = entries[i];
        const int64_t rh = x / NE;
        const int64_t row = rh / Hq;
        int64_t t = row_pos[row];
        t = t < 0 ? 0 : (t > max_pos ? max_pos : t);
        const int64_t lo = j * S;
        int64_t hi = lo + S < t + 1 ? lo + S : t + 1;
        if (hi > cap) hi = cap;
        float qf[EPL];
        to_f32(*reinterpret_cast<const uint4 *>(q + rh * D + c * EPL), qf, T());
        float m = kNegInf, l = 0.f, o[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = 0.f;
        for (int64_t k0 = lo; k0 < hi; k0 += KPW) {
            float z[STEPS];
            float cmax = kNegInf;
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                const int64_t key = k0 + s * RPI + rr;
                const bool ok = key < hi;
                const int64_t kl = ok ? key : hi - 1;
                float kf[EPL];
                to_f32(*reinterpret_cast<const uint4 *>(Kb + kl * D + c * EPL), kf, T());
                float acc = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc = fmaf(qf[e], kf[e], acc);
#pragma unroll
                for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off);
                z[s] = ok ? acc * scale_log2 : kNegInf;
                cmax = fmaxf(cmax, z[s]);
            }
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, off));
            const float mn = fmaxf(m, cmax);  // finite: every chunk has a valid key
            const float a = (m == kNegInf) ? 0.f : exp2f(m - mn);
            float csum = 0.f, co[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) co[e] = 0.f;
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                const int64_t key = k0 + s * RPI + rr;
                const bool ok = key < hi;
                const int64_t kl = ok ? key : hi - 1;
                const float p = ok ? exp2f(z[s] - mn) : 0.f;
                csum += p;
                float vf[EPL];
                to_f32(*reinterpret_cast<const uint4 *>(Vb + kl * D + c * EPL), vf, T());
#pragma unroll
                for (int e = 0; e < EPL; ++e) co[e] = fmaf(p, vf[e], co[e]);
            }
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1) {
                csum += __shfl_xor(csum, off);
#pragma unroll
                for (int e = 0; e < EPL; ++e) co[e] += __shfl_xor(co[e], off);
            }
            l = l * a + csum;
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[e] = o[e] * a + co[e];
            m = mn;
        }
        float *rec = records + x * record_floats(D);
        if (rr == 0) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) rec[4 + c * EPL + e] = o[e];
        }
        if (lane == 0) {
            rec[0] = m;
            rec[1] = l;
        }
    }
}

template <typename T, int D>
hipError_t valu_launch(const TileArgs &t, hipStream_t st) {
    const RowArgs &a = t.a;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    hipLaunchKernelGGL((tile_valu<T, D>), dim3((unsigned)t.max_tiles), dim3(256), 0, st, (const T *)a.q, a.row_pos,
                       (const T *)t.K, (const T *)t.V, t.counts, t.offsets, t.tile_off, t.list, t.tiles, t.records,
                       t.n_exp, t.span_slots, t.NE, a.Hq, a.Hkv, a.S, a.cap, a.max_pos, scale_log2);
    return hipGetLastError();
}

}  // namespace

int prefill_tile_rows(const RowArgs &a) {
    (void)a;
    return kValuTile;
}

hipError_t launch_prefill_tiles(const TileArgs &t, hipStream_t st) {
    const RowArgs &a = t.a;
    if (a.dtype == RA_BF16) return a.d == 64 ? valu_launch<uint16_t, 64>(t, st) : valu_launch<uint16_t, 128>(t, st);
    return a.d == 64 ? valu_launch<float, 64>(t, st) : valu_launch<float, 128>(t, st);
}

}  // namespace ra
