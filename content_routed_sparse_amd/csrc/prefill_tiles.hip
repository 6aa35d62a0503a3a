// Prefill tiles: each tile is up to MT (row-head, entry) pairs that attend to the same span of
// one (sequence, kv head); the tile produces each pair's partial softmax state over the span's
// keys (masked to keys <= the row's position).
//
// tile_mfma (bf16): a block takes up to 128 entries (4 waves x 32 rows) and streams the span's
// keys through LDS in chunks of 32: K row-major, V transposed, so that both products run on
// v_mfma_f32_16x16x32_bf16 -- S = Q K^T (gathered query rows as the A operand, kept in
// registers) and O += P V (P rounded to bf16 through a per-wave LDS tile).  The softmax is
// online, per row, with DPP reductions across the 16 lanes that hold a row's scores.
// Tiles of one span are consecutive in the tile list and are spread over the 8 XCDs in
// contiguous ranges, so the blocks that reread a span's keys share an L2.
//
// tile_valu: one wave per entry, keys streamed in chunks of KPW rows with an online softmax
// (fp32 inputs).  The span's rows are shared by the tile's entries through the caches.
#include "common.h"
#include "prefill_tiles.h"
#include "wave_ops.h"

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

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMfmaTile = 128;  // entries per tile: 4 waves x 32 rows
constexpr int kChunk = 32;      // keys per LDS stage

// XCD-aware order: the hardware hands block b to XCD b % 8; give XCD x a contiguous range of
// the tile list (tiles of one span are consecutive) so that they share its L2.
// Bijective on [0, grid): XCD x owns the range starting at x * (grid / 8) + min(x, grid % 8).
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t grid) {
    const int64_t q = grid / 8, rem = grid % 8, x = b % 8, i = b / 8;
    return x * q + (x < rem ? x : rem) + i;
}

template <int D>
__global__ void __launch_bounds__(256) tile_mfma(const uint16_t *__restrict__ q, const int64_t *__restrict__ row_pos,
                                                 const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
                                                 const int32_t *__restrict__ counts,
                                                 const int32_t *__restrict__ offsets,
                                                 const int32_t *__restrict__ tile_off,
                                                 const int32_t *__restrict__ list, const int2 *__restrict__ tiles,
                                                 float *__restrict__ records, int64_t n_exp, int64_t span_slots,
                                                 int NE, int Hq, int S, int64_t cap, int64_t max_pos,
                                                 float scale_log2) {
    constexpr int KS = D / 32;   // k-steps of the QK product
    constexpr int ET = D / 16;   // 16-wide output tiles of the PV product
    constexpr int KROW = D + 8;  // LDS row pitch of K (bf16 elements)
    constexpr int VROW = kChunk + 8;
    constexpr int PROW = kChunk + 8;
    __shared__ uint16_t Ks[kChunk * KROW];
    __shared__ uint16_t Vt[D * VROW];
    __shared__ uint16_t Ps[4][32 * PROW];
    __shared__ int64_t row_t[kMfmaTile];
    __shared__ int32_t row_x[kMfmaTile];
    __shared__ int64_t tmax_s;

    const int64_t total = tile_off[n_exp];
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    if (tile >= total) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lg = lane >> 4, lr = lane & 15;
    const int2 tl = tiles[tile];
    const int64_t expert = tl.x;
    const int count = counts[expert];
    const int n = count - tl.y < kMfmaTile ? count - tl.y : kMfmaTile;
    const int64_t j = expert % span_slots;
    const int64_t sg = expert / span_slots;
    const int32_t *entries = list + offsets[expert] + tl.y;
    const int64_t lo = j * S;

    // rows of the tile: entry id and position (t = -1 for padding rows: everything masked)
    if (tid < kMfmaTile) {
        int32_t x = -1;
        int64_t t = -1;
        if (tid < n) {
            x = entries[tid];
            t = row_pos[(x / NE) / Hq];
            t = t < 0 ? 0 : (t > max_pos ? max_pos : t);
        }
        row_x[tid] = x;
        row_t[tid] = t;
    }
    if (tid == 0) tmax_s = 0;  // valid rows have t >= 0 (and a tile holds at least one)
    __syncthreads();
    if (tid < n) atomicMax((unsigned long long *)&tmax_s, (unsigned long long)row_t[tid]);
    __syncthreads();
    // keys of the span this tile needs: [lo, hi), hi <= tmax + 1 (keys after every row are skipped)
    const int64_t tmax = tmax_s;
    int64_t hi = lo + S;
    if (hi > tmax + 1) hi = tmax + 1;
    if (hi > cap) hi = cap;

    // A operand: this wave's 2 x 16 gathered query rows, all k-steps, in registers
    bf16x8_t qa[2][KS];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int32_t x = row_x[32 * wave + 16 * a + lr];
        const int64_t rh = x >= 0 ? x / NE : 0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 raw = *reinterpret_cast<const uint4 *>(q + rh * D + 32 * ks + 8 * lg);
            if (x < 0) raw = make_uint4(0, 0, 0, 0);
            qa[a][ks] = __builtin_bit_cast(bf16x8_t, raw);
        }
    }
    // positions of the rows this lane's outputs belong to: rows 32w + 16a + 4lg + i
    int64_t trow[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) trow[a][i] = row_t[32 * wave + 16 * a + 4 * lg + i];

    float m[2][4], l[2][4];
    f32x4_t o[2][ET];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m[a][i] = -__builtin_huge_valf();
            l[a][i] = 0.f;
        }
#pragma unroll
        for (int et = 0; et < ET; ++et) o[a][et] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    const uint16_t *Kb = K + sg * cap * D;
    const uint16_t *Vb = V + sg * cap * D;
    for (int64_t k0 = lo; k0 < hi; k0 += kChunk) {
        // stage K rows [k0, k0+32) (row-major) and V^T (keys contiguous per element)
        __syncthreads();
        for (int v = tid; v < kChunk * (D / 8); v += 256) {
            const int key = v / (D / 8), piece = v % (D / 8);
            int64_t p = k0 + key;
            p = p < hi ? p : hi - 1;
            *reinterpret_cast<uint4 *>(&Ks[key * KROW + piece * 8]) =
                *reinterpret_cast<const uint4 *>(Kb + p * D + piece * 8);
        }
        for (int v = tid; v < (kChunk / 2) * (D / 8); v += 256) {
            const int kp = v / (D / 8), piece = v % (D / 8);
            int64_t p0 = k0 + 2 * kp, p1 = p0 + 1;
            p0 = p0 < hi ? p0 : hi - 1;
            p1 = p1 < hi ? p1 : hi - 1;
            const uint4 r0 = *reinterpret_cast<const uint4 *>(Vb + p0 * D + piece * 8);
            const uint4 r1 = *reinterpret_cast<const uint4 *>(Vb + p1 * D + piece * 8);
            const uint32_t w0[4] = {r0.x, r0.y, r0.z, r0.w}, w1[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = piece * 8 + 2 * i;
                *reinterpret_cast<uint32_t *>(&Vt[e * VROW + 2 * kp]) = (w0[i] & 0xFFFFu) | (w1[i] << 16);
                *reinterpret_cast<uint32_t *>(&Vt[(e + 1) * VROW + 2 * kp]) = (w0[i] >> 16) | (w1[i] & 0xFFFF0000u);
            }
        }
        __syncthreads();

        // S = Q K^T for 2 row tiles x 2 key tiles
        f32x4_t sacc[2][2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            bf16x8_t kb[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kb[ks] = __builtin_bit_cast(bf16x8_t,
                                            *reinterpret_cast<const uint4 *>(&Ks[(16 * nb + lr) * KROW + 32 * ks + 8 * lg]));
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[a][ks], kb[ks], acc, 0, 0, 0);
                sacc[a][nb] = acc;
            }
        }
        // online softmax per row (row = 16 lanes of one DPP row x 2 key tiles)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float z[2];
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const int64_t p = k0 + 16 * nb + lr;
                    z[nb] = (p < hi && p <= trow[a][i]) ? sacc[a][nb][i] * scale_log2 : -__builtin_huge_valf();
                }
                const float cmax = allreduce_max<8>(fmaxf(z[0], z[1]));
                const float mn = fmaxf(m[a][i], cmax);
                const bool live = mn != -__builtin_huge_valf();
                const float alpha = live ? exp2f(m[a][i] - mn) : 1.f;
                float psum = 0.f;
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const float pv = live ? exp2f(z[nb] - mn) : 0.f;
                    const uint32_t pb = f32_to_bf16_bits(pv);
                    psum += bf16_bits_to_f32(pb);
                    Ps[wave][(16 * a + 4 * lg + i) * PROW + 16 * nb + lr] = (uint16_t)pb;
                }
                l[a][i] = l[a][i] * alpha + allreduce_sum<8>(psum);
                m[a][i] = mn;
#pragma unroll
                for (int et = 0; et < ET; ++et) o[a][et][i] *= alpha;
            }
        }
        __builtin_amdgcn_wave_barrier();
        // O += P V
        bf16x8_t pa[2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
            pa[a] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(&Ps[wave][(16 * a + lr) * PROW + 8 * lg]));
#pragma unroll
        for (int et = 0; et < ET; ++et) {
            const bf16x8_t vb = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(&Vt[(16 * et + lr) * VROW + 8 * lg]));
#pragma unroll
            for (int a = 0; a < 2; ++a) o[a][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[a], vb, o[a][et], 0, 0, 0);
        }
    }

    // records: (m, l, o[d]) for each valid row
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int32_t x = row_x[32 * wave + 16 * a + 4 * lg + i];
            if (x < 0) continue;
            float *rec = records + (int64_t)x * record_floats(D);
#pragma unroll
            for (int et = 0; et < ET; ++et) rec[4 + 16 * et + lr] = o[a][et][i];
            if (lr == 0) {
                rec[0] = m[a][i];
                rec[1] = l[a][i];
            }
        }
    }
}

template <int D>
hipError_t mfma_launch(const TileArgs &t, hipStream_t st) {
    const RowArgs &a = t.a;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    hipLaunchKernelGGL((tile_mfma<D>), dim3((unsigned)t.max_tiles), dim3(256), 0, st, (const uint16_t *)a.q, a.row_pos,
                       (const uint16_t *)t.K, (const uint16_t *)t.V, t.counts, t.offsets, t.tile_off, t.list, t.tiles,
                       t.records, t.n_exp, t.span_slots, t.NE, a.Hq, a.S, a.cap, a.max_pos, scale_log2);
    return hipGetLastError();
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

int prefill_tile_rows(const RowArgs &a) { return a.dtype == RA_BF16 ? kMfmaTile : kValuTile; }

hipError_t launch_prefill_tiles(const TileArgs &t, hipStream_t st) {
    const RowArgs &a = t.a;
    if (a.dtype == RA_BF16) return a.d == 64 ? mfma_launch<64>(t, st) : mfma_launch<128>(t, st);
    return a.d == 64 ? valu_launch<float, 64>(t, st) : valu_launch<float, 128>(t, st);
}

}  // namespace ra
