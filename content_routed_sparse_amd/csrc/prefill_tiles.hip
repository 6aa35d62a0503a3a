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

constexpr int kMfmaWaves = 8;                   // waves per block
constexpr int kMfmaQT = 1;                      // 16-query tiles per wave
constexpr int kMfmaTile = kMfmaWaves * 16 * kMfmaQT;  // entries per tile (128)
constexpr int kChunk = 64;                      // keys per LDS stage
constexpr int kMfmaThreads = kMfmaWaves * 64;

// XCD-aware order: the hardware hands block b to XCD b % 8; give XCD x a contiguous range of
// the tile list (tiles of one span are consecutive) so that they share its L2.
// Bijective on [0, grid): XCD x owns the range starting at x * (grid / 8) + min(x, grid % 8).
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t grid) {
    const int64_t q = grid / 8, rem = grid % 8, x = b % 8, i = b / 8;
    return x * q + (x < rem ? x : rem) + i;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
#define RA_LDS __attribute__((address_space(3)))

// LDS layout of a staged chunk: kChunk rows of D bf16, unpadded (global_load_lds writes 1 KB
// contiguous per wave instruction), with the 16-byte pieces of each row permuted by an XOR so
// that the MFMA operand reads do not collide on banks:
//   K: piece p of row r at position p ^ (r mod P), P = D / 8 pieces per row;
//   V: piece p of row r at position p ^ 2 (r mod 4).
template <int D>
__device__ __forceinline__ int kswz(int r) { return r % (D / 8); }
__device__ __forceinline__ int vswz(int r) { return 2 * (r & 3); }

// Issue the direct global -> LDS loads of chunk [c0, c0 + kChunk) into (Kd, Vd); rows past
// `hi` repeat row hi - 1 (masked later).  Each wave instruction fills 1 KB = 1024 / (2 D) rows.
template <int D>
__device__ __forceinline__ void chunk_load(const uint16_t *Kb, const uint16_t *Vb, uint16_t *Kd, uint16_t *Vd,
                                           int64_t c0, int64_t hi, int wave, int lane) {
    constexpr int ROWS = 1024 / (2 * D);     // rows per wave instruction
    constexpr int NI = kChunk / ROWS;        // instructions per tensor per chunk
    constexpr int P = D / 8;                 // pieces per row
#pragma unroll
    for (int ii = wave; ii < NI; ii += kMfmaWaves) {
        const int r = ii * ROWS + lane / P;  // chunk row written by this lane
        const int phys = lane % P;
        int64_t g = c0 + r;
        g = g < hi ? g : hi - 1;
        const uint16_t *ksrc = Kb + g * D + (phys ^ kswz<D>(r)) * 8;
        const uint16_t *vsrc = Vb + g * D + (phys ^ vswz(r)) * 8;
        __builtin_amdgcn_global_load_lds((const void *)ksrc, (RA_LDS void *)(Kd + ii * ROWS * D), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void *)vsrc, (RA_LDS void *)(Vd + ii * ROWS * D), 16, 0, 0);
    }
}

// Transposed formulation.  S^T = K Q^T puts keys on the MFMA rows and queries on the columns,
// so lane (lg, lr) holds keys 16kt + 4lg + i of query lr: every per-query quantity (running
// max, sum, rescale of the output) is lane-local, and only the max/sum across the 4 lane
// groups of a query needs cross-lane steps.  O^T = V^T P^T then takes P straight from the S^T
// registers: its 32-key K dimension is ordered as the lanes hold it (keys 4lg..4lg+3 of two
// 16-key tiles per lane group), and V^T is read from LDS in the same order.
template <int D>
__global__ void __launch_bounds__(kMfmaThreads) tile_mfma(const uint16_t *__restrict__ q, const int64_t *__restrict__ row_pos,
                                                 const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
                                                 const int32_t *__restrict__ counts,
                                                 const int32_t *__restrict__ offsets,
                                                 const int32_t *__restrict__ tile_off,
                                                 const int32_t *__restrict__ list, const int2 *__restrict__ tiles,
                                                 float *__restrict__ records, int64_t n_exp, int64_t span_slots,
                                                 int NE, int Hq, int S, int64_t cap, int64_t max_pos,
                                                 float scale_log2) {
    constexpr int KS = D / 32;   // k-steps of the QK product
    constexpr int ET = D / 16;   // 16-wide e tiles of the PV product
    constexpr int KT = kChunk / 16;
    constexpr int NT = kMfmaThreads, QT = kMfmaQT;
    constexpr float NEG = -__builtin_huge_valf();
    __shared__ uint16_t Ks[2][kChunk * D];
    __shared__ uint16_t Vs[2][kChunk * D];
    __shared__ int64_t row_t[kMfmaTile];
    __shared__ int32_t row_x[kMfmaTile];
    __shared__ unsigned long long tmax_s, tmin_s;

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

    if (tid == 0) {
        tmax_s = 0;
        tmin_s = ~0ull;
    }
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
    __syncthreads();
    if (tid < n) {
        atomicMax(&tmax_s, (unsigned long long)row_t[tid]);
        atomicMin(&tmin_s, (unsigned long long)row_t[tid]);
    }
    __syncthreads();
    const int64_t tmax = (int64_t)tmax_s, tmin = (int64_t)tmin_s;
    int64_t hi = lo + S;  // keys of the span used by the tile: [lo, hi)
    if (hi > tmax + 1) hi = tmax + 1;
    if (hi > cap) hi = cap;

    // B operand of S^T: this wave's 2 x 16 gathered query rows, all k-steps, in registers
    bf16x8_t qb[QT][KS];
    int64_t tq[QT];  // position of query (a, lr); -1 for padding
#pragma unroll
    for (int a = 0; a < QT; ++a) {
        const int r = 16 * QT * wave + 16 * a + lr;
        const int32_t x = row_x[r];
        tq[a] = row_t[r];
        const int64_t rh = x >= 0 ? x / NE : 0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 raw = *reinterpret_cast<const uint4 *>(q + rh * D + 32 * ks + 8 * lg);
            if (x < 0) raw = make_uint4(0, 0, 0, 0);
            qb[a][ks] = __builtin_bit_cast(bf16x8_t, raw);
        }
    }
    float m[QT], l[QT];
    f32x4_t o[QT][ET];
#pragma unroll
    for (int a = 0; a < QT; ++a) {
        m[a] = NEG;
        l[a] = 0.f;
#pragma unroll
        for (int et = 0; et < ET; ++et) o[a][et] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    const uint16_t *Kb = K + sg * cap * D;
    const uint16_t *Vb = V + sg * cap * D;
    // double-buffered chunks: the loads of chunk c+1 fly while chunk c is computed
    if (lo < hi) chunk_load<D>(Kb, Vb, Ks[0], Vs[0], lo, hi, wave, lane);
    int buf = 0;
    for (int64_t k0 = lo; k0 < hi; k0 += kChunk, buf ^= 1) {
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of chunk c landed
        __syncthreads();  // everyone's loads landed, and everyone finished reading the other buffer
        if (k0 + kChunk < hi) chunk_load<D>(Kb, Vb, Ks[buf ^ 1], Vs[buf ^ 1], k0 + kChunk, hi, wave, lane);
        const uint16_t *Kc = Ks[buf];
        const uint16_t *Vc = Vs[buf];
        // a chunk needs masks only where it passes the span's end or some row's position
        const bool full = (k0 + kChunk <= hi) && (k0 + kChunk - 1 <= tmin);

        // S^T = K Q^T: 4 key tiles x 2 query tiles
        f32x4_t sc[KT][QT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            bf16x8_t ka[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int r = 16 * kt + lr;
                ka[ks] = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const uint4 *>(&Kc[r * D + (((4 * ks + lg) ^ kswz<D>(r)) * 8)]));
            }
#pragma unroll
            for (int a = 0; a < QT; ++a) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks], qb[a][ks], acc, 0, 0, 0);
                sc[kt][a] = acc;  // S^T[key 16kt + 4lg + i][query 16a + lr]
            }
        }
        // online softmax, per query (lane-local) with the max/sum across the 4 lane groups
        uint32_t pk[QT][KT][2];  // P as bf16 pairs: [a][kt][i/2]
#pragma unroll
        for (int a = 0; a < QT; ++a) {
            float cmax = NEG;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float z = sc[kt][a][i] * scale_log2;
                    if (!full) {
                        const int64_t p = k0 + 16 * kt + 4 * lg + i;
                        z = (p < hi && p <= tq[a]) ? z : NEG;
                    }
                    sc[kt][a][i] = z;
                    cmax = fmaxf(cmax, z);
                }
            }
            cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
            cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
            const float mn = fmaxf(m[a], cmax);
            const bool live = mn != NEG;
            // v_exp_f32 directly: arguments are <= 0, results in [0, 1] (tiny ones may flush to 0)
            const float alpha = live ? __builtin_amdgcn_exp2f(m[a] - mn) : 1.f;
            float psum = 0.f;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                float pv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pv[i] = live ? __builtin_amdgcn_exp2f(sc[kt][a][i] - mn) : 0.f;
                    psum += pv[i];
                }
                pk[a][kt][0] = pack_bf16x2(pv[0], pv[1]);
                pk[a][kt][1] = pack_bf16x2(pv[2], pv[3]);
            }
            psum += __shfl_xor(psum, 16);
            psum += __shfl_xor(psum, 32);
            l[a] = l[a] * alpha + psum;
            m[a] = mn;
#pragma unroll
            for (int et = 0; et < ET; ++et) o[a][et] *= alpha;
        }
        // O^T += V^T P^T, 32-key steps: K slots 8lg..8lg+7 <-> keys (2kk)16 + 4lg + 0..3 and
        // (2kk+1)16 + 4lg + 0..3 for both operands
#pragma unroll
        for (int kk = 0; kk < KT / 2; ++kk) {
            bf16x8_t pb[QT];
#pragma unroll
            for (int a = 0; a < QT; ++a) {
                const uint4 raw = make_uint4(pk[a][2 * kk][0], pk[a][2 * kk][1], pk[a][2 * kk + 1][0], pk[a][2 * kk + 1][1]);
                pb[a] = __builtin_bit_cast(bf16x8_t, raw);
            }
#pragma unroll
            for (int et = 0; et < ET; ++et) {
                // transposed reads: lane (lg, i) gets V[key][16 et + i] for 4 consecutive keys; the
                // 16 lanes of a group address rows base + j/4, columns 16 et + 4 (j % 4)
                uint32_t vw[4];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = 32 * kk + 16 * h + 4 * lg + (lr >> 2);
                    const int col = 16 * et + 4 * (lr & 3);
                    const int addr = r * D + (((col >> 3) ^ vswz(r)) << 3) + (col & 7);
                    const v4i16_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((RA_LDS v4i16_t *)(Vc + addr));
                    vw[2 * h] = (uint32_t)(uint16_t)t[0] | ((uint32_t)(uint16_t)t[1] << 16);
                    vw[2 * h + 1] = (uint32_t)(uint16_t)t[2] | ((uint32_t)(uint16_t)t[3] << 16);
                }
                const bf16x8_t va = __builtin_bit_cast(bf16x8_t, make_uint4(vw[0], vw[1], vw[2], vw[3]));
#pragma unroll
                for (int a = 0; a < QT; ++a) o[a][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[a], o[a][et], 0, 0, 0);
            }
        }
    }

    // records: (m, l, o[d]) per valid row; lane (lg, lr) holds o[16et + 4lg + i] of query lr
#pragma unroll
    for (int a = 0; a < QT; ++a) {
        const int32_t x = row_x[16 * QT * wave + 16 * a + lr];
        if (x < 0) continue;
        float *rec = records + (int64_t)x * record_floats(D);
#pragma unroll
        for (int et = 0; et < ET; ++et)
            *reinterpret_cast<float4 *>(rec + 4 + 16 * et + 4 * lg) =
                make_float4(o[a][et][0], o[a][et][1], o[a][et][2], o[a][et][3]);
        if (lg == 0) {
            rec[0] = m[a];
            rec[1] = l[a];
        }
    }
}

template <int D>
hipError_t mfma_launch(const TileArgs &t, hipStream_t st) {
    const RowArgs &a = t.a;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    hipLaunchKernelGGL((tile_mfma<D>), dim3((unsigned)t.max_tiles), dim3(kMfmaThreads), 0, st, (const uint16_t *)a.q, a.row_pos,
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
