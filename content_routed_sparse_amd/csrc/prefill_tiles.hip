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

constexpr int kMfmaWaves = 8;                   // waves per block, 16 queries each
constexpr int kMfmaTile = kMfmaWaves * 16;      // entries per tile (128)
constexpr int kChunk = 64;                      // keys per LDS stage
constexpr int kMfmaThreads = kMfmaWaves * 64;

// XCD-aware order: the hardware hands block b to XCD b % 8; give XCD x a contiguous range of
// the tile list (tiles of one span are consecutive) so that they share its L2.
// Bijective on [0, grid): XCD x owns the range starting at x * (grid / 8) + min(x, grid % 8).
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t grid) {
    const int64_t q = grid / 8, rem = grid % 8, x = b % 8, i = b / 8;
    return x * q + (x < rem ? x : rem) + i;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> bf16 (round to nearest even) packed in one register: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
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

// Issue the direct global -> LDS loads of the chunk at key offset c (from the span's first key,
// whose K and V rows start at Ksp, Vsp) into (Kd, Vd); rows at or past `n` (the span's keys in
// use) repeat row n - 1 (masked later).  Each wave instruction fills 1 KB = 1024 / (2 D) rows.
// Offsets are 32-bit (a span's rows span S * D * 2 bytes), so the loads take a scalar base.
template <int D>
__device__ __forceinline__ void chunk_load(const uint16_t *Ksp, const uint16_t *Vsp, uint16_t *Kd, uint16_t *Vd,
                                           int c, int n, int wave, int lane) {
    constexpr int ROWS = 1024 / (2 * D);     // rows per wave instruction
    constexpr int NI = kChunk / ROWS;        // instructions per tensor per chunk
    constexpr int P = D / 8;                 // pieces per row
#pragma unroll
    for (int ii = wave; ii < NI; ii += kMfmaWaves) {
        const int r = ii * ROWS + lane / P;  // chunk row written by this lane
        const int phys = lane % P;
        int g = c + r;
        g = g < n ? g : n - 1;
        const uint32_t kof = (uint32_t)(g * D + (phys ^ kswz<D>(r)) * 8);
        const uint32_t vof = (uint32_t)(g * D + (phys ^ vswz(r)) * 8);
        __builtin_amdgcn_global_load_lds((const void *)(Ksp + kof), (RA_LDS void *)(Kd + ii * ROWS * D), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void *)(Vsp + vof), (RA_LDS void *)(Vd + ii * ROWS * D), 16, 0, 0);
    }
}

// Per-lane LDS byte offsets of the MFMA operand reads inside a staged chunk (every other part
// of an address is an immediate).  K: lane (lg, lr) reads row 16 kt + lr, piece 4 ks + lg, which
// sits at piece (4 ks + lg) ^ (lr mod P).  V (transposed reads): lane (lg, lr) addresses row
// 32 kk + 16 h + 4 lg + c and column 16 et + 4 (lr & 3), c = lr >> 2; with et = 4u + v the
// swizzled 16-byte piece is 2 (4u + (v ^ c)) + ((lr & 3) >> 1).
template <int D>
__device__ __forceinline__ void operand_offsets(int lg, int lr, int (&kof)[D / 32], int (&vof)[4]) {
    constexpr int P = D / 8;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) kof[ks] = 2 * (lr * D + (((4 * ks + lg) ^ (lr % P)) * 8));
    const int c = lr >> 2, b = (lr & 3) >> 1, w = lr & 1;
#pragma unroll
    for (int v = 0; v < 4; ++v) vof[v] = 2 * ((4 * lg + c) * D + 16 * (v ^ c) + 8 * b + 4 * w);
}

// Sum / maximum over the 4 lane groups (lanes l, l^16, l^32, l^48) with the gfx950 lane-swap
// instructions (VALU, no LDS round trip).
__device__ __forceinline__ float group_max4(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum4(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// One 64-key chunk of a wave's 16 queries (lane (lg, lr): query lr, keys 16kt + 4lg + i).
// MASK: some key of the chunk lies past the span's end or past some query's position; `lim` is
// then min(hi, t_query + 1) - k0 for this lane's query (keys at offsets >= lim are masked).
// Scores stay raw until the exponent: 2^(s * c - m) is one FMA and one v_exp_f32.  The output
// is rescaled only when some lane's running maximum moved.
template <int D, bool MASK>
__device__ __forceinline__ void tile_chunk(const char *Kbytes, const char *Vbytes, const int (&kof)[D / 32],
                                           const int (&vof)[4], const bf16x8_t (&qb)[D / 32], float &m, float &l,
                                           f32x4_t (&o)[D / 16], int lim, int lg, float scale_log2) {
    constexpr int KS = D / 32, ET = D / 16, KT = kChunk / 16;
    constexpr float NEG = -__builtin_huge_valf();
    // S^T = K Q^T
    f32x4_t sc[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        bf16x8_t ka[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            ka[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(Kbytes + kof[ks] + 2 * 16 * kt * D));
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks], qb[ks], acc, 0, 0, 0);
        sc[kt] = acc;  // S^T[key 16kt + 4lg + i][query lr]
    }
    float cmax = NEG;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (MASK) sc[kt][i] = 16 * kt + 4 * lg + i < lim ? sc[kt][i] : NEG;
            cmax = fmaxf(cmax, sc[kt][i]);
        }
    }
    const float mn = fmaxf(m, group_max4(cmax) * scale_log2);
    // (masked chunks only: a query with no valid key so far keeps m = -inf, p = 0)
    const bool live = !MASK || mn != NEG;
    const float nmn = live ? -mn : 0.f;
    const float alpha = live ? __builtin_amdgcn_exp2f(m - mn) : 1.f;  // 0 while m = -inf
    float psum = 0.f;
    uint32_t pk[KT][2];  // P as bf16 pairs
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // v_exp_f32 directly: arguments are <= 0 (or -inf), results in [0, 1]
            pv[i] = __builtin_amdgcn_exp2f(fmaf(sc[kt][i], scale_log2, nmn));
            psum += pv[i];
        }
        pk[kt][0] = pack_bf16x2(pv[0], pv[1]);
        pk[kt][1] = pack_bf16x2(pv[2], pv[3]);
    }
    l = fmaf(l, alpha, group_sum4(psum));
    m = live ? mn : m;
#pragma unroll
    for (int et = 0; et < ET; ++et) o[et] *= alpha;
    // O^T += V^T P^T, 32-key steps: K slots 8lg..8lg+7 <-> keys (2kk)16 + 4lg + 0..3 and
    // (2kk+1)16 + 4lg + 0..3 for both operands
#pragma unroll
    for (int kk = 0; kk < KT / 2; ++kk) {
        const bf16x8_t pb =
            __builtin_bit_cast(bf16x8_t, make_uint4(pk[2 * kk][0], pk[2 * kk][1], pk[2 * kk + 1][0], pk[2 * kk + 1][1]));
#pragma unroll
        for (int et = 0; et < ET; ++et) {
            // transposed reads: lane (lg, i) gets V[key][16 et + i] for 4 consecutive keys
            uint2 vw[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const char *pv_addr = Vbytes + vof[et & 3] + 2 * ((32 * kk + 16 * h) * D + 64 * (et >> 2));
                vw[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((RA_LDS v4i16_t *)pv_addr));
            }
            const bf16x8_t va = __builtin_bit_cast(bf16x8_t, make_uint4(vw[0].x, vw[0].y, vw[1].x, vw[1].y));
            o[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[et], 0, 0, 0);
        }
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
    constexpr float NEG = -__builtin_huge_valf();
    // staged chunks: K buffers 0 and 1, then V buffers 0 and 1 (kChunk rows of D bf16 each)
    __shared__ uint16_t stage[4][kChunk * D];
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

    // B operand of S^T: this wave's 16 gathered query rows, all k-steps, in registers
    bf16x8_t qb[KS];
    const int r_own = 16 * wave + lr;
    const int32_t x_own = row_x[r_own];
    const int64_t tq = row_t[r_own];  // position of this lane's query; -1 for padding
    {
        const int64_t rh = x_own >= 0 ? x_own / NE : 0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 raw = *reinterpret_cast<const uint4 *>(q + rh * D + 32 * ks + 8 * lg);
            if (x_own < 0) raw = make_uint4(0, 0, 0, 0);
            qb[ks] = __builtin_bit_cast(bf16x8_t, raw);
        }
    }
    float m = NEG, l = 0.f;
    f32x4_t o[ET];
#pragma unroll
    for (int et = 0; et < ET; ++et) o[et] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const uint16_t *Ksp = K + (sg * cap + lo) * D;  // the span's first key row
    const uint16_t *Vsp = V + (sg * cap + lo) * D;
    const int n_keys = (int)(hi - lo);
    int kof[KS], vof[4];
    operand_offsets<D>(lg, lr, kof, vof);
    // One chunk: wait for its loads (issued one chunk earlier), start the next chunk's loads
    // into the other buffer, compute.  A chunk needs masks only where it passes the span's end
    // or some row's position.  The loop is unrolled over the two buffers so that every LDS
    // address is a per-lane constant plus an immediate offset.
    // (key offsets from lo are ints: a span has S keys).  Chunks that end by full_end need no
    // masks; they come first.  The operand offsets carry the buffer: flipping it is an XOR.
    constexpr int BUF = kChunk * D * 2;  // bytes per staged buffer
    const int full_end = (int)((tmin + 1 < hi ? tmin + 1 : hi) - lo);
    const char *Kbytes = reinterpret_cast<const char *>(stage[0]);
    const char *Vbytes = reinterpret_cast<const char *>(stage[2]);
    int nb = 1;  // buffer that receives the next chunk
    auto flip = [&]() {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kof[ks] ^= BUF;
#pragma unroll
        for (int v = 0; v < 4; ++v) vof[v] ^= BUF;
        nb ^= 1;
    };
    if (n_keys > 0) chunk_load<D>(Ksp, Vsp, stage[0], stage[2], 0, n_keys, wave, lane);
    int c = 0;
    for (; c + kChunk <= full_end; c += kChunk) {
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of the chunk landed
        __syncthreads();  // everyone's loads landed, and everyone finished reading the other buffer
        if (c + kChunk < n_keys) chunk_load<D>(Ksp, Vsp, stage[nb], stage[2 + nb], c + kChunk, n_keys, wave, lane);
        tile_chunk<D, false>(Kbytes, Vbytes, kof, vof, qb, m, l, o, kChunk, lg, scale_log2);
        flip();
    }
    for (; c < n_keys; c += kChunk) {
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (c + kChunk < n_keys) chunk_load<D>(Ksp, Vsp, stage[nb], stage[2 + nb], c + kChunk, n_keys, wave, lane);
        int64_t lim = (hi < tq + 1 ? hi : tq + 1) - (lo + c);
        lim = lim < 0 ? 0 : (lim > kChunk ? kChunk : lim);
        tile_chunk<D, true>(Kbytes, Vbytes, kof, vof, qb, m, l, o, (int)lim, lg, scale_log2);
        flip();
    }

    // records: (m, l, o[d]) per valid row; lane (lg, lr) holds o[16et + 4lg + i] of query lr
    if (x_own >= 0) {
        float *rec = records + (int64_t)x_own * record_floats(D);
#pragma unroll
        for (int et = 0; et < ET; ++et)
            *reinterpret_cast<float4 *>(rec + 4 + 16 * et + 4 * lg) = make_float4(o[et][0], o[et][1], o[et][2], o[et][3]);
        if (lg == 0) {
            rec[0] = m;
            rec[1] = l;
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
