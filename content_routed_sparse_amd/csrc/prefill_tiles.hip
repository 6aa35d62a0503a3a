// Prefill tiles: each tile is up to MT (row-head, entry) pairs that attend to the same span of
// one (sequence, kv head); the tile produces each pair's partial softmax state over the span's
// keys (masked to keys <= the row's position).
//
// tile_mfma (bf16): a block of 4 waves takes up to 128 entries (each wave two groups of 16
// queries) and streams the span's keys through LDS in chunks of 64, loaded straight from
// global memory into LDS (K rows and V rows, XOR-swizzled), double-buffered.  The products run
// transposed on v_mfma_f32_16x16x32_bf16: S^T = K Q^T (the gathered query rows are the B operand,
// kept in registers), so each lane owns one query's scores and its softmax state, and
// O^T += V^T P^T takes P (rounded to bf16) straight from the S^T registers, with V^T read by
// transposed LDS reads.  Each query keeps one reference maximum fixed by its first chunk;
// an entry whose row sum then overflows the fast range gets a second pass with its exact
// maximum (decided per entry).  Tiles of one span are consecutive in the tile list and are
// spread over the 8 XCDs in contiguous ranges, so the blocks that reread a span's keys share an L2.
// Over an 8-bit cache the same pipeline stages E4M3 codes and turns them into bf16 operands as it
// reads them (the 8-bit cache tiles, below).
//
// tile_valu: one wave per entry, keys streamed in chunks of KPW rows with an online softmax
// (fp32 inputs).  The span's rows are shared by the tile's entries through the caches.
#include "common.h"
#include "prefill_tiles.h"
#include "wave_ops.h"

#include <type_traits>

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
__global__ void __launch_bounds__(256) tile_valu(const T *__restrict__ q, const T *__restrict__ K,
                                                 const T *__restrict__ V, const int32_t *__restrict__ tile_off,
                                                 const int32_t *__restrict__ list,
                                                 const int64_t *__restrict__ list_t, const int4 *__restrict__ tiles,
                                                 float *__restrict__ records, int64_t n_exp, int64_t span_slots,
                                                 int NE, int S, int64_t cap, float scale_log2) {
    using L = WaveLayout<T, D>;
    constexpr int EPL = L::EPL, LPR = L::LPR, RPI = L::RPI, KPW = L::KPW, STEPS = L::STEPS;
    if (slot_tile(blockIdx.x, tile_off[n_exp]) < 0) return;
    const int4 tl = tiles[blockIdx.x];
    const int64_t expert = tl.x;
    const int n = tl.z;
    const int64_t j = expert % span_slots;
    const int64_t sg = expert / span_slots;  // sequence * Hkv + kv head
    const int32_t *entries = list + tl.y;
    const int64_t *entries_t = list_t + tl.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane % LPR, rr = lane / LPR;
    const T *Kb = K + sg * cap * D;
    const T *Vb = V + sg * cap * D;

    for (int i = wave; i < n; i += 4) {
        const int64_t x = entries[i];
        const int64_t rh = x / NE;
        const int64_t t = entries_t[i];
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
        float *rec = records + x * prefill_record_words(D, false);
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

// Each wave computes kQG groups of 16 queries against every staged key: the K and V operands
// it reads from LDS serve kQG MFMAs each, which sets the LDS bytes per flop (LDS bandwidth, not
// the matrix core, bounds the chunk step at one group per wave).
constexpr int kQG = 2;                          // groups of 16 queries per wave
constexpr int kMfmaWaves = 4;                   // waves per block
constexpr int kMfmaTile = kMfmaWaves * 16 * kQG;  // entries per tile (128)
constexpr int kChunk = 64;                      // keys per LDS stage
constexpr int kMfmaThreads = kMfmaWaves * 64;
constexpr int kWavesPerEU = kQG == 1 ? 4 : 2;   // register budget: 128 or 256 per lane
static_assert(kMfmaTile <= kMfmaThreads, "one thread per entry in the tile reductions");

// XCD-aware order for a grid of exactly `grid` tiles (the dense tiles): the hardware hands block b
// to XCD b % 8; give XCD x a contiguous range of the tile list so that its tiles share an L2.
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
//   V: piece p of row r at position p ^ (2 (r mod 4) + 8 ((r / 4) mod 2)) for D = 128 (the last
//      term moves rows 4..7 of every 8 to the other half of the banks: a transposed read serves
//      lanes that address rows r and r + 4 in the same cycle), p ^ 2 (r mod 4) for D = 64.
template <int D>
__device__ __forceinline__ int kswz(int r) { return r % (D / 8); }
template <int D>
__device__ __forceinline__ int vswz(int r) { return 2 * (r & 3) + (D >= 128 ? 8 * ((r >> 2) & 1) : 0); }

// Issue the direct global -> LDS loads of one tensor's chunk at key offset c (from the tile's
// first key, whose row starts at `base`) into `dst`: kChunk rows of D bf16, rows at or past `n`
// (the rows that may be read) repeating row n - 1 (masked later).  Each wave instruction fills
// 1 KB = 1024 / (2 D) rows.  Buffer loads: the rows are a buffer resource, the chunk and
// row-block offsets are scalar, and a lane's own part of the address (its row in the block, its
// swizzled piece) is the same for every block of a chunk (the swizzles repeat every 16 rows, a
// wave's blocks every 16), so a whole chunk costs no vector arithmetic.  Only a chunk that
// passes row n - 1 clamps rows per lane.  IS_V selects the V swizzle.
template <int D, bool IS_V>
__device__ __forceinline__ void chunk_rows(const uint16_t *base, uint16_t *dst, int c, int n, int wave, int lane) {
    constexpr int ROWS = 1024 / (2 * D);     // rows per wave instruction
    constexpr int NI = kChunk / ROWS;        // instructions per chunk
    constexpr int P = D / 8;                 // pieces per row
    static_assert(kMfmaWaves % 2 == 0 && (ROWS * kMfmaWaves) % 16 == 0, "swizzles repeat across a wave's blocks");
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, n * D * 2, 0x00020000);
    const int rl = lane / P, phys = lane % P;
    const int r0 = wave * ROWS + rl;  // the lane's row in its wave's first block
    const int part = 16 * (phys ^ (IS_V ? vswz<D>(r0) : kswz<D>(r0)));
    if (c + kChunk <= n) {
#pragma unroll
        for (int ii = wave; ii < NI; ii += kMfmaWaves)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (RA_LDS void *)(dst + ii * ROWS * D), 16, rl * D * 2 + part,
                                                     (c * D + ii * ROWS * D) * 2, 0, 0);
    } else {
        // (the rows are recomputed at every call: hoisted out of the callers' loops, one register
        // per load instruction would stay live through the whole sweep)
        int rlv = rl;
        asm volatile("" : "+v"(rlv));
#pragma unroll
        for (int ii = wave; ii < NI; ii += kMfmaWaves) {
            int g = c + ii * ROWS + rlv;
            g = g < n ? g : n - 1;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (RA_LDS void *)(dst + ii * ROWS * D), 16, g * D * 2 + part, 0, 0, 0);
        }
    }
}

// Per-lane LDS byte offsets of the MFMA operand reads inside a staged chunk (every other part
// of an address is an immediate).  K: lane (lg, lr) reads row 16 kt + lr, piece 4 ks + lg, which
// sits at piece (4 ks + lg) ^ (lr mod P).  V (transposed reads): lane (lg, lr) addresses row
// 32 kk + 16 h + 4 lg + c and column 16 et + 4 (lr & 3), c = lr >> 2; with et = 4u + v the
// swizzled 16-byte piece is 2 (4 (u ^ e) + (v ^ c)) + ((lr & 3) >> 1), e = lg & 1 for D = 128
// (0 for D = 64).  vof[u][v] holds the offset of column group et = 4u + v.
template <int D>
__device__ __forceinline__ void operand_offsets(int lg, int lr, int (&kof)[D / 32], int (&vof)[D / 64][4]) {
    constexpr int P = D / 8;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) kof[ks] = 2 * (lr * D + (((4 * ks + lg) ^ (lr % P)) * 8));
    const int c = lr >> 2, b = (lr & 3) >> 1, w = lr & 1, e = D >= 128 ? (lg & 1) : 0;
#pragma unroll
    for (int u = 0; u < D / 64; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            vof[u][v] = 2 * ((4 * lg + c) * D + 8 * (2 * (4 * (u ^ e) + (v ^ c)) + b) + 4 * w);
}

// Maximum over the 4 lane groups (lanes l, l^16, l^32, l^48) with the gfx950 lane-swap
// instructions (VALU, no LDS round trip).
__device__ __forceinline__ float group_max4(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Sum over the 4 lane groups, in a fixed order: (l + l^32) + (l^16 + l^48).
__device__ __forceinline__ float group_sum4(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// One 64-key chunk of a wave's 16 queries (lane (lg, lr): query lr, keys 16kt + 4lg + i).
// MASK: some key of the chunk lies past the span's end or past some query's position; `lim` is
// then min(hi, t_query + 1) - k0 for this lane's query (keys at offsets >= lim are masked).
// Scores stay raw until the exponent: 2^(s * c - m) is one FMA and one v_exp_f32.
// No rescaling: the reference maximum m of a query is fixed at the maximum of its first chunk
// of keys, and later weights 2^(s c - m) may exceed 1 -- the same partial state, written
// relative to a smaller m.  Only the first chunk takes maxima (TRACK); later chunks just
// exponentiate.  If some query's row sum ends above 2^kFastLog2 (or is not finite), a weight
// may have grown past it: the tile then finds every query's largest score in a sweep over its
// keys (max_chunk) and runs again with m set to it, so that no weight exceeds 1.  Weights thus
// stay below 2^kFastLog2, far from fp32 overflow; a query whose output accumulator still overflows
// (weights up to 2^kFastLog2 times values beyond ~2^87) takes the second pass as well.  So does
// a query whose row sum ends below 2^-kFastLog2: in exact arithmetic the first chunk's largest
// key alone weighs 1, but the fast pass forms each exponent with one fused multiply-add against
// the rounded m, so with scores of magnitude ~2^30 and more the largest key's exponent is m's
// rounding error, up to half an ulp of m either way, and every weight can underflow to 0.
// Row sums l = sum_k P[q][k] are taken over the same bf16 weights that the P.V product uses:
// one v_dot2_f32_bf16 against (1, 1) per packed pair, into a per-lane fp32 sum over the lane's
// own keys (the 4 lane groups of a query are added once, at the end: group_sum4).
constexpr float kFastLog2 = 40.f;
constexpr float kFastLimit = 1099511627776.f;  // 2^kFastLog2

// A query's fast-pass result stands when its row sum is in [2^-kFastLog2, 2^kFastLog2] (false for
// NaN) and its output accumulator is finite.
__device__ __forceinline__ bool fast_sum_ok(float l_total) {
    return l_total >= 1.f / kFastLimit && l_total <= kFastLimit;
}

// S^T = K Q^T for one chunk and kQG query groups: sc[g][kt][i] = S^T[key 16kt + 4lg + i][query lr
// of group g].  Each K operand read from LDS feeds the kQG groups' MFMAs.
template <int D>
__device__ __forceinline__ void qk_chunk(const uint16_t *Kc, const int (&kof)[D / 32], const bf16x8_t (&qb)[kQG][D / 32],
                                         f32x4_t (&sc)[kQG][kChunk / 16]) {
    constexpr int KS = D / 32, KT = kChunk / 16;
    const char *Kbytes = reinterpret_cast<const char *>(Kc);
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        bf16x8_t ka[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            ka[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(Kbytes + kof[ks] + 2 * 16 * kt * D));
#pragma unroll
        for (int g = 0; g < kQG; ++g) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks], qb[g][ks], acc, 0, 0, 0);
            sc[g][kt] = acc;
        }
    }
}

// A key's weight 2^(s c - m).  The fast pass takes the exponent from one fused multiply-add
// (exact before its final rounding).  The pass against the exact maximum (EXACT) rounds the
// product first: with m = RN(max s * c), rounding's monotonicity makes every exponent <= 0 and the
// largest key's exactly 0, whatever the scores' magnitude (with the fused form the largest key's
// exponent is the rounding error of m, up to half an ulp of m: 2^64 and more once |m| >= 2^30).
template <bool EXACT>
__device__ __forceinline__ float key_weight(float s, float c, float nm) {
    if constexpr (EXACT) {
#pragma clang fp contract(off)
        const float z = s * c;
        return __builtin_amdgcn_exp2f(z + nm);
    } else {
        return __builtin_amdgcn_exp2f(fmaf(s, c, nm));
    }
}

// The chunk's weights 2^(s c - m) as bf16 pairs (pk[kt][i/2]); with TRACK, the reference
// bookkeeping (maxima) too.
template <bool MASK, bool TRACK, bool EXACT>
__device__ __forceinline__ void softmax_chunk(f32x4_t (&sc)[kChunk / 16], int lim, int lg, float scale_log2, float &m,
                                              uint32_t (&pk)[kChunk / 16][2]) {
    constexpr int KT = kChunk / 16;
    constexpr float NEG = -__builtin_huge_valf();
    if (MASK) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[kt][i] = 16 * kt + 4 * lg + i < lim ? sc[kt][i] : NEG;
    }
    if (TRACK) {
        float cmax = NEG;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, sc[kt][i]);
        const float mx = group_max4(cmax) * scale_log2;
        m = m == NEG ? mx : m;  // a query's first valid keys fix m (its o and l are still 0)
    }
    // (m is still unset only for a padding query with no key in the first chunk: its results
    // are discarded, 0 keeps them finite)
    const float nm = m != NEG ? -m : 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = key_weight<EXACT>(sc[kt][i], scale_log2, nm);
        pk[kt][0] = pack_bf16x2(pv[0], pv[1]);
        pk[kt][1] = pack_bf16x2(pv[2], pv[3]);
    }
}

// O^T += V^T P^T, 32-key steps: K slots 8lg..8lg+7 <-> keys (2kk)16 + 4lg + 0..3 and
// (2kk+1)16 + 4lg + 0..3 for both operands.  Each V operand read from LDS feeds the kQG groups.
template <int D>
__device__ __forceinline__ void pv_chunk(const uint16_t *Vc, const int (&vof)[D / 64][4],
                                         const uint32_t (&pk)[kQG][kChunk / 16][2], f32x4_t (&o)[kQG][D / 16]) {
    constexpr int ET = D / 16, KT = kChunk / 16;
    const char *Vbytes = reinterpret_cast<const char *>(Vc);
#pragma unroll
    for (int kk = 0; kk < KT / 2; ++kk) {
        bf16x8_t pb[kQG];
#pragma unroll
        for (int g = 0; g < kQG; ++g)
            pb[g] = __builtin_bit_cast(bf16x8_t, make_uint4(pk[g][2 * kk][0], pk[g][2 * kk][1], pk[g][2 * kk + 1][0],
                                                            pk[g][2 * kk + 1][1]));
#pragma unroll
        for (int et = 0; et < ET; ++et) {
            // transposed reads: lane (lg, i) gets V[key][16 et + i] for 4 consecutive keys
            uint2 vw[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const char *pv_addr = Vbytes + vof[et >> 2][et & 3] + 2 * (32 * kk + 16 * h) * D;
                vw[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((RA_LDS v4i16_t *)pv_addr));
            }
            const bf16x8_t va = __builtin_bit_cast(bf16x8_t, make_uint4(vw[0].x, vw[0].y, vw[1].x, vw[1].y));
#pragma unroll
            for (int g = 0; g < kQG; ++g) o[g][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[g], o[g][et], 0, 0, 0);
        }
    }
}

// The sweep of the rare second pass: each query's largest score (times scale_log2) over one
// chunk, folded into mx[g].
template <int D, bool MASK>
__device__ __forceinline__ void max_chunk(const uint16_t *Kc, const int (&kof)[D / 32], const bf16x8_t (&qb)[kQG][D / 32],
                                          float (&mx)[kQG], const int (&lim)[kQG], int lg, float scale_log2) {
    constexpr float NEG = -__builtin_huge_valf();
    f32x4_t sc[kQG][kChunk / 16];
    qk_chunk<D>(Kc, kof, qb, sc);
#pragma unroll
    for (int g = 0; g < kQG; ++g) {
        float cmax = NEG;
#pragma unroll
        for (int kt = 0; kt < kChunk / 16; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                cmax = fmaxf(cmax, (!MASK || 16 * kt + 4 * lg + i < lim[g]) ? sc[g][kt][i] : NEG);
        mx[g] = fmaxf(mx[g], group_max4(cmax) * scale_log2);
    }
}

// The keys of a tile: K and V rows from the tile's first key (Ksp, Vsp), n_load of them
// readable, n_keys attended (chunks cover [0, n_keys)), and chunks ending by full_end need no
// mask.  qlim[g] = keys (from the first) that the lane's query of group g may attend.
struct TileKeys {
    const uint16_t *Ksp, *Vsp;
    int n_load, n_keys, full_end;
};

// The staged chunks: K and V of chunk x sit in kb[x & 1] and vb[x & 1].  Four distinct arrays:
// the compiler then knows that a chunk's LDS loads do not touch the buffers being read, and
// does not wait for them before those reads.
template <int D>
struct Stage {
    uint16_t *kb0, *kb1, *vb0, *vb1;
};

// One pass over a tile's chunks with fixed references.  Chunk c's K and V sit in buffers c & 1;
// at chunk c the loads of chunk c + 1 go to the other buffers, so that they fly while chunk c is
// computed (the buffers are distinct arrays, so the compiler does not wait for those loads
// before reading chunk c).  The first chunk takes maxima and fixes each query's reference where
// it is unset.  `preloaded`: K(0) and V(0) are already being loaded.
template <int D, bool EXACT>
__device__ __forceinline__ void fast_sweep(const Stage<D> &st, const TileKeys &tk, bool preloaded, const int (&qlim)[kQG],
                                           const int (&kof)[D / 32], const int (&vof)[D / 64][4],
                                           const bf16x8_t (&qb)[kQG][D / 32], float (&m)[kQG], float (&l)[kQG],
                                           f32x4_t (&o)[kQG][D / 16], int wave, int lane, int lg, float scale_log2) {
    constexpr int KT = kChunk / 16;
    const int C = (tk.n_keys + kChunk - 1) / kChunk;
    if (!preloaded) {
        __syncthreads();  // everyone is done with the buffers
        chunk_rows<D, false>(tk.Ksp, st.kb0, 0, tk.n_load, wave, lane);
        chunk_rows<D, true>(tk.Vsp, st.vb0, 0, tk.n_load, wave, lane);
    }
    const bf16x2_t one2 = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
    // chunk c with buffer parity P = c & 1
    auto iter = [&](auto par, auto mask, auto track, int c) {
        constexpr int P = decltype(par)::value;
        constexpr bool MASK = decltype(mask)::value, TRACK = decltype(track)::value;
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of chunk c landed
        __syncthreads();  // everyone's landed; everyone is done with chunk c - 1
        if (c + 1 < C) {
            chunk_rows<D, false>(tk.Ksp, P ? st.kb0 : st.kb1, (c + 1) * kChunk, tk.n_load, wave, lane);
            chunk_rows<D, true>(tk.Vsp, P ? st.vb0 : st.vb1, (c + 1) * kChunk, tk.n_load, wave, lane);
        }
        f32x4_t sc[kQG][KT];
        qk_chunk<D>(P ? st.kb1 : st.kb0, kof, qb, sc);
        uint32_t pk[kQG][KT][2];
#pragma unroll
        for (int g = 0; g < kQG; ++g) {
            int lim = qlim[g] - c * kChunk;
            lim = lim < 0 ? 0 : (lim > kChunk ? kChunk : lim);
            softmax_chunk<MASK, TRACK, EXACT>(sc[g], lim, lg, scale_log2, m[g], pk[g]);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    l[g] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[g][kt][h]), one2, l[g], false);
        }
        pv_chunk<D>(P ? st.vb1 : st.vb0, vof, pk, o);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using BF = std::integral_constant<bool, false>;
    using BT = std::integral_constant<bool, true>;
    if (kChunk <= tk.full_end) iter(I0{}, BF{}, BT{}, 0);
    else iter(I0{}, BT{}, BT{}, 0);
    for (int c = 1; c < C; c += 2) {
        if ((c + 1) * kChunk <= tk.full_end) iter(I1{}, BF{}, BF{}, c);
        else iter(I1{}, BT{}, BF{}, c);
        if (c + 1 >= C) break;
        if ((c + 2) * kChunk <= tk.full_end) iter(I0{}, BF{}, BF{}, c + 1);
        else iter(I0{}, BT{}, BF{}, c + 1);
    }
}

// The rare sweep before a second pass: every query's largest score (times scale_log2) over the
// tile's keys, into mx[g].  K only, one chunk ahead.
template <int D>
__device__ __forceinline__ void max_sweep(const Stage<D> &st, const TileKeys &tk, const int (&qlim)[kQG],
                                          const int (&kof)[D / 32], const bf16x8_t (&qb)[kQG][D / 32],
                                          float (&mx)[kQG], int wave, int lane, int lg, float scale_log2) {
    const int C = (tk.n_keys + kChunk - 1) / kChunk;
    __syncthreads();  // everyone is done with the buffers
    chunk_rows<D, false>(tk.Ksp, st.kb0, 0, tk.n_load, wave, lane);
    for (int c = 0; c < C; ++c) {
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (c + 1 < C) chunk_rows<D, false>(tk.Ksp, (c & 1) ? st.kb0 : st.kb1, (c + 1) * kChunk, tk.n_load, wave, lane);
        int lim[kQG];
#pragma unroll
        for (int g = 0; g < kQG; ++g) {
            const int v = qlim[g] - c * kChunk;
            lim[g] = v < 0 ? 0 : (v > kChunk ? kChunk : v);
        }
        if (c & 1) max_chunk<D, true>(st.kb1, kof, qb, mx, lim, lg, scale_log2);
        else max_chunk<D, true>(st.kb0, kof, qb, mx, lim, lg, scale_log2);
    }
}

// ---------------------------------------------------------------------- 8-bit cache tiles
// Over an 8-bit cache (E4M3 codes + one fp32 scale per row) the tiles stage each chunk's codes
// (kChunk rows of D bytes, K and V) and its rows' scales into LDS with direct loads, double-
// buffered like the bf16 rows (one barrier per chunk), and turn codes into MFMA operands as they
// read them: a K operand is 8 codes of one row (one 8-byte read), a V operand 8 codes of one column
// (one transposing read, ds_read_b64_tr_b8), each converted exactly to bf16 by four
// v_cvt_scalef32_pk_bf16_fp8 (an E4M3 value has a 4-bit significand, which bf16 holds exactly).
// The operand reads move half the LDS bytes of the bf16 tiles'.  The scales stay apart: each
// key's score is s_k (q . code_k); the P.V weights carry s_v (P' = bf16(P s_v)) while the row sums
// add the unrounded weights, so the result is sum P s_v code_v / sum P.
//
// LDS layout of a staged code chunk: rows of D bytes, unpadded (a direct load fills 1 KB = 1024 / D
// rows per wave instruction), the 16-byte pieces of each row permuted by an XOR so that each
// half-wave's operand reads (32 lanes x 8 bytes) fall on distinct banks.  Piece p of row r sits at
// position p ^ f(r):
//   D = 128 (two rows per 256-byte line of the 64 banks): K  f = (r >> 1 & 3) | (r >> 3 & 1) << 2
//                                                         V  f = (r >> 1 & 3) | ((r >> 3 ^ r >> 4) & 1) << 2
//   D = 64 (four rows per line):                          K  f = r >> 2 & 3
//                                                         V  f = (r >> 2 & 1) | (r >> 4 & 1) << 1
// (a K read of a half-wave takes rows 16 kt + 0..15 at one piece; a V read takes rows
// 32 kk + 16 (j >> 2) + 4 lg + (j & 3), j < 8, lg < 2 or lg >= 2, at one piece.)
template <int D>
__device__ __forceinline__ int kswz8(int r) {
    return D >= 128 ? (((r >> 1) & 3) | (((r >> 3) & 1) << 2)) : ((r >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int vswz8(int r) {
    return D >= 128 ? (((r >> 1) & 3) | ((((r >> 3) ^ (r >> 4)) & 1) << 2)) : (((r >> 2) & 1) | (((r >> 4) & 1) << 1));
}

// The staged chunks of the 8-bit tiles: the codes of chunk x in kc[x & 1], vc[x & 1] (four distinct
// arrays, as in Stage), its rows' scales in ks[x & 1], vs[x & 1].
struct StageF8 {
    uint8_t *kc0, *kc1, *vc0, *vc1;
    float *ks[2], *vs[2];
};

struct TileKeysF8 {
    const uint8_t *Ksp, *Vsp;  // codes of the tile's first key row
    const float *ksp, *vsp;    // scales of the tile's first key row
    int n_load, n_keys, full_end;
};

// Direct global -> LDS loads of chunk c's code rows (rows at or past n repeat row n - 1; masked
// later) in the swizzled layout, and of the chunk's kChunk row scales.
template <int D, bool IS_V>
__device__ __forceinline__ void chunk_codes(const uint8_t *base, uint8_t *dst, const float *sbase, float *sdst, int c,
                                            int n, int wave, int lane) {
    constexpr int ROWS = 1024 / D;  // rows per wave instruction
    constexpr int NI = kChunk / ROWS;
    constexpr int P = D / 16;       // 16-byte pieces per row
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, n * D, 0x00020000);
    const int rl = lane / P, phys = lane % P;
#pragma unroll
    for (int ii = wave; ii < NI; ii += kMfmaWaves) {
        const int r = ii * ROWS + rl;  // the lane's row in the chunk; its LDS piece phys holds piece phys ^ f(r)
        const int part = 16 * (phys ^ (IS_V ? vswz8<D>(r) : kswz8<D>(r)));
        int g = c + r;
        g = g < n ? g : n - 1;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (RA_LDS void *)(dst + ii * ROWS * D), 16, g * D + part, 0, 0, 0);
    }
    if (wave == kMfmaWaves - 1) {  // the chunk's kChunk = 64 scales: one dword per lane
        const __amdgpu_buffer_rsrc_t rss = __builtin_amdgcn_make_buffer_rsrc((void *)sbase, 0, n * 4, 0x00020000);
        int g = c + lane;
        g = g < n ? g : n - 1;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rss, (RA_LDS void *)sdst, 4, g * 4, 0, 0, 0);
    }
}

// 8 E4M3 codes (little-endian bytes of lo, then hi) -> 8 bf16, exactly.
__device__ __forceinline__ bf16x8_t codes8_to_bf16(uint32_t lo, uint32_t hi) {
    return __builtin_bit_cast(bf16x8_t, make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, false)),
                                                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, true)),
                                                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, false)),
                                                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, true))));
}

// Per-lane LDS offsets of the 8-bit operand reads.  K: lane (lg, lr) reads row 16 kt + lr, bytes
// 32 ks + 8 lg .. + 7 (kof8[ks], plus 16 kt D); V: lane (lg, lr) names row
// 32 kk + 16 (j >> 2) + 4 lg + (j & 3) with j = lr >> 1 and the half lr & 1 of column piece et, so
// that the transposing read gives lane lr the codes of column 16 et + lr for the 8 keys of K-slots
// 8 lg .. 8 lg + 7 (the P.V order): vbase + 32 kk D + 16 (et ^ vsw).
template <int D>
__device__ __forceinline__ void operand_offsets8(int lg, int lr, int (&kof8)[D / 32], int &vbase, int &vsw) {
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) kof8[ks] = lr * D + 16 * ((2 * ks + (lg >> 1)) ^ kswz8<D>(lr)) + 8 * (lg & 1);
    const int j = lr >> 1;
    const int vrow = 16 * (j >> 2) + 4 * lg + (j & 3);
    vbase = vrow * D + 8 * (lr & 1);
    vsw = vswz8<D>(vrow);
}

// S^T = K Q^T for one chunk of codes and kQG query groups (the raw products q . code; the caller
// applies the keys' scales).
template <int D>
__device__ __forceinline__ void qk_chunk_f8(const uint8_t *Kc, const int (&kof8)[D / 32],
                                            const bf16x8_t (&qb)[kQG][D / 32], f32x4_t (&sc)[kQG][kChunk / 16]) {
    constexpr int KS = D / 32, KT = kChunk / 16;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        bf16x8_t ka[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint2 raw = *reinterpret_cast<const uint2 *>(Kc + kof8[ks] + 16 * kt * D);
            ka[ks] = codes8_to_bf16(raw.x, raw.y);
        }
#pragma unroll
        for (int g = 0; g < kQG; ++g) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks], qb[g][ks], acc, 0, 0, 0);
            sc[g][kt] = acc;
        }
    }
}

typedef int v2i32_t __attribute__((ext_vector_type(2)));

// O^T += V^T P^T over a chunk of codes (pk: the weights times the keys' value scales, as bf16
// pairs in the K-slot order of pv_chunk); each V operand read feeds the kQG groups.
template <int D>
__device__ __forceinline__ void pv_chunk_f8(const uint8_t *Vc, int vbase, int vsw,
                                            const uint32_t (&pk)[kQG][kChunk / 16][2], f32x4_t (&o)[kQG][D / 16]) {
    constexpr int ET = D / 16, KT = kChunk / 16;
#pragma unroll
    for (int kk = 0; kk < KT / 2; ++kk) {
        bf16x8_t pb[kQG];
#pragma unroll
        for (int g = 0; g < kQG; ++g)
            pb[g] = __builtin_bit_cast(bf16x8_t, make_uint4(pk[g][2 * kk][0], pk[g][2 * kk][1], pk[g][2 * kk + 1][0],
                                                            pk[g][2 * kk + 1][1]));
#pragma unroll
        for (int et = 0; et < ET; ++et) {
            const v2i32_t w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (RA_LDS v2i32_t *)(Vc + vbase + 32 * kk * D + 16 * (et ^ vsw)));
            const bf16x8_t va = codes8_to_bf16((uint32_t)w.x, (uint32_t)w.y);
#pragma unroll
            for (int g = 0; g < kQG; ++g) o[g][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[g], o[g][et], 0, 0, 0);
        }
    }
}

// softmax_chunk for the 8-bit tiles: the weights 2^(s c - m) are added to the lane's row sum l in
// fp32, and pkv holds them times the keys' value scales as bf16 pairs (for P.V).  (The bf16 tiles
// sum the bf16-rounded weights they multiply with; here the weights that multiply carry s_v, so
// the sum takes the unrounded ones: a difference of bf16 rounding, ~2^-9 per weight.)
template <bool MASK, bool TRACK, bool EXACT>
__device__ __forceinline__ void softmax_chunk_f8(f32x4_t (&sc)[kChunk / 16], int lim, int lg, float scale_log2,
                                                 float &m, float &l, const float *vs_chunk,
                                                 uint32_t (&pkv)[kChunk / 16][2]) {
    constexpr int KT = kChunk / 16;
    constexpr float NEG = -__builtin_huge_valf();
    if (MASK) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[kt][i] = 16 * kt + 4 * lg + i < lim ? sc[kt][i] : NEG;
    }
    if (TRACK) {
        float cmax = NEG;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, sc[kt][i]);
        const float mx = group_max4(cmax) * scale_log2;
        m = m == NEG ? mx : m;
    }
    const float nm = m != NEG ? -m : 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = key_weight<EXACT>(sc[kt][i], scale_log2, nm);
        l += (pv[0] + pv[1]) + (pv[2] + pv[3]);
        const float4 vsc = *reinterpret_cast<const float4 *>(vs_chunk + 16 * kt + 4 * lg);  // keys' value scales
        pkv[kt][0] = pack_bf16x2(pv[0] * vsc.x, pv[1] * vsc.y);
        pkv[kt][1] = pack_bf16x2(pv[2] * vsc.z, pv[3] * vsc.w);
    }
}

// The keys' scales applied to a chunk's raw scores: S = s_k (q . code_k) (lane keys 16 kt + 4 lg + i).
__device__ __forceinline__ void scale_scores(f32x4_t (&sc)[kQG][kChunk / 16], const float *ks_chunk, int lg) {
#pragma unroll
    for (int kt = 0; kt < kChunk / 16; ++kt) {
        const float4 k4 = *reinterpret_cast<const float4 *>(ks_chunk + 16 * kt + 4 * lg);
#pragma unroll
        for (int g = 0; g < kQG; ++g) {
            sc[g][kt][0] *= k4.x;
            sc[g][kt][1] *= k4.y;
            sc[g][kt][2] *= k4.z;
            sc[g][kt][3] *= k4.w;
        }
    }
}

// fast_sweep over the 8-bit cache: the same pipeline as fast_sweep (chunk c's codes and scales in
// buffers c & 1, chunk c + 1's loads issued behind the barrier of chunk c), operands from codes.
template <int D, bool EXACT>
__device__ __forceinline__ void fast_sweep_f8(const StageF8 &st, const TileKeysF8 &tk, bool preloaded,
                                              const int (&qlim)[kQG], const int (&kof8)[D / 32], int vbase, int vsw,
                                              const bf16x8_t (&qb)[kQG][D / 32], float (&m)[kQG], float (&l)[kQG],
                                              f32x4_t (&o)[kQG][D / 16], int wave, int lane, int lg,
                                              float scale_log2) {
    constexpr int KT = kChunk / 16;
    const int C = (tk.n_keys + kChunk - 1) / kChunk;
    if (!preloaded) {
        __syncthreads();  // everyone is done with the buffers
        chunk_codes<D, false>(tk.Ksp, st.kc0, tk.ksp, st.ks[0], 0, tk.n_load, wave, lane);
        chunk_codes<D, true>(tk.Vsp, st.vc0, tk.vsp, st.vs[0], 0, tk.n_load, wave, lane);
    }
    auto iter = [&](auto par, auto mask, auto track, int c) {
        constexpr int P = decltype(par)::value;
        constexpr bool MASK = decltype(mask)::value, TRACK = decltype(track)::value;
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of chunk c landed
        __syncthreads();  // everyone's landed; everyone is done with chunk c - 1
        if (c + 1 < C) {
            chunk_codes<D, false>(tk.Ksp, P ? st.kc0 : st.kc1, tk.ksp, st.ks[P ^ 1], (c + 1) * kChunk, tk.n_load, wave,
                                  lane);
            chunk_codes<D, true>(tk.Vsp, P ? st.vc0 : st.vc1, tk.vsp, st.vs[P ^ 1], (c + 1) * kChunk, tk.n_load, wave,
                                 lane);
        }
        f32x4_t sc[kQG][KT];
        qk_chunk_f8<D>(P ? st.kc1 : st.kc0, kof8, qb, sc);
        scale_scores(sc, st.ks[P], lg);
        uint32_t pkv[kQG][KT][2];
#pragma unroll
        for (int g = 0; g < kQG; ++g) {
            int lim = qlim[g] - c * kChunk;
            lim = lim < 0 ? 0 : (lim > kChunk ? kChunk : lim);
            softmax_chunk_f8<MASK, TRACK, EXACT>(sc[g], lim, lg, scale_log2, m[g], l[g], st.vs[P], pkv[g]);
        }
        pv_chunk_f8<D>(P ? st.vc1 : st.vc0, vbase, vsw, pkv, o);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using BF = std::integral_constant<bool, false>;
    using BT = std::integral_constant<bool, true>;
    if (kChunk <= tk.full_end) iter(I0{}, BF{}, BT{}, 0);
    else iter(I0{}, BT{}, BT{}, 0);
    for (int c = 1; c < C; c += 2) {
        if ((c + 1) * kChunk <= tk.full_end) iter(I1{}, BF{}, BF{}, c);
        else iter(I1{}, BT{}, BF{}, c);
        if (c + 1 >= C) break;
        if ((c + 2) * kChunk <= tk.full_end) iter(I0{}, BF{}, BF{}, c + 1);
        else iter(I0{}, BT{}, BF{}, c + 1);
    }
}

// max_sweep over the 8-bit cache: every query's largest scaled score (times scale_log2).  K codes
// and scales only, one chunk ahead.
template <int D>
__device__ __forceinline__ void max_sweep_f8(const StageF8 &st, const TileKeysF8 &tk, const int (&qlim)[kQG],
                                             const int (&kof8)[D / 32], const bf16x8_t (&qb)[kQG][D / 32],
                                             float (&mx)[kQG], int wave, int lane, int lg, float scale_log2) {
    constexpr float NEG = -__builtin_huge_valf();
    const int C = (tk.n_keys + kChunk - 1) / kChunk;
    __syncthreads();  // everyone is done with the buffers
    chunk_codes<D, false>(tk.Ksp, st.kc0, tk.ksp, st.ks[0], 0, tk.n_load, wave, lane);
    for (int c = 0; c < C; ++c) {
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        const bool odd = c & 1;  // (selects, not a runtime index into st.ks: that would live in memory)
        if (c + 1 < C)
            chunk_codes<D, false>(tk.Ksp, odd ? st.kc0 : st.kc1, tk.ksp, odd ? st.ks[0] : st.ks[1], (c + 1) * kChunk,
                                  tk.n_load, wave, lane);
        f32x4_t sc[kQG][kChunk / 16];
        qk_chunk_f8<D>(odd ? st.kc1 : st.kc0, kof8, qb, sc);
        scale_scores(sc, odd ? st.ks[1] : st.ks[0], lg);
#pragma unroll
        for (int g = 0; g < kQG; ++g) {
            int lim = qlim[g] - c * kChunk;
            lim = lim < 0 ? 0 : (lim > kChunk ? kChunk : lim);
            float cmax = NEG;
#pragma unroll
            for (int kt = 0; kt < kChunk / 16; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, 16 * kt + 4 * lg + i < lim ? sc[g][kt][i] : NEG);
            mx[g] = fmaxf(mx[g], group_max4(cmax) * scale_log2);
        }
    }
}

// 1 when some element of a query's output accumulator (over the 4 lane groups that hold it) is not
// finite: the fast pass's weights (up to 2^kFastLog2 against the first chunk's maximum) times large
// values can overflow fp32 although the row sum stays in range; such a query takes the second pass
// too (weights <= 1).
template <int D>
__device__ __forceinline__ bool acc_overflow(const f32x4_t (&og)[D / 16]) {
    float bad = 0.f;
#pragma unroll
    for (int et = 0; et < D / 16; ++et)
#pragma unroll
        for (int i = 0; i < 4; ++i) bad = __builtin_isfinite(og[et][i]) ? bad : 1.f;
    return group_max4(bad) > 0.f;
}

// Transposed formulation.  S^T = K Q^T puts keys on the MFMA rows and queries on the columns,
// so lane (lg, lr) holds keys 16kt + 4lg + i of query lr: every per-query quantity (running
// max, sum, rescale of the output) is lane-local, and only the max/sum across the 4 lane
// groups of a query needs cross-lane steps.  O^T = V^T P^T then takes P straight from the S^T
// registers: its 32-key K dimension is ordered as the lanes hold it (keys 4lg..4lg+3 of two
// 16-key tiles per lane group), and V^T is read from LDS in the same order.
// F8: the cache holds E4M3 codes (K, V) with one fp32 scale per row (ks, vs); otherwise bf16.
template <int D, bool F8>
__global__ void __launch_bounds__(kMfmaThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU, kWavesPerEU))) tile_mfma(const uint16_t *__restrict__ q,
                                                          const void *__restrict__ K,
                                                          const void *__restrict__ V,
                                                          const float *__restrict__ ks,
                                                          const float *__restrict__ vs,
                                                          const int32_t *__restrict__ tile_off,
                                                          const int32_t *__restrict__ list,
                                                          const int64_t *__restrict__ list_t,
                                                          const int4 *__restrict__ tiles,
                                                          float *__restrict__ records, int64_t n_exp,
                                                          int64_t span_slots, int NE, int S, int64_t cap,
                                                          float scale_log2) {
    constexpr int KS = D / 32;   // k-steps of the QK product
    constexpr int ET = D / 16;   // 16-wide e tiles of the PV product
    constexpr float NEG = -__builtin_huge_valf();
    // staged chunks, buffers 0 and 1 of kChunk rows: bf16 K and V (D bf16 per row), or for the
    // 8-bit tiles K and V codes (D bytes per row) with the rows' scales
    __shared__ __align__(16) uint16_t kb0[F8 ? 8 : kChunk * D], vb0[F8 ? 8 : kChunk * D];
    __shared__ __align__(16) uint16_t kb1[F8 ? 8 : kChunk * D], vb1[F8 ? 8 : kChunk * D];
    __shared__ __align__(16) uint8_t kc0[F8 ? kChunk * D : 16], vc0[F8 ? kChunk * D : 16];
    __shared__ __align__(16) uint8_t kc1[F8 ? kChunk * D : 16], vc1[F8 ? kChunk * D : 16];
    __shared__ __align__(16) float ks8[F8 ? 2 * kChunk : 4], vs8[F8 ? 2 * kChunk : 4];
    __shared__ int redo_s[kMfmaWaves];
    __shared__ unsigned long long wmax_s[kMfmaWaves], wmin_s[kMfmaWaves];
    const Stage<D> st{kb0, kb1, vb0, vb1};
    StageF8 st8;    // (assigned field by field: a braced constant initializer of LDS addresses
    st8.kc0 = kc0;  //  would become a static one, which the device compiler rejects)
    st8.kc1 = kc1;
    st8.vc0 = vc0;
    st8.vc1 = vc1;
    st8.ks[0] = ks8;
    st8.ks[1] = ks8 + kChunk;
    st8.vs[0] = vs8;
    st8.vs[1] = vs8 + kChunk;

    // all kernel arguments in one round trip (otherwise some are fetched only where first used)
    asm volatile("" ::"s"(q), "s"(K), "s"(V), "s"(tile_off), "s"(list), "s"(list_t), "s"(tiles), "s"(records),
                 "s"(n_exp), "s"(span_slots), "s"(NE), "s"(S), "s"(cap), "s"(scale_log2));
    if constexpr (F8) asm volatile("" ::"s"(ks), "s"(vs));
    // the tile count and this block's descriptor slot in one round trip (a slot that holds no
    // tile is stale but in bounds: the grid has max_tiles blocks, one per slot)
    const int64_t total = tile_off[n_exp];
    const int4 tl = tiles[blockIdx.x];
    asm volatile("" ::"s"(total), "s"(tl.x), "s"(tl.y), "s"(tl.z));
    if (slot_tile(blockIdx.x, total) < 0) return;
    const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // (uniform: scalar chunk-load offsets)
    const int64_t expert = tl.x;
    const int n = tl.z;  // entries in the tile (<= kMfmaTile)
    const int64_t j = expert % span_slots;
    const int64_t sg = expert / span_slots;
    const int64_t lo = j * S;
    const uint16_t *Ksp = static_cast<const uint16_t *>(K) + (sg * cap + lo) * D;  // the span's first key row
    const uint16_t *Vsp = static_cast<const uint16_t *>(V) + (sg * cap + lo) * D;
    const uint8_t *Ksp8 = static_cast<const uint8_t *>(K) + (sg * cap + lo) * D;  // (8-bit cache)
    const uint8_t *Vsp8 = static_cast<const uint8_t *>(V) + (sg * cap + lo) * D;
    const float *ksp = F8 ? ks + sg * cap + lo : nullptr;
    const float *vsp = F8 ? vs + sg * cap + lo : nullptr;
    const int n_span = (int)(cap - lo < S ? cap - lo : S);  // keys of the span inside the cache

    // One round trip: the tile's entries and their positions, this lane's own row (for its
    // query), and the first chunk of keys -- loaded up to the span's end, since the rows'
    // positions that may cut it short are not known yet (rows past them are masked).
    // (unconditional loads from clamped indices, masked afterwards: a load under a condition is
    // waited for on its own)
    // entry 16 (kQG wave + g) + lr of the tile is query lr of group g of wave `wave`
    const int i_blk = tid < n ? tid : n - 1;
    const int64_t t_blk = list_t[tl.y + i_blk];
    int32_t x_ld[kQG], x_own[kQG];
    int64_t tq[kQG];  // position of the lane's query in each group (-1: padding)
#pragma unroll
    for (int g = 0; g < kQG; ++g) {
        const int r_own = 16 * (kQG * wave + g) + lr;
        const int i_own = r_own < n ? r_own : n - 1;
        x_ld[g] = list[tl.y + i_own];
        const int64_t t_ld = list_t[tl.y + i_own];
        x_own[g] = r_own < n ? x_ld[g] : -1;
        tq[g] = r_own < n ? t_ld : -1;
    }

    // B operands of S^T: the wave's gathered query rows, all k-steps, in registers
    bf16x8_t qb[kQG][KS];
#pragma unroll
    for (int g = 0; g < kQG; ++g) {
        const int64_t rh = x_ld[g] / NE;  // (a padding row loads a valid row, then zero)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 raw = *reinterpret_cast<const uint4 *>(q + rh * D + 32 * ks + 8 * lg);
            if (x_own[g] < 0) raw = make_uint4(0, 0, 0, 0);
            qb[g][ks] = __builtin_bit_cast(bf16x8_t, raw);
        }
    }
    // the first chunk's LDS loads (K and V of chunk 0) fly with the query loads,
    // up to the span's end (issued after them: the compiler waits for everything before using a
    // load's register while LDS loads are outstanding)
    if constexpr (F8) {
        chunk_codes<D, false>(Ksp8, st8.kc0, ksp, st8.ks[0], 0, n_span, wave, lane);
        chunk_codes<D, true>(Vsp8, st8.vc0, vsp, st8.vs[0], 0, n_span, wave, lane);
    } else {
        chunk_rows<D, false>(Ksp, st.kb0, 0, n_span, wave, lane);
        chunk_rows<D, true>(Vsp, st.vb0, 0, n_span, wave, lane);
    }
    // the tile's first and last positions (wave reductions, then across the waves in LDS)
    {
        unsigned long long vmax = tid < n ? (unsigned long long)t_blk : 0ull;
        unsigned long long vmin = tid < n ? (unsigned long long)t_blk : ~0ull;
        vmax = wave_max_u64(vmax);
        vmin = ~wave_max_u64(~vmin);
        if (lane == 0) {
            wmax_s[wave] = vmax;
            wmin_s[wave] = vmin;
        }
    }
    __syncthreads();
    unsigned long long tmax_u = 0ull, tmin_u = ~0ull;
#pragma unroll
    for (int w = 0; w < kMfmaWaves; ++w) {
        tmax_u = wmax_s[w] > tmax_u ? wmax_s[w] : tmax_u;
        tmin_u = wmin_s[w] < tmin_u ? wmin_s[w] : tmin_u;
    }
    const int64_t tmax = (int64_t)tmax_u, tmin = (int64_t)tmin_u;
    int64_t hi = lo + S;  // keys of the span used by the tile: [lo, hi)
    if (hi > tmax + 1) hi = tmax + 1;
    if (hi > cap) hi = cap;
    const int n_keys = (int)(hi - lo);
    // chunks that end by full_end need no mask (key offsets from lo are ints: a span has S keys)
    const int full_end = (int)((tmin + 1 < hi ? tmin + 1 : hi) - lo);
    const TileKeys tk{Ksp, Vsp, n_keys, n_keys, full_end};
    const TileKeysF8 tk8{Ksp8, Vsp8, ksp, vsp, n_keys, n_keys, full_end};
    int qlim[kQG];
#pragma unroll
    for (int g = 0; g < kQG; ++g) {
        const int64_t v = tq[g] + 1 - lo;
        qlim[g] = tq[g] < 0 ? 0 : (int)(v < n_keys ? v : n_keys);
    }
    int kof[KS], vof[D / 64][4];
    int kof8[KS], vbase8 = 0, vsw8 = 0;
    if constexpr (F8) operand_offsets8<D>(lg, lr, kof8, vbase8, vsw8);
    else operand_offsets<D>(lg, lr, kof, vof);

    float m[kQG], l[kQG];
    f32x4_t o[kQG][ET];
    auto reset = [&](const float (&m0)[kQG]) {
#pragma unroll
        for (int g = 0; g < kQG; ++g) {
            m[g] = m0[g];
            l[g] = 0.f;
#pragma unroll
            for (int et = 0; et < ET; ++et) o[g][et] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    };
    float unset[kQG];
#pragma unroll
    for (int g = 0; g < kQG; ++g) unset[g] = NEG;
    reset(unset);
    if constexpr (F8) fast_sweep_f8<D, false>(st8, tk8, true, qlim, kof8, vbase8, vsw8, qb, m, l, o, wave, lane, lg, scale_log2);
    else fast_sweep<D, false>(st, tk, true, qlim, kof, vof, qb, m, l, o, wave, lane, lg, scale_log2);

    // records: header (m, l, s, 0), then o / (l s) as fp16 per valid row, s = 2^-k with k chosen
    // so that the row's largest |o / l| lands in [2^14, 2^15): every value keeps 11 significant
    // bits relative to that maximum, and the records take half the bytes of fp32 ones.  Lane
    // (lg, lr) holds o[16et + 4lg + i] of query lr.  Only the entries flagged in `which` store.
    typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
    auto store = [&](const bool (&which)[kQG]) {
#pragma unroll
        for (int g = 0; g < kQG; ++g) {
            const float lt = group_sum4(l[g]);
            const float inv = 1.f / lt;
            float amax = 0.f;
#pragma unroll
            for (int et = 0; et < ET; ++et)
#pragma unroll
                for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(o[g][et][i] * inv));
            amax = group_max4(amax);
            int k2 = 0;
            if (amax > 0.f && amax <= 3.4028234663852886e38f) {
                k2 = 14 - ((int)((__float_as_uint(amax) >> 23) & 0xFFu) - 127);
                k2 = k2 < -126 ? -126 : (k2 > 126 ? 126 : k2);
            }
            const float c = inv * __uint_as_float((uint32_t)(127 + k2) << 23);
            if (which[g]) {
                float *rec = records + (int64_t)x_own[g] * prefill_record_words(D, true);
                uint32_t *hv = reinterpret_cast<uint32_t *>(rec + 4);
#pragma unroll
                for (int et = 0; et < ET; ++et) {
                    const half2_t lo = {(_Float16)(o[g][et][0] * c), (_Float16)(o[g][et][1] * c)};
                    const half2_t hi = {(_Float16)(o[g][et][2] * c), (_Float16)(o[g][et][3] * c)};
                    *reinterpret_cast<uint2 *>(hv + (16 * et + 4 * lg) / 2) =
                        make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
                }
                if (lg == 0)
                    *reinterpret_cast<float4 *>(rec) =
                        make_float4(m[g], lt, __uint_as_float((uint32_t)(127 - k2) << 23), 0.f);
            }
        }
    };

    // Each entry decides on its own whether it needs the second pass: its row sum left
    // [2^-kFastLog2, 2^kFastLog2] (or is not finite), or its output accumulator overflowed.  Entries that do not store their records now, and keep
    // them, so an entry's result never depends on which other entries share its tile.  The
    // pass itself runs for the whole block (every wave takes the same path through the loads).
    bool need[kQG], done[kQG];
    bool need_any = false;
#pragma unroll
    for (int g = 0; g < kQG; ++g) {
        need[g] = x_own[g] >= 0 && (!fast_sum_ok(group_sum4(l[g])) || acc_overflow<D>(o[g]));
        done[g] = x_own[g] >= 0 && !need[g];
        need_any = need_any || need[g];
    }
    store(done);
    const bool wave_redo = __ballot(need_any) != 0;  // (all lanes vote: a ballot counts active lanes only)
    if (lane == 0) redo_s[wave] = wave_redo ? 1 : 0;
    __syncthreads();
    int redo = 0;
#pragma unroll
    for (int w = 0; w < kMfmaWaves; ++w) redo |= redo_s[w];
    if (redo) {
        float mx[kQG];
#pragma unroll
        for (int g = 0; g < kQG; ++g) mx[g] = NEG;
        if constexpr (F8) {
            max_sweep_f8<D>(st8, tk8, qlim, kof8, qb, mx, wave, lane, lg, scale_log2);
            reset(mx);
            fast_sweep_f8<D, true>(st8, tk8, false, qlim, kof8, vbase8, vsw8, qb, m, l, o, wave, lane, lg, scale_log2);
        } else {
            max_sweep<D>(st, tk, qlim, kof, qb, mx, wave, lane, lg, scale_log2);
            reset(mx);
            fast_sweep<D, true>(st, tk, false, qlim, kof, vof, qb, m, l, o, wave, lane, lg, scale_log2);
        }
        store(need);
    }
}

template <int D, bool F8>
hipError_t mfma_launch(const TileArgs &t, hipStream_t st) {
    const RowArgs &a = t.a;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    hipLaunchKernelGGL((tile_mfma<D, F8>), dim3((unsigned)t.max_tiles), dim3(kMfmaThreads), 0, st,
                       (const uint16_t *)a.q, t.K, t.V, t.ks, t.vs, t.tile_off, t.list, t.list_t, t.tiles, t.records,
                       t.n_exp, t.span_slots, t.NE, a.S, a.cap, scale_log2);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t valu_launch(const TileArgs &t, hipStream_t st) {
    const RowArgs &a = t.a;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    hipLaunchKernelGGL((tile_valu<T, D>), dim3((unsigned)t.max_tiles), dim3(256), 0, st, (const T *)a.q,
                       (const T *)t.K, (const T *)t.V, t.tile_off, t.list, t.list_t, t.tiles, t.records, t.n_exp,
                       t.span_slots, t.NE, a.S, a.cap, scale_log2);
    return hipGetLastError();
}

// Dense causal attention (every key at or before the row's position: the "k = all spans" case
// of the method, and the reference the routed path is measured against).  The same chunk step
// as the routed tiles, with the span replaced by the whole prefix [0, t].
//
// Tile = (kv head g, RT = 128 / G consecutive rows of the call): its entries are the RT rows x
// G query heads of the kv head (entry 16 w + i of the block belongs to wave w), so all entries
// share the keys.  Rows of different sequences in one tile are handled in successive passes
// (increasing sequence id; one pass for a chunk of one sequence): entries of other sequences
// are padding during a pass.  Each entry's whole softmax state stays in registers, so the
// output o / l is written directly: no workspace and no merge.
template <int D>
__global__ void __launch_bounds__(kMfmaThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU, kWavesPerEU)))
dense_mfma(const uint16_t *__restrict__ q, const int32_t *__restrict__ row_seq, const int64_t *__restrict__ row_pos,
           const uint16_t *__restrict__ K, const uint16_t *__restrict__ V, float *__restrict__ out, int64_t n_rows,
           int Hq, int Hkv, int G, int RT, int B, int64_t cap, int64_t max_pos, float scale_log2, int64_t n_blocks) {
    constexpr int KS = D / 32, ET = D / 16;
    constexpr float NEG = -__builtin_huge_valf();
    __shared__ uint16_t kb0[kChunk * D], kb1[kChunk * D], vb0[kChunk * D], vb1[kChunk * D];
    __shared__ int redo_s[kMfmaWaves];
    __shared__ unsigned long long wred_s[3][kMfmaWaves];
    const Stage<D> st{kb0, kb1, vb0, vb1};
    asm volatile("" ::"s"(q), "s"(row_seq), "s"(row_pos), "s"(K), "s"(V), "s"(out), "s"(n_rows), "s"(Hq), "s"(Hkv),
                 "s"(G), "s"(RT), "s"(B), "s"(cap), "s"(max_pos), "s"(scale_log2), "s"(n_blocks));
    // tiles ordered (kv head, row block); XCD x takes a contiguous range of them (shared L2)
    const int64_t tile = xcd_tile(blockIdx.x, n_blocks);
    const int64_t n_rb = (n_rows + RT - 1) / RT;
    const int g = (int)(tile / n_rb);
    const int64_t r0 = (tile % n_rb) * RT;
    const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // (uniform: scalar chunk-load offsets)

    // this lane's entries: query lr of group gi of wave `wave` is entry e = 16 (kQG wave + gi) + lr
    // of the tile, i.e. row r0 + e / G, query head g G + e mod G
    int64_t row_e[kQG], t_e[kQG];
    uint32_t qrow[kQG];  // the entry's row-head (query and output row; n_rows Hq < 2^31, checked on the host)
    bool valid[kQG];
    int seq_e[kQG];
#pragma unroll
    for (int gi = 0; gi < kQG; ++gi) {
        const int e = 16 * (kQG * wave + gi) + lr;
        row_e[gi] = r0 + e / G;
        valid[gi] = e < RT * G && row_e[gi] < n_rows;
        const int64_t row_c = valid[gi] ? row_e[gi] : r0;  // (a padding entry loads a valid row, then zero)
        const int hq = g * G + (valid[gi] ? e % G : 0);
        const int seq_raw = row_seq[row_c];
        const int64_t t_raw = row_pos[row_c];
        qrow[gi] = (uint32_t)(row_c * Hq + hq);
        seq_e[gi] = seq_raw < 0 ? 0 : (seq_raw >= B ? B - 1 : seq_raw);
        t_e[gi] = t_raw < 0 ? 0 : (t_raw > max_pos ? max_pos : t_raw);
    }

    int kof[KS], vof[D / 64][4];
    operand_offsets<D>(lg, lr, kof, vof);

    // block-wide min/max of three 64-bit values (wave reductions, then across the waves in LDS)
    auto block_reduce = [&](unsigned long long a_min, unsigned long long b_min, unsigned long long c_max,
                            unsigned long long &ra, unsigned long long &rb, unsigned long long &rc) {
        a_min = ~wave_max_u64(~a_min);
        b_min = ~wave_max_u64(~b_min);
        c_max = wave_max_u64(c_max);
        __syncthreads();  // (the previous reduction's values have been read)
        if (lane == 0) {
            wred_s[0][wave] = a_min;
            wred_s[1][wave] = b_min;
            wred_s[2][wave] = c_max;
        }
        __syncthreads();
        ra = ~0ull, rb = ~0ull, rc = 0ull;
#pragma unroll
        for (int w = 0; w < kMfmaWaves; ++w) {
            ra = wred_s[0][w] < ra ? wred_s[0][w] : ra;
            rb = wred_s[1][w] < rb ? wred_s[1][w] : rb;
            rc = wred_s[2][w] > rc ? wred_s[2][w] : rc;
        }
    };

    int64_t prev_seq = -1;
    for (;;) {
        // the next sequence of the tile (smallest id above the last one done), its rows' first and
        // last positions
        unsigned long long nseq, tmin_u, tmax_u;
        unsigned long long pmin = ~0ull;
#pragma unroll
        for (int gi = 0; gi < kQG; ++gi)
            if (valid[gi] && seq_e[gi] > prev_seq && (unsigned long long)seq_e[gi] < pmin) pmin = seq_e[gi];
        block_reduce(pmin, ~0ull, 0ull, nseq, tmin_u, tmax_u);
        if (nseq == ~0ull) break;
        const int seq = (int)nseq;
        bool active[kQG];
        unsigned long long amin = ~0ull, amax = 0ull;
#pragma unroll
        for (int gi = 0; gi < kQG; ++gi) {
            active[gi] = valid[gi] && seq_e[gi] == seq;
            if (active[gi]) {
                amin = (unsigned long long)t_e[gi] < amin ? (unsigned long long)t_e[gi] : amin;
                amax = (unsigned long long)t_e[gi] > amax ? (unsigned long long)t_e[gi] : amax;
            }
        }
        block_reduce(~0ull, amin, amax, nseq, tmin_u, tmax_u);
        const int64_t tmin = (int64_t)tmin_u, tmax = (int64_t)tmax_u;
        int64_t hi = tmax + 1;
        if (hi > cap) hi = cap;
        const int n_keys = (int)hi;
        const TileKeys tk{K + ((int64_t)seq * Hkv + g) * cap * D, V + ((int64_t)seq * Hkv + g) * cap * D, n_keys, n_keys,
                          (int)(tmin + 1 < hi ? tmin + 1 : hi)};
        // the queries, loaded again for each sequence of the tile (zero for entries of other sequences)
        bf16x8_t qb[kQG][KS];
        int qlim[kQG];
#pragma unroll
        for (int gi = 0; gi < kQG; ++gi) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                uint4 raw = *reinterpret_cast<const uint4 *>(q + (int64_t)qrow[gi] * D + 32 * ks + 8 * lg);
                if (!active[gi]) raw = make_uint4(0, 0, 0, 0);
                qb[gi][ks] = __builtin_bit_cast(bf16x8_t, raw);
            }
            qlim[gi] = active[gi] ? (int)(t_e[gi] + 1 < n_keys ? t_e[gi] + 1 : n_keys) : 0;
        }

        float m[kQG], l[kQG];
        f32x4_t o[kQG][ET];
        auto reset = [&](const float (&m0)[kQG]) {
#pragma unroll
            for (int gi = 0; gi < kQG; ++gi) {
                m[gi] = m0[gi];
                l[gi] = 0.f;
#pragma unroll
                for (int et = 0; et < ET; ++et) o[gi][et] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
        };
        float unset[kQG];
#pragma unroll
        for (int gi = 0; gi < kQG; ++gi) unset[gi] = NEG;
        reset(unset);
        fast_sweep<D, false>(st, tk, false, qlim, kof, vof, qb, m, l, o, wave, lane, lg, scale_log2);
        // as in the routed tiles: a row sum outside [2^-kFastLog2, 2^kFastLog2] or an overflowed
        // accumulator sends the tile to a second pass
        bool redo_q = false;
#pragma unroll
        for (int gi = 0; gi < kQG; ++gi)
            redo_q = redo_q || (active[gi] && (!fast_sum_ok(group_sum4(l[gi])) || acc_overflow<D>(o[gi])));
        const bool wave_redo = __ballot(redo_q) != 0;  // (all lanes vote: a ballot counts active lanes only)
        if (lane == 0) redo_s[wave] = wave_redo ? 1 : 0;
        __syncthreads();
        int redo = 0;
#pragma unroll
        for (int w = 0; w < kMfmaWaves; ++w) redo |= redo_s[w];
        if (redo) {
            float mx[kQG];
#pragma unroll
        for (int g = 0; g < kQG; ++g) mx[g] = NEG;
            max_sweep<D>(st, tk, qlim, kof, qb, mx, wave, lane, lg, scale_log2);
            reset(mx);
            fast_sweep<D, true>(st, tk, false, qlim, kof, vof, qb, m, l, o, wave, lane, lg, scale_log2);
        }
        // out = o / l (l summed over the query's 4 lane groups: every lane holds the total)
#pragma unroll
        for (int gi = 0; gi < kQG; ++gi) {
            const float lt = group_sum4(l[gi]);
            if (active[gi]) {
                const float inv = 1.f / lt;
                float *dst = out + (int64_t)qrow[gi] * D;
#pragma unroll
                for (int et = 0; et < ET; ++et)
                    *reinterpret_cast<float4 *>(dst + 16 * et + 4 * lg) =
                        make_float4(o[gi][et][0] * inv, o[gi][et][1] * inv, o[gi][et][2] * inv, o[gi][et][3] * inv);
            }
        }
        prev_seq = seq;
    }
}

template <int D>
hipError_t dense_launch(const RowArgs &a, const void *K, const void *V, float *out, hipStream_t st) {
    const int RT = kMfmaTile / a.G;
    const int64_t blocks = a.Hkv * ((a.n_rows + RT - 1) / RT);
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    hipLaunchKernelGGL((dense_mfma<D>), dim3((unsigned)blocks), dim3(kMfmaThreads), 0, st, (const uint16_t *)a.q,
                       a.row_seq, a.row_pos, (const uint16_t *)K, (const uint16_t *)V, out, a.n_rows, a.Hq, a.Hkv,
                       a.G, RT, a.B, a.cap, a.max_pos, scale_log2, blocks);
    return hipGetLastError();
}

}  // namespace

int prefill_tile_rows(const RowArgs &a) { return a.dtype == RA_BF16 ? kMfmaTile : kValuTile; }

hipError_t launch_dense(const RowArgs &a, const void *K, const void *V, float *out, hipStream_t st) {
    if (a.n_rows == 0) return hipSuccess;
    return a.d == 64 ? dense_launch<64>(a, K, V, out, st) : dense_launch<128>(a, K, V, out, st);
}

hipError_t launch_prefill_tiles(const TileArgs &t, hipStream_t st) {
    const RowArgs &a = t.a;
    if (t.ks != nullptr) return a.d == 64 ? mfma_launch<64, true>(t, st) : mfma_launch<128, true>(t, st);
    if (a.dtype == RA_BF16) return a.d == 64 ? mfma_launch<64, false>(t, st) : mfma_launch<128, false>(t, st);
    return a.d == 64 ? valu_launch<float, 64>(t, st) : valu_launch<float, 128>(t, st);
}

}  // namespace ra
