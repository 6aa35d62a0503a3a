// Token-level cold retrieval (InfiniteKV post: the recent tokens stay exact on the GPU, older
// tokens are found by a Hamming scan over compact signatures, the top_k_cold of them are fetched
// and attended together with the recent window).  Signature = the d sign bits of a key or query;
// distance = popcount(sig_q ^ sig_k); the top_k_cold cold positions by (distance, position).
//
// Kernels:
//  * sig_kernel: signatures of new cache rows, one lane per 32-element word.
//  * cold_tile: the scan.  A block owns one (row, kv head) and a tile of kTile cold positions;
//    every signature of the tile is read once (16-byte loads at d = 128, coalesced) and scored
//    against the G query heads of the kv head.  Per head it keeps the tile's kc smallest
//    (distance, position) keys: an LDS histogram of the distances gives the cut distance D*
//    (all keys below it are kept, in any order), and the first ties at D* in position order come
//    from a tie bitmask and a block-wide prefix count.  Tiles write kc keys per head (padded).
//  * cold_merge: one block per (row, query head) selects the kc smallest keys among the tiles'
//    candidates the same way (histogram -> D*; ties taken tile by tile in position order) and
//    writes them ascending, padded with -1.
//  * cold_attn: exact softmax attention over the fetched positions and the hot window, one block
//    per (row, query head), online softmax per group of lanes, merged through LDS.
// Distances are small integers, so the selection is exact and deterministic.
#include "cold_kernels.h"
#include "common.h"

namespace ra {
namespace {

constexpr int kTile = 8192;                  // cold positions per scan block
constexpr int kTileThreads = 256;
constexpr int kPerThread = kTile / kTileThreads;
constexpr int kMaxGroup = 32;                // query heads per kv head
constexpr int kBins = 129;                   // distances 0 .. 128
constexpr int kBinStride = 132;
constexpr uint64_t kNoKey = ~0ull;

__device__ __forceinline__ uint64_t cold_key(uint32_t dist, int64_t pos) { return ((uint64_t)dist << 40) | (uint64_t)pos; }
__device__ __forceinline__ uint32_t key_dist(uint64_t k) { return (uint32_t)(k >> 40); }
__device__ __forceinline__ int64_t key_pos(uint64_t k) { return (int64_t)(k & ((1ull << 40) - 1)); }

// Word w (elements 32w .. 32w+31) of the signature of a d-element vector: bit i is the sign bit
// of element 32w + i (bit 15 of a bf16 pattern, bit 31 of an fp32 value).
template <typename T>
__device__ __forceinline__ uint32_t sig_word(const T *x, int w) {
    uint32_t s = 0;
    constexpr int EPL = 16 / sizeof(T);
#pragma unroll
    for (int c = 0; c < 32 / EPL; ++c) {
        const uint4 raw = *reinterpret_cast<const uint4 *>(x + 32 * w + c * EPL);
        const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (sizeof(T) == 2) {
                s |= ((u[i] >> 15) & 1u) << (c * 8 + 2 * i);
                s |= (u[i] >> 31) << (c * 8 + 2 * i + 1);
            } else {
                s |= (u[i] >> 31) << (c * 4 + i);
            }
        }
    }
    return s;
}

template <typename T, int D>
__global__ void __launch_bounds__(256) sig_kernel(const T *__restrict__ k, uint32_t *__restrict__ sig,
                                                  const int64_t *__restrict__ old_len,
                                                  const int64_t *__restrict__ new_len, int Hkv, int64_t cap,
                                                  int64_t max_new) {
    constexpr int WPR = D / 32;        // words per row
    constexpr int RPB = 256 / WPR;     // rows per block
    const int tid = threadIdx.x, w = tid % WPR;
    const int64_t per_bg = (max_new + RPB - 1) / RPB;
    const int64_t bg = blockIdx.x / per_bg;
    const int64_t i = (blockIdx.x % per_bg) * RPB + tid / WPR;
    const int b = (int)(bg / Hkv);
    int64_t lo = old_len[b], hi = new_len[b];
    if (lo < 0) lo = 0;
    if (hi > cap) hi = cap;
    const int64_t p = lo + i;
    if (i >= max_new || p >= hi) return;
    const int64_t row = bg * cap + p;
    sig[row * WPR + w] = sig_word(k + row * D, w);
}

template <int D>
struct SigWords {
    uint32_t v[D / 32];
};
template <int D>
__device__ __forceinline__ SigWords<D> load_sig(const uint32_t *p) {
    SigWords<D> s;
    if constexpr (D == 128) {
        const uint4 r = *reinterpret_cast<const uint4 *>(p);
        s.v[0] = r.x;
        s.v[1] = r.y;
        s.v[2] = r.z;
        s.v[3] = r.w;
    } else {
        const uint2 r = *reinterpret_cast<const uint2 *>(p);
        s.v[0] = r.x;
        s.v[1] = r.y;
    }
    return s;
}
template <int D>
__device__ __forceinline__ uint32_t distance(const SigWords<D> &s, const uint32_t *q) {
    uint32_t d = 0;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) d += __popc(s.v[i] ^ q[i]);
    return d;
}

// Exclusive prefix sum over the 256 threads of a block (x >= 0); also returns the total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t *wave_tot, uint32_t &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t inc = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(inc, off);
        if (lane >= off) inc += y;
    }
    if (lane == 63) wave_tot[wave] = inc;
    __syncthreads();
    uint32_t before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t t = wave_tot[w];
        if (w < wave) before += t;
        total += t;
    }
    __syncthreads();
    return before + inc - x;
}

template <typename T, int D>
__global__ void __launch_bounds__(kTileThreads) cold_tile(const T *__restrict__ q, const int32_t *__restrict__ row_seq,
                                                          const int64_t *__restrict__ row_pos,
                                                          const uint32_t *__restrict__ sig, uint64_t *__restrict__ cand,
                                                          int Hq, int Hkv, int G, int B, int64_t cap, int64_t max_pos,
                                                          int H, int kc, int n_tiles) {
    constexpr int WPR = D / 32;
    __shared__ uint32_t qsig[kMaxGroup][WPR];
    __shared__ uint32_t hist[kMaxGroup * kBinStride];
    __shared__ uint32_t tie[kMaxGroup][kTile / 32];
    __shared__ uint32_t cut[kMaxGroup], below[kMaxGroup], need[kMaxGroup], cnt[kMaxGroup];
    __shared__ uint32_t wave_tot[4];
    const int tid = threadIdx.x;
    const int tile = blockIdx.x % n_tiles;
    const int64_t rg = blockIdx.x / n_tiles;
    const int g = (int)(rg % Hkv);
    const int64_t row = rg / Hkv;
    int64_t t = row_pos[row];
    t = t < 0 ? 0 : (t > max_pos ? max_pos : t);
    int seq = row_seq[row];
    seq = seq < 0 ? 0 : (seq >= B ? B - 1 : seq);
    const int64_t n_cold = t - H + 1 > 0 ? t - H + 1 : 0;
    const int64_t lo = (int64_t)tile * kTile;
    const int n_here = (int)(n_cold - lo <= 0 ? 0 : (n_cold - lo < kTile ? n_cold - lo : kTile));
    uint64_t *out0 = cand + ((row * Hq + (int64_t)g * G) * n_tiles + tile) * kc;  // + h * n_tiles * kc
    const int64_t head_stride = (int64_t)n_tiles * kc;
    const int kc_eff = n_here < kc ? n_here : kc;
    if (n_here == 0) {
        for (int x = tid; x < G * kc; x += kTileThreads) out0[(x / kc) * head_stride + x % kc] = kNoKey;
        return;
    }
    // query signatures, cleared histograms and tie masks
    for (int x = tid; x < G * WPR; x += kTileThreads) {
        const int h = x / WPR, w = x % WPR;
        qsig[h][w] = sig_word(q + ((row * Hq + (int64_t)g * G + h) * D), w);
    }
    for (int x = tid; x < G * kBinStride; x += kTileThreads) hist[x] = 0;
    for (int h = 0; h < G; ++h) tie[h][tid] = 0;
    if (tid < G) cnt[tid] = 0;
    __syncthreads();
    const uint32_t *sbase = sig + (((int64_t)seq * Hkv + g) * cap + lo) * WPR;
    // sweep 1: distance histograms
    for (int i = 0; i < kPerThread; ++i) {
        const int x = i * kTileThreads + tid;
        if (x < n_here) {
            const SigWords<D> s = load_sig<D>(sbase + (int64_t)x * WPR);
            for (int h = 0; h < G; ++h) atomicAdd(&hist[h * kBinStride + distance<D>(s, qsig[h])], 1u);
        }
    }
    __syncthreads();
    // cut distance per head: the smallest D* with at least kc_eff keys at or below it
    if (tid < G) {
        uint32_t cum = 0, dstar = kBins - 1;
        for (int x = 0; x < kBins; ++x) {
            const uint32_t c = hist[tid * kBinStride + x];
            if (cum + c >= (uint32_t)kc_eff) {
                dstar = x;
                break;
            }
            cum += c;
        }
        cut[tid] = dstar;
        below[tid] = cum;
        need[tid] = kc_eff - cum;
    }
    __syncthreads();
    // sweep 2: keys below the cut (any order); ties at the cut marked in the bitmask
    for (int i = 0; i < kPerThread; ++i) {
        const int x = i * kTileThreads + tid;
        if (x < n_here) {
            const SigWords<D> s = load_sig<D>(sbase + (int64_t)x * WPR);
            for (int h = 0; h < G; ++h) {
                const uint32_t dd = distance<D>(s, qsig[h]);
                if (dd < cut[h]) {
                    const uint32_t slot = atomicAdd(&cnt[h], 1u);
                    out0[h * head_stride + slot] = cold_key(dd, lo + x);
                } else if (dd == cut[h]) {
                    atomicOr(&tie[h][x >> 5], 1u << (x & 31));
                }
            }
        }
    }
    __syncthreads();
    // the first need[h] ties in position order: thread tid owns mask word tid (positions 32 tid ..)
    for (int h = 0; h < G; ++h) {
        uint32_t word = tie[h][tid];
        uint32_t total;
        const uint32_t pre = block_exclusive_scan(__popc(word), wave_tot, total);
        const uint32_t nd = need[h];
        if (pre < nd) {
            uint32_t take = nd - pre, j = 0;
            while (word && j < take) {
                const int bit = __builtin_ctz(word);
                word &= word - 1;
                out0[h * head_stride + below[h] + pre + j] = cold_key(cut[h], lo + 32 * tid + bit);
                ++j;
            }
        }
    }
    // padding past kc_eff
    for (int x = tid; x < G * kc; x += kTileThreads)
        if (x % kc >= kc_eff) out0[(x / kc) * head_stride + x % kc] = kNoKey;
}

// kc <= kMaxCold
__global__ void __launch_bounds__(256) cold_merge(const uint64_t *__restrict__ cand, int32_t *__restrict__ sel,
                                                  int n_tiles, int kc) {
    __shared__ uint32_t hist[kBins];
    __shared__ int64_t lst[kMaxCold];
    __shared__ uint32_t wave_tot[4];
    __shared__ uint32_t n_valid, n_lt, s_cut, s_need;
    const int tid = threadIdx.x;
    const int64_t rh = blockIdx.x;
    const uint64_t *c = cand + rh * (int64_t)n_tiles * kc;
    const int M = n_tiles * kc;
    for (int x = tid; x < kBins; x += 256) hist[x] = 0;
    if (tid == 0) {
        n_valid = 0;
        n_lt = 0;
    }
    __syncthreads();
    uint32_t mine = 0;
    for (int x = tid; x < M; x += 256) {
        const uint64_t k = c[x];
        if (k != kNoKey) {
            atomicAdd(&hist[key_dist(k)], 1u);
            ++mine;
        }
    }
    atomicAdd(&n_valid, mine);
    __syncthreads();
    const uint32_t kc_eff = n_valid < (uint32_t)kc ? n_valid : (uint32_t)kc;
    if (tid == 0) {
        uint32_t cum = 0, dstar = kBins - 1;
        for (int x = 0; x < kBins; ++x) {
            if (cum + hist[x] >= kc_eff) {
                dstar = x;
                break;
            }
            cum += hist[x];
        }
        s_cut = dstar;
        s_need = kc_eff - cum;
    }
    __syncthreads();
    const uint32_t dstar = s_cut, nd = s_need;
    if (kc_eff > 0) {
        for (int x = tid; x < M; x += 256) {
            const uint64_t k = c[x];
            if (k != kNoKey && key_dist(k) < dstar) lst[atomicAdd(&n_lt, 1u)] = key_pos(k);
        }
    }
    __syncthreads();
    const uint32_t lt = n_lt;
    // ties at D*: tile by tile (tiles cover increasing positions), each tile's smallest positions
    uint32_t carry = 0;
    for (int j0 = 0; j0 < n_tiles && kc_eff > 0; j0 += 256) {
        const int j = j0 + tid;
        uint32_t cj = 0;
        if (j < n_tiles)
            for (int e = 0; e < kc; ++e) {
                const uint64_t k = c[(int64_t)j * kc + e];
                cj += (k != kNoKey && key_dist(k) == dstar) ? 1u : 0u;
            }
        uint32_t total;
        const uint32_t pre = carry + block_exclusive_scan(cj, wave_tot, total);
        if (j < n_tiles && cj > 0 && pre < nd) {
            const uint32_t take = nd - pre < cj ? nd - pre : cj;
            for (int e = 0; e < kc; ++e) {
                const uint64_t k = c[(int64_t)j * kc + e];
                if (k == kNoKey || key_dist(k) != dstar) continue;
                uint32_t rank = 0;
                for (int f = 0; f < kc; ++f) {
                    const uint64_t k2 = c[(int64_t)j * kc + f];
                    rank += (k2 != kNoKey && key_dist(k2) == dstar && key_pos(k2) < key_pos(k)) ? 1u : 0u;
                }
                if (rank < take) lst[lt + pre + rank] = key_pos(k);
            }
        }
        carry += total;
    }
    __syncthreads();
    // ascending order, padded with -1
    int32_t *out = sel + rh * kc;
    if (tid < kc) {
        if ((uint32_t)tid < kc_eff) {
            const int64_t p = lst[tid];
            uint32_t rank = 0;
            for (uint32_t x = 0; x < kc_eff; ++x) rank += lst[x] < p ? 1u : 0u;
            out[rank] = (int32_t)p;
        } else {
            out[tid] = -1;
        }
    }
}

// Attention over fetched + hot positions.  16-byte slices: LPR lanes per key row; the wave's
// RPI row groups take keys x = 4 * (wave * RPI + rr) ... in turn; each group keeps its own online
// softmax state over its slice of the output.
template <typename T, int D>
__global__ void __launch_bounds__(256) cold_attn(const T *__restrict__ q, const int32_t *__restrict__ row_seq,
                                                 const int64_t *__restrict__ row_pos, const T *__restrict__ K,
                                                 const T *__restrict__ V, const int32_t *__restrict__ sel,
                                                 float *__restrict__ out, int Hq, int Hkv, int G, int B, int64_t cap,
                                                 int64_t max_pos, int H, int kc, float scale_log2) {
    constexpr int EPL = 16 / sizeof(T), LPR = D / EPL, RPI = 64 / LPR, NGRP = 4 * RPI;
    __shared__ float gm[NGRP], gl[NGRP], go[NGRP][D];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane % LPR, rr = lane / LPR, grp = wave * RPI + rr;
    const int64_t rh = blockIdx.x;
    const int64_t row = rh / Hq;
    const int h = (int)(rh % Hq), g = h / G;
    int64_t t = row_pos[row];
    t = t < 0 ? 0 : (t > max_pos ? max_pos : t);
    int seq = row_seq[row];
    seq = seq < 0 ? 0 : (seq >= B ? B - 1 : seq);
    const int64_t hot_lo = t - H + 1 > 0 ? t - H + 1 : 0;
    const int32_t *s = sel + rh * kc;
    const int64_t n_keys = kc + (t - hot_lo + 1);  // selection entries, then the hot window
    const T *kb = K + ((int64_t)seq * Hkv + g) * cap * D;
    const T *vb = V + ((int64_t)seq * Hkv + g) * cap * D;
    float qf[EPL];
    {
        const uint4 raw = *reinterpret_cast<const uint4 *>(q + rh * D + c * EPL);
        const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (sizeof(T) == 2) {
                qf[2 * i] = bf16_bits_to_f32(u[i] & 0xFFFFu);
                qf[2 * i + 1] = bf16_bits_to_f32(u[i] >> 16);
            } else {
                qf[i] = __uint_as_float(u[i]);
            }
        }
    }
    float M = -__builtin_huge_valf(), L = 0.f, o[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) o[i] = 0.f;
    for (int64_t x = grp; x < n_keys; x += NGRP) {
        const int64_t p = x < kc ? (int64_t)s[x] : hot_lo + (x - kc);
        if (x < kc && (p < 0 || p >= hot_lo)) continue;  // padding, or not a cold position
        const uint4 kr = *reinterpret_cast<const uint4 *>(kb + p * D + c * EPL);
        const uint4 vr = *reinterpret_cast<const uint4 *>(vb + p * D + c * EPL);
        float kf[EPL], vf[EPL];
        const uint32_t ku[4] = {kr.x, kr.y, kr.z, kr.w}, vu[4] = {vr.x, vr.y, vr.z, vr.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (sizeof(T) == 2) {
                kf[2 * i] = bf16_bits_to_f32(ku[i] & 0xFFFFu);
                kf[2 * i + 1] = bf16_bits_to_f32(ku[i] >> 16);
                vf[2 * i] = bf16_bits_to_f32(vu[i] & 0xFFFFu);
                vf[2 * i + 1] = bf16_bits_to_f32(vu[i] >> 16);
            } else {
                kf[i] = __uint_as_float(ku[i]);
                vf[i] = __uint_as_float(vu[i]);
            }
        }
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) z = fmaf(qf[i], kf[i], z);
#pragma unroll
        for (int off = LPR / 2; off > 0; off >>= 1) z += __shfl_xor(z, off);
        z *= scale_log2;
        const float Mn = fmaxf(M, z);
        const float a = exp2f(M - Mn), e = exp2f(z - Mn);
        L = L * a + e;
#pragma unroll
        for (int i = 0; i < EPL; ++i) o[i] = fmaf(e, vf[i], o[i] * a);
        M = Mn;
    }
    if (c == 0) {
        gm[grp] = M;
        gl[grp] = L;
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) go[grp][c * EPL + i] = o[i];
    __syncthreads();
    if (tid < D) {
        float Mt = -__builtin_huge_valf();
        for (int x = 0; x < NGRP; ++x) Mt = fmaxf(Mt, gm[x]);
        float Lt = 0.f, Ot = 0.f;
        for (int x = 0; x < NGRP; ++x) {
            if (gm[x] == -__builtin_huge_valf()) continue;
            const float f = exp2f(gm[x] - Mt);
            Lt = fmaf(gl[x], f, Lt);
            Ot = fmaf(go[x][tid], f, Ot);
        }
        out[rh * D + tid] = Ot / Lt;
    }
}

template <typename T, int D>
hipError_t sig_launch(const SigArgs &a, hipStream_t st) {
    constexpr int RPB = 256 / (D / 32);
    const int64_t blocks = (int64_t)a.B * a.Hkv * ((a.max_new + RPB - 1) / RPB);
    hipLaunchKernelGGL((sig_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, st, (const T *)a.k, a.sig, a.old_len,
                       a.new_len, a.Hkv, a.cap, a.max_new);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t select_launch(const RowArgs &a, const uint32_t *sig, int H, int kc, int32_t *sel, void *ws,
                         hipStream_t st) {
    const int n_tiles = cold_tiles(a.max_pos, H);
    uint64_t *cand = (uint64_t *)ws;
    hipLaunchKernelGGL((cold_tile<T, D>), dim3((unsigned)(a.n_rows * a.Hkv * n_tiles)), dim3(kTileThreads), 0, st,
                       (const T *)a.q, a.row_seq, a.row_pos, sig, cand, a.Hq, a.Hkv, a.G, a.B, a.cap, a.max_pos, H, kc,
                       n_tiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(cold_merge, dim3((unsigned)(a.n_rows * a.Hq)), dim3(256), 0, st, cand, sel, n_tiles, kc);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t attn_launch(const RowArgs &a, const void *K, const void *V, const int32_t *sel, int H, int kc, float *out,
                       hipStream_t st) {
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    hipLaunchKernelGGL((cold_attn<T, D>), dim3((unsigned)(a.n_rows * a.Hq)), dim3(256), 0, st, (const T *)a.q,
                       a.row_seq, a.row_pos, (const T *)K, (const T *)V, sel, out, a.Hq, a.Hkv, a.G, a.B, a.cap,
                       a.max_pos, H, kc, scale_log2);
    return hipGetLastError();
}

}  // namespace

int cold_tiles(int64_t max_pos, int H) {
    const int64_t n = max_pos - H + 1;
    return n <= 0 ? 1 : (int)((n + kTile - 1) / kTile);
}

size_t cold_workspace_bytes(const RowArgs &a, int H, int kc) {
    return (size_t)a.n_rows * a.Hq * cold_tiles(a.max_pos, H) * kc * sizeof(uint64_t);
}

hipError_t launch_signatures(const SigArgs &a, hipStream_t st) {
    if (a.max_new <= 0) return hipSuccess;
    if (a.dtype == RA_BF16) return a.d == 64 ? sig_launch<uint16_t, 64>(a, st) : sig_launch<uint16_t, 128>(a, st);
    return a.d == 64 ? sig_launch<float, 64>(a, st) : sig_launch<float, 128>(a, st);
}

hipError_t launch_cold_select(const RowArgs &a, const uint32_t *sig, int H, int kc, int32_t *sel, void *ws,
                              hipStream_t st) {
    if (a.n_rows == 0) return hipSuccess;
    if (a.dtype == RA_BF16)
        return a.d == 64 ? select_launch<uint16_t, 64>(a, sig, H, kc, sel, ws, st)
                         : select_launch<uint16_t, 128>(a, sig, H, kc, sel, ws, st);
    return a.d == 64 ? select_launch<float, 64>(a, sig, H, kc, sel, ws, st)
                     : select_launch<float, 128>(a, sig, H, kc, sel, ws, st);
}

hipError_t launch_cold_attn(const RowArgs &a, const void *K, const void *V, const int32_t *sel, int H, int kc,
                            float *out, hipStream_t st) {
    if (a.n_rows == 0) return hipSuccess;
    if (a.dtype == RA_BF16)
        return a.d == 64 ? attn_launch<uint16_t, 64>(a, K, V, sel, H, kc, out, st)
                         : attn_launch<uint16_t, 128>(a, K, V, sel, H, kc, out, st);
    return a.d == 64 ? attn_launch<float, 64>(a, K, V, sel, H, kc, out, st)
                     : attn_launch<float, 128>(a, K, V, sel, H, kc, out, st);
}

}  // namespace ra
