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
//    from ranking the listed ties by position (or, with many ties, from a tie bitmask and a
//    block-wide prefix count).  Tiles write kc keys per head (padded).
//  * cold_merge: one block per (row, query head) selects the kc smallest keys among the tiles'
//    candidates the same way (histogram -> D*; ties taken tile by tile in position order) and
//    writes them ascending, padded with -1.
//  * cold_attn: exact softmax attention over the fetched positions and the hot window, one block
//    per (row, query head), online softmax per group of lanes, merged through LDS.
// Distances are small integers, so the selection is exact and deterministic.
#include "cold_kernels.h"
#include "common.h"

#include <type_traits>

namespace ra {
namespace {

// Scan tiles: TILE cold positions per block of THREADS threads, 16 signatures per thread.  Up to
// 8 query heads per kv head: 16384 positions and 1024 threads (fewer, larger tiles: less per-tile
// overhead here and fewer candidates for the merge); more heads: 8192 and 512, so that the
// per-head LDS (histogram, tie bitmask, candidate buffers) of up to 32 heads fits.
constexpr int kTileBig = 16384, kTileBigThreads = 1024;
constexpr int kTileSmall = 8192, kTileSmallThreads = 512;
constexpr int kTileBigMaxGroup = 8;
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
struct WordRaw {
    uint4 r[32 * sizeof(T) / 16];  // the 32 elements of one signature word
};
template <typename T>
__device__ __forceinline__ WordRaw<T> load_word(const T *x, int w) {
    WordRaw<T> raw;
    constexpr int EPL = 16 / sizeof(T);
#pragma unroll
    for (int c = 0; c < 32 / EPL; ++c) raw.r[c] = *reinterpret_cast<const uint4 *>(x + 32 * w + c * EPL);
    return raw;
}
template <typename T>
__device__ __forceinline__ uint32_t pack_word(const WordRaw<T> &raw) {
    uint32_t s = 0;
    constexpr int EPL = 16 / sizeof(T);
#pragma unroll
    for (int c = 0; c < 32 / EPL; ++c) {
        const uint32_t u[4] = {raw.r[c].x, raw.r[c].y, raw.r[c].z, raw.r[c].w};
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
template <typename T>
__device__ __forceinline__ uint32_t sig_word(const T *x, int w) {
    return pack_word<T>(load_word<T>(x, w));
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
// Hamming distance plus d: one XOR and one v_bcnt_u32_b32 (popcount added to its second operand)
// per word, the counts chained through that operand (written out: the compiler would otherwise
// sum separate counts with extra adds).
template <int D>
__device__ __forceinline__ uint32_t distance(const SigWords<D> &s, const uint32_t *q, uint32_t d = 0) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
        const uint32_t x = s.v[i] ^ q[i];
        asm("v_bcnt_u32_b32 %0, %1, %2" : "=v"(d) : "v"(x), "v"(d));
    }
    return d;
}

// LDS of cold_tile for G query heads (32-bit words): query signatures, distance histograms, tie
// bitmasks, and per-wave candidate buffers of up to 128 entries per head within a 60 KB budget.
constexpr int kTileLdsWords = 60 * 1024 / 4;
template <int TILE, int THREADS>
__host__ __device__ constexpr int tile_buf(int G, int WPR) {
    const int room = (kTileLdsWords - G * (WPR + kBinStride + TILE / 32)) / (G * (THREADS / 64));
    return room < 128 ? room : 128;
}
template <int TILE, int THREADS>
__host__ __device__ constexpr int tile_lds_words(int G, int WPR) {
    return G * (WPR + kBinStride + TILE / 32 + (THREADS / 64) * tile_buf<TILE, THREADS>(G, WPR));
}
static_assert(tile_buf<kTileBig, kTileBigThreads>(kTileBigMaxGroup, 4) >= 32 &&
                  tile_buf<kTileSmall, kTileSmallThreads>(kMaxGroup, 4) >= 8,
              "candidate buffers of a few entries per wave at least");

// Exclusive prefix sum over the NW waves of a block (x >= 0); also returns the total.
template <int NW>
__device__ __forceinline__ uint32_t tile_exclusive_scan(uint32_t x, uint32_t *wave_tot, uint32_t &total) {
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
    for (int w = 0; w < NW; ++w) {
        const uint32_t t = wave_tot[w];
        if (w < wave) before += t;
        total += t;
    }
    __syncthreads();
    return before + inc - x;
}

// Cut distance of a distance histogram: the first bin x <= last with bins 0..x summing to at
// least `target`, found by the 64 lanes of one wave (lane l holds bins l, l + 64, l + 128; a
// scan per group of 64 bins); kBins if there is none.  Every lane returns the same values;
// `below` = the sum of the bins before the cut.
__device__ __forceinline__ uint32_t wave_cut(const uint32_t *hist, int last, uint32_t target, uint32_t &below) {
    const int lane = threadIdx.x & 63;
    uint32_t base = 0;
    for (int seg = 0; seg * 64 <= last; ++seg) {
        const int x = seg * 64 + lane;
        const uint32_t v = x <= last ? hist[x] : 0u;
        uint32_t inc = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_up(inc, off);
            if (lane >= off) inc += y;
        }
        const uint64_t hit = __ballot(x <= last && base + inc >= target);
        if (hit) {
            const int f = (int)__builtin_ctzll(hit);
            below = base + (uint32_t)__shfl((int)(inc - v), f);
            return (uint32_t)(seg * 64 + f);
        }
        base += (uint32_t)__shfl((int)inc, 63);
    }
    below = base;
    return kBins;
}

template <typename T, int D, int kTile, int kTileThreads>
__global__ void __launch_bounds__(kTileThreads) cold_tile(const T *__restrict__ q, const int32_t *__restrict__ row_seq,
                                                          const int64_t *__restrict__ row_pos,
                                                          const uint32_t *__restrict__ sig, uint64_t *__restrict__ cand,
                                                          int Hq, int Hkv, int G, int B, int64_t cap, int64_t max_pos,
                                                          int H, int kc, int n_tiles) {
    constexpr int WPR = D / 32;
    constexpr int kPerThread = kTile / kTileThreads;
    constexpr int kTileWaves = kTileThreads / 64;
    static_assert(kTile % kTileThreads == 0 && kTile / 32 <= kTileThreads && kTile <= 65536, "tile shape");
    extern __shared__ uint32_t lds[];
    const int BW = tile_buf<kTile, kTileThreads>(G, WPR);
    uint32_t *qsig = lds;                              // [G][WPR]
    uint32_t *hist = qsig + G * WPR;                   // [G][kBinStride]
    uint32_t *tie = hist + G * kBinStride;             // [G][kTile / 32]
    uint32_t *cbuf = tie + G * (kTile / 32);           // [G][kTileWaves][BW]: (distance << 16) | index
    __shared__ uint32_t theta[kMaxGroup], cut[kMaxGroup], below[kMaxGroup], need[kMaxGroup], cnt[kMaxGroup];
    __shared__ uint32_t ntie[kMaxGroup], tlist[kMaxGroup][64];  // ties at the cut per head (fast path)
    __shared__ uint32_t wcount[kMaxGroup][kTileWaves];
    __shared__ uint32_t wave_tot[kTileWaves], slow;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
    const uint32_t kc_eff = (uint32_t)(n_here < kc ? n_here : kc);
    if (n_here == 0) {
        for (int x = tid; x < G * kc; x += kTileThreads) out0[(x / kc) * head_stride + x % kc] = kNoKey;
        return;
    }
    // Loads in the order they are needed (each wait is for a load and every load before it): the
    // sample position of this thread and the query words, then the tile's signatures, which stay
    // in registers (token x = i * kTileThreads + tid) and are still arriving while the sample
    // sets the thresholds.
    const uint32_t *sbase = sig + (((int64_t)seq * Hkv + g) * cap + lo) * WPR;
    const int n_s = n_here < kTileThreads ? n_here : kTileThreads;  // sample size
    const SigWords<D> smp = load_sig<D>(sbase + (int64_t)(tid < n_s ? tid * (n_here / n_s) : 0) * WPR);
    static_assert(kMaxGroup * WPR <= kTileThreads, "one query word per thread");
    const bool q_wave = wave * 64 < G * WPR;  // (uniform per wave)
    const int qx = tid < G * WPR ? tid : 0;
    WordRaw<T> qraw;
    if (q_wave) qraw = load_word<T>(q + ((row * Hq + (int64_t)g * G + qx / WPR) * D), qx % WPR);
    SigWords<D> sg[kPerThread];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const int x = i * kTileThreads + tid;
        sg[i] = load_sig<D>(sbase + (int64_t)(x < n_here ? x : 0) * WPR);
    }
    if (q_wave && tid < G * WPR) qsig[tid] = pack_word<T>(qraw);
    for (int x = tid; x < G * kBinStride; x += kTileThreads) hist[x] = 0;
    for (int x = tid; x < G * (kTile / 32); x += kTileThreads) tie[x] = 0;
    if (tid < G) cnt[tid] = 0;
    if (tid == 0) slow = 0;
    __syncthreads();
    // 1. a sample of min(kTileThreads, n) positions spread evenly over the tile sets a threshold
    //    per head below which about 3 * kc of the tile's distances should fall
    if (tid < n_s) {
        for (int h = 0; h < G; ++h) atomicAdd(&hist[h * kBinStride + distance<D>(smp, qsig + h * WPR)], 1u);
    }
    __syncthreads();
    for (int h = wave; h < G; h += kTileWaves) {
        const uint32_t target = (uint32_t)((3 * (int64_t)kc_eff * n_s + n_here - 1) / n_here);
        uint32_t b;
        const uint32_t th = wave_cut(hist + h * kBinStride, kBins - 1, target, b);
        if (lane == 0) theta[h] = th < kBins ? th : kBins - 1;
    }
    __syncthreads();
    // 2. candidates at or below the threshold, appended per wave (ballot + mbcnt: no atomics).
    //    In the tile's last (partial) block of positions, those past n_here start their distance
    //    at 256, above every threshold; a full tile needs no such test.
    auto append = [&](auto ragged) {
        constexpr bool RAGGED = decltype(ragged)::value;
        for (int h = 0; h < G; ++h) {
            const uint32_t th = theta[h];
            uint32_t qw[WPR];
#pragma unroll
            for (int w = 0; w < WPR; ++w) qw[w] = qsig[h * WPR + w];
            uint32_t *wb = cbuf + (h * kTileWaves + wave) * BW;
            uint32_t wc = 0;
#pragma unroll
            for (int i = 0; i < kPerThread; ++i) {
                const int x = i * kTileThreads + tid;
                const uint32_t dd = distance<D>(sg[i], qw, RAGGED && x >= n_here ? 256u : 0u);
                const uint64_t bal = __builtin_amdgcn_ballot_w64(dd <= th);
                if (bal) {
                    const uint32_t idx = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)bal, wc));
                    if (dd <= th && idx < (uint32_t)BW) wb[idx] = (dd << 16) | (uint32_t)x;
                    wc += (uint32_t)__popcll(bal);
                }
            }
            if (lane == 0) wcount[h][wave] = wc;
        }
    };
    if (n_here == kTile) append(std::integral_constant<bool, false>{});
    else append(std::integral_constant<bool, true>{});
    for (int x = tid; x < G * kBinStride; x += kTileThreads) hist[x] = 0;
    __syncthreads();
    // 3. histograms of the candidates (each wave its own buffers); the cut per head, or the slow
    //    path when a wave's buffer overflowed or the threshold left fewer than kc_eff candidates
    auto wave_cands = [&](int h, auto f) {
        const uint32_t wc = wcount[h][wave] < (uint32_t)BW ? wcount[h][wave] : (uint32_t)BW;
        const uint32_t *wb = cbuf + (h * kTileWaves + wave) * BW;
        for (uint32_t k = lane; k < wc; k += 64) f(wb[k]);
    };
    for (int h = 0; h < G; ++h)
        wave_cands(h, [&](uint32_t v) { atomicAdd(&hist[h * kBinStride + (v >> 16)], 1u); });
    __syncthreads();
    for (int h = wave; h < G; h += kTileWaves) {
        uint32_t b;
        const uint32_t ct = wave_cut(hist + h * kBinStride, (int)theta[h], kc_eff, b);
        if (lane == 0) {
            bool over = false;
            for (int w = 0; w < kTileWaves; ++w) over |= wcount[h][w] > (uint32_t)BW;
            cut[h] = ct;
            below[h] = b;
            need[h] = kc_eff - b;
            ntie[h] = 0;
            if (over || ct == kBins) atomicOr(&slow, 1u);
        }
    }
    __syncthreads();
    // 4. keys below the cut, and the ties at the cut: the first need[h] of them in position order.
    //    Fast path: the ties of each head (usually a few) are listed and ranked by position in one
    //    wave; with more than 64 ties for some head, or after the slow path, they are marked in a
    //    bitmask per head and counted in position order by a block-wide prefix sum.
    bool use_mask = slow != 0;
    if (slow) {
        // exact histograms of every distance, then the keys below the cut and the tie bitmasks
        for (int x = tid; x < G * kBinStride; x += kTileThreads) hist[x] = 0;
        __syncthreads();
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int i = 0; i < kPerThread; ++i)
                if (i * kTileThreads + tid < n_here) atomicAdd(&hist[h * kBinStride + distance<D>(sg[i], qsig + h * WPR)], 1u);
        __syncthreads();
        for (int h = wave; h < G; h += kTileWaves) {
            uint32_t b;
            const uint32_t ct = wave_cut(hist + h * kBinStride, kBins - 1, kc_eff, b);
            if (lane == 0) {
                cut[h] = ct;
                below[h] = b;
                need[h] = kc_eff - b;
            }
        }
        __syncthreads();
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int i = 0; i < kPerThread; ++i) {
                const int x = i * kTileThreads + tid;
                if (x >= n_here) continue;
                const uint32_t dd = distance<D>(sg[i], qsig + h * WPR);
                if (dd < cut[h]) {
                    out0[h * head_stride + atomicAdd(&cnt[h], 1u)] = cold_key(dd, lo + x);
                } else if (dd == cut[h]) {
                    atomicOr(&tie[h * (kTile / 32) + (x >> 5)], 1u << (x & 31));
                }
            }
    } else {
        // every distance up to the cut is among the candidates
        for (int h = 0; h < G; ++h)
            wave_cands(h, [&](uint32_t v) {
                const uint32_t dd = v >> 16, x = v & 0xFFFFu;
                if (dd < cut[h]) {
                    out0[h * head_stride + atomicAdd(&cnt[h], 1u)] = cold_key(dd, lo + x);
                } else if (dd == cut[h]) {
                    const uint32_t i = atomicAdd(&ntie[h], 1u);
                    if (i < 64) tlist[h][i] = x;
                }
            });
        __syncthreads();
        for (int h = 0; h < G; ++h) use_mask = use_mask || ntie[h] > 64u;
        if (use_mask) {
            for (int h = 0; h < G; ++h)
                wave_cands(h, [&](uint32_t v) {
                    const uint32_t x = v & 0xFFFFu;
                    if ((v >> 16) == cut[h]) atomicOr(&tie[h * (kTile / 32) + (x >> 5)], 1u << (x & 31));
                });
        }
    }
    __syncthreads();
    if (use_mask) {
        // thread tid < kTile / 32 owns mask word tid
        for (int h = 0; h < G; ++h) {
            uint32_t word = tid < kTile / 32 ? tie[h * (kTile / 32) + tid] : 0u;
            uint32_t total;
            const uint32_t pre = tile_exclusive_scan<kTileWaves>(__popc(word), wave_tot, total);
            const uint32_t nd = need[h];
            if (pre < nd) {
                const uint32_t take = nd - pre;
                uint32_t j = 0;
                while (word && j < take) {
                    const int bit = __builtin_ctz(word);
                    word &= word - 1;
                    out0[h * head_stride + below[h] + pre + j] = cold_key(cut[h], lo + 32 * tid + bit);
                    ++j;
                }
            }
        }
    } else {
        // lane i of a head's wave ranks tie i among the head's ties (positions in the tile are
        // distinct, so the ranks are 0 .. ntie - 1)
        for (int h = wave; h < G; h += kTileWaves) {
            const uint32_t nt = ntie[h], nd = need[h];
            const uint32_t x = (uint32_t)lane < nt ? tlist[h][lane] : 0xFFFFFFFFu;
            uint32_t rank = 0;
            for (uint32_t j = 0; j < nt; ++j) rank += tlist[h][j] < x ? 1u : 0u;
            if ((uint32_t)lane < nt && rank < nd) out0[h * head_stride + below[h] + rank] = cold_key(cut[h], lo + x);
        }
    }
    // padding past kc_eff
    for (int x = tid; x < G * kc; x += kTileThreads)
        if ((uint32_t)(x % kc) >= kc_eff) out0[(x / kc) * head_stride + x % kc] = kNoKey;
}

// kc <= kMaxCold, n_tiles <= kMergeTiles.  Candidates are visited three times, coalesced and in
// batches of kMergeBatch independent loads per thread (the first batch kept in registers, later
// ones read again from L2): the distance histogram;
// keys below the cut and per-tile tie counts; the ties of every tile whose ties are all taken.
// The one tile whose ties are taken in part ranks them by position.
constexpr int kMergeThreads = 512;
constexpr int kMergeBatch = 8;

// The first kMergeThreads * kMergeBatch keys (all of them at 1M: 64 tiles x 64) are loaded once
// and kept in registers for the three passes; later batches are loaded again by each pass.
struct KeyRegs {
    uint64_t k[kMergeBatch];
};
__device__ __forceinline__ KeyRegs load_first_keys(const uint64_t *c, int M) {
    KeyRegs r;
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b) {
        const int x = threadIdx.x + b * kMergeThreads;
        r.k[b] = x < M ? c[x] : kNoKey;
    }
    return r;
}
template <typename F>
__device__ __forceinline__ void for_each_key(const uint64_t *c, int M, const KeyRegs &r, F f) {
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b)
        if (r.k[b] != kNoKey) f((int)threadIdx.x + b * kMergeThreads, r.k[b]);
    for (int x0 = threadIdx.x + kMergeThreads * kMergeBatch; x0 < M; x0 += kMergeThreads * kMergeBatch) {
        uint64_t k[kMergeBatch];
#pragma unroll
        for (int b = 0; b < kMergeBatch; ++b) {
            const int x = x0 + b * kMergeThreads;
            k[b] = x < M ? c[x] : kNoKey;
        }
#pragma unroll
        for (int b = 0; b < kMergeBatch; ++b)
            if (k[b] != kNoKey) f(x0 + b * kMergeThreads, k[b]);
    }
}

__global__ void __launch_bounds__(kMergeThreads) cold_merge(const uint64_t *__restrict__ cand, int32_t *__restrict__ sel,
                                                            int n_tiles, int kc) {
    __shared__ uint32_t hist[kBinStride];
    __shared__ uint32_t tcnt[kMergeTiles], tpre[kMergeTiles];
    __shared__ int64_t lst[kMaxCold];
    __shared__ uint32_t wave_tot[kMergeThreads / 64];
    __shared__ uint32_t n_valid, n_lst, s_cut, s_need, b_tile, b_take;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t rh = blockIdx.x;
    const uint64_t *c = cand + rh * (int64_t)n_tiles * kc;
    const int M = n_tiles * kc;
    const KeyRegs kr = load_first_keys(c, M);  // (in flight while the LDS is cleared)
    for (int x = tid; x < kBinStride; x += kMergeThreads) hist[x] = 0;
    for (int x = tid; x < n_tiles; x += kMergeThreads) tcnt[x] = 0;
    if (tid == 0) {
        n_valid = 0;
        n_lst = 0;
        b_tile = 0xFFFFFFFFu;
        b_take = 0;
    }
    __syncthreads();
    uint32_t mine = 0;
    for_each_key(c, M, kr, [&](int, uint64_t k) {
        atomicAdd(&hist[key_dist(k)], 1u);
        ++mine;
    });
    atomicAdd(&n_valid, mine);
    __syncthreads();
    const uint32_t kc_eff = n_valid < (uint32_t)kc ? n_valid : (uint32_t)kc;
    if (wave == 0) {
        uint32_t b;
        const uint32_t ct = wave_cut(hist, kBins - 1, kc_eff, b);
        if (lane == 0) {
            s_cut = ct;
            s_need = kc_eff - b;
        }
    }
    __syncthreads();
    const uint32_t dstar = s_cut, nd = s_need;
    if (kc_eff > 0) {
        for_each_key(c, M, kr, [&](int x, uint64_t k) {
            const uint32_t dd = key_dist(k);
            if (dd < dstar) lst[atomicAdd(&n_lst, 1u)] = key_pos(k);
            else if (dd == dstar) atomicAdd(&tcnt[x / kc], 1u);
        });
    }
    __syncthreads();
    // exclusive prefix of the tie counts over tiles (tiles cover increasing positions): thread tid
    // owns the contiguous tiles [tid * per, tid * per + per)
    const int per = (n_tiles + kMergeThreads - 1) / kMergeThreads;
    uint32_t local = 0;
    for (int j = tid * per; j < tid * per + per && j < n_tiles; ++j) local += tcnt[j];
    uint32_t run;
    {
        uint32_t inc = local;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_up(inc, off);
            if (lane >= off) inc += y;
        }
        if (lane == 63) wave_tot[wave] = inc;
        __syncthreads();
        uint32_t before = 0;
        for (int w = 0; w < wave; ++w) before += wave_tot[w];
        run = before + inc - local;
    }
    for (int j = tid * per; j < tid * per + per && j < n_tiles; ++j) {
        tpre[j] = run;
        if (run < nd && run + tcnt[j] > nd) {  // the one tile whose ties are taken in part
            b_tile = (uint32_t)j;
            b_take = nd - run;
        }
        run += tcnt[j];
    }
    __syncthreads();
    if (kc_eff > 0) {
        for_each_key(c, M, kr, [&](int x, uint64_t k) {
            const int j = x / kc;
            if (key_dist(k) == dstar && tpre[j] + tcnt[j] <= nd) lst[atomicAdd(&n_lst, 1u)] = key_pos(k);
        });
    }
    const uint32_t bt = b_tile;
    if (bt != 0xFFFFFFFFu && wave == 0) {
        // ties of the boundary tile: lane l holds entries l and l + 64; rank by position
        const uint64_t *ct = c + (int64_t)bt * kc;
        uint64_t k0 = lane < kc ? ct[lane] : kNoKey, k1 = lane + 64 < kc ? ct[lane + 64] : kNoKey;
        const bool t0 = k0 != kNoKey && key_dist(k0) == dstar, t1 = k1 != kNoKey && key_dist(k1) == dstar;
        const int64_t p0 = t0 ? key_pos(k0) : INT64_MAX, p1 = t1 ? key_pos(k1) : INT64_MAX;
        uint32_t r0 = 0, r1 = 0;
        for (int src = 0; src < 64; ++src) {
            const int64_t a = __shfl(p0, src), b = __shfl(p1, src);
            r0 += (a < p0 ? 1u : 0u) + (b < p0 ? 1u : 0u);
            r1 += (a < p1 ? 1u : 0u) + (b < p1 ? 1u : 0u);
        }
        if (t0 && r0 < b_take) lst[atomicAdd(&n_lst, 1u)] = p0;
        if (t1 && r1 < b_take) lst[atomicAdd(&n_lst, 1u)] = p1;
    }
    __syncthreads();
    // ascending order, padded with -1
    int32_t *out = sel + rh * kc;
    if (tid < kc) {
        if ((uint32_t)tid < kc_eff) {
            const int64_t p = lst[tid];
            uint32_t rank = 0, x = 0;
            for (; x + 4 <= kc_eff; x += 4) {  // (four independent reads per step)
                const int64_t a0 = lst[x], a1 = lst[x + 1], a2 = lst[x + 2], a3 = lst[x + 3];
                rank += (a0 < p ? 1u : 0u) + (a1 < p ? 1u : 0u) + (a2 < p ? 1u : 0u) + (a3 < p ? 1u : 0u);
            }
            for (; x < kc_eff; ++x) rank += lst[x] < p ? 1u : 0u;
            out[rank] = (int32_t)p;
        } else {
            out[tid] = -1;
        }
    }
}

// Attention over fetched + hot positions.  16-byte slices: LPR lanes per key row, RPI row groups
// per wave, 16 waves: NGRP groups take keys x = grp, grp + NGRP, ... two at a time (both keys'
// K and V loads issued before either is used); each group keeps its own online softmax state over
// its slice of the output, and the groups are merged through LDS.  The selection is staged in LDS
// first, so key positions cost no dependent global load.
constexpr int kAttnWaves = 16;

template <typename T, int D>
__global__ void __launch_bounds__(kAttnWaves * 64) cold_attn(const T *__restrict__ q, const int32_t *__restrict__ row_seq,
                                                        const int64_t *__restrict__ row_pos, const T *__restrict__ K,
                                                        const T *__restrict__ V, const int32_t *__restrict__ sel,
                                                        float *__restrict__ out, int Hq, int Hkv, int G, int B,
                                                        int64_t cap, int64_t max_pos, int H, int kc,
                                                        float scale_log2) {
    constexpr int EPL = 16 / sizeof(T), LPR = D / EPL, RPI = 64 / LPR, NGRP = kAttnWaves * RPI;
    __shared__ float gm[NGRP], gl[NGRP], go[NGRP][D];
    __shared__ int32_t ssel[kMaxCold];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane % LPR, rr = lane / LPR, grp = wave * RPI + rr;
    const int64_t rh = blockIdx.x;
    const int64_t row = rh / Hq;
    const int h = (int)(rh % Hq), g = h / G;
    if (tid < kc) ssel[tid] = sel[rh * kc + tid];
    __syncthreads();
    // a position repeated in the selection counts once, at its first entry
    bool dup = false;
    if (tid < kc) {
        const int32_t p = ssel[tid];
        for (int x = 0; x < tid; ++x) dup = dup || ssel[x] == p;
    }
    __syncthreads();
    if (dup) ssel[tid] = -1;
    int64_t t = row_pos[row];
    t = t < 0 ? 0 : (t > max_pos ? max_pos : t);
    int seq = row_seq[row];
    seq = seq < 0 ? 0 : (seq >= B ? B - 1 : seq);
    const int64_t hot_lo = t - H + 1 > 0 ? t - H + 1 : 0;
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
    __syncthreads();
    float M = -__builtin_huge_valf(), L = 0.f, o[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) o[i] = 0.f;
    for (int64_t x0 = grp; x0 < n_keys; x0 += 2 * NGRP) {
        bool ok[2];
        uint4 kr[2], vr[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int64_t x = x0 + u * NGRP;
            int64_t p = x < kc ? (int64_t)ssel[x < kc ? x : 0] : hot_lo + (x - kc);
            // padding and entries outside the cold set are skipped; past the end as well
            ok[u] = x < n_keys && (x >= kc || (p >= 0 && p < hot_lo));
            p = ok[u] ? p : t;
            kr[u] = *reinterpret_cast<const uint4 *>(kb + p * D + c * EPL);
            vr[u] = *reinterpret_cast<const uint4 *>(vb + p * D + c * EPL);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float kf[EPL], vf[EPL];
            const uint32_t ku[4] = {kr[u].x, kr[u].y, kr[u].z, kr[u].w}, vu[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
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
            if (!ok[u]) continue;  // uniform over the group's lanes
            z *= scale_log2;
            const float Mn = fmaxf(M, z);
            const float a = exp2f(M - Mn), e = exp2f(z - Mn);
            L = L * a + e;
#pragma unroll
            for (int i = 0; i < EPL; ++i) o[i] = fmaf(e, vf[i], o[i] * a);
            M = Mn;
        }
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

template <typename T, int D, int TILE, int THREADS>
void tile_launch(const RowArgs &a, const uint32_t *sig, int H, int kc, uint64_t *cand, int n_tiles, hipStream_t st) {
    const size_t lds = tile_lds_words<TILE, THREADS>(a.G, D / 32) * sizeof(uint32_t);
    hipLaunchKernelGGL((cold_tile<T, D, TILE, THREADS>), dim3((unsigned)(a.n_rows * a.Hkv * n_tiles)), dim3(THREADS),
                       lds, st, (const T *)a.q, a.row_seq, a.row_pos, sig, cand, a.Hq, a.Hkv, a.G, a.B, a.cap,
                       a.max_pos, H, kc, n_tiles);
}

template <typename T, int D>
hipError_t select_launch(const RowArgs &a, const uint32_t *sig, int H, int kc, int32_t *sel, void *ws,
                         hipStream_t st) {
    const int n_tiles = cold_tiles(a.max_pos, H, a.G);
    uint64_t *cand = (uint64_t *)ws;
    if (a.G <= kTileBigMaxGroup)
        tile_launch<T, D, kTileBig, kTileBigThreads>(a, sig, H, kc, cand, n_tiles, st);
    else
        tile_launch<T, D, kTileSmall, kTileSmallThreads>(a, sig, H, kc, cand, n_tiles, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(cold_merge, dim3((unsigned)(a.n_rows * a.Hq)), dim3(kMergeThreads), 0, st, cand, sel, n_tiles,
                       kc);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t attn_launch(const RowArgs &a, const void *K, const void *V, const int32_t *sel, int H, int kc, float *out,
                       hipStream_t st) {
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    hipLaunchKernelGGL((cold_attn<T, D>), dim3((unsigned)(a.n_rows * a.Hq)), dim3(kAttnWaves * 64), 0, st, (const T *)a.q,
                       a.row_seq, a.row_pos, (const T *)K, (const T *)V, sel, out, a.Hq, a.Hkv, a.G, a.B, a.cap,
                       a.max_pos, H, kc, scale_log2);
    return hipGetLastError();
}

}  // namespace

int cold_tile_positions(int G) { return G <= kTileBigMaxGroup ? kTileBig : kTileSmall; }

int cold_tiles(int64_t max_pos, int H, int G) {
    const int64_t n = max_pos - H + 1;
    const int tile = cold_tile_positions(G);
    return n <= 0 ? 1 : (int)((n + tile - 1) / tile);
}

size_t cold_workspace_bytes(const RowArgs &a, int H, int kc) {
    return (size_t)a.n_rows * a.Hq * cold_tiles(a.max_pos, H, a.G) * kc * sizeof(uint64_t);
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
