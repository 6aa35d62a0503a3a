// Decode attention: exact softmax attention of each row over its window and its selected spans
// (release post, "Key idea": token-level attention inside the chosen spans), for few rows per
// sequence.  HBM-bound: the kernel's job is to stream the chosen K/V rows at full bandwidth.
//
// Work unit = (row, kv head, slot, sub-tile).  Slots are the G*k (query head, selection entry)
// pairs of the kv head, then the window spans.  A span chosen by several query heads of the
// kv head is read once: only the unit of the lowest head that chose it (its "owner") runs, and
// it computes the partial state for every head that chose the span (GQA sharing).  The kv
// head's G*k selection entries are loaded into registers together with the row's position in
// one round trip; the unit's span, its ownership and the list of heads sharing it then come
// from register reads and wave ballots, so the K/V stream starts after a single dependent load
// and no block-wide barrier.  Spans are cut into sub-tiles of 4 x KPW keys so that ~2000
// independent units keep all 256 CUs busy.
//
// Inside a unit each wave streams KPW keys straight from HBM into registers with 16-byte loads
// (LPR consecutive lanes cover one key row, so every load instruction reads whole rows); all K
// and V loads are issued before any arithmetic.  Per head: per-lane partial dot products, a
// butterfly reduce-scatter over the LPR lanes on DPP (each lane ends with one key's score), one
// exp2 per lane, the probabilities broadcast through LDS, P.V in fp32, a reduce-scatter over
// the row groups, and a 4-wave merge through LDS.  Partial states (m, l, o[d]) go to the
// workspace, one record per (row, head, entry, sub-tile), and every record is written on every
// call (units without keys mark theirs empty), so the combine kernel merges each row-head's
// records in a fixed order without looking at the selection.
#include "common.h"
#include "decode_append.h"
#include "kernels.h"
#include "summary_body.h"
#include "wave_ops.h"

#include <type_traits>

namespace ra {

template <typename T, int D, int NWAVE, int KPW_>
struct Lanes {
    static constexpr int EPL = 16 / sizeof(T);          // elements per 16-byte load
    static constexpr int LPR = D / EPL;                 // lanes per key row
    static constexpr int RPI = 64 / LPR;                // key rows per load instruction
    static constexpr int KPW = KPW_;                    // keys per wave
    static constexpr int STEPS = KPW / RPI;             // load instructions per wave (K or V)
    static constexpr int DUP = LPR / STEPS;             // lanes holding the same key's score
    static constexpr int TK = NWAVE * KPW;              // keys per unit
};

__device__ __forceinline__ void unpack16(const uint4 &raw, float *f, uint16_t) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
        f[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
}
// 16 E4M3 codes of an 8-bit cache row (exact conversions; the row scale is applied separately).
__device__ __forceinline__ void unpack16(const uint4 &raw, float *f, uint8_t) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
        f[4 * i] = lo.x;
        f[4 * i + 1] = lo.y;
        f[4 * i + 2] = hi.x;
        f[4 * i + 3] = hi.y;
    }
}
__device__ __forceinline__ void unpack16(const uint4 &raw, float *f, float) {
    f[0] = __uint_as_float(raw.x);
    f[1] = __uint_as_float(raw.y);
    f[2] = __uint_as_float(raw.z);
    f[3] = __uint_as_float(raw.w);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Dot product of 8 bf16 pairs packed in two uint4 (four v_dot2_f32_bf16).
__device__ __forceinline__ float dot8_bf16(const uint4 &a, const uint4 &b) {
    float r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x), __builtin_bit_cast(bf16x2_t, b.x), 0.f,
                                              false);
    r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y), __builtin_bit_cast(bf16x2_t, b.y), r, false);
    r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z), __builtin_bit_cast(bf16x2_t, b.z), r, false);
    r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w), __builtin_bit_cast(bf16x2_t, b.w), r, false);
    return r;
}

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal: the K/V rows are read once per call, so they should not
// displace other lines from the caches (measured: ~11% less time for the decode step's
// attention at 1M context than with ordinary loads).
template <typename T>
__device__ __forceinline__ uint4 load_stream(const T *p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kSelRegChunks = 4;  // selection entries of a kv head kept in registers: G*k <= 256
constexpr int kMaxSelChunks = 32;  // G*k <= 32 * 64

// T: element type of the K/V cache (fp32, bf16 bits, or 8-bit E4M3 codes with row scales ks,
// vs); queries are of the same type, bf16 for an 8-bit cache.
template <typename T, int D, int NWAVE, int KPW_>
__global__ void __launch_bounds__(NWAVE * 64) decode_attn(const void *__restrict__ qv, const int32_t *__restrict__ row_seq,
                                                   const int64_t *__restrict__ row_pos, const T *K, const T *V,
                                                   const float *__restrict__ ks, const float *__restrict__ vs,
                                                   const int32_t *__restrict__ sel, float *__restrict__ part, int Hq,
                                                   int Hkv, int G, int S, int k, int W, int B, int64_t cap,
                                                   int64_t max_pos, int64_t n_rows_total, int NW, int nsub,
                                                   float scale_log2) {
    using L = Lanes<T, D, NWAVE, KPW_>;
    constexpr int EPL = L::EPL, LPR = L::LPR, RPI = L::RPI, KPW = L::KPW, STEPS = L::STEPS, TK = L::TK;
    constexpr bool FP8 = sizeof(T) == 1;
    using TQ = typename std::conditional<FP8, uint16_t, T>::type;
    constexpr int QLOADS = FP8 ? 2 : 1;  // 16-byte loads of the lane's query slice
    const TQ *q = reinterpret_cast<const TQ *>(qv);
    constexpr int DUP = L::DUP;
    __shared__ float pbuf[NWAVE][64];
    __shared__ uint64_t mask_s[NWAVE][kMaxSelChunks];
    __shared__ float wm[NWAVE], wl[NWAVE];
    __shared__ float wo[NWAVE][D];

    // all kernel arguments in one round trip (otherwise some are fetched only where first used)
    asm volatile("" ::"s"(qv), "s"(row_seq), "s"(row_pos), "s"(K), "s"(V), "s"(ks), "s"(vs), "s"(sel), "s"(part), "s"(Hq), "s"(Hkv),
                 "s"(G), "s"(S), "s"(k), "s"(W), "s"(B), "s"(cap), "s"(max_pos), "s"(n_rows_total), "s"(NW),
                 "s"(nsub), "s"(scale_log2));
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Gk = G * k;
    // grid order: all window units first (they serve all G heads, so they carry the most work
    // per block and should not form the tail), then the selected-span units
    // (the grid has fewer than 2^32 blocks: 32-bit index arithmetic)
    const uint32_t n_win_units = (uint32_t)(n_rows_total * Hkv * (int64_t)NW * nsub);
    int sub, slot, g;
    int64_t row;
    {
        uint32_t b = blockIdx.x;
        const bool win = b < n_win_units;
        if (!win) b -= n_win_units;
        const uint32_t per = win ? NW : Gk;
        sub = (int)(b % (uint32_t)nsub);
        b /= (uint32_t)nsub;
        slot = (int)(b % per) + (win ? Gk : 0);
        b /= per;
        g = (int)(b % (uint32_t)Hkv);
        row = b / (uint32_t)Hkv;
    }
    const bool is_window = slot >= Gk;
    const int h_own = slot / k, e_own = slot % k;  // span units: (query head, selection entry)
    const int32_t *sel_rg = sel + (row * Hq + (int64_t)g * G) * k;

    // one round trip: the row's position and sequence, and the kv head's selection entries
    const int64_t t_raw = row_pos[row];
    const int seq_raw = row_seq[row];
    int32_t selv[kSelRegChunks];
    const bool sel_in_regs = Gk <= 64 * kSelRegChunks;
    if (!is_window && sel_in_regs) {
        // unconditional loads from clamped indices, masked afterwards (no per-chunk round trips)
#pragma unroll
        for (int cc = 0; cc < kSelRegChunks; ++cc) {
            const int x = cc * 64 + lane;
            selv[cc] = sel_rg[x < Gk ? x : Gk - 1];
        }
#pragma unroll
        for (int cc = 0; cc < kSelRegChunks; ++cc) selv[cc] = cc * 64 + lane < Gk ? selv[cc] : -1;
    } else {
#pragma unroll
        for (int cc = 0; cc < kSelRegChunks; ++cc) selv[cc] = -1;
    }
    asm volatile("" ::: "memory");  // all of the above are in flight together
    asm volatile("" ::"s"(t_raw), "s"(seq_raw));  // (and the scalar ones are not deferred)
    int64_t t = t_raw < 0 ? 0 : (t_raw > max_pos ? max_pos : t_raw);
    const int seq = seq_raw < 0 ? 0 : (seq_raw >= B ? B - 1 : seq_raw);
    const int64_t r = num_routable(t, S, W);
    const int64_t w0 = r * S;
    const int NE = k + NW;  // entries per row-head in the workspace

    // Which records this unit writes: (head h in `hw`, entry, sub).  Every (head, entry, sub)
    // record of the call is written by exactly one unit, so the combine needs no selection:
    //  - a window unit: all G heads, entry k + w (empty once the span starts after t);
    //  - a span entry whose span id is out of range, or repeats an earlier entry of its head:
    //    its own unit, empty;
    //  - a valid span j: the unit of the lowest entry of the kv head that selects j (its "owner")
    //    reads the span once and computes it for every head that selects j (GQA sharing), at
    //    that head's first entry selecting j.
    const uint32_t all_heads = G == 32 ? 0xFFFFFFFFu : (1u << G) - 1u;
    uint32_t hw;
    int first_e = -1;  // span owner: lane h < G holds the first entry of head h that selects j
    int64_t j, lo, hi;
    if (is_window) {
        j = r + (slot - Gk);
        lo = j * S;
        hi = lo + S < t + 1 ? lo + S : t + 1;
        hw = all_heads;
    } else {
        if (sel_in_regs) {
            const int cc = slot >> 6;
            const int32_t v = cc == 0 ? selv[0] : cc == 1 ? selv[1] : cc == 2 ? selv[2] : selv[3];
            j = __builtin_amdgcn_readlane(v, slot & 63);
        } else {
            j = sel_rg[slot];
        }
        lo = hi = 0;  // empty unless this unit owns a valid span
        hw = 1u << h_own;
        if (j >= 0 && j < r) {
            // bit x of the mask: entry x of the kv head selects j
            uint64_t b0 = 0, b1 = 0, b2 = 0, b3 = 0;
            if (sel_in_regs) {  // (entries past G*k hold -1 and never match)
                b0 = __ballot(selv[0] == (int32_t)j);
                b1 = __ballot(selv[1] == (int32_t)j);
                b2 = __ballot(selv[2] == (int32_t)j);
                b3 = __ballot(selv[3] == (int32_t)j);
            } else {
                for (int cc = 0; cc * 64 < Gk; ++cc) {
                    const int x = cc * 64 + lane;
                    const uint64_t bal = __ballot(x < Gk && sel_rg[x] == (int32_t)j);
                    if (lane == 0) mask_s[wave][cc] = bal;
                }
                __builtin_amdgcn_wave_barrier();
            }
            if (lane < G) {  // head `lane`'s entries are mask bits lane*k .. lane*k + k - 1
                const int pbit = lane * k, wd = pbit >> 6, sh = pbit & 63;
                uint64_t lw, hw2;
                if (sel_in_regs) {
                    lw = wd == 0 ? b0 : wd == 1 ? b1 : wd == 2 ? b2 : b3;
                    hw2 = wd == 0 ? b1 : wd == 1 ? b2 : wd == 2 ? b3 : 0ull;
                } else {
                    lw = mask_s[wave][wd];
                    hw2 = (wd + 1) * 64 < Gk ? mask_s[wave][wd + 1] : 0ull;
                }
                uint64_t f = sh ? (lw >> sh) | (hw2 << (64 - sh)) : lw;
                if (k < 64) f &= (1ull << k) - 1ull;
                first_e = f ? (int)__builtin_ctzll(f) : -1;
            }
            const uint32_t hm = (uint32_t)__ballot(first_e >= 0);  // includes h_own
            const int ho = (int)__builtin_ctz(hm);
            if (ho == h_own && __builtin_amdgcn_readlane(first_e, ho) == e_own) {
                hw = hm;  // the owner
                lo = j * S;
                hi = lo + S;
            } else if (__builtin_amdgcn_readlane(first_e, h_own) == e_own) {
                return;  // the owner writes this entry's records (and counts them)
            }
            // otherwise a repeated entry of its head: written empty below
        }
    }
    const bool owner_or_window = hi > lo;
    auto rec_of = [&](int h, int entry) {
        return part + (((row * Hq + g * G + h) * NE + entry) * (int64_t)nsub + sub) * record_floats(D);
    };
    const int64_t ulo = lo + (int64_t)sub * TK;
    if (ulo >= hi) {
        // no keys: the unit's records are marked empty (m = -inf, l = 0)
        if (tid < G && ((hw >> tid) & 1u)) {
            const int entry = is_window ? k + (slot - Gk) : (owner_or_window ? first_e : e_own);
            *reinterpret_cast<float2 *>(rec_of(tid, entry)) = make_float2(kNegInf, 0.f);
        }
    } else {
        const int64_t uhi = ulo + TK < hi ? ulo + TK : hi;
        const int c = lane % LPR, rr = lane / LPR;
        const int h0 = (int)__builtin_ctz(hw);
        uint4 qraw[QLOADS];
#pragma unroll
        for (int i = 0; i < QLOADS; ++i)
            qraw[i] = *reinterpret_cast<const uint4 *>(q + (row * Hq + g * G + h0) * D + c * EPL + 8 * i);

        // stream this wave's keys: all K and V loads are issued before any use
        const int64_t kv_base = ((int64_t)seq * Hkv + g) * cap;
        const int64_t wkey0 = ulo + (int64_t)wave * KPW;
        uint4 kr[STEPS], vr[STEPS];
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            const int64_t key = wkey0 + s * RPI + rr;
            const int64_t kl = key < uhi ? key : uhi - 1;  // in-bounds, finite row for masked keys
            kr[s] = load_stream(K + (kv_base + kl) * D + c * EPL);
        }
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            const int64_t key = wkey0 + s * RPI + rr;
            const int64_t kl = key < uhi ? key : uhi - 1;
            vr[s] = load_stream(V + (kv_base + kl) * D + c * EPL);
        }
        // the key whose score this lane holds after the reduce-scatter
        const int s_own = c / DUP;
        const int64_t own_key = wkey0 + s_own * RPI + rr;
        const bool own_valid = own_key < uhi;
        // 8-bit cache: that key's K and V row scales
        float ksc = 1.f, vsc = 1.f;
        if constexpr (FP8) {
            const int64_t kl = own_key < uhi ? own_key : uhi - 1;
            ksc = ks[kv_base + kl];
            vsc = vs[kv_base + kl];
        }
        asm volatile("" ::: "memory");  // keep the loads here: nothing may sink them into the head loop

        const bool counts = (c % DUP) == 0;  // one lane per key contributes to the sum

        uint32_t rem = hw;
        bool first = true;
        while (rem) {
            const int h = (int)__builtin_ctz(rem);
            rem &= rem - 1u;
            const int entry = is_window ? k + (slot - Gk) : __builtin_amdgcn_readlane(first_e, h);
            const int hq = g * G + h;
            // the packed K/V registers are "redefined" here, so the compiler cannot hoist their
            // widening out of the head loop (that would hold 2x the registers and stall the loads)
#pragma unroll
            for (int s = 0; s < STEPS; ++s)
                asm volatile("" : "+v"(kr[s].x), "+v"(kr[s].y), "+v"(kr[s].z), "+v"(kr[s].w));
            if (!first) {
#pragma unroll
                for (int i = 0; i < QLOADS; ++i)
                    qraw[i] = *reinterpret_cast<const uint4 *>(q + (row * Hq + hq) * D + c * EPL + 8 * i);
            }
            first = false;
            float acc[STEPS];
            if constexpr (FP8) {
                // bf16 query slice against 16 codes per row; the row scale multiplies the sum
                float qf[EPL];
                unpack16(qraw[0], qf, uint16_t());
                unpack16(qraw[1], qf + 8, uint16_t());
#pragma unroll
                for (int s = 0; s < STEPS; ++s) {
                    float kf[EPL];
                    unpack16(kr[s], kf, T());
                    float a = 0.f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) a = fmaf(qf[e], kf[e], a);
                    acc[s] = a;
                }
            } else if constexpr (sizeof(T) == 2) {
                // bf16: packed pairs straight into v_dot2_f32_bf16 (exact products, fp32 sums)
#pragma unroll
                for (int s = 0; s < STEPS; ++s) acc[s] = dot8_bf16(qraw[0], kr[s]);
            } else {
                float qf[EPL];
                unpack16(qraw[0], qf, T());
#pragma unroll
                for (int s = 0; s < STEPS; ++s) {
                    float kf[EPL];
                    unpack16(kr[s], kf, T());
                    float a = 0.f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) a = fmaf(qf[e], kf[e], a);
                    acc[s] = a;
                }
            }
            ReduceScatter<STEPS, ilog2(STEPS), LPR / 2>::run(acc, lane);
            const float sc = allreduce_sum<DUP / 2>(acc[0]);
            const float z = own_valid ? sc * ksc * scale_log2 : kNegInf;
            const float m = wave_max(z);
            const float p = (own_valid && m != kNegInf) ? exp2f(z - m) : 0.f;
            const float ls = wave_sum(counts ? p : 0.f);
            pbuf[wave][lane] = p * vsc;  // (8-bit cache: the V row scale rides on the weight)
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int s = 0; s < STEPS; ++s)
                asm volatile("" : "+v"(vr[s].x), "+v"(vr[s].y), "+v"(vr[s].z), "+v"(vr[s].w));
            float o[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[e] = 0.f;
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                const float ps = pbuf[wave][rr * LPR + s * DUP];
                float vf[EPL];
                unpack16(vr[s], vf, T());
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[e] = fmaf(ps, vf[e], o[e]);
            }
            // over the row groups (lanes of another row group hold other elements: exact partners)
            ReduceScatter<EPL, ilog2(RPI), 32, true>::run(o, lane);  // EPL -> EPL / RPI values
            constexpr int KEEP = EPL / RPI;
            if (lane == 0) {
                wm[wave] = m;
                wl[wave] = ls;
            }
#pragma unroll
            for (int i = 0; i < KEEP; ++i) wo[wave][c * EPL + rr * KEEP + i] = o[i];
            __syncthreads();
            if (tid < D) {
                float M = wm[0];
#pragma unroll
                for (int w = 1; w < NWAVE; ++w) M = fmaxf(M, wm[w]);
                float Lsum = 0.f, O = 0.f;
#pragma unroll
                for (int w = 0; w < NWAVE; ++w) {
                    if (wm[w] != kNegInf) {
                        const float f = exp2f(wm[w] - M);
                        Lsum = fmaf(wl[w], f, Lsum);
                        O = fmaf(wo[w][tid], f, O);
                    }
                }
                float *rec = rec_of(h, entry);
                rec[4 + tid] = O;
                if (tid == 0) {
                    rec[0] = M;
                    rec[1] = Lsum;
                }
            }
            __syncthreads();
        }
    }

}

// Merge for few row-heads with many records: one block of 16 waves per row-head.  Every record
// slot is written by the decode kernel (empty ones have m = -inf), so each wave loads its records
// (x = wave, wave + 16, ...) in batches with no dependent round trip, merges them with its own
// running maximum, and the 16 wave states are merged in fixed order through LDS.
constexpr int kCombineWaves = 16;

template <int D>
__device__ __forceinline__ void combine_rowhead(const float *__restrict__ part, float *__restrict__ out, int nrec,
                                                int64_t rh, float *wm, float *wl, float (*wo)[D]) {
    constexpr int PER = D / 64;
    constexpr int B = 8;  // records per batch
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float *base = part + rh * (int64_t)nrec * record_floats(D);
    float M = kNegInf, l = 0.f, o[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = 0.f;
    for (int x0 = wave; x0 < nrec; x0 += kCombineWaves * B) {
        float v[B][PER], mv[B], lv[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            int x = x0 + kCombineWaves * b;
            x = x < nrec ? x : nrec - 1;
            const float *rec = base + (int64_t)x * record_floats(D);
            const float2 ml = *reinterpret_cast<const float2 *>(rec);
            mv[b] = ml.x;
            lv[b] = ml.y;
#pragma unroll
            for (int i = 0; i < PER; ++i) v[b][i] = rec[4 + lane + 64 * i];
        }
        // every load of the batch stays here, ahead of the first use (left alone, the compiler
        // sinks the l and o loads under the test of the maxima: a second round trip)
        asm volatile("" ::: "memory");
#pragma unroll
        for (int b = 0; b < B; ++b) {
            asm volatile("" : "+v"(mv[b]), "+v"(lv[b]));
#pragma unroll
            for (int i = 0; i < PER; ++i) asm volatile("" : "+v"(v[b][i]));
        }
        float bm = kNegInf;
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (x0 + kCombineWaves * b >= nrec) mv[b] = kNegInf;
            bm = fmaxf(bm, mv[b]);
        }
        const float Mn = fmaxf(M, bm);
        if (Mn != kNegInf) {
            const float a = exp2f(M - Mn);  // 0 when M = -inf
            l *= a;
#pragma unroll
            for (int i = 0; i < PER; ++i) o[i] *= a;
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const bool ok = mv[b] != kNegInf;
                const float f = ok ? exp2f(mv[b] - Mn) : 0.f;
                l = ok ? fmaf(lv[b], f, l) : l;
#pragma unroll
                for (int i = 0; i < PER; ++i) o[i] = ok ? fmaf(v[b][i], f, o[i]) : o[i];
            }
            M = Mn;
        }
    }
    if (lane == 0) {
        wm[wave] = M;
        wl[wave] = l;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) wo[wave][lane + 64 * i] = o[i];
    __syncthreads();
    if (tid < D) {
        float Mt = kNegInf;
#pragma unroll
        for (int w = 0; w < kCombineWaves; ++w) Mt = fmaxf(Mt, wm[w]);
        float Lt = 0.f, Ot = 0.f;
#pragma unroll
        for (int w = 0; w < kCombineWaves; ++w) {
            if (wm[w] != kNegInf) {
                const float f = exp2f(wm[w] - Mt);
                Lt = fmaf(wl[w], f, Lt);
                Ot = fmaf(wo[w][tid], f, Ot);
            }
        }
        out[rh * D + tid] = Lt > 0.f ? Ot / Lt : 0.f;
    }
}

template <int D>
__global__ void __launch_bounds__(kCombineWaves * 64) combine_block(const float *__restrict__ part,
                                                                   float *__restrict__ out, int nrec) {
    __shared__ float wm[kCombineWaves], wl[kCombineWaves], wo[kCombineWaves][D];
    asm volatile("" ::"s"(part), "s"(out), "s"(nrec));  // all kernel arguments in one round trip
    combine_rowhead<D>(part, out, nrec, blockIdx.x, wm, wl, wo);
}

// The merge with a span-summary append in the same launch: blocks below n_rh merge row-heads,
// the B * Hkv blocks after them add one new token per sequence to the summaries (the update
// reads K and writes span_mean / run_sum, none of which the attention reads).
template <int D, typename T>
__global__ void __launch_bounds__(kCombineWaves * 64) combine_append(const float *__restrict__ part,
                                                                    float *__restrict__ out, int nrec, int64_t n_rh,
                                                                    const T *__restrict__ K,
                                                                    const float *__restrict__ kscale,
                                                                    float *__restrict__ mean,
                                                                    float *__restrict__ run_sum,
                                                                    const int64_t *__restrict__ old_len,
                                                                    const int64_t *__restrict__ new_len, int Hkv,
                                                                    int S, int64_t cap, int64_t max_spans) {
    __shared__ float wm[kCombineWaves], wl[kCombineWaves], wo[kCombineWaves][D];
    __shared__ float stage[kStageTokens][D];
    if ((int64_t)blockIdx.x < n_rh) {
        combine_rowhead<D>(part, out, nrec, blockIdx.x, wm, wl, wo);
    } else {
        summary_unit<T, D>(K, kscale, mean, run_sum, old_len, new_len, Hkv, S, cap, max_spans, 0, 1,
                           (int)(blockIdx.x - n_rh), stage);
    }
}

}  // namespace


namespace {

// Keys per wave: 64 (16 loads of K and 16 of V per lane in flight), 32 for fp32 with d = 128
// (the same 32 registers of data per lane); 4 waves per unit.
constexpr int kDecodeWaves = 4;

int decode_keys_per_wave(const RowArgs &a) { return (a.dtype == RA_F32 && a.d == 128) ? 32 : 64; }

int decode_sub_tile(const RowArgs &a) { return kDecodeWaves * decode_keys_per_wave(a); }

template <typename T, int D, int KPW, int NWAVE = kDecodeWaves>
hipError_t decode_launch_t(const RowArgs &a, const void *K, const void *V, const float *ks, const float *vs,
                           const int32_t *sel, float *out, void *ws, const SummaryArgs *app, hipStream_t st) {
    using L = Lanes<T, D, NWAVE, KPW>;
    const int NW = max_window_spans(a.S, a.W);
    const int n_slots = a.G * a.k + NW;
    const int nsub = (int)ceil_div(a.S, L::TK);
    const int64_t blocks = a.n_rows * a.Hkv * n_slots * nsub;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    float *part = (float *)ws;
    hipLaunchKernelGGL((decode_attn<T, D, NWAVE, KPW>), dim3((unsigned)blocks), dim3(NWAVE * 64), 0, st,
                       a.q, a.row_seq, a.row_pos, (const T *)K, (const T *)V, ks, vs, sel, part, a.Hq, a.Hkv, a.G,
                       a.S, a.k, a.W, a.B, a.cap, a.max_pos, a.n_rows, NW, nsub, scale_log2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nrec = (a.k + NW) * nsub;
    const int64_t n_rh = a.n_rows * a.Hq;
    if (app != nullptr && app->max_new == 1) {
        // one new token per sequence: its summary update rides in the merge launch
        hipLaunchKernelGGL((combine_append<D, T>), dim3((unsigned)(n_rh + (int64_t)app->B * app->Hkv)),
                           dim3(kCombineWaves * 64), 0, st, part, out, nrec, n_rh, (const T *)app->k, app->kscale,
                           app->mean, app->run_sum, app->old_len, app->new_len, app->Hkv, app->S, app->cap,
                           app->max_spans);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((combine_block<D>), dim3((unsigned)n_rh), dim3(kCombineWaves * 64), 0, st, part, out, nrec);
    e = hipGetLastError();
    if (e != hipSuccess || app == nullptr || app->max_new <= 0) return e;
    return launch_summary(*app, st);
}

}  // namespace

size_t decode_workspace_bytes(const RowArgs &a) {
    const int NW = max_window_spans(a.S, a.W);
    const int64_t nsub = ceil_div(a.S, decode_sub_tile(a));
    return (size_t)(a.n_rows * a.Hq * (a.k + NW) * nsub * record_floats(a.d) * sizeof(float));
}

hipError_t launch_decode_app(const RowArgs &a, const void *K, const void *V, const int32_t *sel, float *out, void *ws,
                             const SummaryArgs *app, hipStream_t st) {
    if (a.n_rows == 0) return app != nullptr && app->max_new > 0 ? launch_summary(*app, st) : hipSuccess;
    if (a.dtype == RA_BF16)
        return a.d == 64 ? decode_launch_t<uint16_t, 64, 64>(a, K, V, nullptr, nullptr, sel, out, ws, app, st)
                         : decode_launch_t<uint16_t, 128, 64>(a, K, V, nullptr, nullptr, sel, out, ws, app, st);
    return a.d == 64 ? decode_launch_t<float, 64, 64>(a, K, V, nullptr, nullptr, sel, out, ws, app, st)
                     : decode_launch_t<float, 128, 32>(a, K, V, nullptr, nullptr, sel, out, ws, app, st);
}

// 8-bit cache: 64 keys per wave (a lane's reduce-scatter then ends on one key) and
// kDecodeWavesFp8 waves per unit (measured at 1M: 4 waves 34-36 us per call, 8 waves 40 us,
// 16 waves 56 us: the number of units matters more than the bytes in flight per unit);
// sub-tiles at least as long as bf16's, so the workspace of routed_attn_decode suffices.
constexpr int kDecodeWavesFp8 = 4;
static_assert(kDecodeWavesFp8 >= kDecodeWaves, "decode_workspace_bytes sizes records for the bf16 sub-tiles");

hipError_t launch_decode_fp8_app(const RowArgs &a, const uint8_t *K8, const uint8_t *V8, const float *ks,
                                 const float *vs, const int32_t *sel, float *out, void *ws, const SummaryArgs *app,
                                 hipStream_t st) {
    if (a.n_rows == 0) return app != nullptr && app->max_new > 0 ? launch_summary(*app, st) : hipSuccess;
    return a.d == 64 ? decode_launch_t<uint8_t, 64, 64, kDecodeWavesFp8>(a, K8, V8, ks, vs, sel, out, ws, app, st)
                     : decode_launch_t<uint8_t, 128, 64, kDecodeWavesFp8>(a, K8, V8, ks, vs, sel, out, ws, app, st);
}

hipError_t launch_decode(const RowArgs &a, const void *K, const void *V, const int32_t *sel, float *out, void *ws,
                         hipStream_t st) {
    return launch_decode_app(a, K, V, sel, out, ws, nullptr, st);
}

hipError_t launch_decode_fp8(const RowArgs &a, const uint8_t *K8, const uint8_t *V8, const float *ks,
                             const float *vs, const int32_t *sel, float *out, void *ws, hipStream_t st) {
    return launch_decode_fp8_app(a, K8, V8, ks, vs, sel, out, ws, nullptr, st);
}

int64_t decode_grid_items(const RowArgs &a, bool fp8) {
    const int NW = max_window_spans(a.S, a.W);
    const int64_t tk = fp8 ? (int64_t)kDecodeWavesFp8 * 64 : decode_sub_tile(a);  // keys per unit
    const int waves = fp8 ? kDecodeWavesFp8 : kDecodeWaves;
    const int64_t units = a.n_rows * a.Hkv * (int64_t)(a.G * a.k + NW) * ceil_div(a.S, tk);
    const int64_t merge = (a.n_rows * a.Hq + (int64_t)a.B * a.Hkv) * kCombineWaves * 64;
    const int64_t attn = units * waves * 64;
    return attn > merge ? attn : merge;
}

}  // namespace ra
