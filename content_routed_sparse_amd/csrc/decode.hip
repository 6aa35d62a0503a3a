// Decode attention: exact softmax attention of each row over its window and its selected spans
// (release post, "Key idea": token-level attention inside the chosen spans), for few rows per
// sequence.  HBM-bound: the kernel's job is to stream the chosen K/V rows at full bandwidth.
//
// Work unit = (row, kv head, slot, sub-tile).  Slots are the G*k (query head, selection entry)
// pairs of the kv head, then the window spans.  A span chosen by several query heads of the
// kv head is read once: only the unit of the lowest head that chose it (its "owner") runs, and
// it computes the partial state for every head that chose the span (GQA sharing).  Spans are
// cut into sub-tiles of 4 x KPW keys so that ~2000 independent units keep all 256 CUs busy.
// Inside a unit each wave streams KPW keys straight from HBM into registers with 16-byte loads
// (LPR consecutive lanes cover one key row, so every load instruction reads whole rows), then
// per head: dot products reduced over the LPR lanes, an online-softmax partial per wave, the
// P.V product, and a 4-wave merge through LDS.  The partial states (m, l, o[d]) are written to
// the workspace and merged per row in `combine_kernel` in a fixed order.
#include "common.h"
#include "kernels.h"

namespace ra {

template <typename T, int D>
struct Lanes {
    static constexpr int EPL = 16 / sizeof(T);          // elements per 16-byte load
    static constexpr int LPR = D / EPL;                 // lanes per key row
    static constexpr int RPI = 64 / LPR;                // key rows per load instruction
    static constexpr int KPW = (sizeof(T) == 4 && D == 128) ? 32 : 64;  // keys per wave
    static constexpr int STEPS = KPW / RPI;
    static constexpr int TK = 4 * KPW;                  // keys per unit (4 waves)
};

__device__ __forceinline__ void unpack16(const uint4 &raw, float *f, uint16_t) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
        f[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
}
__device__ __forceinline__ void unpack16(const uint4 &raw, float *f, float) {
    f[0] = __uint_as_float(raw.x);
    f[1] = __uint_as_float(raw.y);
    f[2] = __uint_as_float(raw.z);
    f[3] = __uint_as_float(raw.w);
}

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

template <typename T, int D>
__global__ void __launch_bounds__(256) decode_attn(const T *__restrict__ q, const int32_t *__restrict__ row_seq,
                                                   const int64_t *__restrict__ row_pos, const T *__restrict__ K,
                                                   const T *__restrict__ V, const int32_t *__restrict__ sel,
                                                   float *__restrict__ part, int Hq, int Hkv, int G, int S, int k,
                                                   int W, int B, int64_t cap, int64_t max_pos, int n_slots, int NW,
                                                   int nsub, float scale_log2) {
    using L = Lanes<T, D>;
    constexpr int EPL = L::EPL, LPR = L::LPR, RPI = L::RPI, KPW = L::KPW, STEPS = L::STEPS, TK = L::TK;
    __shared__ int sel_s[32 * 64];
    __shared__ int head_entry[32];
    __shared__ int not_owner;
    __shared__ float wm[4], wl[4];
    __shared__ float wo[4][D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = blockIdx.x % nsub;
    int64_t rest = blockIdx.x / nsub;
    const int slot = (int)(rest % n_slots);
    rest /= n_slots;
    const int g = (int)(rest % Hkv);
    const int64_t row = rest / Hkv;

    int64_t t = row_pos[row];
    t = t < 0 ? 0 : (t > max_pos ? max_pos : t);
    int seq = row_seq[row];
    seq = seq < 0 ? 0 : (seq >= B ? B - 1 : seq);
    const int64_t w0 = window_start(t, S, W);
    const int64_t r = w0 / S;
    const int NE = k + NW;  // entries per row-head in the workspace
    const int32_t *sel_rg = sel + (row * Hq + (int64_t)g * G) * k;

    int64_t j, lo, hi;
    const bool is_window = slot >= G * k;
    if (!is_window) {
        j = sel_rg[slot];  // (head slot / k, entry slot % k)
        if (j < 0 || j >= r) return;
        lo = j * S;
        hi = lo + S;
    } else {
        j = w0 / S + (slot - G * k);
        lo = j * S;
        if (lo > t) return;
        hi = lo + S < t + 1 ? lo + S : t + 1;
    }
    const int64_t ulo = lo + (int64_t)sub * TK;
    if (ulo >= hi) return;
    const int64_t uhi = ulo + TK < hi ? ulo + TK : hi;

    // heads of this kv head that attend to span j, and the unit's ownership
    if (tid < G) head_entry[tid] = is_window ? k + (slot - G * k) : -1;
    if (tid == 0) not_owner = 0;
    if (!is_window)
        for (int x = tid; x < G * k; x += 256) sel_s[x] = sel_rg[x];
    __syncthreads();
    if (!is_window) {
        const int my_head = slot / k;
        for (int x = tid; x < G * k; x += 256) {
            if (sel_s[x] == j) {
                head_entry[x / k] = x % k;
                if (x / k < my_head) not_owner = 1;
            }
        }
        __syncthreads();
        if (not_owner) return;
    }

    // stream this wave's KPW keys into registers
    const int c = lane % LPR, rr = lane / LPR;
    const int64_t kv_base = ((int64_t)seq * Hkv + g) * cap;
    const int64_t wkey0 = ulo + (int64_t)wave * KPW;
    uint4 kr[STEPS], vr[STEPS];
    bool valid[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        const int64_t key = wkey0 + s * RPI + rr;
        valid[s] = key < uhi;
        const int64_t kl = valid[s] ? key : uhi - 1;  // in-bounds, finite row for masked keys
        kr[s] = *reinterpret_cast<const uint4 *>(K + (kv_base + kl) * D + c * EPL);
    }
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        const int64_t key = wkey0 + s * RPI + rr;
        const int64_t kl = key < uhi ? key : uhi - 1;
        vr[s] = *reinterpret_cast<const uint4 *>(V + (kv_base + kl) * D + c * EPL);
    }

    for (int h = 0; h < G; ++h) {
        const int entry = head_entry[h];
        if (entry < 0) continue;  // uniform across the block
        const int hq = g * G + h;
        float qf[EPL];
        unpack16(*reinterpret_cast<const uint4 *>(q + (row * Hq + hq) * D + c * EPL), qf, T());
        float z[STEPS];
        float mloc = kNegInf;
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            float kf[EPL];
            unpack16(kr[s], kf, T());
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc = fmaf(qf[e], kf[e], acc);
#pragma unroll
            for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off);
            z[s] = valid[s] ? acc * scale_log2 : kNegInf;
            mloc = fmaxf(mloc, z[s]);
        }
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off));
        float lsum = 0.f;
        float o[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = 0.f;
        if (mloc != kNegInf) {
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                const float p = valid[s] ? exp2f(z[s] - mloc) : 0.f;
                lsum += p;
                float vf[EPL];
                unpack16(vr[s], vf, T());
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[e] = fmaf(p, vf[e], o[e]);
            }
        }
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) {
            lsum += __shfl_xor(lsum, off);
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[e] += __shfl_xor(o[e], off);
        }
        if (lane == 0) {
            wm[wave] = mloc;
            wl[wave] = lsum;
        }
        if (rr == 0) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) wo[wave][c * EPL + e] = o[e];
        }
        __syncthreads();
        if (tid < D) {
            float M = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
            float Lsum = 0.f, O = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                if (wm[w] != kNegInf) {
                    const float f = exp2f(wm[w] - M);
                    Lsum = fmaf(wl[w], f, Lsum);
                    O = fmaf(wo[w][tid], f, O);
                }
            }
            float *rec = part + (((row * Hq + hq) * NE + entry) * (int64_t)nsub + sub) * record_floats(D);
            rec[4 + tid] = O;
            if (tid == 0) {
                rec[0] = M;
                rec[1] = Lsum;
            }
        }
        __syncthreads();
    }
}

}  // namespace

// Merge of the partial states of one row-head, in fixed order: selected entries ascending by
// entry index, then window spans, each over its sub-tiles.  One wave per row-head.
template <int D>
__global__ void __launch_bounds__(256) combine_kernel(const float *__restrict__ part, const int32_t *__restrict__ sel,
                                                      const int64_t *__restrict__ row_pos, float *__restrict__ out,
                                                      int64_t n_rowheads, int Hq, int S, int k, int W,
                                                      int64_t max_pos, int NW, int nsub, int TK) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t rh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (rh >= n_rowheads) return;
    int64_t t = row_pos[rh / Hq];
    t = t < 0 ? 0 : (t > max_pos ? max_pos : t);
    const int64_t w0 = window_start(t, S, W);
    const int64_t r = w0 / S;
    const int NE = k + NW;
    float M = kNegInf, Lsum = 0.f, O[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) O[i] = 0.f;
    auto merge = [&](int entry, int64_t lo, int64_t hi) {
        for (int sub = 0; sub < nsub && lo + (int64_t)sub * TK < hi; ++sub) {
            const float *rec = part + ((rh * NE + entry) * (int64_t)nsub + sub) * record_floats(D);
            const float m = rec[0], l = rec[1];
            if (m == kNegInf) continue;
            const float Mn = fmaxf(M, m);
            const float a = (M == kNegInf) ? 0.f : exp2f(M - Mn);
            const float b = exp2f(m - Mn);
            Lsum = Lsum * a + l * b;
#pragma unroll
            for (int i = 0; i < PER; ++i) O[i] = O[i] * a + rec[4 + lane + 64 * i] * b;
            M = Mn;
        }
    };
    for (int e = 0; e < k; ++e) {
        const int64_t j = sel[rh * k + e];
        if (j < 0 || j >= r) continue;
        merge(e, j * S, j * S + S);
    }
    for (int w = 0; w < NW; ++w) {
        const int64_t lo = w0 + (int64_t)w * S;
        if (lo > t) break;
        const int64_t hi = lo + S < t + 1 ? lo + S : t + 1;
        merge(k + w, lo, hi);
    }
    const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) out[rh * D + lane + 64 * i] = O[i] * inv;
}

hipError_t launch_combine(const RowArgs &a, const float *part, const int32_t *sel, float *out, int nsub, int TK,
                          hipStream_t st) {
    const int64_t n = a.n_rows * a.Hq;
    const int NW = max_window_spans(a.S, a.W);
    auto kern = a.d == 64 ? combine_kernel<64> : combine_kernel<128>;
    hipLaunchKernelGGL(kern, dim3((unsigned)ceil_div(n, 4)), dim3(256), 0, st, part, sel, a.row_pos, out, n, a.Hq, a.S,
                       a.k, a.W, a.max_pos, NW, nsub, TK);
    return hipGetLastError();
}

namespace {
template <typename T, int D>
int decode_tk() { return Lanes<T, D>::TK; }

int decode_sub_tile(const RowArgs &a) {
    if (a.dtype == RA_BF16) return a.d == 64 ? decode_tk<uint16_t, 64>() : decode_tk<uint16_t, 128>();
    return a.d == 64 ? decode_tk<float, 64>() : decode_tk<float, 128>();
}

template <typename T, int D>
hipError_t decode_launch(const RowArgs &a, const void *K, const void *V, const int32_t *sel, void *ws,
                         hipStream_t st) {
    using L = Lanes<T, D>;
    const int NW = max_window_spans(a.S, a.W);
    const int n_slots = a.G * a.k + NW;
    const int nsub = (int)ceil_div(a.S, L::TK);
    const int64_t blocks = a.n_rows * a.Hkv * n_slots * nsub;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    hipLaunchKernelGGL((decode_attn<T, D>), dim3((unsigned)blocks), dim3(256), 0, st, (const T *)a.q, a.row_seq,
                       a.row_pos, (const T *)K, (const T *)V, sel, (float *)ws, a.Hq, a.Hkv, a.G, a.S, a.k, a.W, a.B,
                       a.cap, a.max_pos, n_slots, NW, nsub, scale_log2);
    return hipGetLastError();
}
}  // namespace

size_t decode_workspace_bytes(const RowArgs &a) {
    const int NW = max_window_spans(a.S, a.W);
    const int64_t nsub = ceil_div(a.S, decode_sub_tile(a));
    return (size_t)(a.n_rows * a.Hq * (a.k + NW) * nsub * record_floats(a.d) * sizeof(float));
}

hipError_t launch_decode(const RowArgs &a, const void *K, const void *V, const int32_t *sel, float *out, void *ws,
                         hipStream_t st) {
    if (a.n_rows == 0) return hipSuccess;
    hipError_t e;
    if (a.dtype == RA_BF16)
        e = a.d == 64 ? decode_launch<uint16_t, 64>(a, K, V, sel, ws, st) : decode_launch<uint16_t, 128>(a, K, V, sel, ws, st);
    else
        e = a.d == 64 ? decode_launch<float, 64>(a, K, V, sel, ws, st) : decode_launch<float, 128>(a, K, V, sel, ws, st);
    if (e != hipSuccess) return e;
    const int TK = decode_sub_tile(a);
    return launch_combine(a, (const float *)ws, sel, out, (int)ceil_div(a.S, TK), TK, st);
}

}  // namespace ra
