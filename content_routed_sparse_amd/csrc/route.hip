// Routing scores: every (row, query head) scores every routable span summary of its sequence
// (release post, "Key idea": score the O(L^0.5) candidate spans).  s_j = q . kappa(mean_j).
//
// Two kernels:
//  * route_mfma (bf16 inputs, many rows): a dense [row-heads x spans] contraction on bf16 MFMA
//    (v_mfma_f32_16x16x32_bf16), fp32 accumulation.  A block owns 64 row-heads of one kv head
//    (4 waves x 16) and a chunk of spans; span summaries are rounded to bf16 once per block and
//    staged in LDS, shared by the 4 waves.  Rows of different sequences in one tile are handled
//    in successive passes (one pass in the usual single-sequence chunk).
//  * route_valu (fp32 inputs, or few rows as in decode): fp32 FMA; lanes split each summary
//    row, 8 query heads per pass, butterfly reduction over the lanes of a row.
#include "common.h"
#include "kernels.h"
#include "wave_ops.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Few rows (decode) or fp32 inputs: a block scores 64 spans of one (row, kv head) for all the
// kv head's query heads.  Lanes split each fp32 summary row (8 elements per lane, LPR lanes per
// row, coalesced 32-byte loads); each lane forms partial dot products for 8 heads at once, and a
// butterfly reduce-scatter over the LPR lanes leaves 2 finished scores per lane.
template <typename T, int D>
__global__ void __launch_bounds__(256) route_valu(const T *__restrict__ q, const int32_t *__restrict__ row_seq,
                                                  const int64_t *__restrict__ row_pos,
                                                  const float *__restrict__ mean, float *__restrict__ scores,
                                                  int64_t stride, int Hq, int Hkv, int G, int S, int W, int B,
                                                  int64_t max_spans, int64_t max_pos) {
    constexpr int LPR = D / 8, RPI = 64 / LPR, STEPS = 16 / RPI, N = STEPS * 8, KEEP = N / LPR;
    // all kernel arguments in one round trip (otherwise some are fetched only where first used)
    asm volatile("" ::"s"(q), "s"(row_seq), "s"(row_pos), "s"(mean), "s"(scores), "s"(stride), "s"(Hq), "s"(Hkv),
                 "s"(G), "s"(S), "s"(W), "s"(B), "s"(max_spans), "s"(max_pos));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane % LPR, rr = lane / LPR;
    const int rg = blockIdx.x;
    const int64_t row = rg / Hkv;
    const int g = rg % Hkv;
    constexpr int QV = sizeof(T) == 2 ? 1 : 2;  // 16-byte pieces per head slice of 8 elements
    uint4 qraw[8][QV];
    auto load_q = [&](int hc) {
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            const int hh = hc + h < G ? hc + h : G - 1;  // clamped head; zeroed later if past G
            const uint4 *qp = reinterpret_cast<const uint4 *>(q + (row * Hq + g * G + hh) * D + c * 8);
#pragma unroll
            for (int v = 0; v < QV; ++v) qraw[h][v] = qp[v];
        }
    };
    // the row's position and sequence together with the first 8 heads' queries (which do not
    // depend on them): one round trip
    const int64_t t_raw = row_pos[row];
    const int seq_raw = row_seq[row];
    load_q(0);
    asm volatile("" ::"s"(t_raw), "s"(seq_raw));
    const int64_t t = t_raw < 0 ? 0 : (t_raw > max_pos ? max_pos : t_raw);
    const int seq = seq_raw < 0 ? 0 : (seq_raw >= B ? B - 1 : seq_raw);
    const int64_t r = num_routable(t, S, W);
    const int64_t jw = (int64_t)blockIdx.y * 64 + wave * 16;  // this wave's first span
    if (jw >= r) return;
    const float *mbase = mean + ((int64_t)seq * Hkv + g) * max_spans * D;
    // then every summary load of the wave, issued before any use and pinned there
    float4 mraw[STEPS][2];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        int64_t n = jw + s * RPI + rr;
        n = n < r ? n : r - 1;
        mraw[s][0] = *reinterpret_cast<const float4 *>(mbase + n * D + c * 8);
        mraw[s][1] = *reinterpret_cast<const float4 *>(mbase + n * D + c * 8 + 4);
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
#pragma unroll
        for (int v = 0; v < 2; ++v)
            asm volatile("" : "+v"(mraw[s][v].x), "+v"(mraw[s][v].y), "+v"(mraw[s][v].z), "+v"(mraw[s][v].w));
    float mv[STEPS][8];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        const float f[8] = {mraw[s][0].x, mraw[s][0].y, mraw[s][0].z, mraw[s][0].w,
                            mraw[s][1].x, mraw[s][1].y, mraw[s][1].z, mraw[s][1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) mv[s][e] = sizeof(T) == 2 ? round_bf16(f[e]) : f[e];
    }
    for (int hc = 0; hc < G; hc += 8) {
        if (hc > 0) load_q(hc);
        float acc[N];
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            float qf[8];
            if constexpr (sizeof(T) == 2) {
                const uint32_t w[4] = {qraw[h][0].x, qraw[h][0].y, qraw[h][0].z, qraw[h][0].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    qf[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
                    qf[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
                }
            } else {
                const uint32_t w[8] = {qraw[h][0].x, qraw[h][0].y, qraw[h][0].z, qraw[h][0].w,
                                       qraw[h][1].x, qraw[h][1].y, qraw[h][1].z, qraw[h][1].w};
#pragma unroll
                for (int i = 0; i < 8; ++i) qf[i] = __uint_as_float(w[i]);
            }
            if (hc + h >= G) {
#pragma unroll
                for (int e = 0; e < 8; ++e) qf[e] = 0.f;
            }
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) d = fmaf(qf[e], mv[s][e], d);
                acc[s * 8 + h] = d;
            }
        }
        ReduceScatter<N, ilog2(LPR), LPR / 2>::run(acc, lane);
#pragma unroll
        for (int i = 0; i < KEEP; ++i) {
            const int v = c * KEEP + i;
            const int s = v / 8, h = v % 8;
            const int64_t n = jw + s * RPI + rr;
            if (n < r && hc + h < G) scores[(row * Hq + g * G + hc + h) * stride + n] = acc[i];
        }
    }
}

constexpr int kRowTile = 64;    // row-heads per block (4 waves x 16)
constexpr int kSpanBlock = 64;  // spans staged per LDS step
constexpr int kSpanChunk = 256; // spans per block (grid y)

template <int D>
__global__ void __launch_bounds__(256) route_mfma(const uint16_t *__restrict__ q, const int32_t *__restrict__ row_seq,
                                                  const int64_t *__restrict__ row_pos,
                                                  const float *__restrict__ mean, float *__restrict__ scores,
                                                  int64_t stride, int64_t n_rows, int Hq, int Hkv, int G, int S,
                                                  int W, int B, int64_t max_spans, int64_t max_pos,
                                                  int64_t tiles_per_head) {
    constexpr int KS = D / 32;          // k-steps of 32
    constexpr int LDS_ROW = D + 8;      // bf16 elements per staged span row (padding vs bank conflicts)
    __shared__ uint16_t bstage[kSpanBlock * LDS_ROW];
    __shared__ int tile_seq[kRowTile];
    __shared__ int pass_seq;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = (int)(blockIdx.x / tiles_per_head);
    const int64_t rh0 = (blockIdx.x % tiles_per_head) * kRowTile;
    const int64_t jc0 = (int64_t)blockIdx.y * kSpanChunk;
    const int64_t n_rh = n_rows * G;

    // sequence of each row-head of the tile (-1 when past the last row)
    if (tid < kRowTile) {
        const int64_t rh = rh0 + tid;
        int s = -1;
        if (rh < n_rh) {
            s = row_seq[rh / G];
            s = s < 0 ? 0 : (s >= B ? B - 1 : s);
        }
        tile_seq[tid] = s;
    }
    // this lane's A row (row-head) and its routable count
    const int64_t my_rh = rh0 + wave * 16 + (lane & 15);
    const bool rh_ok = my_rh < n_rh;
    const int64_t my_row = rh_ok ? my_rh / G : 0;
    const int my_h = rh_ok ? (int)(my_rh % G) : 0;
    bf16x8 a[KS];
    {
        const uint16_t *qp = q + (my_row * Hq + g * G + my_h) * D + 8 * (lane >> 4);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 raw = rh_ok ? *reinterpret_cast<const uint4 *>(qp + 32 * ks) : make_uint4(0, 0, 0, 0);
            a[ks] = __builtin_bit_cast(bf16x8, raw);
        }
    }
    // rows of the 4 outputs this lane holds: D[4*(lane/16)+i][lane%16]
    int64_t out_row[4], out_r[4];
    int out_h[4], out_seq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t rh = rh0 + wave * 16 + 4 * (lane >> 4) + i;
        out_row[i] = rh < n_rh ? rh / G : -1;
        out_h[i] = rh < n_rh ? (int)(rh % G) : 0;
        int64_t t = 0;
        if (out_row[i] >= 0) {
            t = row_pos[out_row[i]];
            t = t < 0 ? 0 : (t > max_pos ? max_pos : t);
        }
        out_r[i] = out_row[i] >= 0 ? num_routable(t, S, W) : 0;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) out_seq[i] = out_row[i] >= 0 ? tile_seq[wave * 16 + 4 * (lane >> 4) + i] : -1;
    const int my_seq = rh_ok ? tile_seq[wave * 16 + (lane & 15)] : -1;

    // largest routable count in the tile bounds the span loop
    int64_t rmax = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) rmax = out_r[i] > rmax ? out_r[i] : rmax;
    for (int off = 32; off > 0; off >>= 1) {
        const int64_t o = __shfl_xor(rmax, off);
        rmax = o > rmax ? o : rmax;
    }
    __shared__ int64_t rmax_w[4];
    if (lane == 0) rmax_w[wave] = rmax;
    __syncthreads();
    rmax = rmax_w[0];
    for (int w = 1; w < 4; ++w) rmax = rmax_w[w] > rmax ? rmax_w[w] : rmax;
    int64_t jend = jc0 + kSpanChunk;
    if (jend > rmax) jend = rmax;
    if (jc0 >= jend) return;

    int done_below = -1;  // passes go over the distinct sequences of the tile in increasing order
    while (true) {
        __syncthreads();
        if (tid == 0) {
            int nxt = 0x7fffffff;
            for (int x = 0; x < kRowTile; ++x)
                if (tile_seq[x] > done_below && tile_seq[x] < nxt) nxt = tile_seq[x];
            pass_seq = nxt;
        }
        __syncthreads();
        const int seq = pass_seq;
        if (seq == 0x7fffffff) break;
        done_below = seq;
        const bf16x8 zero8 = {};
        bf16x8 aa[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) aa[ks] = (my_seq == seq) ? a[ks] : zero8;
        const float *mseq = mean + ((int64_t)seq * Hkv + g) * max_spans * D;
        for (int64_t jb = jc0; jb < jend; jb += kSpanBlock) {
            // stage kappa(mean) of spans [jb, jb+64) as bf16
            for (int x = tid; x < kSpanBlock * (D / 4); x += 256) {
                const int n = x / (D / 4), e4 = (x % (D / 4)) * 4;
                const int64_t j = jb + n;
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (j < jend) v = *reinterpret_cast<const float4 *>(mseq + j * D + e4);
                const uint32_t lo = f32_to_bf16_bits(v.x) | (f32_to_bf16_bits(v.y) << 16);
                const uint32_t hi = f32_to_bf16_bits(v.z) | (f32_to_bf16_bits(v.w) << 16);
                *reinterpret_cast<uint2 *>(&bstage[n * LDS_ROW + e4]) = make_uint2(lo, hi);
            }
            __syncthreads();
#pragma unroll
            for (int nb = 0; nb < kSpanBlock / 16; ++nb) {
                const uint16_t *bp = &bstage[(nb * 16 + (lane & 15)) * LDS_ROW + 8 * (lane >> 4)];
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const uint4 raw = *reinterpret_cast<const uint4 *>(bp + 32 * ks);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aa[ks], __builtin_bit_cast(bf16x8, raw), acc, 0, 0, 0);
                }
                const int64_t j = jb + nb * 16 + (lane & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (out_seq[i] == seq && j < out_r[i] && j < jend)
                        scores[(out_row[i] * Hq + g * G + out_h[i]) * stride + j] = acc[i];
                }
            }
            __syncthreads();
        }
    }
}

template <typename T, int D>
hipError_t route_valu_launch(const RowArgs &a, const float *mean, float *scores, int64_t stride, hipStream_t st) {
    const int64_t rmax = num_routable(a.max_pos, a.S, a.W);
    if (rmax == 0 || a.n_rows == 0) return hipSuccess;
    dim3 grid((unsigned)(a.n_rows * a.Hkv), (unsigned)ceil_div(rmax, 64));
    hipLaunchKernelGGL((route_valu<T, D>), grid, dim3(256), 0, st, (const T *)a.q, a.row_seq, a.row_pos, mean, scores,
                       stride, a.Hq, a.Hkv, a.G, a.S, a.W, a.B, a.max_spans, a.max_pos);
    return hipGetLastError();
}

template <int D>
hipError_t route_mfma_launch(const RowArgs &a, const float *mean, float *scores, int64_t stride, hipStream_t st) {
    const int64_t rmax = num_routable(a.max_pos, a.S, a.W);
    if (rmax == 0 || a.n_rows == 0) return hipSuccess;
    const int64_t tiles = ceil_div(a.n_rows * a.G, kRowTile);
    dim3 grid((unsigned)(tiles * a.Hkv), (unsigned)ceil_div(rmax, kSpanChunk));
    hipLaunchKernelGGL((route_mfma<D>), grid, dim3(256), 0, st, (const uint16_t *)a.q, a.row_seq, a.row_pos, mean,
                       scores, stride, a.n_rows, a.Hq, a.Hkv, a.G, a.S, a.W, a.B, a.max_spans, a.max_pos, tiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const RowArgs &a, const float *mean, float *scores, int64_t stride, hipStream_t st) {
    if (a.dtype == RA_BF16) {
        if (a.n_rows * a.G >= 256) return a.d == 64 ? route_mfma_launch<64>(a, mean, scores, stride, st)
                                                    : route_mfma_launch<128>(a, mean, scores, stride, st);
        return a.d == 64 ? route_valu_launch<uint16_t, 64>(a, mean, scores, stride, st)
                         : route_valu_launch<uint16_t, 128>(a, mean, scores, stride, st);
    }
    return a.d == 64 ? route_valu_launch<float, 64>(a, mean, scores, stride, st)
                     : route_valu_launch<float, 128>(a, mean, scores, stride, st);
}

}  // namespace ra
