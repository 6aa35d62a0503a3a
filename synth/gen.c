/*
 * Seeded, position-addressable synthetic inputs for content-routed sparse attention.
 *
 * This file generates random numbers and nothing else: it holds none of the method's
 * arithmetic (no summaries, scores, selection or attention).  Both the CPU oracle's
 * tests and the GPU path's tests/bench read the buffers it fills, so they always see
 * identical inputs.
 *
 * Uniforms: a counter-based stream.  The 64-bit counter x = (seed XOR stream*phi) + index
 * is passed through the SplitMix64 finaliser (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), and the top 53 bits give u in [0, 1).
 * Normals: the Box-Muller transform (Box and Muller, 1958) of the uniform pair at the
 * even/odd counters (2i, 2i+1); the even element takes the cosine branch, the odd one the
 * sine branch.  Values are computed in double, rounded to fp32 (RN), and for bf16 outputs
 * rounded fp32 -> bf16 with round-to-nearest-even.
 *
 * Element counter layout: idx = (((seq << 8 | head) << 36 | pos) << 8) | e, so any range
 * of positions regenerates identically regardless of how a buffer is chunked
 * (seq < 4096, head < 256, pos < 2^36, e < 256).
 *
 * Streams: 1 = queries, 2 = key noise, 3 = values, 4 = per-span key offset directions,
 * 5 = ragged sequence lengths.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t splitmix64_finalise(uint64_t x) {
    uint64_t z = x + GOLDEN;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline double uniform01(uint64_t seed, uint32_t stream, uint64_t idx) {
    uint64_t x = (seed ^ ((uint64_t)stream * GOLDEN)) + idx;
    return (double)(splitmix64_finalise(x) >> 11) * 0x1.0p-53;
}

static inline uint64_t elem_index(int seq, int head, int64_t pos, int e) {
    return ((((uint64_t)seq << 8 | (uint64_t)head) << 36 | (uint64_t)pos) << 8) | (uint64_t)e;
}

/* Normal pair for counters (base, base|1), base even. */
static inline void normal_pair(uint64_t seed, uint32_t stream, uint64_t base, double *z0, double *z1) {
    double u1 = uniform01(seed, stream, base);
    double u2 = uniform01(seed, stream, base | 1u);
    double rad = sqrt(-2.0 * log(1.0 - u1)); /* 1-u1 in (0, 1] */
    double ang = 6.283185307179586476925286766559 * u2;
    *z0 = rad * cos(ang);
    *z1 = rad * sin(ang);
}

double synth_uniform(uint64_t seed, uint32_t stream, uint64_t idx) { return uniform01(seed, stream, idx); }

double synth_normal(uint64_t seed, uint32_t stream, uint64_t idx) {
    double z0, z1;
    normal_pair(seed, stream, idx & ~(uint64_t)1, &z0, &z1);
    return (idx & 1) ? z1 : z0;
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Direction of norm `norm` for (seq, head, span): d normals from stream 4, rescaled. */
static void offset_direction(uint64_t seed, int seq, int head, int64_t span, int d, double norm, double *u) {
    double ss = 0.0;
    for (int e = 0; e < d; e += 2) {
        double z0, z1;
        normal_pair(seed, 4, elem_index(seq, head, span, e), &z0, &z1);
        u[e] = z0;
        if (e + 1 < d) u[e + 1] = z1;
    }
    for (int e = 0; e < d; ++e) ss += u[e] * u[e];
    double s = norm / sqrt(ss);
    for (int e = 0; e < d; ++e) u[e] *= s;
}

/*
 * Fill `out` with normals for heads [head0, head0+nheads) and positions [pos0, pos0+npos).
 *   dtype 0: fp32, dtype 1: bf16 bit patterns (uint16).
 *   layout 0: out[h][p][e] (a KV-cache slab), layout 1: out[p][h][e] (query rows).
 *   offset_norm > 0 adds, to every element of position p, the direction of span p/span_size
 *   (scaled to that norm) before rounding: the "keys with a per-span offset" recipe.
 */
void synth_fill(void *out, int dtype, uint64_t seed, uint32_t stream, int seq, int head0, int nheads,
                int64_t pos0, int64_t npos, int d, int layout, int64_t span_size, double offset_norm) {
    const int64_t rows = (int64_t)nheads * npos;
#pragma omp parallel
    {
        double dir[256];
        int64_t dir_span = -1;
        int dir_head = -1;
        double vals[256];
#pragma omp for schedule(static)
        for (int64_t rI = 0; rI < rows; ++rI) {
            int hl = (int)(rI / npos);
            int64_t pl = rI % npos;
            int head = head0 + hl;
            int64_t pos = pos0 + pl;
            for (int e = 0; e < d; e += 2) {
                double z0, z1;
                normal_pair(seed, stream, elem_index(seq, head, pos, e), &z0, &z1);
                vals[e] = z0;
                if (e + 1 < d) vals[e + 1] = z1;
            }
            if (offset_norm > 0.0) {
                int64_t span = pos / span_size;
                if (span != dir_span || head != dir_head) {
                    offset_direction(seed, seq, head, span, d, offset_norm, dir);
                    dir_span = span;
                    dir_head = head;
                }
                for (int e = 0; e < d; ++e) vals[e] += dir[e];
            }
            int64_t row = layout == 0 ? ((int64_t)hl * npos + pl) : (pl * nheads + hl);
            if (dtype == 0) {
                float *o = (float *)out + row * d;
                for (int e = 0; e < d; ++e) o[e] = (float)vals[e];
            } else {
                uint16_t *o = (uint16_t *)out + row * d;
                for (int e = 0; e < d; ++e) o[e] = f32_to_bf16_rne((float)vals[e]);
            }
        }
    }
}

/* Ragged lengths: out[b] = lo + floor(u * (hi - lo + 1)), u from stream 5 at counter b. */
void synth_lengths(int64_t *out, uint64_t seed, int n, int64_t lo, int64_t hi) {
    for (int b = 0; b < n; ++b) {
        int64_t span = hi - lo + 1;
        int64_t v = lo + (int64_t)floor(uniform01(seed, 5, (uint64_t)b) * (double)span);
        out[b] = v > hi ? hi : v;
    }
}
