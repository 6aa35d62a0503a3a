// CPU oracle of content-routed sparse attention, in plain C++ -- TEST INFRASTRUCTURE ONLY.
//
// Only the tests, the smoke check and the benchmark's CPU-baseline leg load this library
// (oracle/liboracle.so, through oracle/cpp.py).  The GPU library never calls it, and it shares
// no code, header, table or helper with the GPU path.
//
// Source of the definition.  The release post "Experimental model with subquadratic attention:
// 100 tok/s @ 1M context, 76 tok/s @ 10M context (30B model, single GPU)", section "Key idea":
// the context is searched as O(L^0.5) candidate spans; each query scores the spans, keeps the
// top k and attends token by token inside the chosen spans, so any token stays reachable and
// the total cost is O(L^(3/2)).  The post prints no formula; the points it leaves open are
// fixed by the same readings as the numpy oracle (oracle/routed_attention.py):
//
//   R1  span j = positions [jS, jS+S); its summary is the fp32 mean of its keys: an fp32 running
//       sum in token order, divided by S (IEEE division) when the span completes.
//   R2  window of a query at t: [w0, t] with w0 = S * floor(max(0, t-W+1) / S); routable spans
//       are j < r(t) = w0 / S (complete and before the window).
//   R3  each (token, query head) row routes on its own; query head hq reads kv head hq / G.
//   R4  score s_j = q . kappa(mean_j), no 1/sqrt(d); kappa rounds to bf16 (nearest, ties to
//       even) for bf16 inputs and is the identity for fp32 inputs.
//   R5  keep m = min(k, r) spans by (score descending, index ascending); list them ascending,
//       pad with -1.
//   R6  exact softmax attention with scale 1/sqrt(d) over the window and the selected spans.
//
// Arithmetic: inputs (bf16 bit patterns or fp32) are widened exactly; summaries are fp32 as R1
// says; everything after them runs in double, one term at a time in index order.  No blocking,
// no vector code, no fast-math: a reader can check each function against the list above.
// Work is spread over std::threads, one (query row, query head) task at a time.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// ------------------------------------------------------------------------------------- inputs
// A bf16 value is the upper half of the fp32 with the same bits.
float bf16_bits_to_float(uint16_t bits) {
    const uint32_t u = (uint32_t)bits << 16;
    float f;
    std::memcpy(&f, &u, sizeof f);
    return f;
}

// Element i of a stored array (bf16 bit patterns or fp32), exactly, as float.
float stored(const void *base, int is_bf16, int64_t i) {
    if (is_bf16) return bf16_bits_to_float(static_cast<const uint16_t *>(base)[i]);
    return static_cast<const float *>(base)[i];
}

// kappa of R4 for bf16 inputs: the nearest number with an 8-bit significand, ties to even.
// For |x| in [2^(e-1), 2^e) the bf16 numbers are spaced 2^(e-8), and never closer than the
// smallest subnormal spacing 2^-133.  std::nearbyint rounds half-way cases to even in the
// default rounding mode.  Values past the largest bf16 round to infinity as the format does.
float kappa_bf16(float x) {
    if (!std::isfinite(x) || x == 0.0f) return x;
    int e = 0;
    std::frexp((double)x, &e);
    const double spacing = std::ldexp(1.0, std::max(e - 8, -133));
    return (float)(std::nearbyint((double)x / spacing) * spacing);
}

// ------------------------------------------------------------------------------- spans (R2)
int64_t window_start(int64_t t, int64_t S, int64_t W) {
    const int64_t a = t - W + 1 > 0 ? t - W + 1 : 0;
    return S * (a / S);
}

int64_t num_routable(int64_t t, int64_t S, int64_t W) { return window_start(t, S, W) / S; }

// --------------------------------------------------------------------------- thread helper
// Runs body(i) for i in [0, n) on `threads` threads (0: every hardware thread).
template <typename F>
void parallel_for(int64_t n, int threads, F body) {
    int nt = threads > 0 ? threads : (int)std::thread::hardware_concurrency();
    if (nt < 1) nt = 1;
    if (nt > n) nt = (int)(n > 0 ? n : 1);
    std::atomic<int64_t> next{0};
    auto worker = [&]() {
        for (int64_t i = next.fetch_add(1); i < n; i = next.fetch_add(1)) body(i);
    };
    if (nt == 1) {
        worker();
        return;
    }
    std::vector<std::thread> pool;
    for (int i = 0; i < nt; ++i) pool.emplace_back(worker);
    for (auto &th : pool) th.join();
}

// ---------------------------------------------------------------------- summaries (R1)
// Tokens [p0, p1) of kv head h, all inside one span, added to `sum` one at a time in token
// order with fp32 additions; if p1 closes the span, mean = sum / S and the sum restarts at 0.
void add_tokens(const void *keys, int is_bf16, int64_t cap, int64_t d, int64_t h, int64_t p0, int64_t p1,
                int64_t S, float *sum, float *means, int64_t max_spans) {
    for (int64_t p = p0; p < p1; ++p) {
        for (int64_t e = 0; e < d; ++e) {
            const float kv = stored(keys, is_bf16, (h * cap + p) * d + e);
            sum[e] = sum[e] + kv;  // one fp32 addition, rounded to nearest
        }
        if ((p + 1) % S == 0) {
            const int64_t j = (p + 1) / S - 1;
            for (int64_t e = 0; e < d; ++e) {
                if (j < max_spans) means[(h * max_spans + j) * d + e] = sum[e] / (float)S;
                sum[e] = 0.0f;
            }
        }
    }
}

}  // namespace

extern "C" {

// Appends tokens [old_len, new_len) of one sequence to its summaries, in place.
// keys: [hkv][cap][d] stored values; means: [hkv][max_spans][d] fp32; run_sum: [hkv][d] fp32
// (the sum of the open span's tokens so far).  Each span's additions start from its first
// token in position order; spans are independent, so they are computed on separate threads.
void oracle_summary_update(const void *keys, int is_bf16, int64_t hkv, int64_t cap, int64_t d, float *means,
                           int64_t max_spans, float *run_sum, int64_t old_len, int64_t new_len, int64_t S,
                           int threads) {
    if (new_len <= old_len) return;
    const int64_t j_first = old_len / S, j_last = (new_len - 1) / S;
    const int64_t nspan = j_last - j_first + 1;
    // the running sums as they were before the update (the last span's task overwrites them)
    const std::vector<float> run_before(run_sum, run_sum + hkv * d);
    parallel_for(hkv * nspan, threads, [&](int64_t task) {
        const int64_t h = task / nspan, j = j_first + task % nspan;
        const int64_t p0 = std::max(old_len, j * S), p1 = std::min(new_len, (j + 1) * S);
        // the open span continues the running sum; a span that starts inside the range starts at 0
        std::vector<float> sum(d, 0.0f);
        if (p0 == old_len)
            for (int64_t e = 0; e < d; ++e) sum[e] = run_before[h * d + e];
        add_tokens(keys, is_bf16, cap, d, h, p0, p1, S, sum.data(), means, max_spans);
        if (p1 == new_len)  // the last span's sum is the new running sum (0 if it just closed)
            for (int64_t e = 0; e < d; ++e) run_sum[h * d + e] = sum[e];
    });
}

// kappa on n fp32 values (exported for the pins).
void oracle_kappa_bf16(const float *x, float *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = kappa_bf16(x[i]);
}

// Widening of n stored values to double (exported for the pins).
void oracle_widen(const void *x, int is_bf16, double *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = (double)stored(x, is_bf16, i);
}

int64_t oracle_window_start(int64_t t, int64_t S, int64_t W) { return window_start(t, S, W); }
int64_t oracle_num_routable(int64_t t, int64_t S, int64_t W) { return num_routable(t, S, W); }

// R4: s_j = sum_e q_e kappa(mean_je) for j < r, in double, e in increasing order.
// q: d doubles; means_g: [>= r][d] fp32 of the row's kv head.
void oracle_route_scores(const double *q, const float *means_g, int64_t r, int64_t d, int is_bf16, double *out) {
    for (int64_t j = 0; j < r; ++j) {
        double s = 0.0;
        for (int64_t e = 0; e < d; ++e) {
            const float m = means_g[j * d + e];
            s += q[e] * (double)(is_bf16 ? kappa_bf16(m) : m);
        }
        out[j] = s;
    }
}

// R5: the first m = min(k, r) spans of the order (score descending, index ascending), listed
// ascending, padded with -1 to k entries.  An exhaustive sort on that key.
void oracle_select(const double *scores, int64_t r, int64_t k, int64_t *out) {
    std::vector<int64_t> order(r);
    for (int64_t j = 0; j < r; ++j) order[j] = j;
    std::sort(order.begin(), order.end(), [&](int64_t a, int64_t b) {
        if (scores[a] != scores[b]) return scores[a] > scores[b];
        return a < b;
    });
    const int64_t m = std::min(k, r);
    std::vector<int64_t> kept(order.begin(), order.begin() + m);
    std::sort(kept.begin(), kept.end());
    for (int64_t i = 0; i < k; ++i) out[i] = i < m ? kept[i] : -1;
}

// R6 over the given positions of kv head g: z_p = q . k_p / sqrt(d); M = max z;
// w_p = exp(z_p - M) / sum exp(z - M); o = sum_p w_p v_p.  Returns sum_p w_p.
double oracle_attend(const double *q, const void *keys, const void *values, int is_bf16, int64_t cap, int64_t d,
                     int64_t g, const int64_t *pos, int64_t npos, double *out) {
    std::vector<double> z(npos);
    const double inv_sqrt_d = 1.0 / std::sqrt((double)d);
    double zmax = -INFINITY;
    for (int64_t i = 0; i < npos; ++i) {
        double dot = 0.0;
        for (int64_t e = 0; e < d; ++e) dot += q[e] * (double)stored(keys, is_bf16, (g * cap + pos[i]) * d + e);
        z[i] = dot * inv_sqrt_d;
        zmax = std::max(zmax, z[i]);
    }
    double denom = 0.0;
    for (int64_t i = 0; i < npos; ++i) denom += std::exp(z[i] - zmax);
    for (int64_t e = 0; e < d; ++e) out[e] = 0.0;
    double wsum = 0.0;
    for (int64_t i = 0; i < npos; ++i) {
        const double w = std::exp(z[i] - zmax) / denom;
        wsum += w;
        for (int64_t e = 0; e < d; ++e) out[e] += w * (double)stored(values, is_bf16, (g * cap + pos[i]) * d + e);
    }
    return wsum;
}

// Whole rows of one sequence.  Task i is query vector q[i] ([d] stored values) of query head
// head[i] at position pos[i]:
//   scores (R4) -> own selection (R5) -> attended set: window [w0, t] plus the spans of the
//   selection in use (the task's own, or sel_in[i] if sel_in is given: entries outside [0, r)
//   and repeats are skipped) -> attention (R6).
// dense != 0: attention over [0, t] instead (the k = all special case), no routing.
// Outputs per task: out[i][d] (double), sel_out[i][k], wsum[i], n_att[i], and the r scores into
// scores[i][score_stride] when scores is not null (r <= score_stride is the caller's duty).
// keys, values: [hkv][cap][d] stored; means: [hkv][max_spans][d] fp32.  Returns 0, or -1 when
// some task's position lies outside [0, cap) or its head outside [0, hq).
int oracle_rows(int64_t hq, int64_t hkv, int64_t d, int64_t S, int64_t k, int64_t W, int is_bf16,
                const void *keys, const void *values, int64_t cap, const float *means, int64_t max_spans,
                const void *q, const int32_t *head, const int64_t *pos, int64_t n, const int64_t *sel_in, int dense,
                double *out, int64_t *sel_out, double *wsum, int64_t *n_att, double *scores, int64_t score_stride,
                int threads) {
    for (int64_t i = 0; i < n; ++i)
        if (pos[i] < 0 || pos[i] >= cap || head[i] < 0 || head[i] >= hq) return -1;
    const int64_t G = hq / hkv;
    parallel_for(n, threads, [&](int64_t i) {
        const int64_t t = pos[i], g = head[i] / G;
        std::vector<double> qd(d);
        for (int64_t e = 0; e < d; ++e) qd[e] = (double)stored(q, is_bf16, i * d + e);
        std::vector<int64_t> positions;
        int64_t *own = sel_out + i * k;
        for (int64_t x = 0; x < k; ++x) own[x] = -1;
        if (dense) {
            for (int64_t p = 0; p <= t; ++p) positions.push_back(p);
        } else {
            const int64_t r = num_routable(t, S, W);
            std::vector<double> s(r);
            oracle_route_scores(qd.data(), means + g * max_spans * d, r, d, is_bf16, s.data());
            if (scores)
                for (int64_t j = 0; j < r; ++j) scores[i * score_stride + j] = s[j];
            oracle_select(s.data(), r, k, own);
            std::vector<int64_t> use;
            const int64_t *src = sel_in ? sel_in + i * k : own;
            for (int64_t x = 0; x < k; ++x) {
                const int64_t j = src[x];
                if (j >= 0 && j < r && std::find(use.begin(), use.end(), j) == use.end()) use.push_back(j);
            }
            std::sort(use.begin(), use.end());
            for (int64_t j : use)
                for (int64_t p = j * S; p < j * S + S; ++p) positions.push_back(p);
            for (int64_t p = window_start(t, S, W); p <= t; ++p) positions.push_back(p);
        }
        n_att[i] = (int64_t)positions.size();
        wsum[i] = oracle_attend(qd.data(), keys, values, is_bf16, cap, d, g, positions.data(),
                                (int64_t)positions.size(), out + i * d);
    });
    return 0;
}

int oracle_hardware_threads(void) { return (int)std::thread::hardware_concurrency(); }

}  // extern "C"
