"""CPU oracle for content-routed sparse attention (numpy) -- TEST INFRASTRUCTURE ONLY.

This is the second of two implementations of the same definition; the plain C++ one
(routed_attention.cpp, loaded through oracle/cpp.py) is written apart from it, and the pins in
tests/test_oracle.py check both and compare them with each other.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  The GPU library never calls it, and it shares no code with the GPU path.

Source of the definition.  The release post "Experimental model with subquadratic attention:
100 tok/s @ 1M context, 76 tok/s @ 10M context (30B model, single GPU)" (a Korean re-post of the
LocalLLaMA announcement of superlinear-exp-v0.1), section "Key idea", describes the method: the
context is searched as O(L^0.5) candidate spans; each query scores the spans, keeps the top-k,
and then runs token-level attention inside the chosen spans; routing is content-dependent, so
any token can be selected, and the total cost is O(L^(3/2)).  The post gives no formula, so the
points it leaves open are fixed by the readings below (each is one plain choice; all are listed
with their reasons in the design notes of the repository):

  R1  A span is S consecutive cache positions [jS, jS+S); its summary is the fp32 mean of its
      keys, accumulated in token order in fp32 and scaled by 1/S (IEEE division).  Only complete
      spans have a summary.
  R2  The local window of a query at position t starts at the span boundary at or below
      t-W+1:  w0(t) = S * floor(max(0, t-W+1) / S); the window is [w0(t), t].  The routable spans
      are exactly the complete spans before the window, j < r(t) = w0(t) / S.  This makes every
      position <= t reachable, so "k = all spans" gives dense causal attention.
  R3  Each (token, query head) row routes on its own.  Query head hq reads kv head hq // G.
  R4  Routing score s_j = q . kappa(mean_j) with no 1/sqrt(d); kappa rounds the fp32 mean to
      bf16 (round to nearest, ties to even) for bf16 inputs and is the identity for fp32 inputs.
  R5  Selection keeps m = min(k, r) spans by the total order (score descending, index
      ascending); the result is listed in ascending span order and padded with -1.
  R6  Attention is exact softmax attention with scale 1/sqrt(d) over the union of the window and
      the selected spans' tokens.

Every floating-point step after the fp32 summaries runs in float64 (inputs are widened exactly).
"""
import math

import numpy as np

NO_SPAN = -1


# ---------------------------------------------------------------------------------------------
# Input widening and the bf16 rounding kappa (R4)
# ---------------------------------------------------------------------------------------------
def widen(x, is_bf16):
    """Exact value of stored inputs: bf16 bit patterns (uint16) or float32, as float64."""
    x = np.asarray(x)
    if is_bf16:
        assert x.dtype == np.uint16
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert x.dtype == np.float32
    return x.astype(np.float64)


def widen_f32(x, is_bf16):
    """Exact value of stored inputs as float32 (bf16 and fp32 both embed exactly)."""
    x = np.asarray(x)
    if is_bf16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    return x.astype(np.float32)


def round_to_bf16(x):
    """kappa for bf16 inputs: nearest value with an 8-bit significand, ties to even (R4).

    Written from the definition of the format rather than from bit tricks: for |x| in
    [2^(e-1), 2^e) the bf16 spacing is 2^(e-8) (never below the subnormal spacing 2^-133); the
    value is rounded to a multiple of that spacing with round-half-even (numpy.rint).
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    _, e = np.frexp(x)
    spacing = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(x / spacing) * spacing
    return r.astype(np.float32)


# ---------------------------------------------------------------------------------------------
# Spans, window, routable set (R1, R2)
# ---------------------------------------------------------------------------------------------
def window_start(t, S, W):
    """w0(t): the window start, rounded down to a span boundary (R2)."""
    return S * (max(0, t - W + 1) // S)


def num_routable(t, S, W):
    """r(t): spans 0..r-1 are complete and end before the window (R2)."""
    return window_start(t, S, W) // S


# ---------------------------------------------------------------------------------------------
# Span summaries (R1): fp32 running sum in token order, mean on completion
# ---------------------------------------------------------------------------------------------
def summary_update(keys_f32, means, run_sum, old_len, new_len, S):
    """Append tokens [old_len, new_len) of one sequence to its span summaries, in place.

    keys_f32: [Hkv][>=new_len][d] float32 key values.  means: [Hkv][max_spans][d] float32.
    run_sum: [Hkv][d] float32, the fp32 sum of the open span's tokens seen so far.
    Token p is added to run_sum with one fp32 addition (rounded to nearest); when p closes a
    span (p+1 is a multiple of S) the mean run_sum / S is written and run_sum restarts at 0.
    For long ranges the same additions are issued span by span, vectorised across spans:
    each span's sum still starts at 0 and adds its tokens in increasing position order.
    """
    assert keys_f32.dtype == np.float32 and means.dtype == np.float32 and run_sum.dtype == np.float32
    p = old_len
    S32 = np.float32(S)
    # finish the open span token by token
    while p < new_len and (p % S != 0 or new_len - p < S):
        run_sum[:] = run_sum + keys_f32[:, p, :]
        if (p + 1) % S == 0:
            means[:, (p + 1) // S - 1, :] = run_sum / S32
            run_sum[:] = 0
        p += 1
    # whole spans [p, p + n*S): fresh sums, tokens added in order, all spans at once
    n = (new_len - p) // S
    if n > 0:
        j0 = p // S
        block = keys_f32[:, p:p + n * S, :].reshape(keys_f32.shape[0], n, S, keys_f32.shape[2])
        acc = np.zeros((keys_f32.shape[0], n, keys_f32.shape[2]), dtype=np.float32)
        for i in range(S):
            acc += block[:, :, i, :]
        means[:, j0:j0 + n, :] = acc / S32
        p += n * S
    # trailing partial span
    while p < new_len:
        run_sum[:] = run_sum + keys_f32[:, p, :]
        p += 1
    return means, run_sum


def summaries(keys_f32, length, S, max_spans=None):
    """One-shot summaries of a cache of `length` tokens: (means, run_sum)."""
    hkv, _, d = keys_f32.shape
    if max_spans is None:
        max_spans = length // S
    means = np.zeros((hkv, max_spans, d), dtype=np.float32)
    run_sum = np.zeros((hkv, d), dtype=np.float32)
    return summary_update(keys_f32, means, run_sum, 0, length, S)


# ---------------------------------------------------------------------------------------------
# Routing scores (R4) and selection (R5)
# ---------------------------------------------------------------------------------------------
def route_scores(q, means_g, r, is_bf16):
    """s_j = sum_e q_e * kappa(mean_j)_e for j < r, accumulated in float64 (no 1/sqrt(d))."""
    m = means_g[:r]
    if is_bf16:
        m = round_to_bf16(m)
    return m.astype(np.float64) @ np.asarray(q, dtype=np.float64)


def select_spans(scores, k):
    """Top m = min(k, r) spans by (score desc, index asc); ascending ids padded with -1 to k."""
    r = len(scores)
    m = min(k, r)
    idx = np.arange(r)
    order = np.lexsort((idx, -np.asarray(scores, dtype=np.float64)))  # primary: -score, then index
    chosen = np.sort(order[:m])
    out = np.full(k, NO_SPAN, dtype=np.int64)
    out[:m] = chosen
    return out


# ---------------------------------------------------------------------------------------------
# Attended set and exact attention (R2, R6)
# ---------------------------------------------------------------------------------------------
def attended_positions(t, sel, S, W):
    """Window [w0, t] plus every selected span's tokens (disjoint by construction), ascending."""
    parts = [np.arange(j * S, j * S + S) for j in sel if j >= 0]
    parts.append(np.arange(window_start(t, S, W), t + 1))
    return np.concatenate(parts)


def attend(q, keys_g, values_g, positions, is_bf16):
    """Exact softmax attention of one query over the given positions.

    z_p = q . k_p / sqrt(d); w = softmax(z); o = sum_p w_p v_p.  Returns (o, sum_p w_p), float64.
    """
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[0]
    kk = widen(keys_g[positions], is_bf16)
    vv = widen(values_g[positions], is_bf16)
    z = (kk @ q) / math.sqrt(d)
    zmax = z.max()
    e = np.exp(z - zmax)
    w = e / e.sum()
    return w @ vv, w.sum()


# ---------------------------------------------------------------------------------------------
# Whole rows
# ---------------------------------------------------------------------------------------------
class Problem:
    """One sequence's cache and routing parameters (arrays as stored: uint16 bf16 bits or fp32)."""

    def __init__(self, keys, values, length, num_q_heads, S, k, W, is_bf16, means=None):
        self.keys, self.values = keys, values  # [Hkv][>=length][d]
        self.length = length
        self.hkv = keys.shape[0]
        self.hq = num_q_heads
        self.group = num_q_heads // self.hkv
        self.d = keys.shape[2]
        self.S, self.k, self.W = S, k, W
        self.is_bf16 = is_bf16
        if means is None:
            means, _ = summaries(widen_f32(keys[:, :length, :], is_bf16), length, S)
        self.means = means  # [Hkv][>=length//S][d] float32

    def q64(self, q_row):
        return widen(q_row, self.is_bf16)

    def row_scores(self, q_row_h, hq, t):
        r = num_routable(t, self.S, self.W)
        return route_scores(self.q64(q_row_h), self.means[hq // self.group], r, self.is_bf16)

    def row(self, q_row_h, hq, t, sel=None):
        """Routed attention for one (token, head) row at position t.

        Returns dict(out=float64[d], sel=int64[k], scores=float64[r], weight_sum=float).
        If `sel` is given, the attention uses it instead of the row's own selection.
        """
        assert 0 <= t < self.length
        g = hq // self.group
        scores = self.row_scores(q_row_h, hq, t)
        own = select_spans(scores, self.k)
        use = own if sel is None else np.asarray(sel)
        pos = attended_positions(t, use, self.S, self.W)
        o, wsum = attend(self.q64(q_row_h), self.keys[g], self.values[g], pos, self.is_bf16)
        return {"out": o, "sel": own, "scores": scores, "weight_sum": wsum, "n_attended": len(pos)}

    def dense_row(self, q_row_h, hq, t):
        """Dense causal attention over [0, t] (the k = all special case)."""
        g = hq // self.group
        o, _ = attend(self.q64(q_row_h), self.keys[g], self.values[g], np.arange(t + 1), self.is_bf16)
        return o

    def tasks(self, qvecs, heads, positions, sel=None, dense=False, scores=False):
        """Many (query vector, head, position) tasks, one after another; the same results as the
        C++ oracle's Problem.tasks.  A given selection keeps only the first occurrence of each
        routable span id (ids outside [0, r(t)) and repeats attend nothing)."""
        n = len(positions)
        out = np.zeros((n, self.d))
        sel_out = np.full((n, self.k), NO_SPAN, dtype=np.int64)
        wsum = np.zeros(n)
        n_att = np.zeros(n, dtype=np.int64)
        sc = []
        for i in range(n):
            hq, t = int(heads[i]), int(positions[i])
            if dense:
                out[i] = self.dense_row(qvecs[i], hq, t)
                wsum[i], n_att[i] = 1.0, t + 1
                continue
            use = None
            if sel is not None:
                r = num_routable(t, self.S, self.W)
                use = []
                for j in np.asarray(sel[i]).tolist():
                    if 0 <= j < r and j not in use:
                        use.append(j)
                use = np.array(sorted(use), dtype=np.int64)
            res = self.row(qvecs[i], hq, t, sel=use)
            out[i], sel_out[i], wsum[i], n_att[i] = res["out"], res["sel"], res["weight_sum"], res["n_attended"]
            sc.append(res["scores"])
        res = {"out": out, "sel": sel_out, "weight_sum": wsum, "n_attended": n_att}
        if scores:
            res["scores"] = sc
        return res

    def rows(self, q_rows, positions, heads=None, sel=None, dense=False, scores=False):
        """Every head in `heads` (default all) of rows q_rows[i] ([Hq][d]) at positions[i],
        shaped [n][len(heads)] as the C++ oracle's Problem.rows."""
        heads = list(range(self.hq)) if heads is None else list(heads)
        n, nh = len(positions), len(heads)
        q_rows = np.asarray(q_rows)
        qv = [q_rows[i][h] for i in range(n) for h in heads]
        hh = [h for _ in range(n) for h in heads]
        pp = [int(positions[i]) for i in range(n) for _ in heads]
        sl = None if sel is None else np.asarray(sel).reshape(n * nh, self.k)
        res = self.tasks(qv, hh, pp, sel=sl, dense=dense, scores=scores)
        shaped = {"out": res["out"].reshape(n, nh, self.d), "sel": res["sel"].reshape(n, nh, self.k),
                  "weight_sum": res["weight_sum"].reshape(n, nh), "n_attended": res["n_attended"].reshape(n, nh)}
        if scores:
            shaped["scores"] = [res["scores"][i * nh:(i + 1) * nh] for i in range(n)]
        return shaped


def routed_rows(problem, q_rows, positions, heads=None):
    """Routed attention for rows q_rows[i] ([Hq][d]) at positions[i]; returns (out, sel).

    out: float64 [n][Hq][d]; sel: int64 [n][Hq][k].
    """
    n = len(positions)
    heads = range(problem.hq) if heads is None else heads
    out = np.zeros((n, problem.hq, problem.d))
    sel = np.full((n, problem.hq, problem.k), NO_SPAN, dtype=np.int64)
    for i, t in enumerate(positions):
        for hq in heads:
            res = problem.row(q_rows[i][hq], hq, int(t))
            out[i, hq] = res["out"]
            sel[i, hq] = res["sel"]
    return out, sel
