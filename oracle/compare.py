"""Comparison rules between a tested selection/output and the oracle -- TEST INFRASTRUCTURE ONLY.

Selection.  Routing scores are computed in float64 here and in fp32 (or with fp32 accumulation)
on the device, so when two spans' scores are nearly equal either one may legitimately be kept.
A tested selection G is accepted against the oracle's O when it has the same size m, lists
distinct routable spans in ascending order padded with -1, and every span it swaps in or out
lies inside the tie band around the cut:

    tau_in  = m-th best oracle score, tau_out = (m+1)-th (or -inf when r == m);
    delta   = 1e-3 * max(|tau_in|, |tau_out|) + gamma_d * max_j a_j,
              a_j = sum_e |q_e * kappa(mean_j)_e|,  gamma_d = d u / (1 - d u),  u = 2^-24;
    every j in G \\ O has s_j >= tau_in - delta, every j in O \\ G has s_j <= tau_out + delta.

The relative part is the stated 1e-3 tie tolerance; gamma_d * a_j is the classical bound on the
rounding error of a d-term fp32 dot product (Higham, "Accuracy and Stability of Numerical
Algorithms", section 3.1), which matters only when the scores at the cut are close to zero.
Exact ties are not exempt: identical scores differ by 0, which is inside the band, but the
lowest-index rule is then checked separately by the exact-tie tests.

Outputs.  Compared against the oracle evaluated on the tested selection (a valid near-tie choice
attends a different, equally valid set).  Tolerances: max-abs 1e-5 for fp32 inputs, 2e-2 for
bf16 inputs with fp32 accumulation; for bf16 also a relative L2 error <= 1e-2, which an all-zero
or otherwise wrong output cannot meet.
"""
import numpy as np

from .routed_attention import round_to_bf16

U32 = 2.0 ** -24
TIE_REL = 1e-3
TOL_ABS = {"f32": 1e-5, "bf16": 2e-2}
TOL_REL_L2_BF16 = 1e-2


def gamma(d):
    return d * U32 / (1.0 - d * U32)


def score_abs_bound(q, means_g, r, is_bf16):
    """gamma_d * max_j sum_e |q_e kappa(mean_j)_e| over the routable spans."""
    if r == 0:
        return 0.0
    m = means_g[:r]
    if is_bf16:
        m = round_to_bf16(m)
    a = np.abs(m.astype(np.float64)) @ np.abs(np.asarray(q, dtype=np.float64))
    return gamma(len(q)) * float(a.max())


def selection_verdict(tested, oracle_sel, scores, k, abs_bound):
    """'exact', 'near_tie' or a string starting with 'fail' for one row."""
    tested = np.asarray(tested).astype(np.int64)
    r = len(scores)
    m = min(k, r)
    if tested.shape != (k,):
        return "fail: shape"
    head, tail = tested[:m], tested[m:]
    if np.any(tail != -1):
        return "fail: padding"
    if m and (np.any(head < 0) or np.any(head >= r)):
        return "fail: not routable"
    if m > 1 and np.any(np.diff(head) <= 0):
        return "fail: not ascending/distinct"
    gset = set(head.tolist())
    oset = set(int(j) for j in oracle_sel[:m])
    if gset == oset:
        return "exact"
    order = np.lexsort((np.arange(r), -scores))
    tau_in = scores[order[m - 1]]
    tau_out = scores[order[m]] if r > m else -np.inf
    big = max(abs(tau_in), abs(tau_out)) if np.isfinite(tau_out) else abs(tau_in)
    delta = TIE_REL * big + abs_bound
    for j in gset - oset:
        if scores[j] < tau_in - delta:
            return "fail: swapped in span %d (score %.9g < %.9g)" % (j, scores[j], tau_in - delta)
    for j in oset - gset:
        if scores[j] > tau_out + delta:
            return "fail: dropped span %d (score %.9g > %.9g)" % (j, scores[j], tau_out + delta)
    return "near_tie"


def output_errors(tested, reference):
    """Max-abs and relative L2 error of an output row; a tested value that is not finite
    (NaN or infinite, which no finite reference is close to) counts as an infinite error, so
    that it fails every tolerance and survives max()."""
    tested = np.asarray(tested, dtype=np.float64)
    reference = np.asarray(reference, dtype=np.float64)
    if not np.all(np.isfinite(tested)):
        return float("inf"), float("inf")
    diff = tested - reference
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    denom = float(np.linalg.norm(reference))
    rel = float(np.linalg.norm(diff)) / denom if denom > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def output_ok(tested, reference, is_bf16):
    max_abs, rel = output_errors(tested, reference)
    if is_bf16:
        return max_abs <= TOL_ABS["bf16"] and rel <= TOL_REL_L2_BF16, (max_abs, rel)
    return max_abs <= TOL_ABS["f32"], (max_abs, rel)
