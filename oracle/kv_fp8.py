"""CPU oracle of the 8-bit key/value cache -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this module; the GPU library never calls it and shares no code with it.

Source.  The release post "Experimental model with subquadratic attention: 100 tok/s @ 1M
context, 76 tok/s @ 10M context (30B model, single GPU)", section "Limitations and next steps",
lists 4/8-bit quantisation as planned work without a format.  Decode is bound by the K/V bytes
it streams, so an 8-bit cache halves them.  The readings taken here (one plain choice each,
listed with their reasons in the design notes of the repository):

  Q1  Element format: FP8 E4M3 in its finite variant -- 1 sign bit, 4 exponent bits (bias 7),
      3 fraction bits; exponent field 0 holds the subnormals 2^-6 * f/8; the all-ones
      exponent with fraction 7 is NaN and there is no infinity, so the largest value is
      2^8 * 1.75 = 448.
  Q2  Scale: one fp32 scale per (sequence, kv head, token) row of d values, for K and for V
      separately: s = fl32(max_e |x_e| / 448) (s = 1 for an all-zero row).  A per-row scale
      needs nothing but the row itself, so a token can be stored the moment it is produced.
  Q3  Encoding: c_e = E4M3(fl32(x_e / s)) with round to nearest, ties to even, after clamping
      the quotient to [-448, 448] (it exceeds 448 only by the rounding of s).
  Q4  The cache holds the values fl32(E4M3^-1(c_e) * s) (one fp32 rounding); every step of the
      method (span summaries, routing, attention) reads them exactly as it reads a float32
      cache, while queries and routing stay as for bf16 inputs (kappa = bf16 rounding).
"""
import numpy as np

from .routed_attention import Problem, attend, attended_positions, route_scores, select_spans, summaries, widen

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Values (float64) of E4M3 bit patterns (uint8), from the format definition (Q1)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    f = c & 0x7
    normal = np.ldexp(1.0 + f / 8.0, e - 7)
    sub = np.ldexp(f / 8.0, -6)
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (f == 7), np.nan, v)


def e4m3_encode(x):
    """E4M3 bit patterns of float values in [-448, 448]: round to nearest, ties to even (Q3).

    For |x| in [2^(u-1), 2^u) the spacing of E4M3 values is 2^(u-4), never below the subnormal
    spacing 2^-9; the value is rounded to a multiple of it with round-half-even (numpy.rint),
    then written as sign, biased exponent and fraction.
    """
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.abs(x) <= E4M3_MAX), "clamp before encoding"
    _, u = np.frexp(x)
    spacing = np.ldexp(1.0, np.maximum(u - 4, -9))
    r = np.rint(x / spacing) * spacing  # multiples of the spacing; 448 is representable
    a = np.abs(r)
    sign = np.where(np.signbit(r), 0x80, 0)
    _, ua = np.frexp(np.where(a > 0, a, 1.0))
    e_unb = ua - 1  # a in [2^e_unb, 2^(e_unb+1))
    is_norm = a >= 2.0 ** -6
    e_field = np.where(is_norm, e_unb + 7, 0)
    frac = np.where(is_norm, np.rint((a / np.ldexp(1.0, e_unb) - 1.0) * 8), np.rint(a / 2.0 ** -9))
    code = sign | (e_field << 3) | frac.astype(np.int64)
    return np.where(a == 0, sign, code).astype(np.uint8)


def quantize_rows(x_f32):
    """Codes (uint8) and per-row scales (float32) of rows x [..., d] (Q2, Q3)."""
    x = np.asarray(x_f32, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    quot = (x / s[..., None]).astype(np.float32)  # one fp32 division per element
    quot = np.clip(quot, -E4M3_MAX, E4M3_MAX)
    return e4m3_encode(quot), s


def dequantize_rows(codes, scales):
    """The cache's values fl32(E4M3^-1(c) * s) as float32 (Q4)."""
    v = e4m3_decode(codes).astype(np.float32)  # exact: E4M3 values are float32 values
    return (v * np.asarray(scales, dtype=np.float32)[..., None]).astype(np.float32)


class Fp8Problem(Problem):
    """One sequence with an 8-bit cache: codes [Hkv][L][d] uint8 and scales [Hkv][L] float32 for
    K and V; queries are bf16 bit patterns and routing rounds the means to bf16 (Q4)."""

    def __init__(self, k_codes, k_scales, v_codes, v_scales, length, num_q_heads, S, k, W):
        keys = dequantize_rows(k_codes, k_scales)
        values = dequantize_rows(v_codes, v_scales)
        means, _ = summaries(keys[:, :length, :], length, S)
        super().__init__(keys, values, length, num_q_heads, S, k, W, False, means=means)

    def q64(self, q_row):
        return widen(q_row, True)

    def row_scores(self, q_row_h, hq, t):
        from .routed_attention import num_routable
        r = num_routable(t, self.S, self.W)
        return route_scores(self.q64(q_row_h), self.means[hq // self.group], r, True)

    def row(self, q_row_h, hq, t, sel=None):
        assert 0 <= t < self.length
        g = hq // self.group
        scores = self.row_scores(q_row_h, hq, t)
        own = select_spans(scores, self.k)
        use = own if sel is None else np.asarray(sel)
        pos = attended_positions(t, use, self.S, self.W)
        o, wsum = attend(self.q64(q_row_h), self.keys[g], self.values[g], pos, False)
        return {"out": o, "sel": own, "scores": scores, "weight_sum": wsum, "n_attended": len(pos)}

    def dense_row(self, q_row_h, hq, t):
        g = hq // self.group
        o, _ = attend(self.q64(q_row_h), self.keys[g], self.values[g], np.arange(t + 1), False)
        return o
