"""Python face of the C++ oracle (oracle/routed_attention.cpp) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this module.  It marshals arrays into ``liboracle.so`` and back; every step of the method
(summaries, kappa, scores, selection, attended set, attention) runs in the C++ code, which
follows readings R1-R6 (listed in its header and in oracle/routed_attention.py).

The functions mirror the numpy oracle's names and signatures, so that one set of pins checks
both implementations, and ``Problem.rows`` computes many (row, head) tasks at once on all host
threads.
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SOURCE = os.path.join(HERE, "routed_attention.cpp")
NO_SPAN = -1
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64


def build(force=True):
    """Compile routed_attention.cpp with g++ (-O2, no fast-math, no contraction of a*b+c)."""
    if os.path.exists(LIB_PATH) and not force:
        return LIB_PATH
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-pthread", "-ffp-contract=off", "-fPIC", "-shared",
                           SOURCE, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        h = ctypes.CDLL(LIB_PATH)
        h.oracle_summary_update.argtypes = [_P, _I, _L, _L, _L, _P, _L, _P, _L, _L, _L, _I]
        h.oracle_summary_update.restype = None
        h.oracle_kappa_bf16.argtypes = [_P, _P, _L]
        h.oracle_kappa_bf16.restype = None
        h.oracle_widen.argtypes = [_P, _I, _P, _L]
        h.oracle_widen.restype = None
        h.oracle_window_start.argtypes = [_L, _L, _L]
        h.oracle_window_start.restype = _L
        h.oracle_num_routable.argtypes = [_L, _L, _L]
        h.oracle_num_routable.restype = _L
        h.oracle_route_scores.argtypes = [_P, _P, _L, _L, _I, _P]
        h.oracle_route_scores.restype = None
        h.oracle_select.argtypes = [_P, _L, _L, _P]
        h.oracle_select.restype = None
        h.oracle_attend.argtypes = [_P, _P, _P, _I, _L, _L, _L, _P, _L, _P]
        h.oracle_attend.restype = ctypes.c_double
        h.oracle_rows.argtypes = [_L, _L, _L, _L, _L, _L, _I, _P, _P, _L, _P, _L, _P, _P, _P, _L, _P, _I,
                                  _P, _P, _P, _P, _P, _L, _I]
        h.oracle_rows.restype = _I
        h.oracle_hardware_threads.argtypes = []
        h.oracle_hardware_threads.restype = _I
        _lib = h
    return _lib


def default_threads():
    """Threads the oracle uses: the CPUs this process may run on, capped by OMP_NUM_THREADS when
    that is set (it states the host's share of CPUs where a machine is shared)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _ptr(a):
    return a.ctypes.data if a is not None else None


def _stored(x):
    """(contiguous array, is_bf16) for stored inputs: uint16 bf16 bit patterns or float32."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, 1
    assert x.dtype == np.float32, x.dtype
    return x, 0


# ------------------------------------------------------------------------- element helpers
def widen(x, is_bf16):
    x = np.ascontiguousarray(x)
    assert x.dtype == (np.uint16 if is_bf16 else np.float32)
    out = np.empty(x.shape, dtype=np.float64)
    lib().oracle_widen(_ptr(x), int(is_bf16), _ptr(out), x.size)
    return out


def round_to_bf16(x):
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, dtype=np.float32)
    lib().oracle_kappa_bf16(_ptr(x), _ptr(out), x.size)
    return out


def window_start(t, S, W):
    return int(lib().oracle_window_start(int(t), int(S), int(W)))


def num_routable(t, S, W):
    return int(lib().oracle_num_routable(int(t), int(S), int(W)))


# --------------------------------------------------------------------------------- summaries
def summary_update(keys, means, run_sum, old_len, new_len, S, threads=None):
    """Tokens [old_len, new_len) of one sequence into means [Hkv][max_spans][d] and run_sum
    [Hkv][d] (both float32, updated in place).  keys: [Hkv][cap][d], float32 or bf16 bits."""
    keys, bf = _stored(keys)
    assert means.dtype == np.float32 and run_sum.dtype == np.float32
    assert means.flags.c_contiguous and run_sum.flags.c_contiguous
    hkv, cap, d = keys.shape
    assert means.shape[0] == hkv and means.shape[2] == d and run_sum.shape == (hkv, d) and new_len <= cap
    assert means.shape[1] >= new_len // S
    lib().oracle_summary_update(_ptr(keys), bf, hkv, cap, d, _ptr(means), means.shape[1], _ptr(run_sum),
                                int(old_len), int(new_len), int(S), threads or default_threads())
    return means, run_sum


def summaries(keys, length, S, max_spans=None, threads=None):
    hkv, _, d = keys.shape
    if max_spans is None:
        max_spans = length // S
    means = np.zeros((hkv, max_spans, d), dtype=np.float32)
    run_sum = np.zeros((hkv, d), dtype=np.float32)
    return summary_update(keys, means, run_sum, 0, length, S, threads)


# ----------------------------------------------------------------------- scores, selection
def route_scores(q, means_g, r, is_bf16):
    q = np.ascontiguousarray(np.asarray(q, dtype=np.float64))
    m = np.ascontiguousarray(means_g[:r], dtype=np.float32)
    out = np.empty(r, dtype=np.float64)
    lib().oracle_route_scores(_ptr(q), _ptr(m), int(r), q.shape[0], int(is_bf16), _ptr(out))
    return out


def select_spans(scores, k):
    s = np.ascontiguousarray(np.asarray(scores, dtype=np.float64))
    out = np.empty(k, dtype=np.int64)
    lib().oracle_select(_ptr(s), len(s), int(k), _ptr(out))
    return out


def attend(q, keys_g, values_g, positions, is_bf16):
    """Softmax attention of one query (float64 [d]) over positions of one head's [L][d] cache."""
    q = np.ascontiguousarray(np.asarray(q, dtype=np.float64))
    keys_g, bf = _stored(keys_g)
    values_g, _ = _stored(values_g)
    assert bf == int(is_bf16)
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int64))
    out = np.empty(q.shape[0], dtype=np.float64)
    ws = lib().oracle_attend(_ptr(q), _ptr(keys_g), _ptr(values_g), bf, keys_g.shape[0], q.shape[0], 0, _ptr(pos),
                             len(pos), _ptr(out))
    return out, ws


# ------------------------------------------------------------------------------ whole rows
class Problem:
    """One sequence's cache and routing parameters; the same interface as the numpy oracle's
    Problem, plus ``rows`` for many tasks at once."""

    def __init__(self, keys, values, length, num_q_heads, S, k, W, is_bf16, means=None, threads=None):
        self.keys, bf = _stored(keys)  # [Hkv][cap][d]
        self.values, bfv = _stored(values)
        assert bf == bfv == int(is_bf16) and self.keys.shape == self.values.shape
        self.length = int(length)
        self.hkv, self.cap, self.d = self.keys.shape
        self.hq = num_q_heads
        self.group = num_q_heads // self.hkv
        self.S, self.k, self.W = S, k, W
        self.is_bf16 = bool(is_bf16)
        self.threads = threads or default_threads()
        if means is None:
            means, _ = summaries(self.keys, self.length, S, threads=self.threads)
        self.means = np.ascontiguousarray(means, dtype=np.float32)  # [Hkv][>= length // S][d]

    def q64(self, q_row):
        return widen(q_row, self.is_bf16)

    def row_scores(self, q_row_h, hq, t):
        r = num_routable(t, self.S, self.W)
        return route_scores(self.q64(q_row_h), self.means[hq // self.group], r, self.is_bf16)

    def tasks(self, qvecs, heads, positions, sel=None, dense=False, scores=False):
        """Tasks i = (query vector qvecs[i] [d], head heads[i], position positions[i]).

        Returns dict(out [n][d] float64, sel [n][k] int64, weight_sum [n], n_attended [n],
        scores: list of float64 arrays (when asked))."""
        q = np.ascontiguousarray(qvecs)
        assert q.dtype == (np.uint16 if self.is_bf16 else np.float32) and q.ndim == 2 and q.shape[1] == self.d
        n = q.shape[0]
        head = np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
        pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int64))
        assert head.shape == (n,) and pos.shape == (n,)
        assert np.all(pos < self.length), "a row position lies past the sequence's length"
        sel_in = None
        if sel is not None:
            sel_in = np.ascontiguousarray(np.asarray(sel, dtype=np.int64))
            assert sel_in.shape == (n, self.k)
        out = np.empty((n, self.d), dtype=np.float64)
        sel_out = np.empty((n, self.k), dtype=np.int64)
        wsum = np.empty(n, dtype=np.float64)
        n_att = np.empty(n, dtype=np.int64)
        r = np.array([num_routable(int(t), self.S, self.W) for t in pos], dtype=np.int64) if n else np.zeros(0, np.int64)
        stride = max(1, int(r.max())) if n else 1
        sc = np.empty((n, stride), dtype=np.float64) if scores else None
        assert self.means.shape[1] >= (int(r.max()) if n else 0)
        rc = lib().oracle_rows(self.hq, self.hkv, self.d, self.S, self.k, self.W, int(self.is_bf16),
                               _ptr(self.keys), _ptr(self.values), self.cap, _ptr(self.means), self.means.shape[1],
                               _ptr(q), _ptr(head), _ptr(pos), n, _ptr(sel_in), int(dense), _ptr(out), _ptr(sel_out),
                               _ptr(wsum), _ptr(n_att), _ptr(sc), stride, self.threads)
        assert rc == 0, "oracle_rows rejected a task"
        res = {"out": out, "sel": sel_out, "weight_sum": wsum, "n_attended": n_att}
        if scores:
            res["scores"] = [sc[i, :r[i]].copy() for i in range(n)]
        return res

    def rows(self, q_rows, positions, heads=None, sel=None, dense=False, scores=False):
        """Every head in `heads` (default all) of rows q_rows[i] ([Hq][d]) at positions[i].

        Returns the tasks' results reshaped to [n][len(heads)]."""
        heads = list(range(self.hq)) if heads is None else list(heads)
        n, nh = len(positions), len(heads)
        q_rows = np.asarray(q_rows)
        qv = q_rows[:, heads, :].reshape(n * nh, self.d) if n else q_rows.reshape(0, self.d)
        hh = np.tile(np.asarray(heads, dtype=np.int32), n)
        pp = np.repeat(np.asarray(positions, dtype=np.int64), nh)
        sl = None if sel is None else np.asarray(sel).reshape(n * nh, self.k)
        res = self.tasks(qv, hh, pp, sel=sl, dense=dense, scores=scores)
        shaped = {"out": res["out"].reshape(n, nh, self.d), "sel": res["sel"].reshape(n, nh, self.k),
                  "weight_sum": res["weight_sum"].reshape(n, nh), "n_attended": res["n_attended"].reshape(n, nh)}
        if scores:
            shaped["scores"] = [res["scores"][i * nh:(i + 1) * nh] for i in range(n)]
        return shaped

    def row(self, q_row_h, hq, t, sel=None):
        """One (token, head) row: dict(out, sel, scores, weight_sum, n_attended)."""
        assert 0 <= t < self.length
        res = self.tasks(np.asarray(q_row_h)[None], [hq], [t], sel=None if sel is None else self._pad(sel)[None],
                         scores=True)
        return {"out": res["out"][0], "sel": res["sel"][0], "scores": res["scores"][0],
                "weight_sum": float(res["weight_sum"][0]), "n_attended": int(res["n_attended"][0])}

    def dense_row(self, q_row_h, hq, t):
        return self.tasks(np.asarray(q_row_h)[None], [hq], [t], dense=True)["out"][0]

    def _pad(self, sel):
        s = np.full(self.k, NO_SPAN, dtype=np.int64)
        sel = np.asarray(sel, dtype=np.int64).ravel()
        assert len(sel) <= self.k
        s[:len(sel)] = sel
        return s


def routed_rows(problem, q_rows, positions, heads=None):
    """Routed attention for rows q_rows[i] ([Hq][d]) at positions[i]; returns (out, sel)."""
    res = problem.rows(q_rows, positions, heads)
    return res["out"], res["sel"]
