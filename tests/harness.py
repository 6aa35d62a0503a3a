"""Shared GPU-test harness: builds a workload's cache on the device, runs the library's entry
points through the binding, and checks the results against the CPU oracle (the C++ oracle,
oracle/routed_attention.cpp, on all host threads; the comparison rules are oracle/compare.py).

Inputs come only from the seeded generator (synth); expected values come only from oracle/.
"""
import sys
import time

import numpy as np
import torch

import content_routed_sparse_amd as ra
import oracle as O
import oracle.cpp as OC
from synth import BF16
from synth import workloads as WL


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(arr, is_bf16):
    t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16 if is_bf16 else np.float32))
    if is_bf16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def config_for(w, capacity, batch=None):
    return ra.Config(w.num_q_heads, w.num_kv_heads, w.head_dim, w.span_size, w.top_k, w.window,
                     ra.RA_BF16 if w.dtype == BF16 else ra.RA_F32, batch or w.batch, capacity)


class Case:
    """A workload on the device: K/V cache, host copies, and the step's results."""

    def __init__(self, w, lengths, capacity=None):
        self.w = w
        self.is_bf16 = w.dtype == BF16
        self.lengths = np.asarray(lengths, dtype=np.int64)
        self.B = len(self.lengths)
        self.cap = int(capacity or self.lengths.max())
        self.cfg = config_for(w, self.cap, self.B)
        dt = self.cfg.torch_dtype
        shape = (self.B, w.num_kv_heads, self.cap, w.head_dim)
        self.K = torch.zeros(shape, dtype=dt, device="cuda")
        self.V = torch.zeros(shape, dtype=dt, device="cuda")
        self.host = []
        t0 = time.time()
        for b, L in enumerate(self.lengths):
            kh = WL.kv_slab(w, b, 0, int(L), "k")
            vh = WL.kv_slab(w, b, 0, int(L), "v")
            self.K[b, :, :L] = to_dev(kh, self.is_bf16)
            self.V[b, :, :L] = to_dev(vh, self.is_bf16)
            self.host.append((kh, vh))
        torch.cuda.synchronize()
        log("  cache ready: B=%d cap=%d (%.1fs)" % (self.B, self.cap, time.time() - t0))
        self.pipe = ra.Pipeline(self.cfg)
        self._problems = {}

    # ------------------------------------------------------------------ device steps
    def summarize(self, old, new, max_new=None):
        old = torch.as_tensor(np.asarray(old, dtype=np.int64)).cuda()
        new_np = np.asarray(new, dtype=np.int64)
        new = torch.as_tensor(new_np).cuda()
        if max_new is None:
            max_new = int((new_np - old.cpu().numpy()).max())
        self.pipe.summarize(self.K, old, new, max_new)

    def rows_for(self, seqs, positions):
        w = self.w
        q = np.stack([WL.query_at(w, int(s), int(p)) for s, p in zip(seqs, positions)]) if len(seqs) else \
            np.zeros((0, w.num_q_heads, w.head_dim), dtype=np.uint16 if self.is_bf16 else np.float32)
        rows = ra.Rows(to_dev(q, self.is_bf16), torch.as_tensor(np.asarray(seqs, dtype=np.int32)).cuda(),
                       torch.as_tensor(np.asarray(positions, dtype=np.int64)).cuda(),
                       int(max(positions)) if len(positions) else 0)
        return rows, q

    def chunk_rows(self, seq, pos0, n):
        q = WL.queries(self.w, seq, pos0, n)
        rows = ra.Rows(to_dev(q, self.is_bf16), torch.full((n,), seq, dtype=torch.int32, device="cuda"),
                       torch.arange(pos0, pos0 + n, dtype=torch.int64, device="cuda"), pos0 + n - 1)
        return rows, q

    def attend(self, rows, op):
        out = self.pipe.attend(rows, self.K, self.V, op)
        torch.cuda.synchronize()
        return out

    # ---------------------------------------------------------------- oracle side
    def problem(self, b):
        if b not in self._problems:
            kh, vh = self.host[b]
            w = self.w
            self._problems[b] = OC.Problem(kh, vh, int(self.lengths[b]), w.num_q_heads, w.span_size, w.top_k,
                                           w.window, self.is_bf16)
        return self._problems[b]

    def check_summaries(self, b, L=None):
        """Device span means and running sum vs the oracle, bit for bit."""
        L = int(self.lengths[b] if L is None else L)
        kh, _ = self.host[b]
        means, run = OC.summaries(kh[:, :L, :], L, self.w.span_size)
        n = L // self.w.span_size
        dm = self.pipe.span_mean[b, :, :n].cpu().numpy()
        dr = self.pipe.run_sum[b].cpu().numpy()
        assert np.array_equal(dm.view(np.uint32), means[:, :n].view(np.uint32)), "span means differ"
        assert np.array_equal(dr.view(np.uint32), run.view(np.uint32)), "running sums differ"

    def check(self, seqs, positions, q_rows, row_index, heads=None, scores=True, scale_abs=False):
        """Compare selection (tie-aware), scores and outputs of the given rows with the oracle.

        The oracle computes every (row, head) of a sequence in one call; a row whose device
        selection is a valid near-tie alternative is compared with the oracle evaluated on that
        selection (a second call for those rows only).  With scale_abs, a row's max-abs error is
        taken relative to max(1, the reference row's largest magnitude): for caches that hold
        rows of values near 3e30, where an absolute bound made for unit-scale values means
        nothing."""
        w = self.w
        sel = self.pipe.sel.cpu().numpy()
        out = self.pipe.out.cpu().numpy()
        sc = self.pipe.scores.cpu().numpy() if scores else None
        heads = list(range(w.num_q_heads)) if heads is None else list(heads)
        stats = {"rows": 0, "exact": 0, "near_tie": 0, "fail": [], "max_abs": 0.0, "max_rel": 0.0,
                 "score_fail": 0}
        seqs = np.asarray(seqs, dtype=np.int64)
        positions = np.asarray(positions, dtype=np.int64)
        row_index = np.asarray(row_index, dtype=np.int64)
        q_rows = np.asarray(q_rows)

        def record(ri, h, ref):
            ma, rel = O.output_errors(out[ri, h], ref)
            if scale_abs:
                ma /= max(1.0, float(np.abs(ref).max()))
            stats["max_abs"] = max(stats["max_abs"], ma)
            stats["max_rel"] = max(stats["max_rel"], rel)

        for s in np.unique(seqs):
            idx = np.nonzero(seqs == s)[0]
            prob = self.problem(int(s))
            res = prob.rows(q_rows[idx], positions[idx], heads, scores=True)
            # kappa(mean) once per kv head (kappa is idempotent, so the bound takes it as given)
            mk = [O.round_to_bf16(prob.means[g]) if self.is_bf16 else prob.means[g] for g in range(prob.hkv)]
            redo = []
            for a, i in enumerate(idx):
                t, ri = int(positions[i]), int(row_index[i])
                for hi, h in enumerate(heads):
                    ors = res["scores"][a][hi]
                    r = len(ors)
                    bound = O.score_abs_bound(prob.q64(q_rows[i][h]), mk[h // prob.group], r, False)
                    if sc is not None and r:
                        err = np.abs(sc[ri, h, :r].astype(np.float64) - ors)
                        if np.any(err > bound * 1.0001 + 1e-30):
                            stats["score_fail"] += 1
                    v = O.selection_verdict(sel[ri, h], res["sel"][a, hi], ors, w.top_k, bound)
                    stats["rows"] += 1
                    if v.startswith("fail"):
                        stats["fail"].append((int(s), t, h, v))
                        continue
                    stats[v] += 1
                    if v == "exact":
                        record(ri, h, res["out"][a, hi])
                    else:
                        redo.append((i, h, ri))
            if redo:
                alt = prob.tasks(np.stack([q_rows[i][h] for i, h, _ in redo]), [h for _, h, _ in redo],
                                 [int(positions[i]) for i, _, _ in redo],
                                 sel=np.stack([sel[ri, h] for _, h, ri in redo]))
                for x, (i, h, ri) in enumerate(redo):
                    record(ri, h, alt["out"][x])
        return stats


def assert_stats(stats, is_bf16):
    log("  rows=%d exact=%d near_tie=%d fail=%d score_fail=%d max_abs=%.3g max_rel=%.3g" % (
        stats["rows"], stats["exact"], stats["near_tie"], len(stats["fail"]), stats["score_fail"],
        stats["max_abs"], stats["max_rel"]))
    assert not stats["fail"], stats["fail"][:5]
    assert stats["score_fail"] == 0
    if is_bf16:
        assert stats["max_abs"] <= O.compare.TOL_ABS["bf16"]
        assert stats["max_rel"] <= O.compare.TOL_REL_L2_BF16
    else:
        assert stats["max_abs"] <= O.compare.TOL_ABS["f32"]


def run_decode(w, lengths, capacity=None):
    """Cache of `lengths` tokens per sequence; summaries of all but the last token as setup, then the
    decode step: summary update of the last token, routing, selection, attention."""
    c = Case(w, lengths, capacity)
    L = c.lengths
    c.summarize(np.zeros(c.B, dtype=np.int64), L - 1)
    c.summarize(L - 1, L, 1)
    rows, q = c.rows_for(np.arange(c.B), L - 1)
    c.attend(rows, ra.RA_OP_DECODE)
    return c, rows, q


def run_prefill(w, prefix, chunk, pieces=1, timed=False):
    """Cache of prefix + chunk tokens (one sequence); setup summaries of the prefix, then per
    piece: summary update of the piece's tokens and the prefill of its rows."""
    c = Case(w, [prefix + chunk])
    c.summarize([0], [prefix], max(prefix, 1))
    bounds = np.linspace(0, chunk, pieces + 1).astype(int)
    outs, sels = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        rows, _ = c.chunk_rows(0, prefix + a, b - a)
        torch.cuda.synchronize()
        t0 = time.time()
        c.summarize([prefix + a], [prefix + b], b - a)
        c.attend(rows, ra.RA_OP_PREFILL)
        if timed:
            log("  prefill of %d rows: %.2f ms (first call, includes setup of buffers)" % (b - a, (time.time() - t0) * 1e3))
            for _ in range(2):
                torch.cuda.synchronize()
                t0 = time.time()
                c.attend(rows, ra.RA_OP_PREFILL)
                log("  route+topk+prefill again: %.2f ms" % ((time.time() - t0) * 1e3))
        outs.append(c.pipe.out.clone())
        sels.append(c.pipe.sel.clone())
    q = WL.queries(w, 0, prefix, chunk)
    return c, q, torch.cat(outs), torch.cat(sels)
