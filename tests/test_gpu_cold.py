"""GPU parity of token-level cold retrieval through the C ABI: signatures bit for bit, the Hamming
scan's selection equal to the oracle's (integers: no tolerance, ties to the lower position), and
attention over the selection and the hot window within the bf16 / fp32 tolerances.
"""
import numpy as np
import pytest
import torch

import content_routed_sparse_amd as ra
import oracle as O
from oracle import cold_retrieval as C
from synth import workloads as WL

from harness import Case, log, to_dev

pytestmark = pytest.mark.gpu

W = WL.WORKLOADS


def small(base, **kw):
    return W[base].scaled(**kw)


class ColdCase(Case):
    """A synth cache with its signatures on the device and the oracle's problem per sequence."""

    def __init__(self, w, lengths, H, kc, capacity=None, edit=None):
        super().__init__(w, lengths, capacity)
        if edit is not None:
            edit(self)
        self.H, self.kc = H, kc
        c = self.cfg
        self.sig = torch.full((c.batch, c.num_kv_heads, c.capacity, c.head_dim // 8), 0x5A, dtype=torch.uint8,
                              device="cuda")
        old = torch.zeros(self.B, dtype=torch.int64, device="cuda")
        new = torch.as_tensor(self.lengths).cuda()
        ra.kv_signature_update(c, self.K, self.sig, old, new, int(self.lengths.max()))
        torch.cuda.synchronize()
        self._cold = {}

    def cold_problem(self, b):
        if b not in self._cold:
            kh, vh = self.host[b]
            w = self.w
            self._cold[b] = C.ColdProblem(kh, vh, int(self.lengths[b]), w.num_q_heads, self.H, self.kc, self.is_bf16)
        return self._cold[b]

    def check_signatures(self, b, lo=0, hi=None):
        hi = int(self.lengths[b] if hi is None else hi)
        ref = self.cold_problem(b).sig[:, lo:hi]
        assert np.array_equal(self.sig[b, :, lo:hi].cpu().numpy(), ref), "signatures differ"

    def run(self, rows):
        c, n = self.cfg, rows.q.shape[0]
        ws = torch.empty(max(1, ra.cold_workspace_bytes(c, n, rows.max_pos, self.H, self.kc)), dtype=torch.uint8,
                         device="cuda")
        self.sel = torch.full((n, c.num_q_heads, self.kc), -7, dtype=torch.int32, device="cuda")
        self.out = torch.full((n, c.num_q_heads, c.head_dim), np.nan, dtype=torch.float32, device="cuda")
        ra.cold_select(c, rows, self.sig, self.H, self.kc, self.sel, ws)
        ra.cold_attn_decode(c, rows, self.K, self.V, self.sel, self.H, self.kc, self.out)
        torch.cuda.synchronize()
        return self.sel, self.out

    def check(self, seqs, positions, q_rows, heads=None):
        sel, out = self.sel.cpu().numpy(), self.out.cpu().numpy()
        heads = range(self.w.num_q_heads) if heads is None else heads
        stats = {"rows": 0, "max_abs": 0.0, "max_rel": 0.0, "sel_fail": []}
        for i, (s, t, qi) in enumerate(zip(seqs, positions, q_rows)):
            prob = self.cold_problem(int(s))
            for h in heads:
                res = prob.row(qi[h], h, int(t))
                stats["rows"] += 1
                if not np.array_equal(sel[i, h], res["sel"]):
                    stats["sel_fail"].append((int(s), int(t), h))
                    continue
                ma, rel = O.output_errors(out[i, h], res["out"])
                stats["max_abs"] = max(stats["max_abs"], ma)
                stats["max_rel"] = max(stats["max_rel"], rel)
        log("  rows=%d sel_fail=%d max_abs=%.3g max_rel=%.3g" % (stats["rows"], len(stats["sel_fail"]),
                                                                   stats["max_abs"], stats["max_rel"]))
        assert not stats["sel_fail"], stats["sel_fail"][:5]
        if self.is_bf16:
            assert stats["max_abs"] <= O.compare.TOL_ABS["bf16"] and stats["max_rel"] <= O.compare.TOL_REL_L2_BF16
        else:
            assert stats["max_abs"] <= O.compare.TOL_ABS["f32"]


def few_sign_patterns(c):
    """Keys of sequence 0 drawn from 3 sign patterns (random magnitudes): every distance repeats
    thousands of times, across tile boundaries."""
    rng = np.random.default_rng(21)
    w = c.w
    L = int(c.lengths[0])
    pats = np.where(rng.random((3, w.head_dim)) < 0.5, -1.0, 1.0)
    for g in range(w.num_kv_heads):
        which = rng.integers(0, 3, size=L)
        vals = (np.abs(rng.standard_normal((L, w.head_dim))) + 0.1) * pats[which]
        t = torch.from_numpy(vals.astype(np.float32))
        if c.is_bf16:
            t = t.to(torch.bfloat16)
            c.host[0][0][g, :L] = t.view(torch.int16).numpy().view(np.uint16)
        else:
            c.host[0][0][g, :L] = t.numpy()
        c.K[0, g, :L] = t.cuda()


def query_copies(c):
    """Every 150th key of sequence 0 (about 109 per scan tile of 16384 positions) gets the signs
    of the query of head G g of its kv head g at the last position, so that head has more than 64
    ties at distance 0 in every tile: the ties are ranked from the bitmask, not the short list."""
    rng = np.random.default_rng(22)
    w = c.w
    L = int(c.lengths[0])
    qh = WL.query_at(w, 0, L - 1)
    qf = torch.from_numpy(qh.view(np.int16)).view(torch.bfloat16).float().numpy() if c.is_bf16 else qh
    pos = np.arange(0, L - 256, 150)
    for g in range(w.num_kv_heads):
        signs = np.where(np.signbit(qf[g * w.group]), -1.0, 1.0)
        vals = (np.abs(rng.standard_normal((len(pos), w.head_dim))) + 0.1) * signs
        t = torch.from_numpy(vals.astype(np.float32))
        if c.is_bf16:
            t = t.to(torch.bfloat16)
            c.host[0][0][g, pos] = t.view(torch.int16).numpy().view(np.uint16)
        else:
            c.host[0][0][g, pos] = t.numpy()
        c.K[0, g, torch.from_numpy(pos).cuda()] = t.cuda()


CASES = [
    # name, workload, lengths, H, top_k_cold, edit
    ("d128_G8_kc64_20k", small("decode_1m", decode_len=20000), [20000], 256, 64, None),
    ("d64_G4_kc7_H16", small("decode_1m", num_q_heads=8, num_kv_heads=2, head_dim=64, decode_len=3000), [3000], 16,
     7, None),
    ("fp32_d64_kc96", W["tiny_prefill_fp32"], [9000], 256, 96, None),
    ("batch_ragged_kc128", small("decode_1m", decode_len=17000), [17000, 300, 100, 257], 256, 128, None),
    ("G32_kc32", small("decode_1m", num_q_heads=32, num_kv_heads=1, decode_len=12000), [12000], 64, 32, None),
    ("heavy_ties", small("decode_1m", num_q_heads=8, num_kv_heads=2, decode_len=30000), [30000], 256, 64,
     few_sign_patterns),
    ("over_64_ties_per_tile", small("decode_1m", decode_len=40000), [40000], 256, 64, query_copies),
    # 37 tiles x 128 candidates per head: more than the merge keeps in registers (4096)
    ("kc128_600k_merge_batches", small("decode_1m", decode_len=600000), [600000], 256, 128, None),
]


@pytest.mark.parametrize("name,w,lengths,H,kc,edit", CASES, ids=[c[0] for c in CASES])
def test_cold_retrieval_decode(name, w, lengths, H, kc, edit):
    c = ColdCase(w, lengths, H, kc, edit=edit)
    for b in range(c.B):
        c.check_signatures(b)
    L = c.lengths
    rows, q = c.rows_for(np.arange(c.B), L - 1)
    c.run(rows)
    c.check(np.arange(c.B), L - 1, q)


def test_cold_rows_at_other_positions_and_signature_appends():
    """Rows at several positions of one sequence in one call (their cold sets differ), with the
    signatures built in two appends."""
    w = small("decode_1m", num_q_heads=8, num_kv_heads=2, decode_len=10000)
    c = ColdCase(w, [10000], 128, 16)
    sig0 = c.sig.clone()
    c.sig.fill_(0x5A)
    ra.kv_signature_update(c.cfg, c.K, c.sig, torch.tensor([0]).cuda(), torch.tensor([6000]).cuda(), 6000)
    assert (c.sig[0, :, 6000:] == 0x5A).all()
    ra.kv_signature_update(c.cfg, c.K, c.sig, torch.tensor([6000]).cuda(), torch.tensor([10000]).cuda(), 4000)
    assert torch.equal(c.sig, sig0)
    pos = [0, 127, 128, 129, 5000, 8191 + 128, 8192 + 128, 9999]
    rows, q = c.rows_for([0] * len(pos), pos)
    c.run(rows)
    c.check([0] * len(pos), pos, q)


@pytest.mark.timeout(900)
def test_cold_retrieval_at_1m():
    """decode_1m (1M tokens, 32 query heads / 4 kv heads) with a 256-token hot window and 64 cold
    tokens per head: sampled signature rows, every row-head's selection and output."""
    w = W["decode_1m"]
    L = w.decode_len
    c = ColdCase(w, [L], 256, 64)
    rng = np.random.default_rng(9)
    for p in np.sort(rng.integers(0, L - 4096, size=6)):
        c.check_signatures(0, int(p), int(p) + 4096)
    c.check_signatures(0, L - 1000, L)
    rows, q = c.rows_for([0], [L - 1])
    c.run(rows)
    c.check([0], [L - 1], q)


def test_cold_attn_ignores_repeated_and_out_of_set_entries():
    """cold_attn_decode on a hand-made selection with repeated positions, -1 and positions of the
    hot window (outside the cold set): each distinct cold position is attended once."""
    w = small("decode_1m", num_q_heads=8, num_kv_heads=2, decode_len=5000)
    H, kc = 64, 16
    c = ColdCase(w, [5000], H, kc)
    t = 4999
    rows, q = c.rows_for([0], [t])
    n_cold = t - H + 1
    rng = np.random.default_rng(23)
    sel = np.empty((1, w.num_q_heads, kc), dtype=np.int32)
    for h in range(w.num_q_heads):
        pool = rng.choice(n_cold, size=6, replace=False)
        row = rng.choice(pool, size=kc)
        row[rng.random(kc) < 0.2] = -1
        row[rng.random(kc) < 0.1] = n_cold + rng.integers(0, H)  # a hot position: not cold
        sel[0, h] = row
    out = torch.full((1, w.num_q_heads, w.head_dim), np.nan, dtype=torch.float32, device="cuda")
    ra.cold_attn_decode(c.cfg, rows, c.K, c.V, torch.as_tensor(sel).cuda(), H, kc, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    prob = c.cold_problem(0)
    for h in range(w.num_q_heads):
        used = []
        for p in sel[0, h]:
            if 0 <= p < n_cold and p not in used:
                used.append(int(p))
        ref = prob.row(q[0][h], h, t, sel=np.array(sorted(used), dtype=np.int64))
        assert ref["n_attended"] == len(used) + H
        ma, rel = O.output_errors(got[0, h], ref["out"])
        assert ma <= O.compare.TOL_ABS["bf16"] and rel <= O.compare.TOL_REL_L2_BF16, (h, ma, rel)
