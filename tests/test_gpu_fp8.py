"""GPU parity of the 8-bit key/value cache (E4M3 codes with one fp32 scale per row) through the
C ABI: quantisation bit for bit, span summaries bit for bit, decode attention within the bf16
tolerances of the oracle evaluated on the dequantised cache (selections tie-aware).
"""
import numpy as np
import pytest
import torch

import content_routed_sparse_amd as ra
import oracle as O
from synth import workloads as WL

from harness import Case, assert_stats, log

pytestmark = pytest.mark.gpu

W = WL.WORKLOADS
Q = O.kv_fp8


def small(base, **kw):
    return W[base].scaled(**kw)


def host_quantize(bits, rows_per_piece=1 << 16):
    """Oracle codes and scales of a host bf16 cache [Hkv][L][d] (in pieces, to bound memory)."""
    hkv, L, d = bits.shape
    codes = np.empty((hkv, L, d), dtype=np.uint8)
    scales = np.empty((hkv, L), dtype=np.float32)
    for h in range(hkv):
        for p in range(0, L, rows_per_piece):
            c, s = Q.quantize_rows(O.widen_f32(bits[h, p:p + rows_per_piece], True))
            codes[h, p:p + rows_per_piece] = c
            scales[h, p:p + rows_per_piece] = s
    return codes, scales


class Fp8Case(Case):
    """A bf16 workload whose cache is quantised on the device (kv_quantize_fp8) and, separately, by
    the oracle on the host; summaries, routing and decode then run on the 8-bit cache."""

    def __init__(self, w, lengths, capacity=None, edit=None):
        super().__init__(w, lengths, capacity)
        if edit is not None:  # (special rows, applied to the host and device bf16 caches alike)
            edit(self)
        shape = tuple(self.K.shape)
        self.K8 = torch.full(shape, 0xAA, dtype=torch.uint8, device="cuda")
        self.V8 = torch.full(shape, 0xAA, dtype=torch.uint8, device="cuda")
        self.KS = torch.full(shape[:3], -1.0, dtype=torch.float32, device="cuda")
        self.VS = torch.full(shape[:3], -1.0, dtype=torch.float32, device="cuda")
        old = torch.zeros(self.B, dtype=torch.int64, device="cuda")
        new = torch.as_tensor(self.lengths).cuda()
        mx = int(self.lengths.max())
        ra.kv_quantize_fp8(self.cfg, self.K, self.K8, self.KS, old, new, mx)
        ra.kv_quantize_fp8(self.cfg, self.V, self.V8, self.VS, old, new, mx)
        torch.cuda.synchronize()
        self.host8 = []
        for b, L in enumerate(self.lengths):
            kh, vh = self.host[b]
            self.host8.append(host_quantize(kh[:, :L]) + host_quantize(vh[:, :L]))

    def problem(self, b):
        if b not in self._problems:
            kc, ks, vc, vs = self.host8[b]
            w = self.w
            self._problems[b] = Q.Fp8Problem(kc, ks, vc, vs, int(self.lengths[b]), w.num_q_heads, w.span_size,
                                             w.top_k, w.window)
        return self._problems[b]

    def summarize(self, old, new, max_new=None):
        old = torch.as_tensor(np.asarray(old, dtype=np.int64)).cuda()
        new_np = np.asarray(new, dtype=np.int64)
        new = torch.as_tensor(new_np).cuda()
        if max_new is None:
            max_new = int((new_np - old.cpu().numpy()).max())
        ra.span_summary_update_fp8(self.cfg, self.K8, self.KS, self.pipe.span_mean, self.pipe.run_sum, old, new,
                                   max_new)

    def decode(self, rows):
        p, cfg = self.pipe, self.cfg
        n = rows.q.shape[0]
        if (n, rows.max_pos, ra.RA_OP_DECODE) != (p.n_rows, p.max_pos, p.op):
            p.reserve(n, rows.max_pos, ra.RA_OP_DECODE)
        ra.route_scores(cfg, rows, p.span_mean, p.scores)
        ra.topk_spans(cfg, rows, p.scores, p.sel)
        ra.routed_attn_decode_fp8(cfg, rows, self.K8, self.V8, self.KS, self.VS, p.sel, p.out, p.workspace)
        torch.cuda.synchronize()
        return p.out

    def check_codes(self, b, lo=0, hi=None):
        """Device codes and scales of rows [lo, hi) of sequence b, bit for bit."""
        hi = int(self.lengths[b] if hi is None else hi)
        kc, ks, vc, vs = self.host8[b]
        for dev, ref in ((self.K8, kc), (self.V8, vc)):
            assert np.array_equal(dev[b, :, lo:hi].cpu().numpy(), ref[:, lo:hi]), "codes differ"
        for dev, ref in ((self.KS, ks), (self.VS, vs)):
            assert np.array_equal(dev[b, :, lo:hi].cpu().numpy().view(np.uint32), ref[:, lo:hi].view(np.uint32)), \
                "scales differ"

    def check_summaries(self, b, L=None):
        L = int(self.lengths[b] if L is None else L)
        kc, ks, _, _ = self.host8[b]
        means, run = O.summaries(Q.dequantize_rows(kc[:, :L], ks[:, :L]), L, self.w.span_size)
        n = L // self.w.span_size
        dm = self.pipe.span_mean[b, :, :n].cpu().numpy()
        dr = self.pipe.run_sum[b].cpu().numpy()
        assert np.array_equal(dm.view(np.uint32), means[:, :n].view(np.uint32)), "span means differ"
        assert np.array_equal(dr.view(np.uint32), run.view(np.uint32)), "running sums differ"


def special_rows(c):
    """An all-zero row, a row of huge values, a row whose quotients fall among the subnormal
    codes, a row of one value and its negation (host and device caches)."""
    d = c.w.head_dim
    rows = {3: np.zeros(d, np.float32),
            10: np.linspace(-3e30, 3e30, d).astype(np.float32),
            11: np.concatenate([[448.0], np.geomspace(1e-4, 1.0, d - 1)]).astype(np.float32),
            12: np.where(np.arange(d) % 2 == 0, 1.5, -1.5).astype(np.float32)}
    for p, v in rows.items():
        t = torch.tensor(v).to(torch.bfloat16)
        bits = t.view(torch.int16).numpy().view(np.uint16)
        for h in range(c.w.num_kv_heads):
            for arr, dev in ((c.host[0][0], c.K), (c.host[0][1], c.V)):
                arr[h, p] = bits
                dev[0, h, p] = t.cuda()


@pytest.mark.parametrize("d", [128, 64])
def test_quantisation_matches_the_oracle_bit_for_bit(d):
    w = small("decode_1m", head_dim=d, span_size=64, window=64, top_k=4, decode_len=2500)
    c = Fp8Case(w, [2500], capacity=2600, edit=special_rows)
    c.check_codes(0)
    # rows past the length are left alone
    assert (c.K8[0, :, 2500:] == 0xAA).all() and (c.KS[0, :, 2500:] == -1.0).all()
    # an append of rows [2500, 2600): those rows only
    L2 = 2600
    bits = WL.kv_slab(w, 0, 0, L2, "k")
    c.K[0, :, 2500:L2] = torch.from_numpy(bits[:, 2500:L2].view(np.int16)).view(torch.bfloat16).cuda()
    ra.kv_quantize_fp8(c.cfg, c.K, c.K8, c.KS, torch.tensor([2500]).cuda(), torch.tensor([L2]).cuda(), 100)
    torch.cuda.synchronize()
    kc, ks = host_quantize(bits[:, 2500:L2])
    assert np.array_equal(c.K8[0, :, 2500:L2].cpu().numpy(), kc)
    assert np.array_equal(c.KS[0, :, 2500:L2].cpu().numpy().view(np.uint32), ks.view(np.uint32))
    c.check_codes(0, 0, 2500)  # earlier rows unchanged
    assert (c.K8[0, :, L2:] == 0xAA).all()


def test_summaries_over_the_8bit_cache_bit_for_bit():
    w = small("decode_1m", num_q_heads=8, num_kv_heads=2, span_size=64, window=64, top_k=4, decode_len=3000)
    c = Fp8Case(w, [3000])
    for a, b in ((0, 1000), (1000, 1001), (1001, 2999), (2999, 3000)):
        c.summarize([a], [b])
        c.check_summaries(0, b)


DECODE_CASES = [
    ("d128_G8_k8", small("decode_1m", span_size=64, window=64, top_k=8, decode_len=4000), [4000]),
    ("d64_G4_W3S", small("decode_1m", num_q_heads=8, num_kv_heads=2, head_dim=64, span_size=32, window=96, top_k=5,
                         decode_len=2000), [2000]),
    ("d128_batch3_ragged", small("decode_1m", span_size=128, window=128, top_k=6, decode_len=6000),
     [6000, 3333, 129]),
    ("d128_G32_k16", small("decode_1m", num_q_heads=32, num_kv_heads=1, span_size=64, window=64, top_k=16,
                           decode_len=5000), [5000]),
]


@pytest.mark.parametrize("name,w,lengths", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_over_the_8bit_cache(name, w, lengths):
    c = Fp8Case(w, lengths, capacity=max(lengths))
    L = c.lengths
    c.summarize(np.zeros(c.B, dtype=np.int64), L - 1)
    c.summarize(L - 1, L, 1)
    for b in range(c.B):
        c.check_summaries(b)
    rows, q = c.rows_for(np.arange(c.B), L - 1)
    c.decode(rows)
    stats = c.check(np.arange(c.B), L - 1, q, np.arange(c.B))
    assert_stats(stats, True)


@pytest.mark.timeout(900)
def test_decode_1m_over_the_8bit_cache_full():
    """decode_1m (1M tokens, 32 query heads / 4 kv heads) with the cache quantised on the device:
    codes and scales of a sample of rows, summaries and every row-head against the oracle."""
    w = W["decode_1m"]
    L = w.decode_len
    c = Fp8Case(w, [L])
    rng = np.random.default_rng(7)
    for p in np.sort(rng.integers(0, L - 4096, size=8)):
        c.check_codes(0, int(p), int(p) + 4096)
    c.check_codes(0, L - 2048, L)
    c.summarize([0], [L - 1])
    c.summarize([L - 1], [L], 1)
    c.check_summaries(0)
    rows, q = c.rows_for([0], [L - 1])
    c.decode(rows)
    stats = c.check([0], [L - 1], q, [0])
    log("  decode_1m fp8: max_abs %.3g max_rel %.3g" % (stats["max_abs"], stats["max_rel"]))
    assert_stats(stats, True)


# ----------------------------------------------------------------------------- prefill, 8-bit
def prefill_fp8(c, prefix, chunk, pieces=1):
    """Setup summaries of the prefix, then per piece of the chunk: the piece's summary update,
    routing, selection and routed_attn_prefill_fp8 of its rows; returns (out, sel) of the chunk."""
    c.summarize([0], [prefix], max(prefix, 1))
    bounds = np.linspace(0, chunk, pieces + 1).astype(int)
    outs, sels = [], []
    p = c.pipe
    for a, b in zip(bounds[:-1], bounds[1:]):
        rows, _ = c.chunk_rows(0, prefix + a, b - a)
        c.summarize([prefix + a], [prefix + b], b - a)
        p.reserve(b - a, rows.max_pos, ra.RA_OP_PREFILL)
        ra.route_scores(c.cfg, rows, p.span_mean, p.scores)
        ra.topk_spans(c.cfg, rows, p.scores, p.sel)
        ra.routed_attn_prefill_fp8(c.cfg, rows, c.K8, c.V8, c.KS, c.VS, p.sel, p.out, p.workspace)
        torch.cuda.synchronize()
        outs.append(p.out.clone())
        sels.append(p.sel.clone())
    return torch.cat(outs), torch.cat(sels)


def outlier_rows(c):
    """Keys planted along single queries' vectors past the first chunk of a window span: each of
    these queries sees a score ~160 (log2 units) above the maximum of its first keys, so its entry
    takes the 8-bit tile's second pass."""
    w = c.w
    G = w.num_q_heads // w.num_kv_heads
    prefix = int(c.lengths[0]) - 256
    qs = WL.queries(w, 0, prefix, 256)
    for i, (r, h) in enumerate([(10, 0), (60, 3), (100, 5), (150, 2), (200, 7), (250, 1)]):
        qf = (qs[r, h].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        alpha = 160.0 * np.sqrt(w.head_dim) / (np.log2(np.e) * np.linalg.norm(qf))
        t = torch.tensor(alpha * qf / np.linalg.norm(qf), dtype=torch.float32).to(torch.bfloat16)
        p = prefix - 256 + 70 + 23 * i  # window span of every chunk row, past its first 64 keys
        c.host[0][0][h // G, p] = t.view(torch.int16).numpy().view(np.uint16)
        c.K[0, h // G, p] = t.cuda()


PREFILL_FP8_CASES = [
    # name, workload, prefix, chunk, edit
    ("d128_G8", small("prefill_8k_on_1m", span_size=32, window=32, top_k=4), 2048, 300, None),
    ("d64_G8_S48_W100", small("prefill_8k_on_1m", num_q_heads=8, num_kv_heads=1, head_dim=64, span_size=48,
                              window=100, top_k=5), 1500, 333, None),
    ("d128_special_rows", small("prefill_8k_on_1m", num_q_heads=8, num_kv_heads=2, span_size=16, window=16,
                                top_k=6), 700, 200, special_rows),
    ("d128_outliers_second_pass", small("prefill_8k_on_1m", num_q_heads=8, num_kv_heads=2, span_size=256,
                                        window=256, top_k=4), 3072, 256, outlier_rows),
]


@pytest.mark.parametrize("name,w,prefix,chunk,edit", PREFILL_FP8_CASES, ids=[c[0] for c in PREFILL_FP8_CASES])
def test_prefill_over_the_8bit_cache(name, w, prefix, chunk, edit):
    c = Fp8Case(w, [prefix + chunk], edit=edit)
    out, sel = prefill_fp8(c, prefix, chunk)
    c.check_summaries(0)
    q = WL.queries(w, 0, prefix, chunk)
    c.pipe.reserve(chunk, prefix + chunk - 1, ra.RA_OP_PREFILL)
    c.pipe.out.copy_(out)
    c.pipe.sel.copy_(sel)
    # (rows of values near 3e30: max-abs relative to the row's magnitude)
    stats = c.check([0] * chunk, np.arange(prefix, prefix + chunk), q, np.arange(chunk), scores=False,
                    scale_abs=edit is special_rows)
    log("  %s: max_abs %.3g max_rel %.3g" % (name, stats["max_abs"], stats["max_rel"]))
    assert_stats(stats, True)


def test_prefill_over_the_8bit_cache_chunking_and_decode_agree():
    """Cut into 1 or 3 calls the 8-bit prefill gives the same bits, and its last row equals the
    8-bit decode kernel's result for that row within the rounding of P to bf16."""
    w = small("prefill_8k_on_1m", span_size=64, window=64, top_k=8)
    prefix, chunk = 4000, 200
    c = Fp8Case(w, [prefix + chunk])
    out1, sel1 = prefill_fp8(c, prefix, chunk, pieces=1)
    c3 = Fp8Case(w, [prefix + chunk])
    out3, sel3 = prefill_fp8(c3, prefix, chunk, pieces=3)
    assert torch.equal(sel1, sel3) and torch.equal(out1, out3)
    rows, _ = c.rows_for([0], [prefix + chunk - 1])
    outd = torch.empty(1, w.num_q_heads, w.head_dim, device="cuda")
    ws = torch.empty(ra.workspace_bytes(c.cfg, ra.RA_OP_DECODE, 1, prefix + chunk - 1), dtype=torch.uint8,
                     device="cuda")
    ra.routed_attn_decode_fp8(c.cfg, rows, c.K8, c.V8, c.KS, c.VS, sel1[-1:].contiguous(), outd, ws)
    torch.cuda.synchronize()
    diff = (outd[0] - out1[-1]).abs().max().item()
    assert diff <= max(outd.abs().max().item(), 0.1) * 2.0 ** -8, diff


@pytest.mark.timeout(900)
def test_prefill_8k_on_1m_over_the_8bit_cache_sampled():
    """The 8192-token chunk on the 1M-token cache, quantised on the device: every row computed;
    a seeded sample of 32 positions x 32 heads (chunk edges and span boundaries included) against
    the oracle on the dequantised cache."""
    w = W["prefill_8k_on_1m"]
    P, n = w.prefix_len, w.chunk_len
    c = Fp8Case(w, [P + n])
    out, sel = prefill_fp8(c, P, n)
    rng = np.random.default_rng(w.seed + 1)
    must = [0, n - 1, 1022, 1023, 1024, 2047, 2048, 4095, 4096, n - 1025]
    rest = sorted(set(rng.choice(n, 64, replace=False).tolist()) - set(must))[:32 - len(must)]
    idx = np.array(sorted(set(must) | set(rest)))
    q = WL.queries(w, 0, P, n)
    stats = c.check([0] * len(idx), P + idx, q[idx], idx, scores=False)
    log("  prefill_8k_on_1m fp8: rows %d max_abs %.3g max_rel %.3g" % (stats["rows"], stats["max_abs"],
                                                                      stats["max_rel"]))
    assert_stats(stats, True)
