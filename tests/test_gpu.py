"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Selections must match the oracle exactly except inside the stated near-tie band; outputs must
be within max-abs 1e-5 (fp32 inputs) or 2e-2 plus relative L2 1e-2 (bf16 inputs) of the oracle
evaluated on the device's selection; span summaries must match bit for bit.
"""
import numpy as np
import pytest
import torch

import content_routed_sparse_amd as ra
import oracle as O
from synth import BF16, F32
from synth import workloads as WL

from harness import Case, assert_stats, log, run_decode, run_prefill

pytestmark = pytest.mark.gpu

W = WL.WORKLOADS


def small(base, **kw):
    return W[base].scaled(**kw)


# ----------------------------------------------------------------------------- small cases
PREFILL_CASES = [
    # name, workload, prefix, chunk
    ("fp32_d64_1h", small("tiny_prefill_fp32", chunk_len=700), 0, 700),
    ("fp32_d128_gqa", small("tiny_prefill_fp32", num_q_heads=4, num_kv_heads=2, head_dim=128, span_size=16,
                            top_k=3, window=20), 333, 257),
    ("bf16_d128_gqa8", small("prefill_8k_on_1m", span_size=32, window=32, top_k=4), 2048, 300),
    ("bf16_d64_S48_W100", small("prefill_8k_on_1m", num_q_heads=8, num_kv_heads=1, head_dim=64, span_size=48,
                                window=100, top_k=5), 1500, 333),
    ("bf16_S1_W1", small("prefill_8k_on_1m", num_q_heads=2, num_kv_heads=1, head_dim=64, span_size=1, window=1,
                         top_k=3), 50, 70),
]


@pytest.mark.parametrize("name,w,prefix,chunk", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_small(name, w, prefix, chunk):
    log("prefill case", name)
    c, q, out, sel = run_prefill(w, prefix, chunk)
    c.check_summaries(0)
    pos = np.arange(prefix, prefix + chunk)
    stats = c.check([0] * chunk, pos, q, np.arange(chunk))
    assert_stats(stats, w.dtype == BF16)


DECODE_CASES = [
    ("bf16_d128_ragged", small("ragged_decode_16", batch=3, span_size=64, window=64, top_k=8, ragged=(3000, 9000)),),
    ("bf16_d64_W3S", small("ragged_decode_16", batch=2, head_dim=64, num_q_heads=8, num_kv_heads=2, span_size=32,
                           window=96, top_k=6, ragged=(700, 5000)),),
    ("fp32_d64", small("tiny_prefill_fp32", mode="decode", batch=4, num_q_heads=4, num_kv_heads=4, span_size=64,
                       window=64, top_k=8, ragged=(100, 4000)),),
    ("fp32_d128", small("tiny_prefill_fp32", mode="decode", batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                        span_size=128, window=200, top_k=4, ragged=(129, 3000)),),
    ("bf16_short_rows_r0", small("ragged_decode_16", batch=3, span_size=64, window=64, top_k=8, ragged=(1, 130)),),
    # G*k > 256: the kv head's selection entries are matched from memory, not from registers
    ("bf16_G32_k16", small("ragged_decode_16", batch=2, num_q_heads=32, num_kv_heads=1, span_size=32, window=32,
                           top_k=16, ragged=(2000, 6000)),),
    ("bf16_G8_k64", small("ragged_decode_16", batch=2, num_q_heads=16, num_kv_heads=2, span_size=16, window=40,
                          top_k=64, ragged=(2500, 4000)),),
]


@pytest.mark.parametrize("name,w", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_small(name, w):
    log("decode case", name)
    lengths = w.seq_lengths()
    c, rows, q = run_decode(w, lengths)
    for b in range(c.B):
        c.check_summaries(b)
    stats = c.check(np.arange(c.B), lengths - 1, q, np.arange(c.B))
    assert_stats(stats, w.dtype == BF16)


def test_k_all_spans_equals_dense_causal():
    """With k >= number of spans every past token is attended: the output is dense causal attention
    (max-abs 2e-2 and relative L2 1e-2 against the oracle's dense rows, every row and head)."""
    w = small("prefill_8k_on_1m", num_q_heads=4, num_kv_heads=2, span_size=32, window=32, top_k=64)
    c, q, out, sel = run_prefill(w, 1024, 900)  # at most 60 routable spans < k
    out = out.cpu().numpy()
    pos = 1024 + np.arange(900)
    ref = c.problem(0).rows(q, pos, dense=True)["out"]
    worst_abs, worst_rel = 0.0, 0.0
    for i in range(900):
        for h in range(4):
            ma, rel = O.output_errors(out[i, h], ref[i, h])
            worst_abs, worst_rel = max(worst_abs, ma), max(worst_rel, rel)
    log("  k=all vs dense: max abs %.3g, max rel L2 %.3g" % (worst_abs, worst_rel))
    assert worst_abs <= O.compare.TOL_ABS["bf16"] and worst_rel <= O.compare.TOL_REL_L2_BF16


def test_prefill_outlier_keys_force_the_second_pass():
    """Keys of norm far above the rest, planted past a span's first 64 keys: some rows then see a
    score more than 2^32 (log2 units) above the maximum of their first keys, and the tile kernel
    recomputes those tiles with the final maximum.  The result must still match the oracle."""
    w = small("prefill_8k_on_1m", num_q_heads=8, num_kv_heads=2, span_size=256, window=256, top_k=4)
    prefix, chunk = 3072, 256
    c = Case(w, [prefix + chunk])
    kh, vh = c.host[0]
    big = np.uint16(0x41F0)  # bf16 30.0
    planted = [(g, p) for g in range(2) for p in (100, 700, 1000, 1900, 2500)]  # offsets >= 64 in their spans
    for g, p in planted:
        kh[g, p, :] = big
        c.K[0, g, p, :] = torch.full((w.head_dim,), 30.0, dtype=torch.bfloat16)
    c._problems.clear()
    c.summarize([0], [prefix], prefix)
    rows, q = c.chunk_rows(0, prefix, chunk)
    c.summarize([prefix], [prefix + chunk], chunk)
    c.attend(rows, ra.RA_OP_PREFILL)
    c.check_summaries(0)
    stats = c.check([0] * chunk, np.arange(prefix, prefix + chunk), q, np.arange(chunk))
    assert_stats(stats, True)


def _plant_ramp_rows(c, positions):
    """Key and value rows that ramp from -3e30 to 3e30 (bf16) at the given positions of sequence
    0, every kv head, host and device caches alike."""
    t = torch.tensor(np.linspace(-3e30, 3e30, c.w.head_dim).astype(np.float32)).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16)
    kh, vh = c.host[0]
    for g in range(c.w.num_kv_heads):
        for p in positions:
            kh[g, p] = bits
            vh[g, p] = bits
            c.K[0, g, p] = t.cuda()
            c.V[0, g, p] = t.cuda()
    c._problems.clear()


def test_prefill_and_dense_with_rows_near_3e30():
    """Cache rows of values up to 3e30: scores against them reach ~1e30 (log2 units), where a
    weight's exponent formed by one fused multiply-add against the rounded maximum would be that
    rounding error (2^70 and more).  Routed prefill and dense attention stay finite and match the
    oracle; max-abs is taken relative to the row's magnitude, relative L2 as usual."""
    w = small("prefill_8k_on_1m", num_q_heads=8, num_kv_heads=2, span_size=32, window=32, top_k=4)
    prefix, chunk = 1000, 200
    c = Case(w, [prefix + chunk])
    _plant_ramp_rows(c, [10, 75, 500, 1010, 1100])  # routable spans, chunk rows' windows
    c.summarize([0], [prefix], prefix)
    rows, q = c.chunk_rows(0, prefix, chunk)
    c.summarize([prefix], [prefix + chunk], chunk)
    c.attend(rows, ra.RA_OP_PREFILL)
    c.check_summaries(0)
    pos = np.arange(prefix, prefix + chunk)
    stats = c.check([0] * chunk, pos, q, np.arange(chunk), scale_abs=True)
    assert_stats(stats, True)
    out = torch.empty(chunk, w.num_q_heads, w.head_dim, device="cuda")
    ra.attn_dense_causal(c.cfg, rows, c.K, c.V, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = c.problem(0).rows(q, pos, dense=True)["out"]
    worst_abs, worst_rel, huge = 0.0, 0.0, 0
    for i in range(chunk):
        for h in range(w.num_q_heads):
            ma, rel = O.output_errors(got[i, h], ref[i, h])
            mag = max(1.0, float(np.abs(ref[i, h]).max()))
            huge += mag > 1e20
            worst_abs, worst_rel = max(worst_abs, ma / mag), max(worst_rel, rel)
    log("  dense: rows=%d (%d near 3e30) scaled max_abs=%.3g max_rel=%.3g" % (chunk * w.num_q_heads, huge,
                                                                             worst_abs, worst_rel))
    assert huge > 0
    assert worst_abs <= O.compare.TOL_ABS["bf16"] and worst_rel <= O.compare.TOL_REL_L2_BF16


def test_prefill_chunking_is_bitwise_invariant():
    w = small("prefill_8k_on_1m", span_size=32, window=32, top_k=4)
    _, _, out1, sel1 = run_prefill(w, 1000, 600, pieces=1)
    _, _, out3, sel3 = run_prefill(w, 1000, 600, pieces=3)
    assert torch.equal(sel1, sel3)
    assert torch.equal(out1, out3)


def _outlier_prefill(w, prefix, chunk, pieces, targets):
    """run_prefill with keys planted along single queries' vectors (each target query alone sees
    a score ~160 log2 units above the maximum of its first keys, so its entry takes the second
    pass); returns (out, sel) of the chunk computed in `pieces` calls."""
    G = w.num_q_heads // w.num_kv_heads
    c = Case(w, [prefix + chunk])
    qs = WL.queries(w, 0, prefix, chunk)
    kh, _ = c.host[0]
    for r, h, p in targets:
        bits, kdev = _aligned_outlier_key(qs[r, h], w.head_dim, 160.0)
        kh[h // G, p, :] = bits
        c.K[0, h // G, p, :] = kdev.to("cuda")
    c._problems.clear()
    c.summarize([0], [prefix], prefix)
    bounds = np.linspace(0, chunk, pieces + 1).astype(int)
    outs, sels = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        rows, _ = c.chunk_rows(0, prefix + a, b - a)
        c.summarize([prefix + a], [prefix + b], b - a)
        c.attend(rows, ra.RA_OP_PREFILL)
        outs.append(c.pipe.out.clone())
        sels.append(c.pipe.sel.clone())
    return c, qs, torch.cat(outs), torch.cat(sels)


def test_prefill_chunking_is_bitwise_invariant_with_outlier_keys():
    """Entries that need the second pass share tiles with entries that do not; cutting the chunk
    into 1, 3 or 5 calls regroups the tiles, and every output bit stays the same (each entry
    decides its second pass alone).  The result also matches the oracle."""
    w = small("prefill_8k_on_1m", num_q_heads=8, num_kv_heads=2, span_size=256, window=256, top_k=4)
    prefix, chunk = 3072, 256
    targets = [(r, h, 2816 + 70 + 23 * i) for i, (r, h) in enumerate([(10, 0), (60, 3), (100, 5), (150, 2),
                                                                      (200, 7), (250, 1)])]
    c, q, out1, sel1 = _outlier_prefill(w, prefix, chunk, 1, targets)
    stats = c.check([0] * chunk, np.arange(prefix, prefix + chunk), q, np.arange(chunk))
    assert_stats(stats, True)
    for pieces in (3, 5):
        _, _, outp, selp = _outlier_prefill(w, prefix, chunk, pieces, targets)
        assert torch.equal(sel1, selp), pieces
        assert torch.equal(out1, outp), pieces


@pytest.mark.parametrize("G,k", [(8, 8), (4, 16)])
def test_prefill_ignores_repeated_and_out_of_range_entries(G, k):
    """routed_attn_prefill on a hand-made selection with repeated span ids (inside one head and
    across the heads of a kv head), -1 and ids >= r: the result is attention over the distinct
    routable spans, as the decode entry point computes it (compared with the oracle), and the
    last row equals the decode kernel's result on the same selection."""
    w = small("prefill_8k_on_1m", num_q_heads=2 * G, num_kv_heads=2, span_size=32, window=32, top_k=k)
    prefix, chunk = 3000, 200
    c, q, _, _ = run_prefill(w, prefix, chunk)
    rng = np.random.default_rng(17)
    pos = np.arange(prefix, prefix + chunk)
    sel = np.empty((chunk, w.num_q_heads, k), dtype=np.int32)
    for i, t in enumerate(pos):
        r = c.cfg.num_routable(int(t))
        pool = rng.choice(r, size=3 * k // 2, replace=False)
        for h in range(w.num_q_heads):
            row = rng.choice(pool, size=k)
            row[rng.random(k) < 0.15] = -1
            row[rng.random(k) < 0.1] = r + rng.integers(0, 5)
            sel[i, h] = row
    rows, _ = c.chunk_rows(0, prefix, chunk)
    sel_d = torch.as_tensor(sel).cuda()
    out = torch.empty(chunk, w.num_q_heads, w.head_dim, device="cuda")
    ws = torch.empty(ra.workspace_bytes(c.cfg, ra.RA_OP_PREFILL, chunk, int(pos[-1])), dtype=torch.uint8, device="cuda")
    ra.routed_attn_prefill(c.cfg, rows, c.K, c.V, sel_d, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = c.problem(0).rows(q, pos, sel=sel.astype(np.int64))["out"]
    worst = 0.0
    for i in range(chunk):
        for h in range(w.num_q_heads):
            ma, rel = O.output_errors(got[i, h], ref[i, h])
            worst = max(worst, ma)
            assert ma <= O.compare.TOL_ABS["bf16"] and rel <= O.compare.TOL_REL_L2_BF16, (i, h, ma, rel)
    log("  prefill on repeated/out-of-range entries: max abs %.3g" % worst)
    # the decode kernel on the last row's selection
    rows1, _ = c.rows_for([0], [int(pos[-1])])
    out1 = torch.empty(1, w.num_q_heads, w.head_dim, device="cuda")
    ws1 = torch.empty(ra.workspace_bytes(c.cfg, ra.RA_OP_DECODE, 1, int(pos[-1])), dtype=torch.uint8, device="cuda")
    ra.routed_attn_decode(c.cfg, rows1, c.K, c.V, sel_d[-1:].contiguous(), out1, ws1)
    torch.cuda.synchronize()
    diff = (out1[0] - out[-1]).abs().max().item()
    scale = max(out1.abs().max().item(), 0.1)
    assert diff <= scale * 2.0 ** -8, diff  # decode keeps P in fp32, prefill rounds it to bf16


def test_last_prefill_row_matches_decode():
    """The decode kernel and the prefill kernel give the same result for the same row."""
    w = small("prefill_8k_on_1m", span_size=64, window=64, top_k=8)
    cp, q, out_p, sel_p = run_prefill(w, 4000, 200)
    wd = w.scaled(mode="decode", decode_len=4200)
    cd, rows, qd = run_decode(wd, [4200])
    assert np.array_equal(q[-1], qd[0])
    same = (sel_p[-1] == cd.pipe.sel[0]).all(dim=1).cpu().numpy()
    # routing runs on MFMA for the chunk and on FMA for the single row: selections may differ
    # only inside the near-tie band, which the oracle checks below
    stats = cd.check([0], [4199], qd, [0])
    assert_stats(stats, True)
    # the prefill tile rounds the softmax weights to bf16 for the P.V product (relative error
    # up to 2^-9 per weight), the decode kernel keeps them in fp32: allow 2^-8 of max |o|
    diff = (out_p[-1] - cd.pipe.out[0]).abs().max(dim=1).values.cpu().numpy()
    scale = float(cd.pipe.out[0].abs().max())
    assert same.sum() >= 28 and np.all(diff[same] <= max(scale, 0.1) * 2.0 ** -8), (same, diff)


def test_repeatable_and_row_independent():
    w = small("ragged_decode_16", batch=4, span_size=64, window=64, top_k=8, ragged=(5000, 9000))
    lengths = w.seq_lengths()
    c, rows, q = run_decode(w, lengths)
    out1 = c.pipe.out.clone()
    c.attend(rows, ra.RA_OP_DECODE)
    assert torch.equal(out1, c.pipe.out)
    # the same rows in another order and alone give the same bits
    perm = [2, 0, 3, 1]
    rows2, _ = c.rows_for(perm, lengths[perm] - 1)
    out2 = c.attend(rows2, ra.RA_OP_DECODE).clone()
    assert torch.equal(out2, out1[perm])
    rows3, _ = c.rows_for([3], lengths[[3]] - 1)
    out3 = c.attend(rows3, ra.RA_OP_DECODE).clone()
    assert torch.equal(out3[0], out1[3])


@pytest.mark.parametrize("G,k", [(8, 8), (32, 16)])
def test_decode_ignores_repeated_and_out_of_range_entries(G, k):
    """A hand-made selection with repeated span ids (inside one head and across the heads of a
    kv head) and ids outside [0, r): the result is attention over the distinct valid spans.
    Two calls in a row give the same bits (the workspace counters are back at zero)."""
    w = small("ragged_decode_16", batch=2, num_q_heads=2 * G, num_kv_heads=2, span_size=32, window=32, top_k=k,
              ragged=(3000, 5000))
    lengths = w.seq_lengths()
    c, rows, q = run_decode(w, lengths)
    rng = np.random.default_rng(7)
    sel = np.empty((c.B, w.num_q_heads, k), dtype=np.int32)
    for b in range(c.B):
        r = c.cfg.num_routable(int(lengths[b]) - 1)
        pool = rng.choice(r, size=3 * k // 2, replace=False)  # few distinct spans: heads share them
        for h in range(w.num_q_heads):
            row = rng.choice(pool, size=k)  # repeats inside the head
            row[rng.random(k) < 0.15] = -1
            row[rng.random(k) < 0.1] = r + rng.integers(0, 5)  # not routable
            sel[b, h] = row
    sel_d = torch.as_tensor(sel).cuda()
    out = torch.empty(c.B, w.num_q_heads, w.head_dim, device="cuda")
    ra.routed_attn_decode(c.cfg, rows, c.K, c.V, sel_d, out, c.pipe.workspace)
    torch.cuda.synchronize()
    first = out.clone()
    ra.routed_attn_decode(c.cfg, rows, c.K, c.V, sel_d, out, c.pipe.workspace)
    torch.cuda.synchronize()
    assert torch.equal(first, out)
    got = out.cpu().numpy()
    worst = 0.0
    for b in range(c.B):
        t = int(lengths[b]) - 1
        r = c.cfg.num_routable(t)
        for h in range(w.num_q_heads):
            used = []
            for j in sel[b, h]:
                if 0 <= j < r and j not in used:
                    used.append(int(j))
            ref = c.problem(b).row(q[b][h], h, t, sel=np.array(used, dtype=np.int64))["out"]
            ma, rel = O.output_errors(got[b, h], ref)
            worst = max(worst, ma)
            assert ma <= O.compare.TOL_ABS["bf16"] and rel <= O.compare.TOL_REL_L2_BF16, (b, h, ma, rel)
    log("  repeated/out-of-range entries: max abs %.3g" % worst)


DENSE_CASES = [
    # name, workload, number of rows
    ("d128_G4", small("ragged_decode_16", batch=3, num_q_heads=8, num_kv_heads=2, span_size=64, window=64, top_k=4,
                      ragged=(500, 3000)), 70),
    ("d64_G32", small("ragged_decode_16", batch=2, head_dim=64, num_q_heads=32, num_kv_heads=1, span_size=64,
                      window=64, top_k=4, ragged=(900, 2000)), 21),
    ("d128_G3", small("ragged_decode_16", batch=2, num_q_heads=6, num_kv_heads=2, span_size=32, window=32, top_k=4,
                      ragged=(300, 1500)), 50),
    ("d128_G1", small("ragged_decode_16", batch=2, num_q_heads=4, num_kv_heads=4, span_size=32, window=32, top_k=4,
                      ragged=(100, 700)), 140),
]


@pytest.mark.parametrize("name,w,n", DENSE_CASES, ids=[c[0] for c in DENSE_CASES])
def test_dense_causal_small(name, w, n):
    """attn_dense_causal against the oracle's dense causal attention, rows of several sequences
    in random order (several passes per tile), plus one contiguous run of rows."""
    log("dense case", name)
    lengths = w.seq_lengths()
    c = Case(w, lengths)
    rng = np.random.default_rng(11)
    seqs = rng.integers(0, c.B, size=n)
    pos = np.array([rng.integers(0, lengths[s]) for s in seqs])
    run = np.arange(lengths[0] - 40, lengths[0])  # a chunk-like run of one sequence
    seqs = np.concatenate([seqs, np.zeros(len(run), dtype=np.int64)])
    pos = np.concatenate([pos, run])
    rows, q = c.rows_for(seqs, pos)
    out = torch.empty(len(seqs), w.num_q_heads, w.head_dim, device="cuda")
    ra.attn_dense_causal(c.cfg, rows, c.K, c.V, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    worst_abs, worst_rel = 0.0, 0.0
    for i, (s_, t) in enumerate(zip(seqs, pos)):
        for h in range(w.num_q_heads):
            ref = c.problem(int(s_)).dense_row(q[i][h], h, int(t))
            ma, rel = O.output_errors(got[i, h], ref)
            worst_abs, worst_rel = max(worst_abs, ma), max(worst_rel, rel)
    log("  rows=%d max_abs=%.3g max_rel=%.3g" % (len(seqs), worst_abs, worst_rel))
    assert worst_abs <= O.compare.TOL_ABS["bf16"] and worst_rel <= O.compare.TOL_REL_L2_BF16


def test_dense_equals_routed_with_all_spans():
    """With k >= the number of routable spans the routed prefill is dense causal attention: the
    two GPU paths agree (both round the weights to bf16 for P.V)."""
    w = small("prefill_8k_on_1m", num_q_heads=4, num_kv_heads=2, span_size=32, window=32, top_k=64)
    c, q, out_r, sel = run_prefill(w, 1024, 900)  # at most 60 routable spans < k
    rows, _ = c.chunk_rows(0, 1024, 900)
    out_d = torch.empty_like(out_r)
    ra.attn_dense_causal(c.cfg, rows, c.K, c.V, out_d)
    torch.cuda.synchronize()
    diff = (out_d - out_r).abs().max().item()
    scale = out_r.abs().max().item()
    log("  dense vs routed(k=all): max abs diff %.3g (max |o| %.3g)" % (diff, scale))
    assert diff <= max(scale, 0.1) * 2.0 ** -7


def test_dense_outlier_keys_force_the_second_pass():
    w = small("prefill_8k_on_1m", num_q_heads=8, num_kv_heads=2, span_size=256, window=256, top_k=4)
    L = 2600
    c = Case(w, [L])
    kh, _ = c.host[0]
    for g in range(2):
        for p in (900, 1700, 2300):  # far past the first chunk of every row
            kh[g, p, :] = np.uint16(0x41F0)  # bf16 30.0
            c.K[0, g, p, :] = torch.full((w.head_dim,), 30.0, dtype=torch.bfloat16)
    c._problems.clear()
    pos = np.arange(L - 200, L)
    rows, q = c.rows_for(np.zeros(len(pos), dtype=np.int64), pos)
    out = torch.empty(len(pos), w.num_q_heads, w.head_dim, device="cuda")
    ra.attn_dense_causal(c.cfg, rows, c.K, c.V, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    worst = 0.0
    for i, t in enumerate(pos):
        for h in range(w.num_q_heads):
            ma, rel = O.output_errors(got[i, h], c.problem(0).dense_row(q[i][h], h, int(t)))
            worst = max(worst, ma)
            assert ma <= O.compare.TOL_ABS["bf16"] and rel <= O.compare.TOL_REL_L2_BF16, (i, h, ma, rel)
    log("  outliers: max abs %.3g" % worst)


def _aligned_outlier_key(q_bits, d, log2_units):
    """bf16 bits of a key along one query's vector whose score with that query is about
    `log2_units` in the kernels' log2 domain (other queries see ~|q|^-1 of it)."""
    qf = (q_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    alpha = log2_units * np.sqrt(d) / (np.log2(np.e) * np.linalg.norm(qf))
    k = torch.tensor(alpha * qf / np.linalg.norm(qf), dtype=torch.float32).to(torch.bfloat16)
    return k.view(torch.int16).numpy().view(np.uint16), k


@pytest.mark.parametrize("kind", ["prefill", "dense"])
def test_single_query_overflow_sends_its_tile_to_the_second_pass(kind):
    """Keys planted along single queries' vectors, past the first chunk of keys: each target
    query alone sees a score ~160 (log2 units) above the maximum of its first keys, so its
    weights overflow in the fast pass, while the other entries of its tile stay in range.  The
    whole tile must take the second pass whatever place the query holds in it (every lane
    votes).  Six targets in different rows and heads, so that some sit at no special place."""
    w = small("prefill_8k_on_1m", num_q_heads=8, num_kv_heads=2, span_size=256, window=256, top_k=4)
    G = w.num_q_heads // w.num_kv_heads
    if kind == "prefill":
        prefix, chunk = 3072, 256
        c = Case(w, [prefix + chunk])
        qs = WL.queries(w, 0, prefix, chunk)
        # rows t in [3072, 3328) all see window span 11 = keys [2816, 3072) in full
        targets = [(r, h, 2816 + 70 + 23 * i) for i, (r, h) in enumerate([(10, 0), (60, 3), (100, 5), (150, 2),
                                                                          (200, 7), (250, 1)])]
        qrows = [qs[r, h] for r, h, _ in targets]
    else:
        L = 2600
        c = Case(w, [L])
        pos = np.arange(L - 200, L)
        targets = [(r, h, 700 + 211 * i) for i, (r, h) in enumerate([(5, 0), (40, 3), (100, 5), (130, 2),
                                                                    (170, 7), (199, 1)])]
        qrows = [WL.query_at(w, 0, int(pos[r]))[h] for r, h, _ in targets]
    kh, _ = c.host[0]
    for (r, h, p), qrow in zip(targets, qrows):
        bits, kdev = _aligned_outlier_key(qrow, w.head_dim, 160.0)
        kh[h // G, p, :] = bits
        c.K[0, h // G, p, :] = kdev.to("cuda")
    c._problems.clear()
    if kind == "prefill":
        c.summarize([0], [prefix], prefix)
        rows, q = c.chunk_rows(0, prefix, chunk)
        c.summarize([prefix], [prefix + chunk], chunk)
        c.attend(rows, ra.RA_OP_PREFILL)
        stats = c.check([0] * chunk, np.arange(prefix, prefix + chunk), q, np.arange(chunk))
        assert_stats(stats, True)
    else:
        rows, q = c.rows_for(np.zeros(len(pos), dtype=np.int64), pos)
        out = torch.empty(len(pos), w.num_q_heads, w.head_dim, device="cuda")
        ra.attn_dense_causal(c.cfg, rows, c.K, c.V, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for i, t in enumerate(pos):
            for hh in range(w.num_q_heads):
                ma, rel = O.output_errors(got[i, hh], c.problem(0).dense_row(q[i][hh], hh, int(t)))
                assert ma <= O.compare.TOL_ABS["bf16"] and rel <= O.compare.TOL_REL_L2_BF16, (i, hh, ma, rel)


def test_empty_rows_are_a_no_op():
    w = small("ragged_decode_16", batch=1, span_size=64, window=64, top_k=8, ragged=(0, 0), decode_len=2000)
    c = Case(w, [2000])
    c.summarize([0], [2000])
    c.summarize([2000], [2000], 1)  # old == new: nothing to add
    c.check_summaries(0)
    rows, _ = c.rows_for([], [])
    out = c.attend(rows, ra.RA_OP_DECODE)
    assert out.shape[0] == 0


def test_summary_incremental_bitwise():
    w = small("ragged_decode_16", batch=2, span_size=48, window=64, top_k=8, ragged=(3000, 5000))
    c = Case(w, w.seq_lengths())
    L = c.lengths
    p = np.zeros(2, dtype=np.int64)
    for step in [1, 47, 48, 100, 1000, 5000]:
        nxt = np.minimum(p + step, L)
        c.summarize(p, nxt, min(step, c.cap))
        p = nxt
    assert np.array_equal(p, L)
    for b in range(2):
        c.check_summaries(b)


def test_invalid_arguments_raise():
    w = small("ragged_decode_16", batch=1, span_size=64, window=64, top_k=8, ragged=(0, 0), decode_len=500)
    c = Case(w, [500])
    rows, _ = c.rows_for([0], [499])
    bad = ra.Config(32, 4, 128, 64, 65, 64, ra.RA_BF16, 1, 500)  # top_k > 64
    with pytest.raises(ra.RoutedAttnError) as e:
        ra.topk_spans(bad, rows, torch.zeros(1, 32, 8, device="cuda"), torch.zeros(1, 32, 65, dtype=torch.int32,
                                                                                    device="cuda"))
    assert e.value.status == 2
    small_ws = torch.empty(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(ra.RoutedAttnError) as e:
        ra.routed_attn_decode(c.cfg, rows, c.K, c.V, torch.zeros(1, 32, 8, dtype=torch.int32, device="cuda"),
                              torch.empty(1, 32, 128, device="cuda"), small_ws)
    assert e.value.status == 3


# ------------------------------------------------------------------------------ full sizes
@pytest.mark.timeout(600)
def test_tiny_prefill_fp32_full():
    w = W["tiny_prefill_fp32"]
    log("tiny_prefill_fp32: L=4096, all rows")
    c, q, out, sel = run_prefill(w, 0, w.chunk_len)
    c.check_summaries(0)
    stats = c.check([0] * w.chunk_len, np.arange(w.chunk_len), q, np.arange(w.chunk_len))
    assert_stats(stats, False)


@pytest.mark.timeout(600)
def test_decode_1m_full():
    w = W["decode_1m"]
    log("decode_1m: L=1048576, 32 rows")
    c, rows, q = run_decode(w, w.seq_lengths())
    c.check_summaries(0)
    stats = c.check([0], [w.decode_len - 1], q, [0])
    assert_stats(stats, True)


@pytest.mark.timeout(900)
def test_ragged_decode_16_full():
    """Ragged decode of 16 sequences (64K..512K tokens): every sequence's summaries, and all
    16 x 32 = 512 row-heads against the oracle."""
    w = W["ragged_decode_16"]
    lengths = w.seq_lengths()
    log("ragged_decode_16: lengths", lengths.tolist())
    c, rows, q = run_decode(w, lengths)
    for b in range(c.B):
        c.check_summaries(b)
    every = np.arange(c.B)
    stats = c.check(every, lengths - 1, q, every)
    assert stats["rows"] == 16 * w.num_q_heads
    assert_stats(stats, True)


@pytest.mark.timeout(900)
def test_prefill_8k_on_1m_full_sampled():
    """8192-token chunk on a 1M-token cache: every row is computed; a seeded sample of 32
    positions x 32 heads (always the chunk's first and last rows and span-boundary rows) is
    compared with the oracle."""
    w = W["prefill_8k_on_1m"]
    P, n = w.prefix_len, w.chunk_len
    log("prefill_8k_on_1m: prefix=%d chunk=%d" % (P, n))
    c, q, out, sel = run_prefill(w, P, n, timed=True)
    c.check_summaries(0)
    rng = np.random.default_rng(w.seed)
    must = [0, n - 1, 1022, 1023, 1024, 2047, 2048, 4095, 4096, n - 1025]
    rest = sorted(set(rng.choice(n, 64, replace=False).tolist()) - set(must))[:32 - len(must)]
    idx = np.array(sorted(set(must) | set(rest)))
    stats = c.check([0] * len(idx), P + idx, q[idx], idx)
    assert_stats(stats, True)


def _topk_case(r_values, pattern, k, seed):
    """topk_spans on hand-made scores: rows at positions with the given routable counts."""
    S = W = 4
    rng = np.random.default_rng(seed)
    n = len(r_values)
    pos = np.array([4 * r + 3 for r in r_values], dtype=np.int64)  # r(t) = (t - 3) // 4 for t >= 3
    stride = max(1, max(r_values))
    sc = np.zeros((n, 1, stride), dtype=np.float32)
    for i, r in enumerate(r_values):
        if pattern == "normal":
            sc[i, 0, :r] = rng.standard_normal(r)
        elif pattern == "equal":
            sc[i, 0, :r] = 0.25
        elif pattern == "few_values":
            sc[i, 0, :r] = rng.integers(-2, 3, r) * 0.5
        elif pattern == "signed_zero":
            sc[i, 0, :r] = np.where(rng.random(r) < 0.5, -0.0, 0.0)
            sc[i, 0, :r:7] = -1.0
        elif pattern == "one_lane":  # every large score sits in lane 0 (j = 0, 64, 128, ...)
            sc[i, 0, :r] = rng.standard_normal(r) - 10.0
            sc[i, 0, :r:64] = 100.0 + rng.standard_normal(len(range(0, r, 64)))
        elif pattern == "descending":
            sc[i, 0, :r] = -np.arange(r, dtype=np.float32)
    cfg = ra.Config(1, 1, 64, S, k, W, ra.RA_BF16, 1, int(pos.max()) + 1)
    rows = ra.Rows(torch.zeros(n, 1, 64, dtype=torch.bfloat16, device="cuda"),
                   torch.zeros(n, dtype=torch.int32, device="cuda"), torch.as_tensor(pos).cuda(), int(pos.max()))
    sel = torch.full((n, 1, k), 77, dtype=torch.int32, device="cuda")
    ra.topk_spans(cfg, rows, torch.as_tensor(sc).cuda(), sel)
    got = sel.cpu().numpy()
    for i, r in enumerate(r_values):
        want = O.select_spans(sc[i, 0, :r].astype(np.float64), k)
        assert np.array_equal(got[i, 0], want), (pattern, r, got[i, 0], want)


@pytest.mark.parametrize("pattern", ["normal", "equal", "few_values", "signed_zero", "one_lane", "descending"])
def test_topk_spans_exact(pattern):
    """Selection is exactly the oracle's on given scores, for every register width and the
    fallback paths (r from 0 to beyond 64 x 40 candidates per lane)."""
    for k in (1, 8, 16, 64):
        for group in ([0, 1, 2, 15, 16, 17, 63, 64, 65, 100, 128], [129, 300, 511, 512], [513, 1000, 1031, 1088],
                      [1089, 2000, 2559, 2560], [2561, 4000, 5000]):
            _topk_case(group, pattern, k, seed=k * 1000 + len(group))


@pytest.mark.timeout(1200)
def test_decode_10m_full():
    """Decode at L = 10,485,760 (20 GiB of bf16 K/V for one layer): all 32 rows."""
    w = W["decode_10m"]
    log("decode_10m: L=%d, 32 rows" % w.decode_len)
    c, rows, q = run_decode(w, w.seq_lengths())
    c.check_summaries(0)
    stats = c.check([0], [w.decode_len - 1], q, [0])
    assert_stats(stats, True)


def test_decode_step_replays_from_a_hip_graph():
    """The decode step captured in a HIP graph: every replay, with eager work and host
    synchronisation in between, equals the eager result bit for bit."""
    w = small("ragged_decode_16", batch=2, span_size=64, window=64, top_k=8, ragged=(3000, 6000))
    lengths = w.seq_lengths()
    c, rows, q = run_decode(w, lengths)
    eager_out = c.pipe.out.clone()
    eager_sel = c.pipe.sel.clone()
    L = torch.as_tensor(lengths).cuda()
    Lm1 = L - 1
    cap_stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap_stream):
        c.pipe.summarize(c.K, Lm1, L, 1)
        c.pipe.attend(rows, c.K, c.V, ra.RA_OP_DECODE)
    for rep in range(3):
        c.pipe.out.zero_()
        c.pipe.sel.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(c.pipe.out, eager_out), rep
        assert torch.equal(c.pipe.sel, eager_sel), rep
        # eager work between replays
        c.attend(rows, ra.RA_OP_DECODE)
        assert torch.equal(c.pipe.out, eager_out)


@pytest.mark.parametrize("d,G,S,W,nseq", [(128, 8, 32, 32, 1), (64, 4, 16, 40, 3), (128, 32, 64, 64, 2)])
def test_route_and_topk_do_not_depend_on_the_score_stride(d, G, S, W, nseq):
    """Scores and selections (bf16, enough rows for the MFMA routing kernel, rows of several
    sequences mixed in its tiles) are bitwise the same for an odd stride, the stride plus one and
    the 32-float multiple that score_stride gives; entries past a row's r(t) are never written."""
    rng = np.random.default_rng(d + G + nseq)
    Hkv = 2 if G < 32 else 1
    n, cap, k = 300, 5000, 4
    cfg = ra.Config(G * Hkv, Hkv, d, S, k, W, ra.RA_BF16, nseq, cap)
    mean = torch.from_numpy(rng.standard_normal((nseq, Hkv, cfg.max_spans, d)).astype(np.float32)).cuda()
    q = torch.from_numpy(rng.standard_normal((n, G * Hkv, d)).astype(np.float32)).to(torch.bfloat16).cuda()
    seqs = np.sort(rng.integers(0, nseq, n)).astype(np.int32)
    pos = rng.integers(0, cap, n)
    rows = ra.Rows(q, torch.from_numpy(seqs).cuda(), torch.from_numpy(pos).cuda(), int(pos.max()))
    r_max = cfg.num_routable(int(pos.max()))
    r = np.array([cfg.num_routable(int(t)) for t in pos])
    got = []
    for stride in (r_max, r_max + 1, ra.score_stride(cfg, int(pos.max()))):
        scores = torch.full((n, G * Hkv, stride), np.nan, dtype=torch.float32, device="cuda")
        sel = torch.full((n, G * Hkv, k), -7, dtype=torch.int32, device="cuda")
        ra.route_scores(cfg, rows, mean, scores)
        ra.topk_spans(cfg, rows, scores, sel)
        sc = scores.cpu().numpy()
        for i in range(n):
            assert not np.isnan(sc[i, :, :r[i]]).any() and np.isnan(sc[i, :, r[i]:]).all()
        got.append((np.concatenate([sc[i, :, :r[i]].ravel() for i in range(n)]), sel.cpu().numpy()))
    for sc, sel in got[1:]:
        assert np.array_equal(sc.view(np.uint32), got[0][0].view(np.uint32))
        assert np.array_equal(sel, got[0][1])


ROUTE_TOPK_CASES = [
    ("bf16_d128_G8", small("ragged_decode_16", batch=3, span_size=64, window=64, top_k=16, ragged=(3000, 60000))),
    ("bf16_d64_G4_W3S", small("ragged_decode_16", batch=2, head_dim=64, num_q_heads=8, num_kv_heads=2, span_size=32,
                              window=96, top_k=6, ragged=(700, 30000))),
    ("bf16_G32_k16", small("ragged_decode_16", batch=2, num_q_heads=32, num_kv_heads=1, span_size=64, window=64,
                           top_k=16, ragged=(2000, 20000))),
    ("bf16_r1000_k64", small("ragged_decode_16", batch=2, num_q_heads=8, num_kv_heads=2, span_size=16, window=16,
                             top_k=64, ragged=(12000, 17000))),
    ("fp32_d128_G4", small("tiny_prefill_fp32", mode="decode", batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                           span_size=128, window=200, top_k=4, ragged=(129, 50000))),
    ("bf16_short_rows_r0", small("ragged_decode_16", batch=3, span_size=64, window=64, top_k=8, ragged=(1, 130))),
    ("bf16_all_rows_r0", small("ragged_decode_16", batch=2, span_size=64, window=64, top_k=8, ragged=(1, 100))),
]


@pytest.mark.parametrize("name,w", ROUTE_TOPK_CASES, ids=[c[0] for c in ROUTE_TOPK_CASES])
def test_route_topk_spans_equals_route_then_topk(name, w):
    """The fused routing + selection gives exactly the selection of route_scores then
    topk_spans (the same fp32 scores, the same order), for every row and head; rows of several
    sequences and extra rows at earlier positions (other r) in one call.  Twenty calls in a row on
    one workspace (the last-arriving block of each (row, kv head) selects, and leaves its
    counter at zero) all give the same selection."""
    lengths = w.seq_lengths()
    c, rows, q = run_decode(w, lengths)
    rng = np.random.default_rng(5)
    seqs = np.concatenate([np.arange(c.B), rng.integers(0, c.B, 5)])
    pos = np.concatenate([lengths - 1, [rng.integers(0, lengths[s]) for s in seqs[c.B:]]])
    rows2, q2 = c.rows_for(seqs, pos)
    n = len(seqs)
    scores = torch.empty(n, w.num_q_heads, ra.score_stride(c.cfg, int(pos.max())), device="cuda")
    sel_ref = torch.full((n, w.num_q_heads, w.top_k), -7, dtype=torch.int32, device="cuda")
    ra.route_scores(c.cfg, rows2, c.pipe.span_mean, scores)
    ra.topk_spans(c.cfg, rows2, scores, sel_ref)
    ws = torch.zeros(ra.workspace_bytes(c.cfg, ra.RA_OP_ROUTE_TOPK, n, int(pos.max())), dtype=torch.uint8,
                     device="cuda")
    for rep in range(20):
        sel = torch.full_like(sel_ref, -9)
        ra.route_topk_spans(c.cfg, rows2, c.pipe.span_mean, sel, ws)
        torch.cuda.synchronize()
        assert torch.equal(sel, sel_ref), rep
    counters = ws[:4 * n * w.num_kv_heads].view(torch.int32)
    assert int(counters.abs().sum()) == 0
    # and the decode rows' selection is the oracle's (exact or a valid near tie)
    c.pipe.sel.copy_(sel[:c.B])
    stats = c.check(np.arange(c.B), lengths - 1, q, np.arange(c.B), scores=False)
    assert not stats["fail"], stats["fail"][:3]


# few rows up to 4000 routable spans: one launch up to 1088 spans (the largest call, 1088, with
# rows at block edges below it), route_scores + topk_spans inside the call beyond
FEW_LONG_ROUTE_TOPK_CASES = [
    # name, workload, cache length, the r of each row, edit
    ("r1088_k16_one_launch", small("ragged_decode_16", batch=1, span_size=16, window=16, top_k=16), 17450,
     [1088, 1087, 1024, 1023, 257, 256, 255, 129, 128, 127, 16, 15, 0], None),
    ("r1088_k64_one_launch", small("ragged_decode_16", batch=1, span_size=16, window=16, top_k=64), 17450,
     [1088, 1000, 200, 65, 64, 63, 0], None),
    ("r2559_k16", small("ragged_decode_16", batch=1, span_size=16, window=16, top_k=16), 41000,
     [2559, 2000, 1500, 1089, 1088, 700, 257, 256, 255, 128, 127, 5, 0], None),
    ("r4000_k16", small("ragged_decode_16", batch=1, span_size=16, window=16, top_k=16), 64100,
     [4000, 3999, 3000, 2049, 2048, 33], None),
    ("r4000_k1", small("ragged_decode_16", batch=1, span_size=16, window=16, top_k=1), 64100, [4000, 300, 1, 0],
     None),
    ("r2048_k64", small("ragged_decode_16", batch=1, span_size=16, window=16, top_k=64), 32800,
     [2048, 1500, 129, 64, 63, 0], None),
    ("r2100_k64_two_calls", small("ragged_decode_16", batch=1, span_size=16, window=16, top_k=64), 34000,
     [2100, 1000], None),
    ("r2559_all_scores_tie", small("ragged_decode_16", batch=1, span_size=16, window=16, top_k=16), 41000,
     [2559, 1000, 129, 3], "constant_keys"),
]


@pytest.mark.parametrize("name,w,length,want_r,edit", FEW_LONG_ROUTE_TOPK_CASES,
                         ids=[c[0] for c in FEW_LONG_ROUTE_TOPK_CASES])
def test_route_topk_spans_few_rows_many_spans(name, w, length, want_r, edit):
    """Decode-shaped calls (fewer than 256 row-heads per kv head) with up to 4000 routable spans:
    route_topk_spans equals route_scores then topk_spans for every row and head, on three calls in
    a row, with its counters back at zero; rows with r from 0 up, across the one-launch path's
    128-span block edges and its largest call (r = 1088), k = 1, 16 and 64, a cache whose keys are
    all equal (every score ties: the lowest indices win), and calls past the one-launch limit."""
    c = Case(w, [length])
    if edit == "constant_keys":
        one = torch.full((w.head_dim,), 0.5, dtype=torch.bfloat16)
        kh = c.host[0][0]
        kh[:] = one.view(torch.int16).numpy().view(np.uint16)
        c.K[0, :, :length] = one.cuda()
        c._problems.clear()
    L = c.lengths
    c.summarize(np.zeros(c.B, dtype=np.int64), L)
    rng = np.random.default_rng(31)
    S, Wn = w.span_size, w.window
    pos = np.array([min(length - 1, r * S + Wn - 1 + int(rng.integers(0, S))) for r in want_r])
    got_r = [c.cfg.num_routable(int(t)) for t in pos]
    assert got_r == want_r, got_r
    seqs = np.zeros(len(pos), dtype=np.int64)
    rows, _ = c.rows_for(seqs, pos)
    n = len(seqs)
    assert n * w.group < 256  # the few-row regime
    scores = torch.empty(n, w.num_q_heads, ra.score_stride(c.cfg, int(pos.max())), device="cuda")
    sel_ref = torch.full((n, w.num_q_heads, w.top_k), -7, dtype=torch.int32, device="cuda")
    ra.route_scores(c.cfg, rows, c.pipe.span_mean, scores)
    ra.topk_spans(c.cfg, rows, scores, sel_ref)
    ws = torch.zeros(ra.workspace_bytes(c.cfg, ra.RA_OP_ROUTE_TOPK, n, int(pos.max())), dtype=torch.uint8,
                     device="cuda")
    for rep in range(3):
        sel = torch.full_like(sel_ref, -9)
        ra.route_topk_spans(c.cfg, rows, c.pipe.span_mean, sel, ws)
        torch.cuda.synchronize()
        if not torch.equal(sel, sel_ref):
            bad = (sel != sel_ref).any(dim=2).nonzero()[:4].tolist()
            raise AssertionError("rep %d: %d row-heads differ, e.g. %s: %s vs %s" % (
                rep, int((sel != sel_ref).any(dim=2).sum()), bad, sel[bad[0][0], bad[0][1]].tolist(),
                sel_ref[bad[0][0], bad[0][1]].tolist()))
    counters = ws[:4 * n * w.num_kv_heads].view(torch.int32)
    assert int(counters.abs().sum()) == 0
    if edit == "constant_keys":  # every score ties: the m lowest routable indices
        for i, r in enumerate(want_r):
            m = min(w.top_k, r)
            want = np.concatenate([np.arange(m), np.full(w.top_k - m, -1)]).astype(np.int32)
            assert (sel[i].cpu().numpy() == want[None, :]).all(), (r, sel[i, 0].tolist())
    log("  %s: %d rows x %d heads, r up to %d" % (name, n, w.num_q_heads, max(want_r)))


# many rows and long rows: route_topk_spans runs route_scores + topk_spans through its workspace;
# the selection must be that of the two calls, bit for bit
MANY_ROUTE_TOPK_CASES = [
    # name, workload, lengths, rows: (sequence, position) pairs drawn per sequence, edit
    ("d128_G8_r999", small("ragged_decode_16", batch=1, span_size=64, window=64, top_k=16), [64000], 48, None),
    ("d128_G8_r1025_to_1061", small("ragged_decode_16", batch=1, span_size=64, window=64, top_k=16), [68000], 48,
     "late_rows"),
    ("d64_G4_two_seqs", small("ragged_decode_16", batch=2, head_dim=64, num_q_heads=16, num_kv_heads=4, span_size=32,
                              window=32, top_k=8), [32000, 20000], 40, None),
    ("d128_small_r", small("ragged_decode_16", batch=1, span_size=64, window=64, top_k=16), [64000], 0, "small_r"),
    ("d128_all_scores_tie", small("ragged_decode_16", batch=1, span_size=64, window=64, top_k=16), [40000], 48,
     "constant_keys"),
    ("d128_k32", small("ragged_decode_16", batch=1, span_size=64, window=64, top_k=32), [64000], 48,
     None),
    ("d128_r1249", small("ragged_decode_16", batch=1, span_size=16, window=16, top_k=16), [20000], 48,
     None),
    ("d128_k64", small("ragged_decode_16", batch=1, span_size=64, window=64, top_k=64), [64000], 48, None),
    ("d128_k64_small_r", small("ragged_decode_16", batch=1, span_size=64, window=64, top_k=64), [64000], 0,
     "small_r"),
]


@pytest.mark.parametrize("name,w,lengths,per_seq,edit", MANY_ROUTE_TOPK_CASES,
                         ids=[c[0] for c in MANY_ROUTE_TOPK_CASES])
def test_route_topk_spans_many_rows_equals_route_then_topk(name, w, lengths, per_seq, edit):
    """Prefill-shaped calls (at least 256 row-heads per kv head): route_topk_spans equals
    route_scores then topk_spans for every row and head, on two calls in a row.  Cases: r near
    1000 and from 1025 to 1061, rows of two sequences interleaved, rows with r from 0 to 1000, a
    cache whose keys are all equal (every score ties), k = 32 and 64 (the largest, also with r
    from 0 to 1000), and r up to 1249."""
    c = Case(w, lengths)
    if edit == "constant_keys":
        one = torch.full((w.head_dim,), 0.5, dtype=torch.bfloat16)
        kh = c.host[0][0]
        kh[:] = one.view(torch.int16).numpy().view(np.uint16)
        c.K[0, :, :lengths[0]] = one.cuda()
        c._problems.clear()
    L = c.lengths
    c.summarize(np.zeros(c.B, dtype=np.int64), L)
    rng = np.random.default_rng(23)
    if edit == "small_r":
        S, W = w.span_size, w.window
        want_r = [0, 1, 5, 16, 31, 32, 33, 40, 100, 255, 256, 300, 700, 999]
        pos = np.array([min(int(L[0]) - 1, r * S + W - 1 + int(rng.integers(0, S))) for r in want_r for _ in range(24)])
        seqs = np.zeros(len(pos), dtype=np.int64)
    elif edit == "late_rows":  # r from 1025 to 1061
        seqs = np.zeros(per_seq, dtype=np.int64)
        pos = rng.integers(1025 * w.span_size + w.window - 1, int(L[0]), per_seq)
    else:
        seqs = np.repeat(np.arange(c.B), per_seq)
        pos = np.concatenate([rng.integers(int(L[b]) // 2, int(L[b]), per_seq) for b in range(c.B)])
        order = rng.permutation(len(seqs))  # sequences interleaved within tiles
        seqs, pos = seqs[order], pos[order]
    rows, _ = c.rows_for(seqs, pos)
    n = len(seqs)
    assert n * w.group >= 256  # the many-row regime
    scores = torch.empty(n, w.num_q_heads, ra.score_stride(c.cfg, int(pos.max())), device="cuda")
    sel_ref = torch.full((n, w.num_q_heads, w.top_k), -7, dtype=torch.int32, device="cuda")
    ra.route_scores(c.cfg, rows, c.pipe.span_mean, scores)
    ra.topk_spans(c.cfg, rows, scores, sel_ref)
    ws = torch.zeros(ra.workspace_bytes(c.cfg, ra.RA_OP_ROUTE_TOPK, n, int(pos.max())), dtype=torch.uint8,
                     device="cuda")
    for rep in range(2):
        sel = torch.full_like(sel_ref, -9)
        ra.route_topk_spans(c.cfg, rows, c.pipe.span_mean, sel, ws)
        torch.cuda.synchronize()
        if not torch.equal(sel, sel_ref):
            bad = (sel != sel_ref).any(dim=2).nonzero()[:4].tolist()
            raise AssertionError("rep %d: %d row-heads differ, e.g. %s: %s vs %s" % (
                rep, int((sel != sel_ref).any(dim=2).sum()), bad, sel[bad[0][0], bad[0][1]].tolist(),
                sel_ref[bad[0][0], bad[0][1]].tolist()))
    log("  %s: %d rows x %d heads, r up to %d" % (name, n, w.num_q_heads, c.cfg.num_routable(int(pos.max()))))
