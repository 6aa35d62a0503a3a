"""GPU tests of the decode calls that carry the step's summary update
(routed_attn_decode_append, routed_attn_decode_fp8_append): routing on the summaries before the
update, then the call, gives bit for bit the outputs and summaries of the unfused order (update,
route, select, attend), which the other GPU tests compare with the oracle.
"""
import numpy as np
import pytest
import torch

import content_routed_sparse_amd as ra
from synth import workloads as WL

from harness import Case

pytestmark = pytest.mark.gpu

W = WL.WORKLOADS


def small(base, **kw):
    return W[base].scaled(**kw)


def fresh_summaries(c, upto):
    """span_mean / run_sum of the first upto[b] tokens of each sequence (device)."""
    p = ra.Pipeline(c.cfg)
    zero = torch.zeros(c.B, dtype=torch.int64, device="cuda")
    up = torch.as_tensor(np.asarray(upto, dtype=np.int64)).cuda()
    ra.span_summary_update(c.cfg, c.K, p.span_mean, p.run_sum, zero, up, int(max(upto)))
    return p


def unfused(c, rows, before, after, n_new):
    """The reference order: update, route, select, attend."""
    p = fresh_summaries(c, before)
    b_t = torch.as_tensor(np.asarray(before, dtype=np.int64)).cuda()
    a_t = torch.as_tensor(np.asarray(after, dtype=np.int64)).cuda()
    ra.span_summary_update(c.cfg, c.K, p.span_mean, p.run_sum, b_t, a_t, n_new)
    out = p.attend(rows, c.K, c.V, ra.RA_OP_DECODE).clone()
    torch.cuda.synchronize()
    return out, p


def fused(c, rows, before, after, n_new):
    """Route and select on the summaries before the update, then attend with the append."""
    p = fresh_summaries(c, before)
    p.reserve(rows.q.shape[0], rows.max_pos, ra.RA_OP_DECODE)
    ra.route_scores(c.cfg, rows, p.span_mean, p.scores)
    ra.topk_spans(c.cfg, rows, p.scores, p.sel)
    b_t = torch.as_tensor(np.asarray(before, dtype=np.int64)).cuda()
    a_t = torch.as_tensor(np.asarray(after, dtype=np.int64)).cuda()
    ra.routed_attn_decode_append(c.cfg, rows, c.K, c.V, p.sel, p.out, p.workspace, p.span_mean, p.run_sum, b_t, a_t,
                                 n_new)
    torch.cuda.synchronize()
    return p.out.clone(), p


def assert_same(u, f):
    (o1, p1), (o2, p2) = u, f
    assert torch.equal(o1, o2), "outputs differ"
    assert torch.equal(p1.span_mean, p2.span_mean), "span means differ"
    assert torch.equal(p1.run_sum, p2.run_sum), "running sums differ"


CASES = [
    # name, workload, lengths (the last token of each closes a span when L % S == 0)
    ("bf16_d128_closing", small("decode_1m", span_size=64, window=64, top_k=8, decode_len=4096), [4096]),
    ("bf16_d128_open", small("decode_1m", span_size=64, window=64, top_k=8, decode_len=4000), [4000]),
    ("bf16_ragged3", small("ragged_decode_16", batch=3, span_size=64, window=96, top_k=6, ragged=(3000, 9000)), None),
    ("fp32_d64", W["tiny_prefill_fp32"], [4096, 1500]),
    ("bf16_d64_G4_W1", small("decode_1m", num_q_heads=8, num_kv_heads=2, head_dim=64, span_size=32, window=1,
                             top_k=5, decode_len=3200), [3200, 3199, 40]),
]


@pytest.mark.parametrize("name,w,lengths", CASES, ids=[c[0] for c in CASES])
def test_decode_append_equals_update_then_decode(name, w, lengths):
    L = np.asarray(lengths if lengths is not None else w.seq_lengths(), dtype=np.int64)
    c = Case(w, L)
    rows, _ = c.rows_for(np.arange(c.B), L - 1)
    assert_same(unfused(c, rows, L - 1, L, 1), fused(c, rows, L - 1, L, 1))


def test_decode_append_of_several_tokens_runs_after_the_merge():
    """Five new tokens per sequence (its own launches after the merge), window >= span."""
    w = small("decode_1m", span_size=32, window=64, top_k=4, decode_len=2050)
    L = np.array([2050, 1600], dtype=np.int64)
    c = Case(w, L)
    rows, _ = c.rows_for(np.arange(2), L - 1)
    assert_same(unfused(c, rows, L - 5, L, 5), fused(c, rows, L - 5, L, 5))


def test_decode_append_with_no_rows_only_updates():
    w = small("decode_1m", span_size=64, window=64, top_k=4, decode_len=1000)
    c = Case(w, [1000])
    p = fresh_summaries(c, [999])
    q = torch.zeros(0, w.num_q_heads, w.head_dim, dtype=torch.bfloat16, device="cuda")
    rows = ra.Rows(q, torch.zeros(0, dtype=torch.int32, device="cuda"), torch.zeros(0, dtype=torch.int64,
                                                                                     device="cuda"), 999)
    empty = torch.empty(0, w.num_q_heads, w.top_k, dtype=torch.int32, device="cuda")
    out = torch.empty(0, w.num_q_heads, w.head_dim, dtype=torch.float32, device="cuda")
    ws = torch.empty(1, dtype=torch.uint8, device="cuda")
    ra.routed_attn_decode_append(c.cfg, rows, c.K, c.V, empty, out, ws, p.span_mean, p.run_sum,
                                 torch.tensor([999]).cuda(), torch.tensor([1000]).cuda(), 1)
    ref = fresh_summaries(c, [1000])
    torch.cuda.synchronize()
    assert torch.equal(p.span_mean, ref.span_mean) and torch.equal(p.run_sum, ref.run_sum)


def test_fp8_decode_append_equals_update_then_decode():
    w = small("decode_1m", span_size=64, window=64, top_k=8, decode_len=4096)
    L = np.array([4096, 2500], dtype=np.int64)
    c = Case(w, L)
    cfg = c.cfg
    K8 = torch.empty(tuple(c.K.shape), dtype=torch.uint8, device="cuda")
    V8 = torch.empty_like(K8)
    KS = torch.empty(tuple(c.K.shape[:3]), dtype=torch.float32, device="cuda")
    VS = torch.empty_like(KS)
    zero = torch.zeros(2, dtype=torch.int64, device="cuda")
    full = torch.as_tensor(L).cuda()
    ra.kv_quantize_fp8(cfg, c.K, K8, KS, zero, full, int(L.max()))
    ra.kv_quantize_fp8(cfg, c.V, V8, VS, zero, full, int(L.max()))
    rows, _ = c.rows_for(np.arange(2), L - 1)
    before = torch.as_tensor(L - 1).cuda()
    results = []
    for mode in ("unfused", "fused"):
        p = ra.Pipeline(cfg)
        ra.span_summary_update_fp8(cfg, K8, KS, p.span_mean, p.run_sum, zero, before, int(L.max() - 1))
        p.reserve(2, rows.max_pos, ra.RA_OP_DECODE)
        if mode == "unfused":
            ra.span_summary_update_fp8(cfg, K8, KS, p.span_mean, p.run_sum, before, full, 1)
        ra.route_scores(cfg, rows, p.span_mean, p.scores)
        ra.topk_spans(cfg, rows, p.scores, p.sel)
        if mode == "unfused":
            ra.routed_attn_decode_fp8(cfg, rows, K8, V8, KS, VS, p.sel, p.out, p.workspace)
        else:
            ra.routed_attn_decode_fp8_append(cfg, rows, K8, V8, KS, VS, p.sel, p.out, p.workspace, p.span_mean,
                                             p.run_sum, before, full, 1)
        torch.cuda.synchronize()
        results.append((p.out.clone(), p))
    assert_same(results[0], results[1])
