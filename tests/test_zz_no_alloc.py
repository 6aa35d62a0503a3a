"""routed_attn_decode_noalloc (the decode entry point that allocates nothing: its partial records
go to the library's fixed device scratch) against routed_attn_decode with a caller workspace,
through the C ABI: bit for bit, on two calls in a row, the second with fewer rows and other
sequences (the scratch keeps the first call's contents), and a call past the scratch limit is
rejected before any launch."""
import numpy as np
import pytest
import torch

import content_routed_sparse_amd as ra
from synth import workloads as WL

from harness import Case, assert_stats, log, run_decode

pytestmark = pytest.mark.gpu


def _both(c, rows, sel):
    n = rows.q.shape[0]
    w = c.w
    ref = torch.full((n, w.num_q_heads, w.head_dim), np.nan, device="cuda")
    ws = torch.empty(ra.workspace_bytes(c.cfg, ra.RA_OP_DECODE, n, rows.max_pos), dtype=torch.uint8, device="cuda")
    ra.routed_attn_decode(c.cfg, rows, c.K, c.V, sel, ref, ws)
    got = torch.full_like(ref, np.nan)
    ra.routed_attn_decode_noalloc(c.cfg, rows, c.K, c.V, sel, got)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_decode_equals_the_workspace_entry_point():
    w = WL.WORKLOADS["ragged_decode_16"].scaled(batch=6, span_size=64, window=64, top_k=8, ragged=(3000, 9000))
    lengths = w.seq_lengths()
    c, rows, q = run_decode(w, lengths)
    sel = c.pipe.sel
    # first call: all 6 sequences
    ref, got = _both(c, rows, sel)
    assert torch.equal(ref, c.pipe.out)
    assert torch.equal(got, ref)
    stats = c.check(np.arange(c.B), lengths - 1, q, np.arange(c.B))
    assert_stats(stats, True)
    # second call: 2 other rows in another order (fewer records than the first call left behind)
    pick = [4, 1]
    rows2, q2 = c.rows_for(pick, lengths[pick] - 1)
    sel2 = sel[pick].contiguous()
    ref2, got2 = _both(c, rows2, sel2)
    assert torch.equal(got2, ref2)
    assert torch.equal(got2, ref[pick])
    log("  noalloc decode: bitwise equal on %d then %d rows" % (c.B, len(pick)))


def test_noalloc_decode_rejects_calls_past_its_scratch():
    w = WL.WORKLOADS["decode_1m"].scaled(span_size=64, window=64, top_k=64, decode_len=70000)
    c = Case(w, [70000])
    n = 80  # 80 rows x 32 heads x (64 + 2) entries x 1 sub-tile x 528 bytes > 32 MiB
    rows, _ = c.rows_for([0] * n, [69999] * n)
    need = ra.workspace_bytes(c.cfg, ra.RA_OP_DECODE, n, 69999)
    assert need > 32 << 20
    sel = torch.full((n, w.num_q_heads, w.top_k), -1, dtype=torch.int32, device="cuda")
    out = torch.empty(n, w.num_q_heads, w.head_dim, device="cuda")
    with pytest.raises(ra.RoutedAttnError) as e:
        ra.routed_attn_decode_noalloc(c.cfg, rows, c.K, c.V, sel, out)
    assert e.value.status == 3 and "scratch" in str(e.value)
