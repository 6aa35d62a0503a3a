"""Benchmark: one decode step of content-routed sparse attention at 1M context, on one GPU.

A step is the whole hot path for one new token of one sequence at L = 1,048,576 (32 query
heads, 4 kv heads, d = 128, bf16 cache, spans of 1024, top-16 + window of 1024):
route_topk_spans (route_scores and topk_spans in one launch) -> routed_attn_decode_append (the
attention and, in its merge launch, the new token's span-summary update; equivalent to updating
first, since the token completes no routable span).
Inputs are synthetic (seeded generator), resident in HBM before timing starts.

So that every step reads its keys and values from HBM rather than from the 256 MB Infinity
Cache, the bench keeps `--caches` independent 1M-token sequences (2 GiB of K/V each) and step
i works on sequence i mod caches; each step is the same single-sequence workload.

Further objects in the same line (each with its own roofline): the 8-bit cache decode step, the
token-level cold retrieval step, a session snapshot of one 1M-token state, the chunked prefill
(8192 tokens on 1M) with dense causal attention beside it and the routed-vs-dense ladder (the same
chunk after 128K, 256K, 512K and 1M tokens), the CPU oracle's rate, and the decode steps of the
10M-token and ragged 16-sequence workloads.

Prints one JSON line.  `--gpus` above 1 is refused: this path runs on one GPU.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed-attn decode & prefill tokens/s per layer @1M ctx; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--caches", type=int, default=4)
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", action="store_true", help="replay the step from HIP graphs instead of launching")
    p.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill measurement")
    p.add_argument("--prefill-steps", type=int, default=10)
    p.add_argument("--dense-steps", type=int, default=2,
                   help="timed calls of dense causal attention on the prefill rows (0: skip)")
    p.add_argument("--no-ladder", action="store_true",
                   help="skip the routed-vs-dense ladder (the same chunk after 128K, 256K and 512K tokens)")
    p.add_argument("--no-fp8", action="store_true", help="skip the decode and prefill steps over the 8-bit cache")
    p.add_argument("--no-snapshot", action="store_true", help="skip the session snapshot / restore measurement")
    p.add_argument("--no-cold", action="store_true", help="skip the token-level cold retrieval decode step")
    p.add_argument("--no-tiny", action="store_true", help="skip the tiny fp32 prefill (4096 tokens, d = 64)")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the decode steps of the 10M-token and ragged 16-sequence workloads")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a 256 MiB device copy (reference kernel for HBM byte counters)")
    return p.parse_args()


def progress(msg):
    """One line on stderr as each leg ends (stdout carries only the JSON line)."""
    print("[bench] %s (%.0f s)" % (msg, time.time() - T_START), file=sys.stderr, flush=True)


T_START = time.time()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs the single-GPU path only (one GPU per process, no sharding); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import content_routed_sparse_amd as ra
    from synth import BF16
    from synth import workloads as WL

    w = WL.WORKLOADS["decode_1m"]
    L = w.decode_len
    NC = args.caches
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg1 = ra.Config(w.num_q_heads, w.num_kv_heads, w.head_dim, w.span_size, w.top_k, w.window, ra.RA_BF16, 1, L)

    # ---- inputs: NC independent sequences, generated on the host, copied once into HBM
    t0 = time.time()
    K = torch.empty(NC, w.num_kv_heads, L, w.head_dim, dtype=torch.bfloat16, device=dev)
    V = torch.empty_like(K)
    for s in range(NC):
        K[s] = torch.from_numpy(WL.kv_slab(w, s, 0, L, "k").view(np.int16)).view(torch.bfloat16).to(dev)
        V[s] = torch.from_numpy(WL.kv_slab(w, s, 0, L, "v").view(np.int16)).view(torch.bfloat16).to(dev)
    qs = [torch.from_numpy(WL.query_at(w, s, L - 1)[None].view(np.int16)).view(torch.bfloat16).to(dev)
          for s in range(NC)]
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    progress("decode_1m caches ready")

    # ---- per-sequence state and buffers (allocated once)
    stride = ra.score_stride(cfg1, L - 1)
    st = []
    for s in range(NC):
        d = {
            "k": K[s:s + 1], "v": V[s:s + 1],
            "mean": torch.zeros(1, w.num_kv_heads, cfg1.max_spans, w.head_dim, dtype=torch.float32, device=dev),
            "run": torch.zeros(1, w.num_kv_heads, w.head_dim, dtype=torch.float32, device=dev),
            "rows": ra.Rows(qs[s], torch.zeros(1, dtype=torch.int32, device=dev),
                            torch.full((1,), L - 1, dtype=torch.int64, device=dev), L - 1),
            "scores": torch.empty(1, w.num_q_heads, stride, dtype=torch.float32, device=dev),
            "sel": torch.empty(1, w.num_q_heads, w.top_k, dtype=torch.int32, device=dev),
            "out": torch.empty(1, w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev),
        }
        st.append(d)
    ws = torch.empty(ra.workspace_bytes(cfg1, ra.RA_OP_DECODE, 1, L - 1), dtype=torch.uint8, device=dev)
    zero = torch.zeros(1, dtype=torch.int64, device=dev)
    before = torch.full((1,), L - 1, dtype=torch.int64, device=dev)
    after = torch.full((1,), L, dtype=torch.int64, device=dev)
    # setup (untimed): summaries of the L-1 tokens already in each cache
    for d in st:
        ra.span_summary_update(cfg1, d["k"], d["mean"], d["run"], zero, before, L - 1)
    torch.cuda.synchronize()

    # the step's calls, validated once per sequence and replayed (ctypes only per call): routing
    # and selection, then the attention with the new token's summary update in its merge launch.
    # The new token (position L-1) completes no span that is routable at L-1 (that span lies in
    # the window) and routing does not read the running sum, so this order selects exactly what
    # update-then-route does.  Re-running the step re-closes that span: every step is the same work.
    for d in st:
        d["calls_front"], front_kind = front_calls(ra, cfg1, d["rows"], d["mean"], d["scores"], d["sel"])
        d["call_attn"] = ra.prepare("routed_attn_decode_append", cfg1, d["rows"], d["k"], d["v"], d["sel"], d["out"],
                                    ws, d["mean"], d["run"], before, after, 1)

    def front(d):
        for c in d["calls_front"]:
            c()

    def attend(d):
        d["call_attn"]()

    # eager reference outputs of each sequence's step
    for d in st:
        front(d)
        attend(d)
    torch.cuda.synchronize()
    first = [d["out"].clone() for d in st]

    # Optionally the step is captured as two HIP graphs per sequence (summary + routing +
    # selection, then the attention).  Each graph launch costs a few microseconds of queue time,
    # so back-to-back launches of prepared calls are the default.
    graphs = []
    if args.graph:
        cap = torch.cuda.Stream()
        for d in st:
            ga, gb = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(ga, stream=cap):
                front(d)
            with torch.cuda.graph(gb, stream=cap):
                attend(d)
            graphs.append((ga, gb))
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    # HIP events around routed_attn_decode on every EV_EVERY-th timed step (an event pair adds a
    # few microseconds of queue gaps, so it is not recorded on every step)
    EV_EVERY = 8
    timed_ev = list(range(0, args.steps, EV_EVERY))
    ev = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for i in timed_ev}

    def step(i, timed):
        s = i % NC
        if graphs:
            graphs[s][0].replay()
        else:
            front(st[s])
        if timed and i in ev:
            ev[i][0].record(stream)
        if graphs:
            graphs[s][1].replay()
        else:
            attend(st[s])
        if timed and i in ev:
            ev[i][1].record(stream)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    warm_same = all(torch.equal(first[s], st[s]["out"]) for s in range(NC))

    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start

    ms_per_step = t_total * 1e3 / args.steps
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in ev.values()]))
    same = warm_same and all(torch.equal(first[s], st[s]["out"]) for s in range(NC))

    # ---- algorithmic bytes of routed_attn_decode: K and V rows of the union of the spans the
    # query heads of each kv head selected, plus the window, plus q (bf16) and out (fp32)
    G = w.group
    win = (L - 1) - (w.span_size * (max(0, L - 1 - w.window + 1) // w.span_size)) + 1
    per_seq = []
    for d in st:
        sel = d["sel"][0].cpu().numpy()
        uni = sum(len(set(sel[g * G:(g + 1) * G].ravel().tolist()) - {-1}) for g in range(w.num_kv_heads))
        kv = (uni * w.span_size + w.num_kv_heads * win) * w.head_dim * 2 * 2
        # + the summary update: the new K row, the running sum read and written, per kv head
        per_seq.append(kv + w.num_q_heads * w.head_dim * (2 + 4) + w.num_kv_heads * w.head_dim * (2 + 8))
    bytes_step = float(np.mean([per_seq[i % NC] for i in timed_ev]))
    achieved = bytes_step / (attn_ms * 1e-3) / 1e9
    # the whole step also reads the summaries of every routable span (routing)
    route_bytes = ((L - w.window) // w.span_size) * w.num_kv_heads * w.head_dim * 4
    step_gbs = (bytes_step + route_bytes) / (ms_per_step * 1e-3) / 1e9

    traffic = counter_traffic("routed_attn_decode_1m")

    result = {
        "metric": METRIC,
        "value": round(1000.0 / ms_per_step, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_1m", "context": L, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "span": w.span_size, "top_k": w.top_k, "window": w.window, "batch": 1,
                   "rotated_sequences": NC, "hip_graphs": bool(args.graph), "routing_calls": front_kind},
        "roofline": {"bound": "hbm",
                     "kernel": "routed_attn_decode_append (decode_attn + merge launch with the token's summary update)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": int(bytes_step), "avg_launch_ms": round(attn_ms, 5)},
        "step_roofline": {"bound": "hbm", "what": "the whole step (route + top-k + attention with the update)",
                          "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                          "algorithmic_bytes_per_step": int(bytes_step + route_bytes)},
        "repeat_bitwise_identical": bool(same),
        "setup_seconds": round(gen_s, 1),
    }
    progress("decode_1m done")

    if not args.no_fp8:
        result["decode_fp8"] = bench_decode_fp8(args, w, K, V, qs)
        progress("decode_fp8 done")

    if not args.no_cold:
        result["cold_retrieval"] = bench_cold(args, w, K, V, qs)
        progress("cold_retrieval done")

    if not args.no_snapshot:
        result["snapshot"] = bench_snapshot(w, st[0], cfg1)
        progress("snapshot done")

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    if not args.no_cpu_baseline:
        kv0 = [(WL.kv_slab(w, 0, 0, L, "k"), WL.kv_slab(w, 0, 0, L, "v"))]
        result["cpu_baseline"], result["oracle_check"] = oracle_decode_baseline(
            w, kv0, [L], [WL.query_at(w, 0, L - 1)], args.cpu_seconds, st[0]["sel"].cpu().numpy(),
            st[0]["out"].cpu().numpy())
        del kv0
        progress("decode_1m cpu baseline done")

    if not args.no_prefill:
        del K, V, st
        torch.cuda.empty_cache()
        result["prefill"] = bench_prefill(args.prefill_steps, args.dense_steps, not args.no_ladder,
                                          0.0 if args.no_cpu_baseline else args.cpu_seconds, not args.no_fp8,
                                          args.warmup)
        progress("prefill done")

    if not args.no_extra:
        if args.no_prefill:
            del K, V, st
            torch.cuda.empty_cache()
        result["decode_other"] = [bench_decode_workload(name, max(8, args.steps // 2), args.warmup,
                                                        0.0 if args.no_cpu_baseline else args.cpu_seconds)
                                  for name in ("decode_10m", "ragged_decode_16")]
        progress("decode_other done")

    if not args.no_tiny:
        result["tiny_prefill"] = bench_tiny_prefill(max(20, args.steps // 4), 0.0 if args.no_cpu_baseline else
                                                    args.cpu_seconds)
        progress("tiny_prefill done")

    print(json.dumps(result), flush=True)


def front_calls(ra, cfg, rows, mean, scores, sel):
    """The step's routing and selection: route_topk_spans (its zeroed workspace is allocated here,
    untimed; one launch for these shapes up to 1088 routable spans, route_scores + topk_spans inside
    the call beyond).  `scores` is unused: the call keeps its scores in its workspace."""
    import torch

    n = rows.q.shape[0]
    ws = torch.zeros(ra.workspace_bytes(cfg, ra.RA_OP_ROUTE_TOPK, n, rows.max_pos), dtype=torch.uint8,
                     device=rows.q.device)
    fused = ra.prepare("route_topk_spans", cfg, rows, mean, sel, ws)
    fused._ws = ws  # keeps the workspace alive with the prepared call
    r = cfg.num_routable(rows.max_pos)
    return [fused], "route_topk_spans" if r <= 64 * 17 else "route_topk_spans (route_scores + topk_spans inside)"


def counter_traffic(tag):
    """HBM bytes per call measured with rocprofv3 counters (profiles/<tag>_traffic.json), or
    None when the kernel sources changed since they were taken."""
    tf = os.path.join(ROOT, "profiles", tag + "_traffic.json")
    if not os.path.exists(tf):
        return None
    rec = json.load(open(tf))
    h = hashlib.sha256()
    for f in rec.get("sources", []):
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return rec.get("bytes_per_launch") if rec.get("source_sha256") == h.hexdigest() else None


def bench_prefill(steps, dense_steps=2, ladder=True, cpu_seconds=0.0, fp8=True, warmup=10):
    """Chunked prefill: 8192 new tokens appended to a 1M-token cache (the chunk's K/V are in
    the cache before timing).  A step = span_summary_update of the chunk + route_topk_spans
    (route_scores + topk_spans in one call) + routed_attn_prefill for its 8192 x 32 row-heads.
    With fp8, the same step over the cache quantised to E4M3 codes (kv_quantize_fp8, untimed
    setup)."""
    import torch

    import content_routed_sparse_amd as ra
    from synth import workloads as WL

    w = WL.WORKLOADS["prefill_8k_on_1m"]
    P, n = w.prefix_len, w.chunk_len
    L = P + n
    dev = torch.device("cuda:0")
    cfg = ra.Config(w.num_q_heads, w.num_kv_heads, w.head_dim, w.span_size, w.top_k, w.window, ra.RA_BF16, 1, L)
    kh, vh, qh = WL.kv_slab(w, 0, 0, L, "k"), WL.kv_slab(w, 0, 0, L, "v"), WL.queries(w, 0, P, n)
    K = torch.from_numpy(kh.view(np.int16)).view(torch.bfloat16)[None].to(dev)
    V = torch.from_numpy(vh.view(np.int16)).view(torch.bfloat16)[None].to(dev)
    q = torch.from_numpy(qh.view(np.int16)).view(torch.bfloat16).to(dev)
    rows = ra.Rows(q, torch.zeros(n, dtype=torch.int32, device=dev),
                   torch.arange(P, L, dtype=torch.int64, device=dev), L - 1)
    mean = torch.zeros(1, w.num_kv_heads, cfg.max_spans, w.head_dim, dtype=torch.float32, device=dev)
    run = torch.zeros(1, w.num_kv_heads, w.head_dim, dtype=torch.float32, device=dev)
    t_p, t_l = torch.tensor([P], device=dev), torch.tensor([L], device=dev)
    ra.span_summary_update(cfg, K, mean, run, torch.zeros(1, dtype=torch.int64, device=dev), t_p, P)  # setup
    progress("prefill cache ready")
    sel = torch.empty(n, w.num_q_heads, w.top_k, dtype=torch.int32, device=dev)
    out = torch.empty(n, w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev)
    ws = torch.empty(ra.workspace_bytes(cfg, ra.RA_OP_PREFILL, n, L - 1), dtype=torch.uint8, device=dev)
    # the chunk starts and ends on span boundaries, so re-running the step recomputes the same
    # summaries and leaves the running sum at zero: every step is the same work
    # routing + selection in one call (route_topk_spans: the scores stay on chip; the same selection
    # as route_scores + topk_spans); its workspace starts zeroed, untimed
    ws_rt = torch.zeros(ra.workspace_bytes(cfg, ra.RA_OP_ROUTE_TOPK, n, L - 1), dtype=torch.uint8, device=dev)
    calls = [ra.prepare("span_summary_update", cfg, K, mean, run, t_p, t_l, n),
             ra.prepare("route_topk_spans", cfg, rows, mean, sel, ws_rt)]
    attn = ra.prepare("routed_attn_prefill", cfg, rows, K, V, sel, out, ws)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for _ in range(max(1, warmup)):  # untimed steps, as for decode (clocks and caches settle)
        for c in calls:
            c()
        attn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        for c in calls:
            c()
        ev[i][0].record(stream)
        attn()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / steps
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    alg_bytes = prefill_algorithmic_bytes(w, sel.cpu().numpy(), 2)
    # algorithmic work: 4 d flops per (row-head, attended key) for Q.K^T and P.V, plus 2 d per
    # (row-head, routable span) for routing; attended keys = selected spans' keys + window
    pos = np.arange(P, L)
    S, W = w.span_size, w.window
    w0 = S * (np.maximum(0, pos - W + 1) // S)
    r = w0 // S
    m = np.minimum(w.top_k, r)
    keys = (m * S + (pos - w0 + 1)).astype(np.float64)
    d = w.head_dim
    attn_flops = 4.0 * d * keys.sum() * w.num_q_heads
    route_flops = 2.0 * d * r.astype(np.float64).sum() * w.num_q_heads
    tflops = attn_flops / (attn_ms * 1e-3) / 1e12

    progress("prefill bf16 done")
    fp8_leg = bench_prefill_fp8(w, cfg, K, V, rows, t_p, t_l, steps, attn_flops, route_flops, out, warmup) if fp8 else None
    if fp8:
        progress("prefill fp8 done")

    # the same rows with dense causal attention over the whole prefix (the brute-force scan that
    # routing replaces; its flops are 4 d per (row-head, key <= t))
    dense = None
    if dense_steps > 0:
        out_d = torch.empty_like(out)
        call = ra.prepare("attn_dense_causal", cfg, rows, K, V, out_d)
        call()
        torch.cuda.synchronize()
        evd = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(dense_steps)]
        for a, b in evd:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        dense_ms = float(np.mean([a.elapsed_time(b) for a, b in evd]))
        dense_flops = 4.0 * d * (pos + 1).astype(np.float64).sum() * w.num_q_heads
        dtf = dense_flops / (dense_ms * 1e-3) / 1e12
        dense = {"kernel": "attn_dense_causal (bf16 MFMA tiles)", "ms_per_call": round(dense_ms, 3),
                 "tokens_per_s": round(n / (dense_ms * 1e-3), 1), "flops_per_call": dense_flops,
                 "achieved_tflops": round(dtf, 1), "mfma_frac": round(dtf / 2500.0, 4),
                 "traffic": counter_traffic("attn_dense_causal_8k_on_1m"),
                 "routed_attn_speedup": round(dense_ms / attn_ms, 2)}

    # the routed-vs-dense ladder: the same 8192-row chunk after shorter prefixes of the same cache
    rungs = []
    if ladder and dense_steps > 0:
        rungs = prefill_ladder(w, cfg, K, V, q, mean, ws, dense_steps,
                               {"prefix": P, "routed_path_ms": None, "routed_attn_ms": round(attn_ms, 4),
                                "dense_ms": dense["ms_per_call"] if dense else None})
    cpu, check = None, None
    if cpu_seconds > 0:
        cpu, check = oracle_prefill_baseline(w, kh, vh, P, n, qh, cpu_seconds, sel.cpu().numpy(), out.cpu().numpy())
    step_tflops = (attn_flops + route_flops) / (step_ms * 1e-3) / 1e12
    return {
        "workload": "prefill_8k_on_1m", "chunk": n, "context": L, "steps": steps,
        "value": round(n / (step_ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(step_ms, 4),
        "roofline": {"bound": "mfma", "kernel": "routed_attn_prefill (dispatch + bf16 MFMA tiles + merge)",
                     "achieved": round(tflops, 1), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(tflops / 2500.0, 4), "traffic": counter_traffic("routed_attn_prefill_8k_on_1m"),
                     "algorithmic_flops_per_launch": attn_flops, "algorithmic_bytes_per_launch": alg_bytes,
                     "avg_launch_ms": round(attn_ms, 4)},
        "step_flops": attn_flops + route_flops,
        "step_tflops": round(step_tflops, 1),
        "step_roofline": {"bound": "mfma", "what": "the whole step (summary update + route + top-k + attention)",
                          "achieved": round(step_tflops, 1), "peak": 2500.0, "unit": "TFLOP/s",
                          "frac": round(step_tflops / 2500.0, 4)},
        "cpu_baseline": cpu, "oracle_check": check,
        "fp8_cache": fp8_leg,
        "dense_causal": dense,
        "ladder": rungs,
    }


def prefill_algorithmic_bytes(w, sel_h, elem_bytes, row_scale_bytes=0):
    """Bytes a routed_attn_prefill call of the chunk must move at least: the K and V rows of every
    attended (kv head, span) once (the routed spans the selection names, complete, and the window
    spans up to the chunk's last row), with their row scales for an 8-bit cache, plus q (bf16),
    the selection, the rows' positions and sequences, and out (fp32)."""
    P, n, L = w.prefix_len, w.chunk_len, w.prefix_len + w.chunk_len
    S, W, G, d = w.span_size, w.window, w.group, w.head_dim
    w_first = (max(0, P - W + 1) // S) * S // S
    w_last = (L - 1) // S
    keys = 0
    for g in range(w.num_kv_heads):
        spans = np.unique(sel_h[:, g * G:(g + 1) * G, :])
        spans = spans[(spans >= 0) & (spans < w_first)]
        keys += len(spans) * S
        for j in range(w_first, w_last + 1):
            keys += min(S, L - j * S)
    kv = keys * 2 * (d * elem_bytes + row_scale_bytes)
    return int(kv + n * w.num_q_heads * (d * 2 + w.top_k * 4 + d * 4) + n * 12)


def bench_prefill_fp8(w, cfg, K, V, rows, t_p, t_l, steps, attn_flops, route_flops, out_bf16, warmup=10):
    """The prefill step over the 8-bit cache: span_summary_update_fp8 of the chunk +
    route_topk_spans + routed_attn_prefill_fp8.  The tiles convert the codes to bf16 in LDS and run the
    same bf16 MFMA products, so the flops and the peak are those of the bf16 step."""
    import torch

    import content_routed_sparse_amd as ra

    dev = K.device
    P, n, L = w.prefix_len, w.chunk_len, w.prefix_len + w.chunk_len
    K8 = torch.empty(K.shape, dtype=torch.uint8, device=dev)
    V8 = torch.empty_like(K8)
    KS = torch.empty(K.shape[:3], dtype=torch.float32, device=dev)
    VS = torch.empty_like(KS)
    zero = torch.zeros(1, dtype=torch.int64, device=dev)
    ra.kv_quantize_fp8(cfg, K, K8, KS, zero, t_l, L)
    ra.kv_quantize_fp8(cfg, V, V8, VS, zero, t_l, L)
    mean = torch.zeros(1, w.num_kv_heads, cfg.max_spans, w.head_dim, dtype=torch.float32, device=dev)
    run = torch.zeros(1, w.num_kv_heads, w.head_dim, dtype=torch.float32, device=dev)
    ra.span_summary_update_fp8(cfg, K8, KS, mean, run, zero, t_p, P)  # setup
    sel = torch.empty(n, w.num_q_heads, w.top_k, dtype=torch.int32, device=dev)
    out = torch.empty(n, w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev)
    ws = torch.empty(ra.workspace_bytes(cfg, ra.RA_OP_PREFILL, n, L - 1), dtype=torch.uint8, device=dev)
    ws_rt = torch.zeros(ra.workspace_bytes(cfg, ra.RA_OP_ROUTE_TOPK, n, L - 1), dtype=torch.uint8, device=dev)
    calls = [ra.prepare("span_summary_update_fp8", cfg, K8, KS, mean, run, t_p, t_l, n),
             ra.prepare("route_topk_spans", cfg, rows, mean, sel, ws_rt)]
    attn = ra.prepare("routed_attn_prefill_fp8", cfg, rows, K8, V8, KS, VS, sel, out, ws)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for _ in range(max(1, warmup)):
        for c in calls:
            c()
        attn()
    torch.cuda.synchronize()
    first = out.clone()
    t0 = time.perf_counter()
    for i in range(steps):
        for c in calls:
            c()
        ev[i][0].record(stream)
        attn()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / steps
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    tflops = attn_flops / (attn_ms * 1e-3) / 1e12
    step_tflops = (attn_flops + route_flops) / (step_ms * 1e-3) / 1e12
    alg_bytes = prefill_algorithmic_bytes(w, sel.cpu().numpy(), 1, 4)
    # quantisation's effect on the result: largest |out_fp8 - out_bf16| over the chunk
    diff = float((out - out_bf16).abs().max().item())
    return {"workload": "prefill_8k_on_1m, 8-bit cache (E4M3 codes, one fp32 scale per kv-head row)",
            "value": round(n / (step_ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(step_ms, 4),
            "roofline": {"bound": "mfma", "kernel": "routed_attn_prefill_fp8 (dispatch + 8-bit MFMA tiles + merge)",
                         "achieved": round(tflops, 1), "peak": 2500.0, "unit": "TFLOP/s",
                         "frac": round(tflops / 2500.0, 4),
                         "traffic": counter_traffic("routed_attn_prefill_fp8_8k_on_1m"),
                         "algorithmic_flops_per_launch": attn_flops, "algorithmic_bytes_per_launch": alg_bytes,
                         "avg_launch_ms": round(attn_ms, 4)},
            "step_tflops": round(step_tflops, 1),
            "max_abs_vs_bf16_cache": round(diff, 5),
            "repeat_bitwise_identical": bool(torch.equal(first, out))}


def time_calls(calls, reps):
    """Mean ms of one pass over `calls` (HIP events on the current stream around each pass)."""
    import torch

    stream = torch.cuda.current_stream()
    for c in calls:
        c()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        for c in calls:
            c()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def prefill_ladder(w, cfg, K, V, q, mean, ws, dense_steps, top):
    """Routed against dense attention for the chunk of 8192 rows placed after prefixes of 128K,
    256K, 512K and 1M tokens (the last rung is the prefill leg's own chunk; its routed path is timed
    here like the others).  Every span the rows can route to lies in the cache's first 1M tokens,
    which the prefill leg has summarised, so the summaries need no update.  Reported per rung: the
    routed attention call, the routed path (route_topk_spans + routed_attn_prefill) and
    attn_dense_causal, and the dense time over each."""
    import torch

    import content_routed_sparse_amd as ra

    n = w.chunk_len
    dev = q.device
    out = []
    for P in (131072, 262144, 524288, w.prefix_len):
        L = P + n
        rows = ra.Rows(q, torch.zeros(n, dtype=torch.int32, device=dev),
                       torch.arange(P, L, dtype=torch.int64, device=dev), L - 1)
        sel = torch.empty(n, w.num_q_heads, w.top_k, dtype=torch.int32, device=dev)
        o = torch.empty(n, w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev)
        ws_rt = torch.zeros(ra.workspace_bytes(cfg, ra.RA_OP_ROUTE_TOPK, n, L - 1), dtype=torch.uint8, device=dev)
        front = [ra.prepare("route_topk_spans", cfg, rows, mean, sel, ws_rt)]
        attn = ra.prepare("routed_attn_prefill", cfg, rows, K, V, sel, o, ws)
        path_ms = time_calls(front + [attn], 3)
        attn_ms = time_calls([attn], 3)
        if P == w.prefix_len and top["dense_ms"] is not None:
            dense_ms = top["dense_ms"]
        else:
            dense_ms = time_calls([ra.prepare("attn_dense_causal", cfg, rows, K, V, o)], dense_steps)
        out.append({"prefix": P, "context": L, "routed_path_ms": round(path_ms, 3), "routed_attn_ms": round(attn_ms, 3),
                    "dense_ms": round(dense_ms, 3), "dense_over_routed_path": round(dense_ms / path_ms, 2),
                    "dense_over_routed_attn": round(dense_ms / attn_ms, 2)})
    return out


def bench_decode_fp8(args, w, K, V, qs):
    """The decode step over the 8-bit cache: the same sequences quantised to E4M3 codes with one
    fp32 scale per (kv head, token) row (kv_quantize_fp8, untimed setup); a step is route_scores ->
    topk_spans -> routed_attn_decode_fp8_append (the attention and the new token's summary update)."""
    import torch

    import content_routed_sparse_amd as ra

    L, NC, dev = w.decode_len, K.shape[0], K.device
    cfg1 = ra.Config(w.num_q_heads, w.num_kv_heads, w.head_dim, w.span_size, w.top_k, w.window, ra.RA_BF16, 1, L)
    K8 = torch.empty(K.shape, dtype=torch.uint8, device=dev)
    V8 = torch.empty_like(K8)
    KS = torch.empty(K.shape[:3], dtype=torch.float32, device=dev)
    VS = torch.empty_like(KS)
    zero = torch.zeros(1, dtype=torch.int64, device=dev)
    full = torch.full((1,), L, dtype=torch.int64, device=dev)
    before = torch.full((1,), L - 1, dtype=torch.int64, device=dev)
    stride = ra.score_stride(cfg1, L - 1)
    ws = torch.empty(ra.workspace_bytes(cfg1, ra.RA_OP_DECODE, 1, L - 1), dtype=torch.uint8, device=dev)
    st = []
    for s in range(NC):
        ra.kv_quantize_fp8(cfg1, K[s:s + 1], K8[s:s + 1], KS[s:s + 1], zero, full, L)
        ra.kv_quantize_fp8(cfg1, V[s:s + 1], V8[s:s + 1], VS[s:s + 1], zero, full, L)
        d = {"k": K8[s:s + 1], "v": V8[s:s + 1], "ks": KS[s:s + 1], "vs": VS[s:s + 1],
             "mean": torch.zeros(1, w.num_kv_heads, cfg1.max_spans, w.head_dim, dtype=torch.float32, device=dev),
             "run": torch.zeros(1, w.num_kv_heads, w.head_dim, dtype=torch.float32, device=dev),
             "rows": ra.Rows(qs[s], torch.zeros(1, dtype=torch.int32, device=dev),
                             torch.full((1,), L - 1, dtype=torch.int64, device=dev), L - 1),
             "scores": torch.empty(1, w.num_q_heads, stride, dtype=torch.float32, device=dev),
             "sel": torch.empty(1, w.num_q_heads, w.top_k, dtype=torch.int32, device=dev),
             "out": torch.empty(1, w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev)}
        ra.span_summary_update_fp8(cfg1, d["k"], d["ks"], d["mean"], d["run"], zero, before, L - 1)
        d["front"], _ = front_calls(ra, cfg1, d["rows"], d["mean"], d["scores"], d["sel"])
        d["attn"] = ra.prepare("routed_attn_decode_fp8_append", cfg1, d["rows"], d["k"], d["v"], d["ks"], d["vs"],
                               d["sel"], d["out"], ws, d["mean"], d["run"], before, full, 1)
        st.append(d)
    torch.cuda.synchronize()
    for d in st:
        for c in d["front"]:
            c()
        d["attn"]()
    torch.cuda.synchronize()
    first = [d["out"].clone() for d in st]
    stream = torch.cuda.current_stream()
    EV_EVERY = 8
    timed_ev = list(range(0, args.steps, EV_EVERY))
    ev = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for i in timed_ev}

    def step(i, timed):
        d = st[i % NC]
        for c in d["front"]:
            c()
        if timed and i in ev:
            ev[i][0].record(stream)
        d["attn"]()
        if timed and i in ev:
            ev[i][1].record(stream)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in ev.values()]))
    same = all(torch.equal(first[s], st[s]["out"]) for s in range(NC))
    # algorithmic bytes: codes (1 byte per value) and row scales (4 bytes) of the K and V rows of
    # each kv head's union of selected spans plus the window, q (bf16) and out (fp32)
    G = w.group
    win = (L - 1) - (w.span_size * (max(0, L - 1 - w.window + 1) // w.span_size)) + 1
    per_seq = []
    for d in st:
        sel = d["sel"][0].cpu().numpy()
        uni = sum(len(set(sel[g * G:(g + 1) * G].ravel().tolist()) - {-1}) for g in range(w.num_kv_heads))
        rows_kv = uni * w.span_size + w.num_kv_heads * win
        per_seq.append(rows_kv * (w.head_dim + 4) * 2 + w.num_q_heads * w.head_dim * (2 + 4) +
                       w.num_kv_heads * (w.head_dim + 4 + w.head_dim * 8))
    bytes_step = float(np.mean([per_seq[i % NC] for i in timed_ev]))
    achieved = bytes_step / (attn_ms * 1e-3) / 1e9
    return {"workload": "decode_1m, 8-bit cache (E4M3 codes, one fp32 scale per kv-head row)",
            "value": round(1000.0 / ms, 2), "unit": "tokens/s", "ms_per_step": round(ms, 5),
            "roofline": {"bound": "hbm",
                         "kernel": "routed_attn_decode_fp8_append (decode_attn + merge launch with the summary update)",
                         "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": counter_traffic("routed_attn_decode_fp8_1m"),
                         "algorithmic_bytes_per_launch": int(bytes_step), "avg_launch_ms": round(attn_ms, 5)},
            "repeat_bitwise_identical": bool(same)}


COLD_HOT, COLD_K = 256, 64


def bench_cold(args, w, K, V, qs):
    """Token-level cold retrieval decode step on the same sequences: a 256-token hot window and 64
    cold tokens per query head found by a Hamming scan over sign-bit signatures.  A step is
    kv_signature_update (the new token) -> cold_select (scan + merge) -> cold_attn_decode."""
    import torch

    import content_routed_sparse_amd as ra

    L, NC, dev = w.decode_len, K.shape[0], K.device
    cfg1 = ra.Config(w.num_q_heads, w.num_kv_heads, w.head_dim, w.span_size, w.top_k, w.window, ra.RA_BF16, 1, L)
    sig = torch.empty(NC, w.num_kv_heads, L, w.head_dim // 8, dtype=torch.uint8, device=dev)
    zero = torch.zeros(1, dtype=torch.int64, device=dev)
    before = torch.full((1,), L - 1, dtype=torch.int64, device=dev)
    full = torch.full((1,), L, dtype=torch.int64, device=dev)
    ws = torch.empty(ra.cold_workspace_bytes(cfg1, 1, L - 1, COLD_HOT, COLD_K), dtype=torch.uint8, device=dev)
    st = []
    for s in range(NC):
        ra.kv_signature_update(cfg1, K[s:s + 1], sig[s:s + 1], zero, before, L - 1)
        rows = ra.Rows(qs[s], torch.zeros(1, dtype=torch.int32, device=dev),
                       torch.full((1,), L - 1, dtype=torch.int64, device=dev), L - 1)
        d = {"rows": rows, "sel": torch.empty(1, w.num_q_heads, COLD_K, dtype=torch.int32, device=dev),
             "out": torch.empty(1, w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev)}
        d["sig"] = ra.prepare("kv_signature_update", cfg1, K[s:s + 1], sig[s:s + 1], before, full, 1)
        d["select"] = ra.prepare("cold_select", cfg1, rows, sig[s:s + 1], COLD_HOT, COLD_K, d["sel"], ws)
        d["attn"] = ra.prepare("cold_attn_decode", cfg1, rows, K[s:s + 1], V[s:s + 1], d["sel"], COLD_HOT, COLD_K,
                               d["out"])
        st.append(d)
    torch.cuda.synchronize()
    for d in st:
        d["sig"]()
        d["select"]()
        d["attn"]()
    torch.cuda.synchronize()
    first = [(d["sel"].clone(), d["out"].clone()) for d in st]
    stream = torch.cuda.current_stream()
    EV_EVERY = 8
    timed_ev = list(range(0, args.steps, EV_EVERY))
    ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in timed_ev}

    def step(i, timed):
        d = st[i % NC]
        d["sig"]()
        if timed and i in ev:
            ev[i][0].record(stream)
        d["select"]()
        if timed and i in ev:
            ev[i][1].record(stream)
        d["attn"]()
        if timed and i in ev:
            ev[i][2].record(stream)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    sel_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev.values()]))
    attn_ms = float(np.mean([b.elapsed_time(c) for _, b, c in ev.values()]))
    same = all(torch.equal(f[0], d["sel"]) and torch.equal(f[1], d["out"]) for f, d in zip(first, st))
    # algorithmic bytes of cold_select: the signatures of every cold position of each kv head, q,
    # and the selection written; cold_attn_decode: K and V rows of each kv head's union of fetched
    # positions plus its hot window, q and out
    n_cold = L - 1 - COLD_HOT + 1
    sel_bytes = w.num_kv_heads * n_cold * (w.head_dim // 8) + w.num_q_heads * (w.head_dim * 2 + COLD_K * 4)
    G = w.group
    per_seq = []
    for d in st:
        sel = d["sel"][0].cpu().numpy()
        uni = sum(len(set(sel[g * G:(g + 1) * G].ravel().tolist()) - {-1}) for g in range(w.num_kv_heads))
        per_seq.append((uni + w.num_kv_heads * COLD_HOT) * w.head_dim * 2 * 2 + w.num_q_heads * w.head_dim * 6)
    attn_bytes = float(np.mean(per_seq))
    achieved = sel_bytes / (sel_ms * 1e-3) / 1e9
    # the scan is vector-ALU work: per (query head, cold position) pair at least COLD_OPS_PER_PAIR
    # lane-instructions (the Hamming distance of d/32 words: d/32 XOR + d/32 popcount-and-add,
    # then one compare with the threshold)
    pairs = w.num_q_heads * n_cold
    ops = pairs * cold_ops_per_pair(w.head_dim)
    alu = ops / (sel_ms * 1e-3) / 1e12
    return {"workload": "decode_1m, cold retrieval (hot window 256, top_k_cold 64, sign-bit signatures)",
            "value": round(1000.0 / ms, 2), "unit": "tokens/s", "ms_per_step": round(ms, 5),
            "roofline": {"bound": "alu", "kernel": "cold_select (cold_tile scan + cold_merge)",
                         "achieved": round(alu, 3), "peak": round(VALU_PEAK_TOPS, 2), "unit": "T lane-ops/s",
                         "frac": round(alu / VALU_PEAK_TOPS, 4), "traffic": counter_traffic("cold_select_1m"),
                         "algorithmic_ops_per_launch": int(ops), "pairs_per_launch": int(pairs),
                         "avg_launch_ms": round(sel_ms, 5)},
            "hbm_view": {"algorithmic_bytes_per_launch": int(sel_bytes), "achieved_GBps": round(achieved, 1),
                         "frac_of_8TBps": round(achieved / HBM_PEAK_GBS, 4)},
            "cold_attn_decode": {"avg_launch_ms": round(attn_ms, 5), "algorithmic_bytes_per_launch": int(attn_bytes),
                                 "achieved_GBps": round(attn_bytes / (attn_ms * 1e-3) / 1e9, 1)},
            "repeat_bitwise_identical": bool(same)}


# Integer vector-ALU peak: 256 CUs x 64 lane-instructions per clock (4 SIMDs of 16 lanes) x 2.4 GHz.
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12


def cold_ops_per_pair(d):
    """Lane-instructions of one Hamming distance and threshold test at head dimension d: d/32 XOR
    and d/32 popcount-and-accumulate (v_bcnt_u32_b32 adds its count to an accumulator), one compare."""
    return 2 * (d // 32) + 1


# SHA-256 of one 64-byte block takes at least 1,400 VALU instructions on gfx950: 48 schedule words
# x 10 (two sigmas of 2 rotations + 1 shift + one three-input xor, two adds), 64 rounds x 14 (two
# Sigmas x 4, choice 1, majority 1, four adds as three-input or plain adds), 8 final adds and 16
# byte swaps.  The vector ALUs retire 64 lane-instructions per clock per CU: 256 CUs x 64 x 2.4 GHz
# / 1400 x 64 bytes = 1.80 TB/s of hashed data.
SHA_PEAK_GBS = 256 * 64 * 2.4e9 / 1400 * 64 / 1e9


def bench_snapshot(w, d0, cfg1, reps=3):
    """Session snapshot of one 1M-token sequence's state (2 GiB of bf16 K/V rows, span means,
    running sums): kv_snapshot_pack (header, payload copies, SHA-256 digest levels),
    kv_snapshot_verify (every digest recomputed and compared), kv_snapshot_unpack into a second
    set of buffers, and the image's copies to and from pinned host memory (PCIe)."""
    import torch

    import content_routed_sparse_amd as ra

    L, dev = w.decode_len, d0["k"].device
    lengths = [L]
    n = ra.snapshot_bytes(cfg1, lengths)
    img = torch.empty(n, dtype=torch.uint8, device=dev)
    img2 = torch.empty_like(img)
    bad = torch.empty(1, dtype=torch.int64, device=dev)
    K2, V2 = torch.empty_like(d0["k"]), torch.empty_like(d0["v"])
    M2, R2 = torch.zeros_like(d0["mean"]), torch.zeros_like(d0["run"])
    host = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    stream = torch.cuda.current_stream()

    def timed(fn):
        ts = []
        for r in range(reps + 1):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            if r > 0:
                ts.append(a.elapsed_time(b))
        return float(np.mean(ts))

    t_pack = timed(lambda: ra.kv_snapshot_pack(cfg1, d0["k"], d0["v"], d0["mean"], d0["run"], lengths, img))
    header = img[:4096].cpu().numpy()
    info, _ = ra.kv_snapshot_parse(header)
    header = header[:info["header_bytes"]].copy()
    t_verify = timed(lambda: ra.kv_snapshot_verify(header, img, bad))
    intact = int(bad.item()) == -1
    t_unpack = timed(lambda: ra.kv_snapshot_unpack(cfg1, header, img, K2, V2, M2, R2, guard=bad))
    restored = (torch.equal(K2, d0["k"]) and torch.equal(V2, d0["v"]) and torch.equal(R2, d0["run"]) and
                torch.equal(M2[:, :, :L // w.span_size], d0["mean"][:, :, :L // w.span_size]))
    del K2, V2
    d2h, h2d = [], []
    for r in range(2):
        t0 = time.perf_counter()
        host.copy_(img)
        d2h.append(time.perf_counter() - t0)
        t0 = time.perf_counter()
        img2.copy_(host, non_blocking=True)
        torch.cuda.synchronize()
        h2d.append(time.perf_counter() - t0)
    round_trip = torch.equal(img, img2)
    gbs = lambda ms: round(n / (ms * 1e-3) / 1e9, 1)
    achieved = n / (t_verify * 1e-3) / 1e9
    return {"workload": "decode_1m state of one sequence (1M tokens x 4 kv heads, bf16)",
            "image_bytes": n, "root": bytes(host[-32:].numpy()).hex(),
            "pack_ms": round(t_pack, 3), "pack_GBps": gbs(t_pack),
            "verify_ms": round(t_verify, 3), "verify_GBps": gbs(t_verify),
            "unpack_ms": round(t_unpack, 3), "unpack_GBps": gbs(t_unpack),
            "d2h_pinned_GBps": round(n / min(d2h) / 1e9, 1), "h2d_pinned_GBps": round(n / min(h2d) / 1e9, 1),
            "roofline": {"bound": "alu", "kernel": "kv_snapshot_verify (sha_chunks, every level)",
                         "achieved": round(achieved, 1), "peak": round(SHA_PEAK_GBS, 1), "unit": "GB/s",
                         "frac": round(achieved / SHA_PEAK_GBS, 4), "traffic": None,
                         "algorithmic_bytes_per_launch": n, "avg_launch_ms": round(t_verify, 5)},
            "intact": intact, "restored_bitwise": bool(restored), "pcie_round_trip_bitwise": bool(round_trip)}


def bench_tiny_prefill(steps, cpu_seconds=0.0):
    """The tiny causal prefill (fp32, 1 head, d = 64, 4096 tokens from an empty cache, spans of 64,
    top-8 + window 64): a step is span_summary_update of the 4096 tokens + route_scores +
    topk_spans + routed_attn_prefill for the 4096 rows, all fp32 FMA.  Its work (0.6 GFLOP) is far
    too small to fill the GPU: the leg reports the time, and the fraction of the fp32 vector peak
    as a number, not a target."""
    import torch

    import content_routed_sparse_amd as ra
    from synth import workloads as WL

    w = WL.WORKLOADS["tiny_prefill_fp32"]
    n = w.chunk_len
    dev = torch.device("cuda:0")
    cfg = ra.Config(w.num_q_heads, w.num_kv_heads, w.head_dim, w.span_size, w.top_k, w.window, ra.RA_F32, 1, n)
    kh, vh, qh = WL.kv_slab(w, 0, 0, n, "k"), WL.kv_slab(w, 0, 0, n, "v"), WL.queries(w, 0, 0, n)
    K = torch.from_numpy(kh)[None].to(dev)
    V = torch.from_numpy(vh)[None].to(dev)
    q = torch.from_numpy(qh).to(dev)
    rows = ra.Rows(q, torch.zeros(n, dtype=torch.int32, device=dev), torch.arange(n, dtype=torch.int64, device=dev),
                   n - 1)
    mean = torch.zeros(1, w.num_kv_heads, cfg.max_spans, w.head_dim, dtype=torch.float32, device=dev)
    run = torch.zeros(1, w.num_kv_heads, w.head_dim, dtype=torch.float32, device=dev)
    zero, full = torch.zeros(1, dtype=torch.int64, device=dev), torch.full((1,), n, dtype=torch.int64, device=dev)
    scores = torch.empty(n, w.num_q_heads, ra.score_stride(cfg, n - 1), dtype=torch.float32, device=dev)
    sel = torch.empty(n, w.num_q_heads, w.top_k, dtype=torch.int32, device=dev)
    out = torch.empty(n, w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev)
    ws = torch.empty(ra.workspace_bytes(cfg, ra.RA_OP_PREFILL, n, n - 1), dtype=torch.uint8, device=dev)
    # every step starts from the empty cache: the summary update rebuilds all 64 means
    calls = [ra.prepare("span_summary_update", cfg, K, mean, run, zero, full, n),
             ra.prepare("route_scores", cfg, rows, mean, scores),
             ra.prepare("topk_spans", cfg, rows, scores, sel)]
    attn = ra.prepare("routed_attn_prefill", cfg, rows, K, V, sel, out, ws)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        for c in calls:
            c()
        attn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        for c in calls:
            c()
        a.record(stream)
        attn()
        b.record(stream)
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / steps
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    pos = np.arange(n)
    S, W = w.span_size, w.window
    w0 = S * (np.maximum(0, pos - W + 1) // S)
    r = w0 // S
    keys = (np.minimum(w.top_k, r) * S + (pos - w0 + 1)).astype(np.float64)
    attn_flops = 4.0 * w.head_dim * keys.sum() * w.num_q_heads
    route_flops = 2.0 * w.head_dim * r.astype(np.float64).sum() * w.num_q_heads
    FP32_PEAK = 157.3
    tf = attn_flops / (attn_ms * 1e-3) / 1e12
    stf = (attn_flops + route_flops) / (step_ms * 1e-3) / 1e12
    cpu, check = None, None
    if cpu_seconds > 0:
        cpu, check = oracle_prefill_baseline(w, kh, vh, 0, n, qh, cpu_seconds, sel.cpu().numpy(), out.cpu().numpy())
    return {"workload": "tiny_prefill_fp32", "chunk": n, "context": n, "steps": steps,
            "value": round(n / (step_ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(step_ms, 4),
            "dtype": "f32",
            "roofline": {"bound": "alu", "kernel": "routed_attn_prefill (dispatch + fp32 tiles + merge)",
                         "achieved": round(tf, 3), "peak": FP32_PEAK, "unit": "TFLOP/s",
                         "frac": round(tf / FP32_PEAK, 5), "traffic": None,
                         "algorithmic_flops_per_launch": attn_flops, "avg_launch_ms": round(attn_ms, 4)},
            "step_roofline": {"bound": "alu", "what": "the whole step (summary update + route + top-k + attention)",
                              "achieved": round(stf, 3), "peak": FP32_PEAK, "unit": "TFLOP/s",
                              "frac": round(stf / FP32_PEAK, 5)},
            "cpu_baseline": cpu, "oracle_check": check}


def bench_decode_workload(name, steps, warmup, cpu_seconds=0.0):
    """The decode step of another decode workload: decode_10m (one 10M-token sequence, spans of
    4096) or ragged_decode_16 (16 sequences of 64K..512K tokens, spans of 512).  A step appends
    one token to every sequence: route_scores -> topk_spans -> routed_attn_decode_append (with the
    tokens' summary update) for the last position of each; its working set (1-2 GB) is larger than
    the 256 MB Infinity Cache, so steps repeat on the same caches."""
    import torch

    import content_routed_sparse_amd as ra
    from synth import workloads as WL

    w = WL.WORKLOADS[name]
    dev = torch.device("cuda:0")
    lengths = np.asarray(w.seq_lengths(), dtype=np.int64)
    B, cap = len(lengths), int(lengths.max())
    cfg = ra.Config(w.num_q_heads, w.num_kv_heads, w.head_dim, w.span_size, w.top_k, w.window, ra.RA_BF16, B, cap)
    t0 = time.time()
    K = torch.empty(B, w.num_kv_heads, cap, w.head_dim, dtype=torch.bfloat16, device=dev)
    V = torch.empty_like(K)
    kv = []  # host copies, kept for the oracle's baseline
    for b, L in enumerate(lengths):
        pair = (WL.kv_slab(w, b, 0, int(L), "k"), WL.kv_slab(w, b, 0, int(L), "v"))
        K[b, :, :L] = torch.from_numpy(pair[0].view(np.int16)).view(torch.bfloat16).to(dev)
        V[b, :, :L] = torch.from_numpy(pair[1].view(np.int16)).view(torch.bfloat16).to(dev)
        if cpu_seconds > 0:
            kv.append(pair)
    qh = np.stack([WL.query_at(w, b, int(L) - 1) for b, L in enumerate(lengths)])
    q = torch.from_numpy(qh.view(np.int16)).view(torch.bfloat16).to(dev)
    rows = ra.Rows(q, torch.arange(B, dtype=torch.int32, device=dev), torch.as_tensor(lengths - 1).to(dev), cap - 1)
    mean = torch.zeros(B, w.num_kv_heads, cfg.max_spans, w.head_dim, dtype=torch.float32, device=dev)
    run = torch.zeros(B, w.num_kv_heads, w.head_dim, dtype=torch.float32, device=dev)
    zero = torch.zeros(B, dtype=torch.int64, device=dev)
    before, after = torch.as_tensor(lengths - 1).to(dev), torch.as_tensor(lengths).to(dev)
    ra.span_summary_update(cfg, K, mean, run, zero, before, int(lengths.max() - 1))  # setup, untimed
    scores = torch.empty(B, w.num_q_heads, ra.score_stride(cfg, cap - 1), dtype=torch.float32, device=dev)
    sel = torch.empty(B, w.num_q_heads, w.top_k, dtype=torch.int32, device=dev)
    out = torch.empty(B, w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev)
    ws = torch.empty(ra.workspace_bytes(cfg, ra.RA_OP_DECODE, B, cap - 1), dtype=torch.uint8, device=dev)
    front, front_kind = front_calls(ra, cfg, rows, mean, scores, sel)
    attn = ra.prepare("routed_attn_decode_append", cfg, rows, K, V, sel, out, ws, mean, run, before, after, 1)
    torch.cuda.synchronize()
    setup = time.time() - t0
    for c in front:
        c()
    attn()
    torch.cuda.synchronize()
    first = out.clone()
    stream = torch.cuda.current_stream()
    ev = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for i in range(0, steps, 4)}

    def step(i, timed):
        for c in front:
            c()
        if timed and i in ev:
            ev[i][0].record(stream)
        attn()
        if timed and i in ev:
            ev[i][1].record(stream)

    for i in range(warmup):
        step(i, False)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        step(i, True)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t1) * 1e3 / steps
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in ev.values()]))
    same = torch.equal(first, out)
    # algorithmic bytes of routed_attn_decode: per row and kv head, K and V rows of the union of
    # the spans its query heads selected plus its window; q (bf16) and out (fp32)
    G, S = w.group, w.span_size
    selh = sel.cpu().numpy()
    rows_kv = 0
    for b, L in enumerate(lengths):
        t = int(L) - 1
        win = t - S * (max(0, t - w.window + 1) // S) + 1
        for g in range(w.num_kv_heads):
            uni = len(set(selh[b, g * G:(g + 1) * G].ravel().tolist()) - {-1})
            rows_kv += uni * S + win
    nbytes = rows_kv * w.head_dim * 2 * 2 + B * w.num_q_heads * w.head_dim * (2 + 4)
    # + the summary update: the new K row, the running sum read and written, per kv head
    nbytes += B * w.num_kv_heads * w.head_dim * (2 + 8)
    achieved = nbytes / (attn_ms * 1e-3) / 1e9
    # the whole step also reads the summaries of every routable span (routing)
    route_bytes = sum(((int(L) - 1 - w.window + 1) // S) * w.num_kv_heads * w.head_dim * 4 for L in lengths)
    step_gbs = (nbytes + route_bytes) / (ms * 1e-3) / 1e9
    gsel, gout = sel.cpu().numpy(), out.cpu().numpy()
    del K, V
    torch.cuda.empty_cache()
    cpu, check = None, None
    if cpu_seconds > 0:
        cpu, check = oracle_decode_baseline(w, kv, lengths, qh, cpu_seconds, gsel, gout)
        del kv
    return {"workload": name, "sequences": B, "context_max": cap, "span": S, "top_k": w.top_k, "window": w.window,
            "routing_calls": front_kind,
            "value": round(B * 1000.0 / ms, 2), "unit": "tokens/s", "ms_per_step": round(ms, 5),
            "roofline": {"bound": "hbm",
                     "kernel": "routed_attn_decode_append (decode_attn + merge launch with the token's summary update)",
                         "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": counter_traffic({"decode_10m": "routed_attn_decode_10m",
                                                     "ragged_decode_16": "routed_attn_decode_ragged16"}[name]),
                         "algorithmic_bytes_per_launch": int(nbytes), "avg_launch_ms": round(attn_ms, 5)},
            "step_roofline": {"bound": "hbm", "what": "the whole step (route + top-k + attention with the update)",
                              "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                              "algorithmic_bytes_per_step": int(nbytes + route_bytes)},
            "repeat_bitwise_identical": bool(same), "setup_seconds": round(setup, 1),
            "cpu_baseline": cpu, "oracle_check": check}


# ------------------------------------------------------------------------------ CPU baseline
BF16 = 1  # synth's code for bf16 inputs
# The oracle (the plain C++ implementation in oracle/, fp64, one std::thread task per (row, head))
# timed on the host's cores over a bounded sample of each workload, on the same seeded inputs.
# Its setup (summaries of the cache that precedes the step) is untimed, as on the GPU.  The
# oracle's results for the sampled rows are also compared with the GPU's (selection exact or a
# valid near tie, largest output error).

def _host_cpu():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_check(w, prob, q_rows, positions, gsel, gout):
    """Oracle vs GPU for rows of one sequence (all heads): selection verdicts and max-abs error."""
    import oracle as O

    res = prob.rows(q_rows, positions, scores=True)
    kinds, worst = {"exact": 0, "near_tie": 0, "fail": 0}, 0.0
    mk = [O.round_to_bf16(prob.means[g]) if prob.is_bf16 else prob.means[g] for g in range(prob.hkv)]
    for i, t in enumerate(positions):
        for h in range(w.num_q_heads):
            sc = res["scores"][i][h]
            bound = O.score_abs_bound(prob.q64(q_rows[i][h]), mk[h // prob.group], len(sc), False)
            v = O.selection_verdict(gsel[i, h], res["sel"][i, h], sc, w.top_k, bound)
            kinds["fail" if v.startswith("fail") else v] += 1
            if v.startswith("fail"):
                continue
            ref = res["out"][i, h] if v == "exact" else prob.row(q_rows[i][h], h, int(t), sel=gsel[i, h])["out"]
            worst = max(worst, O.output_errors(gout[i, h], ref)[0])
    return kinds, worst


def oracle_decode_baseline(w, kv, lengths, q_rows, seconds, gsel=None, gout=None):
    """Decode steps of the oracle: every sequence's new token folded into its summaries, then its
    row (all query heads) routed, selected and attended; repeated until `seconds` have passed.
    kv: per sequence (K, V) host arrays [Hkv][L_b][d]; q_rows [B][Hq][d]."""
    import oracle.cpp as OC

    threads = OC.default_threads()
    S = w.span_size
    base = []
    for (kh, vh), L in zip(kv, lengths):
        L = int(L)
        means, run = OC.summaries(kh, L - 1, S, max_spans=L // S, threads=threads)  # setup, untimed
        base.append((means, run))
    steps, probs = 0, None
    t0 = time.perf_counter()
    while True:
        probs = []
        for b, ((kh, vh), L) in enumerate(zip(kv, lengths)):
            L = int(L)
            m2, r2 = base[b][0].copy(), base[b][1].copy()
            OC.summary_update(kh, m2, r2, L - 1, L, S, threads=threads)
            prob = OC.Problem(kh, vh, L, w.num_q_heads, S, w.top_k, w.window, True, means=m2, threads=threads)
            prob.rows(q_rows[b][None], [L - 1])
            probs.append(prob)
        steps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    out = {"value": round(steps * len(lengths) / el, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": "%d decode steps of the %s workload (%d sequence%s: summary update of the new token + %d query "
                     "heads each), C++ oracle, fp64, %d threads, %s" % (
                         steps, w.name, len(lengths), "s" if len(lengths) > 1 else "", w.num_q_heads, threads,
                         _host_cpu())}
    check = None
    if gsel is not None:
        kinds, worst = {"exact": 0, "near_tie": 0, "fail": 0}, 0.0
        for b, L in enumerate(lengths):
            k_, w_ = _oracle_check(w, probs[b], q_rows[b][None], [int(L) - 1], gsel[b:b + 1], gout[b:b + 1])
            for key in kinds:
                kinds[key] += k_[key]
            worst = max(worst, w_)
        check = {"rows": int(len(lengths) * w.num_q_heads), "selection": kinds, "max_abs_err": worst}
    return out, check


def oracle_prefill_baseline(w, kh, vh, prefix, chunk, q, seconds, gsel=None, gout=None, sample_rows=None):
    """Prefill of the oracle: the chunk's summary update (timed once), then rows of the chunk
    (all query heads) spread evenly over it, in batches, until `seconds` have passed; the rate is
    per token of the whole step: 1 / (update time / chunk + row time / rows done)."""
    import oracle.cpp as OC

    threads = OC.default_threads()
    S = w.span_size
    L = prefix + chunk
    means, run = OC.summaries(kh, prefix, S, max_spans=L // S, threads=threads)  # setup, untimed
    t0 = time.perf_counter()
    OC.summary_update(kh, means, run, prefix, L, S, threads=threads)
    t_upd = time.perf_counter() - t0
    prob = OC.Problem(kh, vh, L, w.num_q_heads, S, w.top_k, w.window, w.dtype == BF16, means=means,
                       threads=threads)
    order = np.argsort((np.arange(chunk) * 0.6180339887498949) % 1.0, kind="stable")  # evenly spread rows
    if sample_rows is not None:
        order = order[:sample_rows]
    done, t_rows = 0, 0.0
    batch = 16 if chunk > 4096 else chunk
    while done < len(order):
        idx = np.sort(order[done:done + batch])
        t1 = time.perf_counter()
        prob.rows(q[idx], prefix + idx)
        t_rows += time.perf_counter() - t1
        done += len(idx)
        if t_upd + t_rows >= seconds:
            break
    rate = 1.0 / (t_upd / chunk + t_rows / done)
    out = {"value": round(rate, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": "the %s chunk's summary update (%d tokens) + %d of its %d rows (all %d query heads), "
                     "C++ oracle, fp64, %d threads, %s" % (w.name, chunk, done, chunk, w.num_q_heads, threads,
                                                           _host_cpu())}
    check = None
    if gsel is not None:
        idx = np.sort(order[:min(done, 64)])
        kinds, worst = _oracle_check(w, prob, q[idx], prefix + idx, gsel[idx], gout[idx])
        check = {"rows": int(len(idx) * w.num_q_heads), "selection": kinds, "max_abs_err": worst}
    return out, check


if __name__ == "__main__":
    main()
