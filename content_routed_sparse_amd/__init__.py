"""Python binding of the gfx950 content-routed sparse attention library (``libroutedattn.so``).

Thin ctypes wrappers with the C entry points' names.  They check tensor devices, dtypes and
shapes, then pass raw device pointers and torch's current HIP stream; every step of the
computation runs in the library's HIP kernels.  PyTorch only provides device memory and
streams.  If the library has not been built the first call raises (no fallback exists).

The method (release post "Experimental model with subquadratic attention: 100 tok/s @ 1M
context, 76 tok/s @ 10M context", section "Key idea"): spans of S keys are summarised by their
mean; each query row scores the spans, keeps the top k and attends exactly to those spans'
tokens plus a local window.
"""
import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libroutedattn.so")

RA_F32, RA_BF16 = 0, 1
RA_OP_DECODE, RA_OP_PREFILL, RA_OP_ROUTE_TOPK = 0, 1, 2
EXPORTED = ("span_summary_update", "route_scores", "topk_spans", "route_topk_spans", "routed_attn_decode",
            "routed_attn_prefill",
            "routed_attn_decode_noalloc",
            "attn_dense_causal", "kv_quantize_fp8", "span_summary_update_fp8", "routed_attn_decode_fp8",
            "routed_attn_prefill_fp8",
            "routed_attn_decode_append", "routed_attn_decode_fp8_append",
            "kv_signature_update", "ra_cold_workspace_bytes", "cold_select", "cold_attn_decode",
            "kv_snapshot_bytes", "kv_snapshot_pack", "kv_snapshot_parse", "kv_snapshot_verify", "kv_snapshot_unpack",
            "kv_snapshot_bytes_fp8", "kv_snapshot_pack_fp8", "kv_snapshot_unpack_fp8",
            "kv_snapshot_write_file", "kv_snapshot_read_file", "ra_workspace_bytes", "ra_status_string",
            "ra_last_error")
SNAPSHOT_INTACT = (1 << 64) - 1  # kv_snapshot_verify's word when every digest matches
RA_SNAPSHOT_E4M3 = 2  # image element type of the 8-bit cache


class RoutedAttnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("routed_attn status %d (%s): %s" % (status, _status_string(status), message))
        self.status = status


class _Config(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("span_size", ctypes.c_int32), ("top_k", ctypes.c_int32), ("window", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("batch", ctypes.c_int32), ("capacity", ctypes.c_int64),
                ("max_spans", ctypes.c_int64)]


class _SnapshotInfo(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("span_size", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("header_bytes", ctypes.c_uint64), ("payload_bytes", ctypes.c_uint64),
                ("image_bytes", ctypes.c_uint64)]


class _Rows(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("row_seq", ctypes.c_void_p), ("row_pos", ctypes.c_void_p),
                ("n_rows", ctypes.c_int64), ("max_pos", ctypes.c_int64)]


_lib = None


def lib():
    """The loaded library; raises if it was not built (never falls back)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libroutedattn.so is not built: run `python -m content_routed_sparse_amd.build` "
                               "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        CP, RP = ctypes.POINTER(_Config), ctypes.POINTER(_Rows)
        sigs = {
            "span_summary_update": [CP, P, P, P, P, P, I64, P],
            "route_scores": [CP, RP, P, P, I64, P],
            "topk_spans": [CP, RP, P, I64, P, P],
            "route_topk_spans": [CP, RP, P, P, P, SZ, P],
            "routed_attn_decode": [CP, RP, P, P, P, P, P, SZ, P],
            "routed_attn_decode_noalloc": [CP, RP, P, P, P, P, P],
            "routed_attn_prefill": [CP, RP, P, P, P, P, P, SZ, P],
            "attn_dense_causal": [CP, RP, P, P, P, P],
            "kv_quantize_fp8": [CP, P, P, P, P, P, I64, P],
            "span_summary_update_fp8": [CP, P, P, P, P, P, P, I64, P],
            "routed_attn_decode_fp8": [CP, RP, P, P, P, P, P, P, P, SZ, P],
            "routed_attn_prefill_fp8": [CP, RP, P, P, P, P, P, P, P, SZ, P],
            "routed_attn_decode_append": [CP, RP, P, P, P, P, P, SZ, P, P, P, P, I64, P],
            "routed_attn_decode_fp8_append": [CP, RP, P, P, P, P, P, P, P, SZ, P, P, P, P, I64, P],
            "kv_signature_update": [CP, P, P, P, P, I64, P],
            "cold_select": [CP, RP, P, I32, I32, P, P, SZ, P],
            "cold_attn_decode": [CP, RP, P, P, P, I32, I32, P, P],
            "kv_snapshot_pack": [CP, P, P, P, P, P, P, SZ, P],
            "kv_snapshot_parse": [P, SZ, ctypes.POINTER(_SnapshotInfo), P, I32],
            "kv_snapshot_verify": [P, SZ, P, SZ, P, P],
            "kv_snapshot_unpack": [CP, P, SZ, P, SZ, P, P, P, P, P, P],
            "kv_snapshot_pack_fp8": [CP, P, P, P, P, P, P, P, P, SZ, P],
            "kv_snapshot_unpack_fp8": [CP, P, SZ, P, SZ, P, P, P, P, P, P, P, P],
            "kv_snapshot_write_file": [ctypes.c_char_p, P, SZ],
            "kv_snapshot_read_file": [ctypes.c_char_p, P, SZ, ctypes.POINTER(SZ)],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = I32
        L.ra_cold_workspace_bytes.argtypes = [CP, I64, I64, I32, I32]
        L.ra_cold_workspace_bytes.restype = SZ
        for name in ("kv_snapshot_bytes", "kv_snapshot_bytes_fp8"):
            getattr(L, name).argtypes = [CP, P]
            getattr(L, name).restype = SZ
        L.ra_workspace_bytes.argtypes = [CP, I32, I64, I64]
        L.ra_workspace_bytes.restype = SZ
        L.ra_status_string.argtypes = [I32]
        L.ra_status_string.restype = ctypes.c_char_p
        L.ra_last_error.argtypes = []
        L.ra_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _status_string(status):
    try:
        return lib().ra_status_string(status).decode()
    except Exception:  # pragma: no cover - only while formatting an error
        return "?"


def _check(status):
    if status != 0:
        raise RoutedAttnError(status, lib().ra_last_error().decode())


@dataclass(frozen=True)
class Config:
    """Shapes and method parameters (mirror of ra_config)."""
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    span_size: int
    top_k: int
    window: int
    dtype: int
    batch: int
    capacity: int
    max_spans: int = -1

    def __post_init__(self):
        if self.max_spans < 0:
            object.__setattr__(self, "max_spans", -(-self.capacity // self.span_size))

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == RA_BF16 else torch.float32

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads

    def c(self):
        return _Config(self.num_q_heads, self.num_kv_heads, self.head_dim, self.span_size, self.top_k, self.window,
                       self.dtype, self.batch, self.capacity, self.max_spans)

    def num_routable(self, t):
        return (self.span_size * (max(0, t - self.window + 1) // self.span_size)) // self.span_size


@dataclass
class Rows:
    """Query rows: q [n][Hq][d], row_seq int32 [n], row_pos int64 [n], host bound max_pos."""
    q: torch.Tensor
    row_seq: torch.Tensor
    row_pos: torch.Tensor
    max_pos: int

    def c(self):
        return _Rows(self.q.data_ptr(), self.row_seq.data_ptr(), self.row_pos.data_ptr(), self.q.shape[0],
                     int(self.max_pos))


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, dtype, shape=None, name="tensor"):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return t.data_ptr()


def _rows(cfg, rows):
    n = rows.q.shape[0]
    _dev(rows.q, cfg.torch_dtype, (n, cfg.num_q_heads, cfg.head_dim), "q")
    _dev(rows.row_seq, torch.int32, (n,), "row_seq")
    _dev(rows.row_pos, torch.int64, (n,), "row_pos")
    return rows.c()


def _kv_shape(cfg):
    return (cfg.batch, cfg.num_kv_heads, cfg.capacity, cfg.head_dim)


# Each entry point is split into an argument builder (validation + marshalling into ctypes
# values) and the call itself, so that a caller in a tight loop can validate once and replay the
# prepared call (see `prepare`).

def _args_span_summary_update(cfg, k_cache, span_mean, run_sum, old_len, new_len, max_new_tokens, stream=None):
    c = cfg.c()
    return (ctypes.byref(c), _dev(k_cache, cfg.torch_dtype, _kv_shape(cfg), "k_cache"),
            _dev(span_mean, torch.float32, (cfg.batch, cfg.num_kv_heads, cfg.max_spans, cfg.head_dim), "span_mean"),
            _dev(run_sum, torch.float32, (cfg.batch, cfg.num_kv_heads, cfg.head_dim), "run_sum"),
            _dev(old_len, torch.int64, (cfg.batch,), "old_len"), _dev(new_len, torch.int64, (cfg.batch,), "new_len"),
            int(max_new_tokens), _stream(stream)), (c,)


def score_stride(cfg, max_pos):
    """Floats per (row, head) for a scores buffer of rows up to max_pos: r(max_pos) rounded up to a
    multiple of 32, so that every score row starts on a 128-byte cache line (the bf16 routing
    kernel's 16-byte stores then fill whole lines; for an 8192-row chunk on 1M tokens routing and
    top-k together measured ~600 us against ~750 us with an odd stride and ~660 us with a
    multiple of 16).  Any stride >= r(max_pos) is valid."""
    return max(32, -(-cfg.num_routable(max_pos) // 32) * 32)


def _scores_shape_check(cfg, rows, scores):
    n = rows.q.shape[0]
    if scores.dim() != 3 or tuple(scores.shape[:2]) != (n, cfg.num_q_heads):
        raise ValueError("scores must have shape [n_rows, Hq, stride]")


def _args_route_scores(cfg, rows, span_mean, scores, stream=None):
    c, r = cfg.c(), _rows(cfg, rows)
    _scores_shape_check(cfg, rows, scores)
    return (ctypes.byref(c), ctypes.byref(r),
            _dev(span_mean, torch.float32, (cfg.batch, cfg.num_kv_heads, cfg.max_spans, cfg.head_dim), "span_mean"),
            _dev(scores, torch.float32, None, "scores"), scores.shape[2], _stream(stream)), (c, r)


def _args_route_topk_spans(cfg, rows, span_mean, sel, workspace, stream=None):
    c, r = cfg.c(), _rows(cfg, rows)
    n = rows.q.shape[0]
    return (ctypes.byref(c), ctypes.byref(r),
            _dev(span_mean, torch.float32, (cfg.batch, cfg.num_kv_heads, cfg.max_spans, cfg.head_dim), "span_mean"),
            _dev(sel, torch.int32, (n, cfg.num_q_heads, cfg.top_k), "sel"),
            _dev(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream(stream)), (c, r)


def _args_topk_spans(cfg, rows, scores, sel, stream=None):
    c, r = cfg.c(), _rows(cfg, rows)
    _scores_shape_check(cfg, rows, scores)
    n = rows.q.shape[0]
    return (ctypes.byref(c), ctypes.byref(r), _dev(scores, torch.float32, None, "scores"), scores.shape[2],
            _dev(sel, torch.int32, (n, cfg.num_q_heads, cfg.top_k), "sel"), _stream(stream)), (c, r)


def _args_attn(cfg, rows, k_cache, v_cache, sel, out, workspace, stream=None):
    c, r = cfg.c(), _rows(cfg, rows)
    n = rows.q.shape[0]
    return (ctypes.byref(c), ctypes.byref(r), _dev(k_cache, cfg.torch_dtype, _kv_shape(cfg), "k_cache"),
            _dev(v_cache, cfg.torch_dtype, _kv_shape(cfg), "v_cache"),
            _dev(sel, torch.int32, (n, cfg.num_q_heads, cfg.top_k), "sel"),
            _dev(out, torch.float32, (n, cfg.num_q_heads, cfg.head_dim), "out"),
            _dev(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream(stream)), (c, r)


def _args_dense(cfg, rows, k_cache, v_cache, out, stream=None):
    c, r = cfg.c(), _rows(cfg, rows)
    n = rows.q.shape[0]
    return (ctypes.byref(c), ctypes.byref(r), _dev(k_cache, cfg.torch_dtype, _kv_shape(cfg), "k_cache"),
            _dev(v_cache, cfg.torch_dtype, _kv_shape(cfg), "v_cache"),
            _dev(out, torch.float32, (n, cfg.num_q_heads, cfg.head_dim), "out"), _stream(stream)), (c, r)


# 8-bit cache: codes [B][Hkv][cap][d] uint8, scales [B][Hkv][cap] float32; queries bf16.
def _scale_shape(cfg):
    return (cfg.batch, cfg.num_kv_heads, cfg.capacity)


def _bf16_cfg(cfg):
    if cfg.dtype != RA_BF16:
        raise ValueError("8-bit caches go with bf16 queries: cfg.dtype must be RA_BF16")


def _args_kv_quantize_fp8(cfg, src, codes, scales, old_len, new_len, max_new_tokens, stream=None):
    _bf16_cfg(cfg)
    c = cfg.c()
    return (ctypes.byref(c), _dev(src, torch.bfloat16, _kv_shape(cfg), "src"),
            _dev(codes, torch.uint8, _kv_shape(cfg), "codes"), _dev(scales, torch.float32, _scale_shape(cfg), "scales"),
            _dev(old_len, torch.int64, (cfg.batch,), "old_len"), _dev(new_len, torch.int64, (cfg.batch,), "new_len"),
            int(max_new_tokens), _stream(stream)), (c,)


def _args_span_summary_update_fp8(cfg, k_codes, k_scales, span_mean, run_sum, old_len, new_len, max_new_tokens,
                                  stream=None):
    _bf16_cfg(cfg)
    c = cfg.c()
    return (ctypes.byref(c), _dev(k_codes, torch.uint8, _kv_shape(cfg), "k_codes"),
            _dev(k_scales, torch.float32, _scale_shape(cfg), "k_scales"),
            _dev(span_mean, torch.float32, (cfg.batch, cfg.num_kv_heads, cfg.max_spans, cfg.head_dim), "span_mean"),
            _dev(run_sum, torch.float32, (cfg.batch, cfg.num_kv_heads, cfg.head_dim), "run_sum"),
            _dev(old_len, torch.int64, (cfg.batch,), "old_len"), _dev(new_len, torch.int64, (cfg.batch,), "new_len"),
            int(max_new_tokens), _stream(stream)), (c,)


def _args_attn_fp8(cfg, rows, k_codes, v_codes, k_scales, v_scales, sel, out, workspace, stream=None):
    _bf16_cfg(cfg)
    c, r = cfg.c(), _rows(cfg, rows)
    n = rows.q.shape[0]
    return (ctypes.byref(c), ctypes.byref(r), _dev(k_codes, torch.uint8, _kv_shape(cfg), "k_codes"),
            _dev(v_codes, torch.uint8, _kv_shape(cfg), "v_codes"),
            _dev(k_scales, torch.float32, _scale_shape(cfg), "k_scales"),
            _dev(v_scales, torch.float32, _scale_shape(cfg), "v_scales"),
            _dev(sel, torch.int32, (n, cfg.num_q_heads, cfg.top_k), "sel"),
            _dev(out, torch.float32, (n, cfg.num_q_heads, cfg.head_dim), "out"),
            _dev(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream(stream)), (c, r)


# Decode with the step's summary append (the token's update rides in the merge launch).
def _append_tail(cfg, span_mean, run_sum, old_len, new_len, max_new_tokens):
    return (_dev(span_mean, torch.float32, (cfg.batch, cfg.num_kv_heads, cfg.max_spans, cfg.head_dim), "span_mean"),
            _dev(run_sum, torch.float32, (cfg.batch, cfg.num_kv_heads, cfg.head_dim), "run_sum"),
            _dev(old_len, torch.int64, (cfg.batch,), "old_len"), _dev(new_len, torch.int64, (cfg.batch,), "new_len"),
            int(max_new_tokens))


def _args_attn_append(cfg, rows, k_cache, v_cache, sel, out, workspace, span_mean, run_sum, old_len, new_len,
                      max_new_tokens, stream=None):
    head, keep = _args_attn(cfg, rows, k_cache, v_cache, sel, out, workspace, stream)
    return head[:-1] + _append_tail(cfg, span_mean, run_sum, old_len, new_len, max_new_tokens) + head[-1:], keep


def _args_attn_fp8_append(cfg, rows, k_codes, v_codes, k_scales, v_scales, sel, out, workspace, span_mean, run_sum,
                          old_len, new_len, max_new_tokens, stream=None):
    head, keep = _args_attn_fp8(cfg, rows, k_codes, v_codes, k_scales, v_scales, sel, out, workspace, stream)
    return head[:-1] + _append_tail(cfg, span_mean, run_sum, old_len, new_len, max_new_tokens) + head[-1:], keep


# Cold retrieval: signatures [B][Hkv][cap][d/8] uint8, sel_cold [n][Hq][top_k_cold] int32.
def _sig_shape(cfg):
    return (cfg.batch, cfg.num_kv_heads, cfg.capacity, cfg.head_dim // 8)


def _args_kv_signature_update(cfg, k_cache, sig, old_len, new_len, max_new_tokens, stream=None):
    c = cfg.c()
    return (ctypes.byref(c), _dev(k_cache, cfg.torch_dtype, _kv_shape(cfg), "k_cache"),
            _dev(sig, torch.uint8, _sig_shape(cfg), "sig"), _dev(old_len, torch.int64, (cfg.batch,), "old_len"),
            _dev(new_len, torch.int64, (cfg.batch,), "new_len"), int(max_new_tokens), _stream(stream)), (c,)


def _args_cold_select(cfg, rows, sig, hot_window, top_k_cold, sel_cold, workspace, stream=None):
    c, r = cfg.c(), _rows(cfg, rows)
    n = rows.q.shape[0]
    return (ctypes.byref(c), ctypes.byref(r), _dev(sig, torch.uint8, _sig_shape(cfg), "sig"), int(hot_window),
            int(top_k_cold), _dev(sel_cold, torch.int32, (n, cfg.num_q_heads, top_k_cold), "sel_cold"),
            _dev(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream(stream)), (c, r)


def _args_cold_attn_decode(cfg, rows, k_cache, v_cache, sel_cold, hot_window, top_k_cold, out, stream=None):
    c, r = cfg.c(), _rows(cfg, rows)
    n = rows.q.shape[0]
    return (ctypes.byref(c), ctypes.byref(r), _dev(k_cache, cfg.torch_dtype, _kv_shape(cfg), "k_cache"),
            _dev(v_cache, cfg.torch_dtype, _kv_shape(cfg), "v_cache"),
            _dev(sel_cold, torch.int32, (n, cfg.num_q_heads, top_k_cold), "sel_cold"), int(hot_window),
            int(top_k_cold), _dev(out, torch.float32, (n, cfg.num_q_heads, cfg.head_dim), "out"),
            _stream(stream)), (c, r)


_BUILDERS = {
    "span_summary_update": _args_span_summary_update,
    "route_scores": _args_route_scores,
    "topk_spans": _args_topk_spans,
    "route_topk_spans": _args_route_topk_spans,
    "routed_attn_decode": _args_attn,
    "routed_attn_prefill": _args_attn,
    "attn_dense_causal": _args_dense,
    "kv_quantize_fp8": _args_kv_quantize_fp8,
    "span_summary_update_fp8": _args_span_summary_update_fp8,
    "routed_attn_decode_fp8": _args_attn_fp8,
    "routed_attn_prefill_fp8": _args_attn_fp8,
    "routed_attn_decode_append": _args_attn_append,
    "routed_attn_decode_fp8_append": _args_attn_fp8_append,
    "kv_signature_update": _args_kv_signature_update,
    "cold_select": _args_cold_select,
    "cold_attn_decode": _args_cold_attn_decode,
}


class Prepared:
    """A validated call of one entry point with fixed arguments; calling it launches again.

    The tensors given at preparation are the ones used by every call; the caller keeps them
    alive and unchanged in shape.  With stream=None the call goes to torch's current stream at
    call time (so a prepared call can be captured into a graph); otherwise to the given stream.
    """

    def __init__(self, name, *args, stream=None):
        self.fn = getattr(lib(), name)
        self.args, self._keep = _BUILDERS[name](*args, stream=stream)
        self._tensors = args
        self.dynamic_stream = stream is None
        self._head = self.args[:-1]

    def __call__(self):
        if self.dynamic_stream:
            _check(self.fn(*self._head, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
        else:
            _check(self.fn(*self.args))


def prepare(name, *args, stream=None):
    return Prepared(name, *args, stream=stream)


def span_summary_update(cfg, k_cache, span_mean, run_sum, old_len, new_len, max_new_tokens, stream=None):
    """Append tokens [old_len[b], new_len[b]) of each sequence to its span summaries."""
    args, _keep = _args_span_summary_update(cfg, k_cache, span_mean, run_sum, old_len, new_len, max_new_tokens,
                                            stream)
    _check(lib().span_summary_update(*args))


def route_scores(cfg, rows, span_mean, scores, stream=None):
    """scores[row][h][j] = q . kappa(mean_j) for every routable span j of the row."""
    args, _keep = _args_route_scores(cfg, rows, span_mean, scores, stream)
    _check(lib().route_scores(*args))


def topk_spans(cfg, rows, scores, sel, stream=None):
    """sel[row][h] = the row's top-k routable spans, ascending, padded with -1."""
    args, _keep = _args_topk_spans(cfg, rows, scores, sel, stream)
    _check(lib().topk_spans(*args))


def route_topk_spans(cfg, rows, span_mean, sel, workspace, stream=None):
    """route_scores then topk_spans in one launch (few rows).  The workspace (RA_OP_ROUTE_TOPK
    bytes) must start zeroed (torch.zeros); every call leaves its counters at zero."""
    args, _keep = _args_route_topk_spans(cfg, rows, span_mean, sel, workspace, stream)
    _check(lib().route_topk_spans(*args))


def workspace_bytes(cfg, op, n_rows, max_pos):
    c = cfg.c()
    n = lib().ra_workspace_bytes(ctypes.byref(c), op, n_rows, max_pos)
    if n == 0 and n_rows > 0:
        raise RoutedAttnError(1, lib().ra_last_error().decode())
    return n


def routed_attn_decode(cfg, rows, k_cache, v_cache, sel, out, workspace, stream=None):
    """Exact attention over window + selected spans, split-K over span sub-tiles (few rows)."""
    args, _keep = _args_attn(cfg, rows, k_cache, v_cache, sel, out, workspace, stream)
    _check(lib().routed_attn_decode(*args))


def routed_attn_decode_noalloc(cfg, rows, k_cache, v_cache, sel, out, stream=None):
    """routed_attn_decode with the library's own fixed device scratch (no workspace, nothing
    allocated); calls that overlap on one GPU race."""
    c, r = cfg.c(), _rows(cfg, rows)
    n = rows.q.shape[0]
    _check(lib().routed_attn_decode_noalloc(
        ctypes.byref(c), ctypes.byref(r), _dev(k_cache, cfg.torch_dtype, _kv_shape(cfg), "k_cache"),
        _dev(v_cache, cfg.torch_dtype, _kv_shape(cfg), "v_cache"),
        _dev(sel, torch.int32, (n, cfg.num_q_heads, cfg.top_k), "sel"),
        _dev(out, torch.float32, (n, cfg.num_q_heads, cfg.head_dim), "out"), _stream(stream)))


def routed_attn_prefill(cfg, rows, k_cache, v_cache, sel, out, workspace, stream=None):
    """Exact attention over window + selected spans, rows grouped span by span (many rows)."""
    args, _keep = _args_attn(cfg, rows, k_cache, v_cache, sel, out, workspace, stream)
    _check(lib().routed_attn_prefill(*args))


def attn_dense_causal(cfg, rows, k_cache, v_cache, out, stream=None):
    """Exact attention over every key at or before each row's position (bf16; no workspace)."""
    args, _keep = _args_dense(cfg, rows, k_cache, v_cache, out, stream)
    _check(lib().attn_dense_causal(*args))


def kv_quantize_fp8(cfg, src, codes, scales, old_len, new_len, max_new_tokens, stream=None):
    """8-bit cache: E4M3 codes and per-row scales of rows [old_len[b], new_len[b]) of a bf16 cache."""
    args, _keep = _args_kv_quantize_fp8(cfg, src, codes, scales, old_len, new_len, max_new_tokens, stream)
    _check(lib().kv_quantize_fp8(*args))


def span_summary_update_fp8(cfg, k_codes, k_scales, span_mean, run_sum, old_len, new_len, max_new_tokens,
                            stream=None):
    """span_summary_update over an 8-bit K cache (sums of the dequantised values)."""
    args, _keep = _args_span_summary_update_fp8(cfg, k_codes, k_scales, span_mean, run_sum, old_len, new_len,
                                                max_new_tokens, stream)
    _check(lib().span_summary_update_fp8(*args))


def routed_attn_decode_fp8(cfg, rows, k_codes, v_codes, k_scales, v_scales, sel, out, workspace, stream=None):
    """routed_attn_decode over an 8-bit K/V cache (bf16 queries)."""
    args, _keep = _args_attn_fp8(cfg, rows, k_codes, v_codes, k_scales, v_scales, sel, out, workspace, stream)
    _check(lib().routed_attn_decode_fp8(*args))


def routed_attn_prefill_fp8(cfg, rows, k_codes, v_codes, k_scales, v_scales, sel, out, workspace, stream=None):
    """routed_attn_prefill over an 8-bit K/V cache (bf16 queries); the prefill workspace."""
    args, _keep = _args_attn_fp8(cfg, rows, k_codes, v_codes, k_scales, v_scales, sel, out, workspace, stream)
    _check(lib().routed_attn_prefill_fp8(*args))


def routed_attn_decode_append(cfg, rows, k_cache, v_cache, sel, out, workspace, span_mean, run_sum, old_len, new_len,
                              max_new_tokens, stream=None):
    """routed_attn_decode, then span_summary_update of tokens [old_len[b], new_len[b]) (one launch
    less when a single token per sequence is appended)."""
    args, _keep = _args_attn_append(cfg, rows, k_cache, v_cache, sel, out, workspace, span_mean, run_sum, old_len,
                                    new_len, max_new_tokens, stream)
    _check(lib().routed_attn_decode_append(*args))


def routed_attn_decode_fp8_append(cfg, rows, k_codes, v_codes, k_scales, v_scales, sel, out, workspace, span_mean,
                                  run_sum, old_len, new_len, max_new_tokens, stream=None):
    """routed_attn_decode_fp8, then span_summary_update_fp8 of tokens [old_len[b], new_len[b])."""
    args, _keep = _args_attn_fp8_append(cfg, rows, k_codes, v_codes, k_scales, v_scales, sel, out, workspace,
                                        span_mean, run_sum, old_len, new_len, max_new_tokens, stream)
    _check(lib().routed_attn_decode_fp8_append(*args))


def kv_signature_update(cfg, k_cache, sig, old_len, new_len, max_new_tokens, stream=None):
    """Cold retrieval: sign-bit signatures of K rows [old_len[b], new_len[b])."""
    args, _keep = _args_kv_signature_update(cfg, k_cache, sig, old_len, new_len, max_new_tokens, stream)
    _check(lib().kv_signature_update(*args))


def cold_workspace_bytes(cfg, n_rows, max_pos, hot_window, top_k_cold):
    c = cfg.c()
    n = lib().ra_cold_workspace_bytes(ctypes.byref(c), n_rows, max_pos, hot_window, top_k_cold)
    if n == 0 and n_rows > 0:
        raise RoutedAttnError(1, lib().ra_last_error().decode())
    return n


def cold_select(cfg, rows, sig, hot_window, top_k_cold, sel_cold, workspace, stream=None):
    """Hamming scan: the top_k_cold cold positions of every (row, head), ascending, -1 padded."""
    args, _keep = _args_cold_select(cfg, rows, sig, hot_window, top_k_cold, sel_cold, workspace, stream)
    _check(lib().cold_select(*args))


def cold_attn_decode(cfg, rows, k_cache, v_cache, sel_cold, hot_window, top_k_cold, out, stream=None):
    """Exact attention over the selected cold positions and the hot window."""
    args, _keep = _args_cold_attn_decode(cfg, rows, k_cache, v_cache, sel_cold, hot_window, top_k_cold, out, stream)
    _check(lib().cold_attn_decode(*args))


# ------------------------------------------------------------------------ session snapshots
# Image = header | payload (live K/V rows, span means, running sums) | SHA-256 digest levels |
# root; layout in include/routed_attn.h.  `lengths` are host token counts per sequence, headers
# are host bytes, images are uint8 device tensors (or pinned host tensors for the file helpers).

def _host_lengths(cfg, lengths):
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(lengths, dtype=np.int64))
    if arr.shape != (cfg.batch,):
        raise ValueError("lengths must have cfg.batch = %d entries" % cfg.batch)
    return arr


def _host_bytes(header):
    """(pointer, size, keep-alive) of host bytes: bytes, bytearray, numpy or a CPU tensor."""
    import numpy as np
    if isinstance(header, torch.Tensor):
        if header.is_cuda:
            raise TypeError("header must be host memory")
        header = header.contiguous().numpy()
    arr = np.ascontiguousarray(np.frombuffer(header, dtype=np.uint8) if isinstance(header, (bytes, bytearray))
                               else np.asarray(header).view(np.uint8).reshape(-1))
    return arr.ctypes.data, arr.nbytes, arr


def snapshot_bytes(cfg, lengths):
    """Image bytes of the state of sequences with these host lengths."""
    arr = _host_lengths(cfg, lengths)
    c = cfg.c()
    n = lib().kv_snapshot_bytes(ctypes.byref(c), arr.ctypes.data)
    if n == 0:
        raise RoutedAttnError(1, lib().ra_last_error().decode())
    return n


def kv_snapshot_pack(cfg, k_cache, v_cache, span_mean, run_sum, lengths, image, stream=None):
    """Write the snapshot image of the cache state into the uint8 device tensor `image`."""
    arr = _host_lengths(cfg, lengths)
    c = cfg.c()
    _check(lib().kv_snapshot_pack(
        ctypes.byref(c), _dev(k_cache, cfg.torch_dtype, _kv_shape(cfg), "k_cache"),
        _dev(v_cache, cfg.torch_dtype, _kv_shape(cfg), "v_cache"),
        _dev(span_mean, torch.float32, (cfg.batch, cfg.num_kv_heads, cfg.max_spans, cfg.head_dim), "span_mean"),
        _dev(run_sum, torch.float32, (cfg.batch, cfg.num_kv_heads, cfg.head_dim), "run_sum"), arr.ctypes.data,
        _dev(image, torch.uint8, None, "image"), image.numel(), _stream(stream)))


def _fp8_cache_args(cfg, k_codes, v_codes, k_scales, v_scales):
    shape = _kv_shape(cfg)
    return (_dev(k_codes, torch.uint8, shape, "k_codes"), _dev(v_codes, torch.uint8, shape, "v_codes"),
            _dev(k_scales, torch.float32, shape[:3], "k_scales"), _dev(v_scales, torch.float32, shape[:3], "v_scales"))


def snapshot_bytes_fp8(cfg, lengths):
    """Image bytes of the state of sequences with these host lengths over the 8-bit cache."""
    arr = _host_lengths(cfg, lengths)
    c = cfg.c()
    n = lib().kv_snapshot_bytes_fp8(ctypes.byref(c), arr.ctypes.data)
    if n == 0:
        raise RoutedAttnError(1, lib().ra_last_error().decode())
    return n


def kv_snapshot_pack_fp8(cfg, k_codes, v_codes, k_scales, v_scales, span_mean, run_sum, lengths, image, stream=None):
    """Write the snapshot image of the 8-bit cache state (codes, row scales, summaries)."""
    arr = _host_lengths(cfg, lengths)
    c = cfg.c()
    _check(lib().kv_snapshot_pack_fp8(
        ctypes.byref(c), *_fp8_cache_args(cfg, k_codes, v_codes, k_scales, v_scales),
        _dev(span_mean, torch.float32, (cfg.batch, cfg.num_kv_heads, cfg.max_spans, cfg.head_dim), "span_mean"),
        _dev(run_sum, torch.float32, (cfg.batch, cfg.num_kv_heads, cfg.head_dim), "run_sum"), arr.ctypes.data,
        _dev(image, torch.uint8, None, "image"), image.numel(), _stream(stream)))


def kv_snapshot_unpack_fp8(cfg, header, image, k_codes, v_codes, k_scales, v_scales, span_mean, run_sum, guard=None,
                           stream=None):
    """Copy the saved 8-bit state of the device image into the caches (only if *guard reads intact)."""
    ptr, n, _keep = _host_bytes(header)
    g = None if guard is None else _dev(guard, torch.int64, (1,), "guard")
    _check(lib().kv_snapshot_unpack_fp8(
        ctypes.byref(cfg.c()), ctypes.c_void_p(ptr), n, _dev(image, torch.uint8, None, "image"), image.numel(), g,
        *_fp8_cache_args(cfg, k_codes, v_codes, k_scales, v_scales),
        _dev(span_mean, torch.float32, (cfg.batch, cfg.num_kv_heads, cfg.max_spans, cfg.head_dim), "span_mean"),
        _dev(run_sum, torch.float32, (cfg.batch, cfg.num_kv_heads, cfg.head_dim), "run_sum"), _stream(stream)))


def kv_snapshot_parse(header, max_batch=1 << 20):
    """(info dict, lengths numpy array) of a host header."""
    import numpy as np
    ptr, n, _keep = _host_bytes(header)
    info = _SnapshotInfo()
    _check(lib().kv_snapshot_parse(ctypes.c_void_p(ptr), n, ctypes.byref(info), None, 0))
    lengths = np.zeros(info.batch, dtype=np.int64)
    _check(lib().kv_snapshot_parse(ctypes.c_void_p(ptr), n, ctypes.byref(info), lengths.ctypes.data, info.batch))
    return {f: getattr(info, f) for f, _ in _SnapshotInfo._fields_ if f != "reserved"}, lengths


def kv_snapshot_verify(header, image, bad_offset, stream=None):
    """Recompute every digest of the device image; bad_offset (int64 device tensor [1]) receives
    SNAPSHOT_INTACT (as int64: -1) or the smallest offset of a chunk whose digest differs."""
    ptr, n, _keep = _host_bytes(header)
    _check(lib().kv_snapshot_verify(ctypes.c_void_p(ptr), n, _dev(image, torch.uint8, None, "image"), image.numel(),
                                    _dev(bad_offset, torch.int64, (1,), "bad_offset"), _stream(stream)))


def kv_snapshot_unpack(cfg, header, image, k_cache, v_cache, span_mean, run_sum, guard=None, stream=None):
    """Copy the saved state of the device image into the caches (only if *guard reads intact)."""
    ptr, n, _keep = _host_bytes(header)
    g = None if guard is None else _dev(guard, torch.int64, (1,), "guard")
    _check(lib().kv_snapshot_unpack(
        ctypes.byref(cfg.c()), ctypes.c_void_p(ptr), n, _dev(image, torch.uint8, None, "image"), image.numel(), g,
        _dev(k_cache, cfg.torch_dtype, _kv_shape(cfg), "k_cache"),
        _dev(v_cache, cfg.torch_dtype, _kv_shape(cfg), "v_cache"),
        _dev(span_mean, torch.float32, (cfg.batch, cfg.num_kv_heads, cfg.max_spans, cfg.head_dim), "span_mean"),
        _dev(run_sum, torch.float32, (cfg.batch, cfg.num_kv_heads, cfg.head_dim), "run_sum"), _stream(stream)))


def kv_snapshot_write_file(path, host_image):
    """Write a host uint8 tensor or buffer to `path` (through a temporary file renamed into place)."""
    ptr, n, _keep = _host_bytes(host_image)
    _check(lib().kv_snapshot_write_file(os.fsencode(path), ctypes.c_void_p(ptr), n))


def kv_snapshot_read_file(path, pin=True):
    """The bytes of a file as a host uint8 tensor (pinned by default)."""
    n = ctypes.c_size_t(0)
    _check(lib().kv_snapshot_read_file(os.fsencode(path), None, 0, ctypes.byref(n)))
    buf = torch.empty(n.value, dtype=torch.uint8, pin_memory=pin)
    _check(lib().kv_snapshot_read_file(os.fsencode(path), ctypes.c_void_p(buf.data_ptr()), n.value, ctypes.byref(n)))
    return buf


def save_snapshot(path, cfg, k_cache, v_cache, span_mean, run_sum, lengths):
    """Pack the state on the device, copy the image to pinned host memory and write it to
    `path`.  Returns the root digest (hex)."""
    image = torch.empty(snapshot_bytes(cfg, lengths), dtype=torch.uint8, device=k_cache.device)
    kv_snapshot_pack(cfg, k_cache, v_cache, span_mean, run_sum, lengths, image)
    host = torch.empty(image.numel(), dtype=torch.uint8, pin_memory=True)
    host.copy_(image)  # stream-ordered after the pack; synchronous for the host
    kv_snapshot_write_file(path, host)
    return bytes(host[-32:].numpy()).hex()


def load_snapshot(path, cfg, k_cache, v_cache, span_mean, run_sum):
    """Read `path`, check every digest on the device and restore the state into the caches.
    Returns the restored lengths; raises (restoring nothing) if any digest differs."""
    host = kv_snapshot_read_file(path)
    info, lengths = kv_snapshot_parse(host[:min(host.numel(), 64 + 8 * (1 << 20))])
    image = host.to(k_cache.device, non_blocking=True)
    bad = torch.empty(1, dtype=torch.int64, device=k_cache.device)
    header = host[:info["header_bytes"]]
    kv_snapshot_verify(header, image, bad)
    kv_snapshot_unpack(cfg, header, image, k_cache, v_cache, span_mean, run_sum, guard=bad)
    b = int(bad.item()) & SNAPSHOT_INTACT
    if b != SNAPSHOT_INTACT:
        raise RoutedAttnError(6, "%s: digest mismatch in the chunk at byte %d; nothing restored" % (path, b))
    return lengths


def save_snapshot_fp8(path, cfg, k_codes, v_codes, k_scales, v_scales, span_mean, run_sum, lengths):
    """save_snapshot for the 8-bit cache (codes and row scales).  Returns the root digest (hex)."""
    image = torch.empty(snapshot_bytes_fp8(cfg, lengths), dtype=torch.uint8, device=k_codes.device)
    kv_snapshot_pack_fp8(cfg, k_codes, v_codes, k_scales, v_scales, span_mean, run_sum, lengths, image)
    host = torch.empty(image.numel(), dtype=torch.uint8, pin_memory=True)
    host.copy_(image)
    kv_snapshot_write_file(path, host)
    return bytes(host[-32:].numpy()).hex()


def load_snapshot_fp8(path, cfg, k_codes, v_codes, k_scales, v_scales, span_mean, run_sum):
    """load_snapshot for the 8-bit cache: every digest checked on the device, then the state
    restored (nothing restored if any digest differs, which raises).  Returns the lengths."""
    host = kv_snapshot_read_file(path)
    info, lengths = kv_snapshot_parse(host[:min(host.numel(), 64 + 8 * (1 << 20))])
    image = host.to(k_codes.device, non_blocking=True)
    bad = torch.empty(1, dtype=torch.int64, device=k_codes.device)
    header = host[:info["header_bytes"]]
    kv_snapshot_verify(header, image, bad)
    kv_snapshot_unpack_fp8(cfg, header, image, k_codes, v_codes, k_scales, v_scales, span_mean, run_sum, guard=bad)
    b = int(bad.item()) & SNAPSHOT_INTACT
    if b != SNAPSHOT_INTACT:
        raise RoutedAttnError(6, "%s: digest mismatch in the chunk at byte %d; nothing restored" % (path, b))
    return lengths


class Pipeline:
    """Device buffers for one configuration and the four calls of a step, in order.

    Owns span_mean / run_sum (the summary table), the scores, selection, output and workspace
    buffers; the K/V cache tensors belong to the caller.  Allocation happens in the
    constructor and in `reserve`, never inside `step`.
    """

    def __init__(self, cfg, device="cuda"):
        self.cfg = cfg
        self.device = device
        self.span_mean = torch.zeros(cfg.batch, cfg.num_kv_heads, cfg.max_spans, cfg.head_dim, dtype=torch.float32,
                                     device=device)
        self.run_sum = torch.zeros(cfg.batch, cfg.num_kv_heads, cfg.head_dim, dtype=torch.float32, device=device)
        self.n_rows = -1
        self.max_pos = -1
        self.op = None

    def reserve(self, n_rows, max_pos, op):
        cfg = self.cfg
        stride = score_stride(cfg, max_pos)
        self.scores = torch.empty(n_rows, cfg.num_q_heads, stride, dtype=torch.float32, device=self.device)
        self.sel = torch.empty(n_rows, cfg.num_q_heads, cfg.top_k, dtype=torch.int32, device=self.device)
        self.out = torch.empty(n_rows, cfg.num_q_heads, cfg.head_dim, dtype=torch.float32, device=self.device)
        self.workspace = torch.empty(max(1, workspace_bytes(cfg, op, n_rows, max_pos)), dtype=torch.uint8,
                                     device=self.device)
        self.n_rows, self.max_pos, self.op = n_rows, max_pos, op

    def summarize(self, k_cache, old_len, new_len, max_new_tokens, stream=None):
        span_summary_update(self.cfg, k_cache, self.span_mean, self.run_sum, old_len, new_len, max_new_tokens, stream)

    def attend(self, rows, k_cache, v_cache, op, stream=None):
        """route_scores -> topk_spans -> routed_attn_{decode,prefill}; returns the output tensor."""
        n = rows.q.shape[0]
        if (n, rows.max_pos, op) != (self.n_rows, self.max_pos, self.op):
            self.reserve(n, rows.max_pos, op)
        route_scores(self.cfg, rows, self.span_mean, self.scores, stream)
        topk_spans(self.cfg, rows, self.scores, self.sel, stream)
        fn = routed_attn_decode if op == RA_OP_DECODE else routed_attn_prefill
        fn(self.cfg, rows, k_cache, v_cache, self.sel, self.out, self.workspace, stream)
        return self.out
