"""The five synthetic workloads (shapes, sizes and value recipes) and their input builders.

Recipe (the release post's performance table is measured at 1M and 10M tokens of context;
these inputs stand in for those long-context workloads):
  * queries  ~ N(0, 1) per element (stream 1), rounded to the workload dtype;
  * keys     ~ N(0, 1) (stream 2), plus, for the bf16 workloads, a per-(sequence, kv head, span)
             random direction of Euclidean norm 2 (stream 4) added to every key of the span before
             rounding, so that span means differ and routing is not trivial;
  * values   ~ N(0, 1) (stream 3);
  * ragged lengths ~ U{lo..hi} (stream 5).
Seeds are 0x5EED0000 + workload number.
"""
from dataclasses import dataclass, field
from typing import Tuple

import numpy as np

from . import BF16, F32, fill, lengths


@dataclass(frozen=True)
class Workload:
    name: str
    number: int
    mode: str  # "prefill" or "decode"
    dtype: int  # F32 or BF16
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    span_size: int
    top_k: int
    window: int
    offset_norm: float
    # prefill: cache length before the chunk and chunk length; decode: per-sequence lengths
    # (the length includes the token being decoded, whose K/V is already in the cache).
    prefix_len: int = 0
    chunk_len: int = 0
    batch: int = 1
    decode_len: int = 0
    ragged: Tuple[int, int] = (0, 0)
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def seed(self):
        return 0x5EED0000 + self.number

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads

    def seq_lengths(self):
        """Per-sequence cache length after the step (decode) or after the chunk (prefill)."""
        if self.mode == "prefill":
            return np.array([self.prefix_len + self.chunk_len] * self.batch, dtype=np.int64)
        if self.ragged != (0, 0):
            return lengths(self.seed, self.batch, self.ragged[0], self.ragged[1])
        return np.array([self.decode_len] * self.batch, dtype=np.int64)

    def capacity(self):
        return int(self.seq_lengths().max())

    def scaled(self, **kw):
        """A copy with some sizes changed (used for small parity cases)."""
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "tiny_prefill_fp32": Workload("tiny_prefill_fp32", 1, "prefill", F32, 1, 1, 64, 64, 8, 64, 0.0,
                                  prefix_len=0, chunk_len=4096),
    "decode_1m": Workload("decode_1m", 2, "decode", BF16, 32, 4, 128, 1024, 16, 1024, 2.0,
                          decode_len=1048576),
    "prefill_8k_on_1m": Workload("prefill_8k_on_1m", 3, "prefill", BF16, 32, 4, 128, 1024, 16, 1024, 2.0,
                                 prefix_len=1048576, chunk_len=8192),
    "decode_10m": Workload("decode_10m", 4, "decode", BF16, 32, 4, 128, 4096, 16, 4096, 2.0,
                           decode_len=10485760),
    "ragged_decode_16": Workload("ragged_decode_16", 5, "decode", BF16, 32, 4, 128, 512, 16, 512, 2.0,
                                 batch=16, ragged=(65536, 524288)),
}


def kv_slab(w: Workload, seq: int, pos0: int, npos: int, which: str, out=None):
    """Keys or values of one sequence for positions [pos0, pos0+npos): shape [Hkv][npos][d]."""
    if which == "k":
        return fill(w.dtype, w.seed, 2, seq, 0, w.num_kv_heads, pos0, npos, w.head_dim, 0,
                    w.span_size, w.offset_norm, out=out)
    return fill(w.dtype, w.seed, 3, seq, 0, w.num_kv_heads, pos0, npos, w.head_dim, 0, out=out)


def queries(w: Workload, seq: int, pos0: int, npos: int, out=None):
    """Query rows of one sequence at positions [pos0, pos0+npos): shape [npos][Hq][d]."""
    return fill(w.dtype, w.seed, 1, seq, 0, w.num_q_heads, pos0, npos, w.head_dim, 1, out=out)


def query_at(w: Workload, seq: int, pos: int):
    """One query row [Hq][d] at position pos."""
    return queries(w, seq, pos, 1)[0]
