"""CPU oracle of token-level cold retrieval -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this module; the GPU library never calls it and shares no code with it.

Source.  The InfiniteKV post ("InfiniteKV open source release: a KV cache that stores old tokens
as 104-byte searchable records in RAM or on disk instead of deleting them") describes a second,
token-level way of reaching old context: the most recent 256 tokens stay exact on the GPU; older
tokens become compact searchable records with small signatures kept in GPU memory; for every
generated token the cache fetches the most relevant old tokens (top_k_cold of them, 32 to 64 in
the published runs, 96 for dense documents), found by a Hamming scan over the signatures, and
the model attends to those plus the recent window.  The post gives no signature or record
format.  Readings (one plain choice each, listed with their reasons in the design notes):

  C1  Hot window: the last H positions [max(0, t-H+1), t] of a query at position t (H = 256 in
      the post), attended exactly.
  C2  Cold tokens: every earlier position [0, t-H+1).
  C3  Signature of a key or query vector of d elements: its d sign bits (bit e set iff element e
      has its sign bit set, so -0 counts as negative), packed little-endian: bit e is bit e % 8
      of byte e // 8.  A sign code with the identity as projection; the post names no projection.
  C4  Relevance: the Hamming distance between the query head's signature and the key's.  The
      m = min(top_k_cold, number of cold tokens) cold positions with the smallest distance are
      fetched, ties going to the lower position; they are listed ascending, padded with -1.
  C5  Attention: exact softmax(q . k / sqrt(d)) over the hot window and the fetched positions,
      reading K and V from the cache at its own precision (the post's compressed records have
      no given format; here the cold keys and values stay in the cache).
  Query head h reads kv head h // (Hq / Hkv); each (token, query head) row selects on its own.
"""
import numpy as np

from .routed_attention import attend, widen


def sign_bits(x, is_bf16):
    """Sign bits (0/1, uint8) of stored values: bf16 bit patterns (uint16) or float32."""
    x = np.asarray(x)
    if is_bf16:
        assert x.dtype == np.uint16
        return (x >> 15).astype(np.uint8)
    assert x.dtype == np.float32
    return (x.view(np.uint32) >> 31).astype(np.uint8)


def signatures(x, is_bf16):
    """Packed signatures [..., d/8] (uint8) of vectors [..., d] (C3)."""
    return np.packbits(sign_bits(x, is_bf16), axis=-1, bitorder="little")


def hamming(sig_q, sig_k):
    """Hamming distances between one packed signature [d/8] and rows of signatures [n, d/8]."""
    x = np.bitwise_xor(np.asarray(sig_k, dtype=np.uint8), np.asarray(sig_q, dtype=np.uint8)[None, :])
    return np.unpackbits(x, axis=-1).sum(axis=-1).astype(np.int64)


def cold_count(t, H):
    """Number of cold positions of a query at position t (C2)."""
    return max(0, t - H + 1)


def select_cold(sig_q, sig_k_g, t, H, kc):
    """Fetched cold positions (C4): ascending, padded with -1 to kc entries."""
    n = cold_count(t, H)
    out = np.full(kc, -1, dtype=np.int64)
    if n == 0:
        return out
    dist = hamming(sig_q, sig_k_g[:n])
    order = np.lexsort((np.arange(n), dist))  # primary: distance, then position
    m = min(kc, n)
    out[:m] = np.sort(order[:m])
    return out


def hot_positions(t, H):
    return np.arange(max(0, t - H + 1), t + 1)


class ColdProblem:
    """One sequence's cache (arrays as stored: uint16 bf16 bits or fp32) with H and top_k_cold."""

    def __init__(self, keys, values, length, num_q_heads, H, kc, is_bf16):
        self.keys, self.values = keys, values  # [Hkv][>=length][d]
        self.length = length
        self.hkv = keys.shape[0]
        self.hq = num_q_heads
        self.group = num_q_heads // self.hkv
        self.H, self.kc = H, kc
        self.is_bf16 = is_bf16
        self.sig = signatures(keys[:, :length, :], is_bf16)  # [Hkv][length][d/8]

    def row(self, q_row_h, hq, t, sel=None):
        """Cold-retrieval attention of one (token, head) row at position t.  With `sel` given
        (the GPU's selection), attention runs over it instead of the row's own selection."""
        assert 0 <= t < self.length
        g = hq // self.group
        own = select_cold(signatures(q_row_h, self.is_bf16), self.sig[g], t, self.H, self.kc)
        use = own if sel is None else np.asarray(sel)
        pos = np.concatenate([np.asarray([p for p in use if p >= 0], dtype=np.int64), hot_positions(t, self.H)])
        o, wsum = attend(widen(q_row_h, self.is_bf16), self.keys[g], self.values[g], pos, self.is_bf16)
        return {"out": o, "sel": own, "weight_sum": wsum, "n_attended": len(pos)}

    def distances(self, q_row_h, hq, t):
        """Hamming distances of the row's cold positions (for tie-aware comparisons)."""
        g = hq // self.group
        return hamming(signatures(q_row_h, self.is_bf16), self.sig[g][:cold_count(t, self.H)])
