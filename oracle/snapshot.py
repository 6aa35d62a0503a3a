"""CPU oracle of the session snapshot image -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this module; the GPU library never calls it and shares no code with it.

Source.  The release post "Experimental model with subquadratic attention: 100 tok/s @ 1M
context, 76 tok/s @ 10M context (30B model, single GPU)", section on why fast long context
matters: the point is to keep the cache instead of reprocessing it, with the KV cache in memory
and sessions saved to and restored from disk; its stack lists session snapshots.  The
InfiniteKV post ("InfiniteKV open source release") backs every result with a receipt carrying a
hash, and checks tensors byte for byte with SHA-256.  Neither fixes a format, so this one is the
library's own (readings, one plain choice each):

  N1  What is saved: for every sequence b of the batch, the live rows [0, L_b) of K and V of
      each kv head, the complete span means [0, floor(L_b / S)) and the running sum of the open
      span -- everything the routed attention reads; rows past L_b and unused summary slots are
      not state.  Restoring writes exactly these and nothing else.
  N2  Integrity: SHA-256 (FIPS 180-4) over 4096-byte chunks of header + payload, then over
      groups of 16 digests (512 bytes) of each digest level while a level has more than 16
      digests, and a root digest over the last level.  Every stored digest can be checked, and a
      mismatch names the chunk whose bytes changed.  (Small groups keep the hashing of the upper
      levels short: SHA-256 of one message is sequential, 9 blocks for a group of 16.)
  N3  The 8-bit cache (the release post's planned quantised cache: E4M3 codes with one fp32
      scale per (sequence, kv head, token) row, as oracle/kv_fp8.py defines them) is saved as
      element type 2: for each (b, g) the K codes and the V codes of rows [0, L_b) (one byte
      per value), then the K scales and the V scales of those rows, each run of scales
      zero-padded to a multiple of 16 bytes so that every later part starts 16-byte aligned.
      The summaries follow as for the other element types.

Image (all integers little-endian):

  header   64 bytes of fields, then int64 lengths[B], zero-padded to a multiple of 16 bytes
             0  8  magic "CRSASNP1"
             8  4  version = 1
            12  4  element type of K and V: 0 = float32, 1 = bfloat16, 2 = E4M3 codes + fp32 row
                   scales (N3)
            16  4  B         20  4  Hkv        24  4  d        28  4  S
            32  8  payload bytes                40  8  header bytes
            48  4  chunk bytes = 4096           52  4  fan-in = 16
            56  8  zero
  payload  for b, for g: K[b][g][0:L_b][:] then V[b][g][0:L_b][:]  (element bytes; type 2 then
           k_scale[b][g][0:L_b] and v_scale[b][g][0:L_b], float32, each zero-padded to a
           multiple of 16 bytes)
           then for b, for g: span_mean[b][g][0:floor(L_b/S)][:] then run_sum[b][g][:]  (float32)
  levels   D_1 = SHA-256 of each 4096-byte chunk of header + payload (the last one may be short);
           D_(l+1) = SHA-256 of each 512-byte chunk (16 digests) of the bytes of D_l, while
           |D_l| > 16; root = SHA-256 of the bytes of the last level.
  image    = header | payload | D_1 | D_2 | ... | D_m | root

A chunk's "offset" is where its bytes start in the image (the root covers all of D_m, so its
chunk starts at D_m).  `verify` returns the smallest offset of a chunk whose stored digest differs
from the digest of its bytes, or None.
"""
import hashlib
import struct

import numpy as np

MAGIC = b"CRSASNP1"
VERSION = 1
CHUNK = 4096
FAN_IN = 16
DIGEST = 32
FIELDS = 64


def sha256(data):
    """SHA-256 digest (FIPS 180-4) of a bytes-like object, by hashlib."""
    return hashlib.sha256(bytes(data)).digest()


def header_bytes(B):
    return -(-(FIELDS + 8 * B) // 16) * 16


def scale_run_bytes(L):
    """Bytes of one run of L fp32 row scales in a type-2 image: 4 L, zero-padded to 16 (N3)."""
    return -(-4 * int(L) // 16) * 16


def payload_bytes(lengths, Hkv, d, S, elem_bytes):
    """Payload bytes; elem_bytes 1 means the 8-bit cache (codes plus scale runs, N3)."""
    rows = sum(int(L) for L in lengths)
    spans = sum(int(L) // S for L in lengths)
    scales = 2 * Hkv * sum(scale_run_bytes(L) for L in lengths) if elem_bytes == 1 else 0
    return 2 * Hkv * rows * d * elem_bytes + scales + Hkv * (spans + len(lengths)) * d * 4


def level_counts(data_bytes):
    """Digest counts of the levels D_1 .. D_m for header + payload of `data_bytes` bytes."""
    counts = [-(-data_bytes // CHUNK)]
    while counts[-1] > FAN_IN:
        counts.append(-(-counts[-1] // FAN_IN))
    return counts


def image_bytes(lengths, Hkv, d, S, elem_bytes):
    data = header_bytes(len(lengths)) + payload_bytes(lengths, Hkv, d, S, elem_bytes)
    return data + DIGEST * sum(level_counts(data)) + DIGEST


def chunk_digests(data, size=CHUNK):
    """SHA-256 of each `size`-byte piece of `data` (the last piece may be short)."""
    return b"".join(sha256(data[i:i + size]) for i in range(0, len(data), size))


def digest_levels(data):
    """[D_1, ..., D_m] (bytes each) and the root digest of header + payload bytes `data` (N2)."""
    levels = [chunk_digests(data)]
    while len(levels[-1]) > FAN_IN * DIGEST:
        levels.append(chunk_digests(levels[-1], FAN_IN * DIGEST))
    return levels, sha256(levels[-1])


def _elem(dtype):
    """(element type code, bytes per element) of a cache array: uint16 holds bf16 bit patterns,
    uint8 E4M3 codes."""
    if dtype == np.uint16:
        return 1, 2
    if dtype == np.float32:
        return 0, 4
    if dtype == np.uint8:
        return 2, 1
    raise TypeError("cache arrays are float32, uint16 (bf16 bit patterns) or uint8 (E4M3 codes)")


def _scale_run(scales, L):
    """The bytes of L fp32 scales, zero-padded to scale_run_bytes(L) (N3)."""
    raw = np.ascontiguousarray(scales[:L], dtype=np.float32).tobytes()
    return raw + b"\0" * (scale_run_bytes(L) - len(raw))


def build_image(k_cache, v_cache, span_mean, run_sum, lengths, S, k_scale=None, v_scale=None):
    """Snapshot image (bytes) of caches [B][Hkv][cap][d], span_mean [B][Hkv][max_spans][d] and
    run_sum [B][Hkv][d] (host arrays), following the layout above.  For the 8-bit cache (uint8
    codes) k_scale and v_scale [B][Hkv][cap] (float32) are the rows' scales."""
    B, Hkv, cap, d = k_cache.shape
    assert v_cache.shape == k_cache.shape and v_cache.dtype == k_cache.dtype
    assert len(lengths) == B and all(0 <= int(L) <= cap for L in lengths)
    code, esz = _elem(k_cache.dtype)
    if code == 2:
        assert k_scale is not None and v_scale is not None
        assert k_scale.shape == (B, Hkv, cap) and v_scale.shape == (B, Hkv, cap)
    parts = []
    for b in range(B):
        L = int(lengths[b])
        for g in range(Hkv):
            parts.append(np.ascontiguousarray(k_cache[b, g, :L]).tobytes())
            parts.append(np.ascontiguousarray(v_cache[b, g, :L]).tobytes())
            if code == 2:
                parts.append(_scale_run(k_scale[b, g], L))
                parts.append(_scale_run(v_scale[b, g], L))
    for b in range(B):
        n = int(lengths[b]) // S
        for g in range(Hkv):
            parts.append(np.ascontiguousarray(span_mean[b, g, :n], dtype=np.float32).tobytes())
            parts.append(np.ascontiguousarray(run_sum[b, g], dtype=np.float32).tobytes())
    payload = b"".join(parts)
    assert len(payload) == payload_bytes(lengths, Hkv, d, S, esz)
    H = header_bytes(B)
    head = MAGIC + struct.pack("<IIIIIIQQIIQ", VERSION, code, B, Hkv, d, S, len(payload), H, CHUNK, FAN_IN, 0)
    head += struct.pack("<%dq" % B, *[int(L) for L in lengths])
    head += b"\0" * (H - len(head))
    data = head + payload
    levels, root = digest_levels(data)
    return data + b"".join(levels) + root


def parse_header(img):
    """Header fields of an image as a dict (raises ValueError on a malformed header)."""
    img = bytes(img[:FIELDS])
    if len(img) < FIELDS or img[:8] != MAGIC:
        raise ValueError("not a snapshot image")
    version, code, B, Hkv, d, S, P, H, chunk, fan, zero = struct.unpack("<IIIIIIQQIIQ", img[8:FIELDS])
    if version != VERSION or chunk != CHUNK or fan != FAN_IN or code not in (0, 1, 2) or H != header_bytes(B):
        raise ValueError("unsupported snapshot header")
    return {"dtype": code, "B": B, "Hkv": Hkv, "d": d, "S": S, "payload": P, "header": H}


def parse_image(img):
    """(header dict, lengths, per-sequence dict of arrays) of a well-formed image."""
    h = parse_header(img)
    B, Hkv, d, S = h["B"], h["Hkv"], h["d"], h["S"]
    lengths = np.frombuffer(img, dtype="<i8", count=B, offset=FIELDS).astype(np.int64)
    dt, esz = {0: (np.float32, 4), 1: (np.uint16, 2), 2: (np.uint8, 1)}[h["dtype"]]
    pos = h["header"]
    seqs = []
    for b in range(B):
        L = int(lengths[b])
        ks, vs, kss, vss = [], [], [], []
        for g in range(Hkv):
            for out in (ks, vs):
                n = L * d * esz
                out.append(np.frombuffer(img, dtype=dt, count=L * d, offset=pos).reshape(L, d))
                pos += n
            if h["dtype"] == 2:
                for out in (kss, vss):
                    out.append(np.frombuffer(img, dtype="<f4", count=L, offset=pos))
                    pos += scale_run_bytes(L)
        seqs.append({"k": ks, "v": vs})
        if h["dtype"] == 2:
            seqs[-1]["k_scale"], seqs[-1]["v_scale"] = kss, vss
    for b in range(B):
        n = int(lengths[b]) // S
        seqs[b]["mean"], seqs[b]["run"] = [], []
        for g in range(Hkv):
            seqs[b]["mean"].append(np.frombuffer(img, dtype="<f4", count=n * d, offset=pos).reshape(n, d))
            pos += n * d * 4
            seqs[b]["run"].append(np.frombuffer(img, dtype="<f4", count=d, offset=pos))
            pos += d * 4
    assert pos == h["header"] + h["payload"]
    return h, lengths, seqs


def verify(img, header=None):
    """Smallest image offset of a chunk whose stored digest differs from its bytes' digest, or
    None when every digest matches (N2).  The layout comes from `header` (a separate copy of
    the header bytes) when given, else from the image's own header."""
    img = bytes(img)
    h = parse_header(img if header is None else header)
    data_end = h["header"] + h["payload"]
    counts = level_counts(data_end)
    bad = None
    src, src_len, size = 0, data_end, CHUNK  # the byte range whose chunks level l digests
    pos = data_end  # where level l is stored
    for n in counts:
        stored = img[pos:pos + DIGEST * n]
        for i in range(n):
            lo = src + i * size
            if sha256(img[lo:min(lo + size, src + src_len)]) != stored[DIGEST * i:DIGEST * (i + 1)]:
                bad = lo if bad is None else min(bad, lo)
        src, src_len, size = pos, DIGEST * n, FAN_IN * DIGEST
        pos += DIGEST * n
    if sha256(img[src:src + src_len]) != img[pos:pos + DIGEST]:
        bad = src if bad is None else min(bad, src)
    assert pos + DIGEST == len(img)
    return bad
