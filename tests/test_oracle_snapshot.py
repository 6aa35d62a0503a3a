"""Pins for the snapshot oracle (oracle/snapshot.py): the hash primitive against the standard's
printed examples, the image layout against its written definition (byte offsets worked out here
by hand, not by the oracle's code), the digest-level sizes against closed forms, and the
integrity check against single-byte corruptions whose location is known.
"""
import json
import os
import struct

import numpy as np
import pytest

from oracle import snapshot as N

HERE = os.path.dirname(os.path.abspath(__file__))


def test_sha256_matches_the_standards_examples():
    with open(os.path.join(HERE, "golden", "sha256_fips180.json")) as f:
        vectors = json.load(f)["vectors"]
    for v in vectors:
        assert N.sha256((v["message"] * v["repeat"]).encode()).hex() == v["digest"]


@pytest.mark.parametrize("nbytes,counts", [
    (64, [1]), (4096, [1]), (4097, [2]), (16 * 4096, [16]), (16 * 4096 + 16, [17, 2]),
    (256 * 4096, [256, 16]), (256 * 4096 + 16, [257, 17, 2]),
])
def test_level_counts_closed_forms(nbytes, counts):
    assert N.level_counts(nbytes) == counts


def caches(dtype, B=3, Hkv=2, cap=300, d=64, S=16, lengths=(300, 17, 0), seed=0):
    rng = np.random.default_rng(seed)
    if dtype == np.uint16:
        k = rng.integers(0, 1 << 16, size=(B, Hkv, cap, d), dtype=np.uint16)
        v = rng.integers(0, 1 << 16, size=(B, Hkv, cap, d), dtype=np.uint16)
    else:
        k = rng.standard_normal((B, Hkv, cap, d)).astype(np.float32)
        v = rng.standard_normal((B, Hkv, cap, d)).astype(np.float32)
    mean = rng.standard_normal((B, Hkv, cap // S, d)).astype(np.float32)
    run = rng.standard_normal((B, Hkv, d)).astype(np.float32)
    return k, v, mean, run, np.array(lengths, dtype=np.int64), S


@pytest.mark.parametrize("dtype", [np.uint16, np.float32], ids=["bf16", "fp32"])
def test_image_layout_follows_the_definition(dtype):
    k, v, mean, run, lengths, S = caches(dtype)
    B, Hkv, cap, d = k.shape
    esz = 2 if dtype == np.uint16 else 4
    img = N.build_image(k, v, mean, run, lengths, S)
    # header: 64 bytes of fields + 3 lengths = 88 -> padded to 96
    H = 96
    assert img[:8] == b"CRSASNP1"
    assert struct.unpack("<I", img[8:12])[0] == 1
    assert struct.unpack("<I", img[12:16])[0] == (1 if dtype == np.uint16 else 0)
    assert struct.unpack("<4I", img[16:32]) == (3, 2, 64, 16)
    rows = 300 + 17
    P = 2 * 2 * rows * 64 * esz + 2 * (300 // 16 + 17 // 16 + 3) * 64 * 4
    assert struct.unpack("<QQII", img[32:56]) == (P, H, 4096, 16)
    assert struct.unpack("<3q", img[64:88]) == (300, 17, 0) and img[88:96] == b"\0" * 8
    # payload: K then V of (b=0, g=0), (0, 1), (1, 0), (1, 1); sequence 2 is empty
    row = 64 * esz
    at = H
    for b, L in ((0, 300), (1, 17)):
        for g in range(2):
            assert img[at:at + L * row] == k[b, g, :L].tobytes()
            at += L * row
            assert img[at:at + L * row] == v[b, g, :L].tobytes()
            at += L * row
    for b, n in ((0, 18), (1, 1), (2, 0)):
        for g in range(2):
            assert img[at:at + n * 256] == mean[b, g, :n].tobytes()
            at += n * 256
            assert img[at:at + 256] == run[b, g].tobytes()
            at += 256
    assert at == H + P
    # levels: (H + P) bytes in 4096-byte chunks (43 or 83 of them), their digests in groups of
    # 16 (3 or 6 digests), then the root over those
    n1 = -(-(H + P) // 4096)
    n2 = -(-n1 // 16)
    assert (n1, n2) == ((43, 3) if esz == 2 else (83, 6))
    d1, d2 = H + P, H + P + 32 * n1
    assert len(img) == d2 + 32 * n2 + 32 == N.image_bytes(lengths, 2, 64, 16, esz)
    for i in (0, n1 - 1):
        chunk = img[4096 * i:min(4096 * (i + 1), H + P)]
        assert img[d1 + 32 * i:d1 + 32 * (i + 1)] == N.sha256(chunk)
    for i in (0, n2 - 1):
        group = img[d1 + 512 * i:min(d1 + 512 * (i + 1), d2)]
        assert img[d2 + 32 * i:d2 + 32 * (i + 1)] == N.sha256(group)
    assert img[-32:] == N.sha256(img[d2:d2 + 32 * n2])


def test_parse_recovers_every_saved_array():
    k, v, mean, run, lengths, S = caches(np.uint16, lengths=(250, 33, 1))
    img = N.build_image(k, v, mean, run, lengths, S)
    h, L, seqs = N.parse_image(img)
    assert list(L) == [250, 33, 1] and h["B"] == 3
    for b in range(3):
        for g in range(2):
            assert np.array_equal(seqs[b]["k"][g], k[b, g, :L[b]])
            assert np.array_equal(seqs[b]["v"][g], v[b, g, :L[b]])
            assert np.array_equal(seqs[b]["mean"][g], mean[b, g, :L[b] // S])
            assert np.array_equal(seqs[b]["run"][g], run[b, g])


def test_rows_past_the_length_are_not_saved():
    k, v, mean, run, lengths, S = caches(np.float32)
    img = N.build_image(k, v, mean, run, lengths, S)
    k2, v2, m2 = k.copy(), v.copy(), mean.copy()
    k2[1, :, 17:] = 7.0
    v2[2] = -1.0
    m2[1, :, 1:] = 3.0
    assert N.build_image(k2, v2, m2, run, lengths, S) == img


def fp8_caches(B=3, Hkv=2, cap=300, d=64, S=16, lengths=(300, 17, 0), seed=3):
    rng = np.random.default_rng(seed)
    k = rng.integers(0, 256, size=(B, Hkv, cap, d), dtype=np.uint8)
    v = rng.integers(0, 256, size=(B, Hkv, cap, d), dtype=np.uint8)
    ks = rng.random((B, Hkv, cap)).astype(np.float32) + 0.5
    vs = rng.random((B, Hkv, cap)).astype(np.float32) + 0.5
    mean = rng.standard_normal((B, Hkv, cap // S, d)).astype(np.float32)
    run = rng.standard_normal((B, Hkv, d)).astype(np.float32)
    return k, v, ks, vs, mean, run, np.array(lengths, dtype=np.int64), S


def test_image_layout_of_the_8bit_cache():
    """Element type 2 (N3): per (b, g) K codes, V codes, then the K and V scale runs of L_b
    floats, each zero-padded to 16 bytes (17 rows: 68 bytes + 12 zeros).  Offsets by hand."""
    k, v, ks, vs, mean, run, lengths, S = fp8_caches()
    img = N.build_image(k, v, mean, run, lengths, S, ks, vs)
    H = 96
    assert struct.unpack("<I", img[12:16])[0] == 2
    # codes 2 x 2 x 317 rows x 64 bytes; scale runs 2 x (2 x 1200 + 2 x 80); summaries 2 x 22 x 256
    P = 81152 + 5120 + 11264
    assert struct.unpack("<QQ", img[32:48]) == (P, H)
    at = H
    for b, L, run_bytes in ((0, 300, 1200), (1, 17, 80)):
        for g in range(2):
            assert img[at:at + 64 * L] == k[b, g, :L].tobytes()
            at += 64 * L
            assert img[at:at + 64 * L] == v[b, g, :L].tobytes()
            at += 64 * L
            for sc in (ks, vs):
                assert img[at:at + 4 * L] == sc[b, g, :L].tobytes()
                assert img[at + 4 * L:at + run_bytes] == b"\0" * (run_bytes - 4 * L)
                at += run_bytes
    for b, n in ((0, 18), (1, 1), (2, 0)):
        for g in range(2):
            assert img[at:at + n * 256] == mean[b, g, :n].tobytes()
            at += n * 256 + 256
    assert at == H + P
    # (H + P) = 97632 bytes: 24 chunks, then 2 digests of groups of 16, then the root
    assert len(img) == H + P + 32 * (24 + 2) + 32 == N.image_bytes(lengths, 2, 64, 16, 1)
    assert N.verify(img) is None


def test_8bit_image_parse_and_rows_past_the_length():
    k, v, ks, vs, mean, run, lengths, S = fp8_caches(lengths=(250, 33, 1))
    img = N.build_image(k, v, mean, run, lengths, S, ks, vs)
    h, L, seqs = N.parse_image(img)
    assert h["dtype"] == 2 and list(L) == [250, 33, 1]
    for b in range(3):
        for g in range(2):
            assert np.array_equal(seqs[b]["k"][g], k[b, g, :L[b]])
            assert np.array_equal(seqs[b]["v"][g], v[b, g, :L[b]])
            assert np.array_equal(seqs[b]["k_scale"][g], ks[b, g, :L[b]])
            assert np.array_equal(seqs[b]["v_scale"][g], vs[b, g, :L[b]])
    ks2, vs2, k2 = ks.copy(), vs.copy(), k.copy()
    ks2[1, :, 33:] = 9.0
    vs2[2, :, 1:] = -2.0
    k2[0, :, 250:] = 1
    assert N.build_image(k2, v, mean, run, lengths, S, ks2, vs2) == img
    ks2[1, 1, 32] = 9.0  # a saved scale changes the image
    assert N.build_image(k, v, mean, run, lengths, S, ks2, vs) != img


def two_level_image():
    # K and V: 2 x 2 x 300 rows of 256 bytes each (bf16, d = 128) = 614400 bytes; summaries
    # 2 kv heads x (4 + 4 means + 2 running sums) x 512 bytes = 10240; header 80 -> 624720 bytes
    # = 153 chunks -> D_1 (153 digests), D_2 (10 digests, groups of 16)
    k, v, mean, run, lengths, S = caches(np.uint16, B=2, Hkv=2, cap=300, d=128, S=64, lengths=(300, 300))
    img = N.build_image(k, v, mean, run, lengths, S)
    h = N.parse_header(img)
    data = h["header"] + h["payload"]
    assert data == 624720 and N.level_counts(data) == [153, 10]
    return bytearray(img), data


def test_verify_accepts_an_intact_image():
    img, _ = two_level_image()
    assert N.verify(img) is None


@pytest.mark.parametrize("where", ["header", "payload", "last_data_byte"])
def test_verify_names_the_corrupted_data_chunk(where):
    img, data = two_level_image()
    header = bytes(img[:80])
    x = {"header": 70, "payload": 4096 * 77 + 1234, "last_data_byte": data - 1}[where]
    img[x] ^= 0x01
    assert N.verify(img, header) == 4096 * (x // 4096)
    if where != "header":
        assert N.verify(img) == 4096 * (x // 4096)


def test_verify_names_the_chunk_of_a_corrupted_digest():
    img, data = two_level_image()
    # a byte of D_1's digest of chunk 140: chunk 140's stored digest no longer matches
    img[data + 32 * 140 + 5] ^= 0x80
    assert N.verify(img) == 4096 * 140
    img, data = two_level_image()
    # a byte of D_2's second digest (over D_1's second group, digests 16..31)
    d2 = data + 32 * 153
    img[d2 + 32 + 3] ^= 0x10
    assert N.verify(img) == data + 512
    img, data = two_level_image()
    img[-1] ^= 0xFF  # the root covers D_2
    assert N.verify(img) == d2


def test_header_checks():
    img, _ = two_level_image()
    bad = bytearray(img)
    bad[0] = ord("X")
    with pytest.raises(ValueError):
        N.parse_header(bad)
    bad = bytearray(img)
    bad[48:52] = struct.pack("<I", 2048)
    with pytest.raises(ValueError):
        N.parse_header(bad)
