"""The C ABI without a GPU: the library loads, exports every declared entry point, and rejects
invalid arguments on the host before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import content_routed_sparse_amd as ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            names += re.findall(r"^(?:ra_status|size_t|const char \*)\s*(\w+)\(", text, flags=re.M)
    return names


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(ra.EXPORTED) <= set(names)
    lib = ra.lib()
    for n in names:
        assert hasattr(lib, n), n


def cfg(**kw):
    base = dict(num_q_heads=32, num_kv_heads=4, head_dim=128, span_size=1024, top_k=16, window=1024,
                dtype=ra.RA_BF16, batch=1, capacity=1 << 20)
    base.update(kw)
    if base["span_size"] < 1:
        base["max_spans"] = 1
    return ra.Config(**base)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def rows(n=1, max_pos=(1 << 20) - 1):
    return ra._Rows(0x1000, 0x1000, 0x1000, n, max_pos)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), 2), (dict(num_q_heads=30), 1), (dict(top_k=0), 1), (dict(top_k=65), 2),
    (dict(span_size=0), 1), (dict(window=0), 1), (dict(dtype=7), 2), (dict(batch=0), 1),
    (dict(max_spans=3), 3), (dict(num_q_heads=64, num_kv_heads=1), 2),
])
def test_config_validation(kw, status):
    c = cfg(**kw).c()
    r = rows()
    lib = ra.lib()
    assert lib.topk_spans(ctypes.byref(c), ctypes.byref(r), FAKE, 1024, FAKE, None) == status
    assert lib.ra_last_error().decode() != ""


def test_argument_validation_before_launch():
    lib = ra.lib()
    c = cfg().c()
    assert lib.route_scores(None, ctypes.byref(rows()), FAKE, FAKE, 1023, None) == 1
    # score stride below the routable count at max_pos
    assert lib.route_scores(ctypes.byref(c), ctypes.byref(rows()), FAKE, FAKE, 1022, None) == 3
    # max_pos outside the cache
    assert lib.topk_spans(ctypes.byref(c), ctypes.byref(rows(max_pos=1 << 20)), FAKE, 1023, FAKE, None) == 3
    # NULL outputs
    assert lib.routed_attn_decode(ctypes.byref(c), ctypes.byref(rows()), FAKE, FAKE, FAKE, None, FAKE, 1 << 30,
                                  None) == 1
    # workspace too small
    assert lib.routed_attn_prefill(ctypes.byref(c), ctypes.byref(rows(8192)), FAKE, FAKE, FAKE, FAKE, FAKE, 16,
                                   None) == 3
    # summary: max_new beyond capacity
    assert lib.span_summary_update(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, (1 << 20) + 1, None) == 3
    assert lib.span_summary_update(ctypes.byref(c), None, FAKE, FAKE, FAKE, FAKE, 1, None) == 1
    # dense attention: bf16 only, capacity * d below 2^31, non-NULL buffers
    c32 = cfg(dtype=ra.RA_F32).c()
    assert lib.attn_dense_causal(ctypes.byref(c32), ctypes.byref(rows()), FAKE, FAKE, FAKE, None) == 2
    big = cfg(capacity=1 << 24, max_spans=1 << 14).c()
    assert lib.attn_dense_causal(ctypes.byref(big), ctypes.byref(rows()), FAKE, FAKE, FAKE, None) == 2
    assert lib.attn_dense_causal(ctypes.byref(c), ctypes.byref(rows()), FAKE, FAKE, None, None) == 1


def test_fp8_entry_points_validate_before_launch():
    lib = ra.lib()
    c = cfg().c()
    c32 = cfg(dtype=ra.RA_F32).c()
    n = ctypes.c_int64(10)
    # 8-bit caches go with bf16 queries
    assert lib.kv_quantize_fp8(ctypes.byref(c32), FAKE, FAKE, FAKE, FAKE, FAKE, 10, None) == 2
    assert lib.span_summary_update_fp8(ctypes.byref(c32), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, None) == 2
    # NULL pointers, negative or oversized token counts
    assert lib.kv_quantize_fp8(ctypes.byref(c), FAKE, None, FAKE, FAKE, FAKE, 10, None) == 1
    assert lib.kv_quantize_fp8(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, -1, None) == 1
    assert lib.kv_quantize_fp8(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, (1 << 20) + 1, None) == 3
    assert lib.span_summary_update_fp8(ctypes.byref(c), FAKE, None, FAKE, FAKE, FAKE, FAKE, 10, None) == 1
    ws = 1 << 30
    assert lib.routed_attn_decode_fp8(ctypes.byref(c), ctypes.byref(rows()), FAKE, FAKE, None, FAKE, FAKE, FAKE,
                                      FAKE, ws, None) == 1
    assert lib.routed_attn_decode_fp8(ctypes.byref(c32), ctypes.byref(rows()), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, ws, None) == 2
    assert lib.routed_attn_decode_fp8(ctypes.byref(c), ctypes.byref(rows()), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, 16, None) == 3
    assert lib.ra_last_error().decode() != ""
    # prefill over the 8-bit cache: the same checks
    assert lib.routed_attn_prefill_fp8(ctypes.byref(c), ctypes.byref(rows()), FAKE, FAKE, None, FAKE, FAKE, FAKE,
                                       FAKE, ws, None) == 1
    assert lib.routed_attn_prefill_fp8(ctypes.byref(c32), ctypes.byref(rows()), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       FAKE, ws, None) == 2
    assert lib.routed_attn_prefill_fp8(ctypes.byref(c), ctypes.byref(rows(8192)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       FAKE, 16, None) == 3


def test_workspace_sizes():
    c = cfg()
    d = ra.workspace_bytes(c, ra.RA_OP_DECODE, 1, (1 << 20) - 1)
    # 32 heads x (16 selected + 2 window entries) x 4 sub-tiles x (4 + 128) floats
    assert d == 32 * 18 * 4 * 132 * 4
    p = ra.workspace_bytes(cfg(capacity=(1 << 20) + 8192), ra.RA_OP_PREFILL, 8192, (1 << 20) + 8191)
    # at least the partial records: bf16 inputs keep them as a 16-byte header + d fp16 values
    assert p > 8192 * 32 * 18 * (16 + 128 * 2)
    p32 = ra.workspace_bytes(cfg(capacity=(1 << 20) + 8192, dtype=ra.RA_F32), ra.RA_OP_PREFILL, 8192, (1 << 20) + 8191)
    assert p32 > 8192 * 32 * 18 * 132 * 4  # fp32 inputs: fp32 records
    assert ra.lib().ra_workspace_bytes(ctypes.byref(c.c()), 5, 1, 0) == 0
    assert ra.lib().ra_status_string(3) == b"buffer too small"


# ------------------------------------------------------------------------- session snapshots
def small_snapshot(dtype=np.uint16, lengths=(300, 17, 0)):
    from oracle import snapshot as N
    rng = np.random.default_rng(3)
    B, Hkv, cap, d, S = len(lengths), 2, 300, 64, 16
    k = rng.integers(0, 1 << 16, size=(B, Hkv, cap, d), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=(B, Hkv, cap, d), dtype=np.uint16)
    if dtype == np.float32:
        k, v = k.astype(np.float32), v.astype(np.float32)
    mean = rng.standard_normal((B, Hkv, cap // S, d)).astype(np.float32)
    run = rng.standard_normal((B, Hkv, d)).astype(np.float32)
    c = ra.Config(num_q_heads=4, num_kv_heads=Hkv, head_dim=d, span_size=S, top_k=4, window=S,
                  dtype=ra.RA_BF16 if dtype == np.uint16 else ra.RA_F32, batch=B, capacity=cap)
    return c, N.build_image(k, v, mean, run, np.array(lengths), S)


@pytest.mark.parametrize("dtype", [np.uint16, np.float32], ids=["bf16", "fp32"])
def test_snapshot_header_parse_and_size(dtype):
    from oracle import snapshot as N
    c, img = small_snapshot(dtype)
    info, lengths = ra.kv_snapshot_parse(img)
    assert list(lengths) == [300, 17, 0]
    assert (info["dtype"], info["batch"], info["num_kv_heads"], info["head_dim"], info["span_size"]) == \
        (c.dtype, 3, 2, 64, 16)
    assert info["image_bytes"] == len(img) == ra.snapshot_bytes(c, [300, 17, 0])
    assert info["header_bytes"] == N.header_bytes(3)
    # only the header is needed; an unaligned copy of it parses the same
    odd = bytearray(b"x") + img[:info["header_bytes"]]
    info2, lengths2 = ra.kv_snapshot_parse(np.frombuffer(bytes(odd), dtype=np.uint8)[1:])
    assert info2 == info and list(lengths2) == [300, 17, 0]


@pytest.mark.parametrize("offset,value", [(0, b"X"), (8, b"\x02"), (12, b"\x05"), (32, b"\x01"), (48, b"\x00\x08"),
                                          (64, b"\xff\xff\xff\xff\xff\xff\xff\xff")])
def test_snapshot_parse_rejects_malformed_headers(offset, value):
    _, img = small_snapshot()
    bad = bytearray(img[:96])
    bad[offset:offset + len(value)] = value
    with pytest.raises(ra.RoutedAttnError) as e:
        ra.kv_snapshot_parse(bytes(bad))
    assert e.value.status == 6
    with pytest.raises(ra.RoutedAttnError):
        ra.kv_snapshot_parse(img[:80])  # shorter than the header


def test_snapshot_entry_points_validate_before_launch():
    c, img = small_snapshot()
    lib = ra.lib()
    cc = c.c()
    L = np.array([300, 17, 0], dtype=np.int64)
    Lp = ctypes.c_void_p(L.ctypes.data)
    n = ra.snapshot_bytes(c, L)
    # NULL buffers, an image too small, lengths past the capacity
    assert lib.kv_snapshot_pack(ctypes.byref(cc), None, FAKE, FAKE, FAKE, Lp, FAKE, n, None) == 1
    assert lib.kv_snapshot_pack(ctypes.byref(cc), FAKE, FAKE, FAKE, FAKE, Lp, FAKE, n - 1, None) == 3
    L2 = np.array([301, 0, 0], dtype=np.int64)
    assert lib.kv_snapshot_pack(ctypes.byref(cc), FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(L2.ctypes.data), FAKE,
                                1 << 30, None) == 3
    assert lib.kv_snapshot_bytes(ctypes.byref(cc), ctypes.c_void_p(L2.ctypes.data)) == 0
    # verify: an image shorter than the header says
    hdr = np.frombuffer(img, dtype=np.uint8)
    assert lib.kv_snapshot_verify(ctypes.c_void_p(hdr.ctypes.data), 96, FAKE, len(img) - 1, FAKE, None) == 6
    # unpack into a configuration of another shape / dtype / batch
    for kw, status in ((dict(head_dim=128), 1), (dict(dtype=ra.RA_F32), 1), (dict(span_size=32, window=32), 1),
                       (dict(batch=2), 3), (dict(capacity=200), 3)):
        c2 = ra.Config(**{**c.__dict__, **kw, "max_spans": -1})
        cc2 = c2.c()
        st = lib.kv_snapshot_unpack(ctypes.byref(cc2), ctypes.c_void_p(hdr.ctypes.data), 96, FAKE, len(img), None,
                                    FAKE, FAKE, FAKE, FAKE, None)
        assert st == status, (kw, st, lib.ra_last_error())


def test_snapshot_of_the_8bit_cache_header_size_and_validation():
    """Element type 2 (codes + row scales): the library parses the oracle's image, sizes it alike,
    and rejects NULL or misaligned scale arrays, a short image and images of the other kind."""
    from oracle import snapshot as N
    rng = np.random.default_rng(5)
    B, Hkv, cap, d, S = 3, 2, 300, 64, 16
    lengths = np.array([300, 17, 0], dtype=np.int64)
    k, v = (rng.integers(0, 256, (B, Hkv, cap, d), dtype=np.uint8) for _ in range(2))
    ks, vs = (rng.random((B, Hkv, cap)).astype(np.float32) for _ in range(2))
    mean = rng.standard_normal((B, Hkv, cap // S, d)).astype(np.float32)
    run = rng.standard_normal((B, Hkv, d)).astype(np.float32)
    img = N.build_image(k, v, mean, run, lengths, S, ks, vs)
    c = ra.Config(num_q_heads=4, num_kv_heads=Hkv, head_dim=d, span_size=S, top_k=4, window=S, dtype=ra.RA_BF16,
                  batch=B, capacity=cap)
    info, L = ra.kv_snapshot_parse(img)
    assert info["dtype"] == ra.RA_SNAPSHOT_E4M3 and list(L) == [300, 17, 0]
    assert info["image_bytes"] == len(img) == ra.snapshot_bytes_fp8(c, lengths)
    assert ra.snapshot_bytes(c, lengths) != len(img)  # the bf16 image of the same state differs in size
    lib = ra.lib()
    cc = c.c()
    Lp = ctypes.c_void_p(lengths.ctypes.data)
    n = len(img)
    pack = lib.kv_snapshot_pack_fp8
    assert pack(ctypes.byref(cc), FAKE, FAKE, None, FAKE, FAKE, FAKE, Lp, FAKE, n, None) == 1
    assert pack(ctypes.byref(cc), FAKE, FAKE, FAKE, ctypes.c_void_p(0x1002), FAKE, FAKE, Lp, FAKE, n, None) == 1
    assert pack(ctypes.byref(cc), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, Lp, FAKE, n - 1, None) == 3
    hdr = np.frombuffer(img, dtype=np.uint8)
    assert lib.kv_snapshot_unpack(ctypes.byref(cc), ctypes.c_void_p(hdr.ctypes.data), 96, FAKE, n, None, FAKE, FAKE,
                                  FAKE, FAKE, None) == 1
    assert lib.kv_snapshot_unpack_fp8(ctypes.byref(cc), ctypes.c_void_p(hdr.ctypes.data), 96, FAKE, n - 1, None,
                                      FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 6
    _, img16 = small_snapshot()
    h16 = np.frombuffer(img16, dtype=np.uint8)
    assert lib.kv_snapshot_unpack_fp8(ctypes.byref(cc), ctypes.c_void_p(h16.ctypes.data), 96, FAKE, len(img16),
                                      None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1


def test_snapshot_file_helpers_round_trip(tmp_path):
    _, img = small_snapshot()
    p = str(tmp_path / "s.bin")
    ra.kv_snapshot_write_file(p, img)
    back = ra.kv_snapshot_read_file(p, pin=False)
    assert bytes(back.numpy()) == img
    assert not os.path.exists(p + ".tmp")
    with pytest.raises(ra.RoutedAttnError) as e:
        ra.kv_snapshot_read_file(str(tmp_path / "missing.bin"), pin=False)
    assert e.value.status == 5


# ------------------------------------------------------------------- token-level cold retrieval
def test_cold_entry_points_validate_before_launch():
    lib = ra.lib()
    c = cfg(batch=1)
    cc = c.c()
    r = rows()
    L = 1 << 20
    need = lib.ra_cold_workspace_bytes(ctypes.byref(cc), 1, L - 1, 256, 64)
    assert need == 32 * ((L - 256 + 16383) // 16384) * 64 * 8  # G = 8: tiles of 16384 positions
    g32 = cfg(batch=1, num_q_heads=32, num_kv_heads=1).c()
    assert lib.ra_cold_workspace_bytes(ctypes.byref(g32), 1, L - 1, 256, 64) == 32 * ((L - 256 + 8191) // 8192) * 64 * 8
    for hot, kc, status in ((0, 64, 1), (256, 0, 2), (256, 129, 2)):
        assert lib.cold_select(ctypes.byref(cc), ctypes.byref(r), FAKE, hot, kc, FAKE, FAKE, 1 << 30, None) == status
        assert lib.cold_attn_decode(ctypes.byref(cc), ctypes.byref(r), FAKE, FAKE, FAKE, hot, kc, FAKE, None) == status
        assert lib.ra_cold_workspace_bytes(ctypes.byref(cc), 1, L - 1, hot, kc) == 0
    assert lib.cold_select(ctypes.byref(cc), ctypes.byref(r), FAKE, 256, 64, FAKE, FAKE, need - 1, None) == 3
    assert lib.cold_select(ctypes.byref(cc), ctypes.byref(r), None, 256, 64, FAKE, FAKE, need, None) == 1
    assert lib.cold_attn_decode(ctypes.byref(cc), ctypes.byref(r), FAKE, None, FAKE, 256, 64, FAKE, None) == 1
    big = cfg(capacity=1 << 31).c()
    assert lib.cold_select(ctypes.byref(big), ctypes.byref(r), FAKE, 256, 64, FAKE, FAKE, 1 << 40, None) == 2
    one = np.zeros(1, dtype=np.int64)
    op = ctypes.c_void_p(one.ctypes.data)
    assert lib.kv_signature_update(ctypes.byref(cc), FAKE, None, op, op, 1, None) == 1
    assert lib.kv_signature_update(ctypes.byref(cc), FAKE, ctypes.c_void_p(0x1008), op, op, 1, None) == 1  # alignment
    assert lib.kv_signature_update(ctypes.byref(cc), FAKE, FAKE, op, op, (1 << 20) + 1, None) == 3


def test_grid_limits_are_checked_before_launch():
    """A launch needs fewer than 2^32 work-items (blocks x threads) per grid dimension.  A
    chunk-sized call through the decode entry point (8192 rows, 4 kv heads, 130 slots, 4
    sub-tiles: 17.04M units of 256 threads) is rejected on the host as unsupported, while the
    same call with 4096 rows (8.52M units) passes validation and fails only on the workspace."""
    lib = ra.lib()
    c = cfg(capacity=(1 << 20) + 8192).c()
    big_ws = ctypes.c_size_t(1 << 62)
    st = lib.routed_attn_decode(ctypes.byref(c), ctypes.byref(rows(8192, (1 << 20) + 8191)), FAKE, FAKE, FAKE, FAKE,
                                FAKE, big_ws, None)
    assert st == 2 and "2^32" in lib.ra_last_error().decode()
    st = lib.routed_attn_decode(ctypes.byref(c), ctypes.byref(rows(4096, (1 << 20) + 8191)), FAKE, FAKE, FAKE, FAKE,
                                FAKE, 16, None)
    assert st == 3
    # the 8-bit entry point has the same units
    st = lib.routed_attn_decode_fp8(ctypes.byref(c), ctypes.byref(rows(8192, (1 << 20) + 8191)), FAKE, FAKE, FAKE,
                                    FAKE, FAKE, FAKE, FAKE, big_ws, None)
    assert st == 2
    # every entry point indexes row-heads with 32 bits: 2^26 rows x 32 query heads is refused
    st = lib.attn_dense_causal(ctypes.byref(c), ctypes.byref(rows(1 << 26, (1 << 20) + 8191)), FAKE, FAKE, FAKE, None)
    assert st == 2 and "too many rows" in lib.ra_last_error().decode()
    st = lib.attn_dense_causal(ctypes.byref(c), ctypes.byref(rows(1 << 25, (1 << 20) + 8191)), FAKE, FAKE, None, None)
    assert st == 1  # (below the limit: the NULL output is what fails)


def test_noalloc_decode_validates_before_launch():
    """routed_attn_decode_noalloc: invalid arguments and calls whose records would not fit the
    library's fixed 32 MiB scratch are rejected on the host."""
    lib = ra.lib()
    c = cfg().c()
    assert lib.routed_attn_decode_noalloc(None, ctypes.byref(rows()), FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.routed_attn_decode_noalloc(ctypes.byref(c), ctypes.byref(rows()), FAKE, FAKE, None, FAKE, None) == 1
    # 1.16 MiB of records per 1M-context row: 40 rows need more than 32 MiB
    assert lib.routed_attn_decode_noalloc(ctypes.byref(c), ctypes.byref(rows(40)), FAKE, FAKE, FAKE, FAKE, None) == 3
    assert "scratch" in lib.ra_last_error().decode()


def test_route_topk_spans_validates_before_launch():
    """The fused routing + selection: a workspace of the stated size (counters + room for the
    scores) for every shape (2559 routable spans included), no NULL buffers."""
    lib = ra.lib()
    c = cfg().c()
    big = ctypes.c_size_t(1 << 40)
    assert lib.route_topk_spans(ctypes.byref(c), ctypes.byref(rows()), FAKE, None, FAKE, big, None) == 1
    c10m = cfg(span_size=4096, window=4096, capacity=10485760)  # 2559 routable spans
    need10 = ra.workspace_bytes(c10m, ra.RA_OP_ROUTE_TOPK, 1, 10485759)
    assert need10 == 256 + 32 * 2560 * 4
    st = lib.route_topk_spans(ctypes.byref(c10m.c()), ctypes.byref(rows(1, 10485759)), FAKE, FAKE, FAKE, need10 - 1,
                              None)
    assert st == 3
    need = ra.workspace_bytes(cfg(), ra.RA_OP_ROUTE_TOPK, 1, (1 << 20) - 1)
    assert need == 256 + 32 * 1024 * 4  # 4 counters (one 256-byte line), 32 heads x 1023 scores padded to 1024
    assert lib.route_topk_spans(ctypes.byref(c), ctypes.byref(rows()), FAKE, FAKE, FAKE, need - 1, None) == 3
