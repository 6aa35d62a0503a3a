"""GPU parity of session snapshots through the C ABI: the device-built image byte for byte
against the oracle's image of the same host arrays, the device check against the oracle's check
on the same corrupted bytes, restore into fresh buffers (rows and slots outside the saved state
untouched, nothing restored from a damaged image), a file round trip after which decoding
continues bit for bit, and the 1M-token cache (five digest levels).
"""
import numpy as np
import pytest
import torch

import content_routed_sparse_amd as ra
from oracle import snapshot as N
from synth import workloads as WL

from harness import Case, log, to_dev

pytestmark = pytest.mark.gpu

W = WL.WORKLOADS


def small(base, **kw):
    return W[base].scaled(**kw)


class SnapCase(Case):
    """A synth cache plus span means / running sums filled with seeded values (the snapshot does
    not interpret them), mirrored on the host."""

    def __init__(self, w, lengths, capacity=None, seed=11):
        super().__init__(w, lengths, capacity)
        rng = np.random.default_rng(seed)
        c = self.cfg
        self.mean_h = rng.standard_normal((c.batch, c.num_kv_heads, c.max_spans, c.head_dim)).astype(np.float32)
        self.run_h = rng.standard_normal((c.batch, c.num_kv_heads, c.head_dim)).astype(np.float32)
        self.pipe.span_mean.copy_(torch.from_numpy(self.mean_h))
        self.pipe.run_sum.copy_(torch.from_numpy(self.run_h))
        kind = np.uint16 if self.is_bf16 else np.float32
        self.K_h = np.zeros((c.batch, c.num_kv_heads, c.capacity, c.head_dim), dtype=kind)
        self.V_h = np.zeros_like(self.K_h)
        for b, L in enumerate(self.lengths):
            self.K_h[b, :, :L], self.V_h[b, :, :L] = self.host[b]

    def oracle_image(self):
        return N.build_image(self.K_h, self.V_h, self.mean_h, self.run_h, self.lengths, self.w.span_size)

    def pack(self, slack=0):
        n = ra.snapshot_bytes(self.cfg, self.lengths)
        img = torch.full((n + slack,), 0xAA, dtype=torch.uint8, device="cuda")
        ra.kv_snapshot_pack(self.cfg, self.K, self.V, self.pipe.span_mean, self.pipe.run_sum, self.lengths, img)
        torch.cuda.synchronize()
        return img, n


def first_difference(a, b):
    a = np.frombuffer(a, dtype=np.uint8)
    b = np.frombuffer(b, dtype=np.uint8)
    if len(a) != len(b):
        return "lengths %d vs %d" % (len(a), len(b))
    d = np.flatnonzero(a != b)
    return None if len(d) == 0 else int(d[0])


PACK_CASES = [
    ("bf16_d128_ragged_2levels", small("decode_1m", span_size=64, window=64, top_k=4, decode_len=5000),
     [5000, 1, 0, 777]),
    ("fp32_d64", W["tiny_prefill_fp32"], [3000, 129]),
    ("bf16_d64_Hkv2", small("decode_1m", num_q_heads=8, num_kv_heads=2, head_dim=64, span_size=32, window=32,
                            top_k=4, decode_len=2000), [2000, 31]),
]

@pytest.mark.parametrize("name,w,lengths", PACK_CASES, ids=[c[0] for c in PACK_CASES])
def test_pack_matches_the_oracle_image(name, w, lengths):
    c = SnapCase(w, lengths)
    img, n = c.pack(slack=4096)
    dev = img.cpu().numpy()
    ref = c.oracle_image()
    assert n == len(ref)
    assert first_difference(dev[:n].tobytes(), ref) is None, first_difference(dev[:n].tobytes(), ref)
    assert (dev[n:] == 0xAA).all()  # nothing written past the image


def corruptions(n_data, levels, image_len):
    """(name, offset) of single-byte flips: header, payload, last data byte, each digest level, root."""
    out = [("header", 70), ("payload", n_data // 2 + 3), ("last_data", n_data - 1)]
    at = n_data
    for i, cnt in enumerate(levels):
        out.append(("level%d" % (i + 1), at + 32 * (cnt - 1) + 7))
        at += 32 * cnt
    out.append(("root", image_len - 1))
    return out


def test_verify_agrees_with_the_oracle_on_corruptions():
    w = small("decode_1m", span_size=64, window=64, top_k=4, decode_len=5000)
    c = SnapCase(w, [5000, 1, 0, 777])
    img, n = c.pack()
    ref = bytearray(c.oracle_image())
    bad = torch.empty(1, dtype=torch.int64, device="cuda")
    h = N.parse_header(ref)
    data = h["header"] + h["payload"]
    header = bytes(ref[:h["header"]])
    ra.kv_snapshot_verify(header, img, bad)
    assert int(bad.item()) == -1 and N.verify(ref) is None
    for name, x in corruptions(data, N.level_counts(data), n):
        img2 = img.clone()
        img2[x] ^= 0x20
        ref2 = bytearray(ref)
        ref2[x] ^= 0x20
        expect = N.verify(ref2, header)
        ra.kv_snapshot_verify(header, img2, bad)
        got = int(bad.item())
        log("  corruption %s at %d -> %d (oracle %s)" % (name, x, got, expect))
        assert got == expect, name


def fresh_buffers(c):
    cfg = c.cfg
    shape = (cfg.batch, cfg.num_kv_heads, cfg.capacity, cfg.head_dim)
    K = torch.full(shape, 3.0, dtype=cfg.torch_dtype, device="cuda")
    V = torch.full(shape, -5.0, dtype=cfg.torch_dtype, device="cuda")
    M = torch.full(tuple(c.pipe.span_mean.shape), 7.0, dtype=torch.float32, device="cuda")
    R = torch.full(tuple(c.pipe.run_sum.shape), 9.0, dtype=torch.float32, device="cuda")
    return K, V, M, R


def bits(t):
    return t.cpu().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy()


def test_unpack_restores_exactly_the_saved_state():
    w = small("decode_1m", span_size=64, window=64, top_k=4, decode_len=3000)
    c = SnapCase(w, [3000, 100, 0], capacity=3100)
    img, n = c.pack()
    header = c.oracle_image()[:N.header_bytes(3)]
    K, V, M, R = fresh_buffers(c)
    ra.kv_snapshot_unpack(c.cfg, header, img, K, V, M, R)
    torch.cuda.synchronize()
    Kb, Vb, Mb, Rb = bits(K), bits(V), M.cpu().numpy(), R.cpu().numpy()
    k_fill, v_fill = bits(torch.full((1,), 3.0, dtype=K.dtype))[0], bits(torch.full((1,), -5.0, dtype=K.dtype))[0]
    for b, L in enumerate(c.lengths):
        assert np.array_equal(Kb[b, :, :L].view(c.K_h.dtype), c.K_h[b, :, :L])
        assert np.array_equal(Vb[b, :, :L].view(c.V_h.dtype), c.V_h[b, :, :L])
        assert (Kb[b, :, L:] == k_fill).all() and (Vb[b, :, L:] == v_fill).all()
        ns = L // w.span_size
        assert np.array_equal(Mb[b, :, :ns], c.mean_h[b, :, :ns]) and (Mb[b, :, ns:] == 7.0).all()
        assert np.array_equal(Rb[b], c.run_h[b])
    # a damaged image restores nothing when unpack is guarded by verify's word
    img[n // 3] ^= 1
    bad = torch.empty(1, dtype=torch.int64, device="cuda")
    K2, V2, M2, R2 = fresh_buffers(c)
    ra.kv_snapshot_verify(header, img, bad)
    ra.kv_snapshot_unpack(c.cfg, header, img, K2, V2, M2, R2, guard=bad)
    torch.cuda.synchronize()
    assert int(bad.item()) != -1
    assert (bits(K2) == k_fill).all() and (M2 == 7.0).all() and (R2 == 9.0).all()


def test_file_round_trip_then_decode_continues(tmp_path):
    w = small("decode_1m", span_size=64, window=64, top_k=8, decode_len=6000)
    L = np.array([6000, 2500])
    c = Case(w, L, capacity=6100)
    c.summarize(np.zeros(2, dtype=np.int64), L)
    rows, _ = c.rows_for([0, 1], L - 1)
    out0 = c.attend(rows, ra.RA_OP_DECODE).clone()
    path = str(tmp_path / "session.crsnap")
    root = ra.save_snapshot(path, c.cfg, c.K, c.V, c.pipe.span_mean, c.pipe.run_sum, L)
    with open(path, "rb") as f:
        on_disk = f.read()
    assert N.verify(on_disk) is None and on_disk[-32:].hex() == root
    K, V, M, R = fresh_buffers(c)
    got = ra.load_snapshot(path, c.cfg, K, V, M, R)
    assert list(got) == list(L)
    c.K, c.V = K, V
    c.pipe.span_mean.copy_(M)
    c.pipe.run_sum.copy_(R)
    out1 = c.attend(rows, ra.RA_OP_DECODE)
    assert torch.equal(out0, out1)
    # a damaged file is refused and restores nothing
    bad = bytearray(on_disk)
    bad[len(bad) // 2] ^= 0x04
    with open(path, "wb") as f:
        f.write(bad)
    K2, V2, M2, R2 = fresh_buffers(c)
    with pytest.raises(ra.RoutedAttnError):
        ra.load_snapshot(path, c.cfg, K2, V2, M2, R2)
    assert (M2 == 7.0).all() and (R2 == 9.0).all()


@pytest.mark.timeout(900)
def test_snapshot_of_the_1m_cache():
    """decode_1m (1M tokens x 4 kv heads, 2 GiB of bf16 K/V): the whole image against the
    oracle's (five digest levels), then a check that names one flipped byte."""
    w = W["decode_1m"]
    c = SnapCase(w, [w.decode_len])
    img, n = c.pack()
    ref = c.oracle_image()
    h = N.parse_header(ref)
    assert len(N.level_counts(h["header"] + h["payload"])) == 5  # 524801, 32801, 2051, 129, 9 digests
    assert first_difference(img.cpu().numpy().tobytes(), ref) is None
    bad = torch.empty(1, dtype=torch.int64, device="cuda")
    header = ref[:h["header"]]
    ra.kv_snapshot_verify(header, img, bad)
    assert int(bad.item()) == -1
    x = 1_234_567_891
    img[x] ^= 0x40
    ra.kv_snapshot_verify(header, img, bad)
    assert int(bad.item()) == 4096 * (x // 4096)


# ------------------------------------------------------------------------- the 8-bit cache
class Fp8SnapCase(SnapCase):
    """SnapCase whose bf16 cache is quantised on the device to the 8-bit cache (E4M3 codes and
    one fp32 scale per row); rows past the lengths keep sentinel codes and scales."""

    def __init__(self, w, lengths, capacity=None, seed=11):
        super().__init__(w, lengths, capacity, seed)
        c = self.cfg
        shape = (c.batch, c.num_kv_heads, c.capacity, c.head_dim)
        self.K8 = torch.full(shape, 0xAA, dtype=torch.uint8, device="cuda")
        self.V8 = torch.full(shape, 0x55, dtype=torch.uint8, device="cuda")
        self.KS = torch.full(shape[:3], -1.0, dtype=torch.float32, device="cuda")
        self.VS = torch.full(shape[:3], -2.0, dtype=torch.float32, device="cuda")
        zero = torch.zeros(c.batch, dtype=torch.int64, device="cuda")
        L = torch.as_tensor(self.lengths).cuda()
        most = max(1, int(self.lengths.max()))
        ra.kv_quantize_fp8(c, self.K, self.K8, self.KS, zero, L, most)
        ra.kv_quantize_fp8(c, self.V, self.V8, self.VS, zero, L, most)
        torch.cuda.synchronize()

    def oracle_image(self):
        return N.build_image(self.K8.cpu().numpy(), self.V8.cpu().numpy(), self.mean_h, self.run_h, self.lengths,
                             self.w.span_size, self.KS.cpu().numpy(), self.VS.cpu().numpy())

    def pack(self, slack=0):
        n = ra.snapshot_bytes_fp8(self.cfg, self.lengths)
        img = torch.full((n + slack,), 0xAA, dtype=torch.uint8, device="cuda")
        ra.kv_snapshot_pack_fp8(self.cfg, self.K8, self.V8, self.KS, self.VS, self.pipe.span_mean, self.pipe.run_sum,
                                self.lengths, img)
        torch.cuda.synchronize()
        return img, n


FP8_PACK_CASES = [
    # capacities that are not multiples of 4: the scale rows of most (sequence, kv head) pairs do
    # not start on 16 bytes; lengths 1 and 777 leave 12 bytes of padding after each scale run
    ("d128_ragged_cap5003", small("decode_1m", span_size=64, window=64, top_k=4, decode_len=5000),
     [5000, 1, 0, 777], 5003),
    ("d64_Hkv2_cap2001", small("decode_1m", num_q_heads=8, num_kv_heads=2, head_dim=64, span_size=32, window=32,
                               top_k=4, decode_len=2000), [2000, 30], 2001),
]


@pytest.mark.parametrize("name,w,lengths,cap", FP8_PACK_CASES, ids=[c[0] for c in FP8_PACK_CASES])
def test_pack_of_the_8bit_cache_matches_the_oracle_image(name, w, lengths, cap):
    c = Fp8SnapCase(w, lengths, capacity=cap)
    img, n = c.pack(slack=4096)
    dev = img.cpu().numpy()
    ref = c.oracle_image()
    assert n == len(ref)
    assert first_difference(dev[:n].tobytes(), ref) is None, first_difference(dev[:n].tobytes(), ref)
    assert (dev[n:] == 0xAA).all()
    # the device check names the chunk of a flipped scale byte and of a flipped padding byte
    h = N.parse_header(ref)
    header = bytes(ref[:h["header"]])
    bad = torch.empty(1, dtype=torch.int64, device="cuda")
    L0 = int(c.lengths[0])
    d = w.head_dim
    k_scale_at = h["header"] + 2 * L0 * d  # sequence 0, kv head 0: after its K and V codes
    L1 = int(c.lengths[1])
    seq1 = h["header"] + w.num_kv_heads * (2 * L0 * d + 2 * N.scale_run_bytes(L0))
    pad_at = seq1 + 2 * L1 * d + 4 * L1  # first padding byte after sequence 1's K scales
    for x in (k_scale_at + 5, pad_at):
        img2 = img.clone()
        img2[x] ^= 0x10
        ref2 = bytearray(ref)
        ref2[x] ^= 0x10
        ra.kv_snapshot_verify(header, img2, bad)
        assert int(bad.item()) == N.verify(ref2, header) == 4096 * (x // 4096)


def fp8_sentinels(c):
    cfg = c.cfg
    shape = (cfg.batch, cfg.num_kv_heads, cfg.capacity, cfg.head_dim)
    return (torch.full(shape, 0x11, dtype=torch.uint8, device="cuda"),
            torch.full(shape, 0x22, dtype=torch.uint8, device="cuda"),
            torch.full(shape[:3], 3.0, dtype=torch.float32, device="cuda"),
            torch.full(shape[:3], 4.0, dtype=torch.float32, device="cuda"),
            torch.full(tuple(c.pipe.span_mean.shape), 7.0, dtype=torch.float32, device="cuda"),
            torch.full(tuple(c.pipe.run_sum.shape), 9.0, dtype=torch.float32, device="cuda"))


def test_unpack_of_the_8bit_cache_restores_exactly_the_saved_state():
    """Codes, scales and summaries of the live rows restored; every other code, scale slot (the
    image's padding included) and summary slot untouched; a damaged image restores nothing."""
    w = small("decode_1m", span_size=64, window=64, top_k=4, decode_len=3000)
    c = Fp8SnapCase(w, [3000, 101, 0], capacity=3103)
    img, n = c.pack()
    header = c.oracle_image()[:N.header_bytes(3)]
    K8, V8, KS, VS, M, R = fp8_sentinels(c)
    ra.kv_snapshot_unpack_fp8(c.cfg, header, img, K8, V8, KS, VS, M, R)
    torch.cuda.synchronize()
    src = [t.cpu().numpy() for t in (c.K8, c.V8, c.KS, c.VS)]
    got = [t.cpu().numpy() for t in (K8, V8, KS, VS)]
    fills = (0x11, 0x22, 3.0, 4.0)
    for b, L in enumerate(c.lengths):
        for s_, g_, f in zip(src, got, fills):
            assert np.array_equal(g_[b, :, :L], s_[b, :, :L])
            assert (g_[b, :, L:] == f).all()
        ns = L // w.span_size
        Mb, Rb = M.cpu().numpy(), R.cpu().numpy()
        assert np.array_equal(Mb[b, :, :ns], c.mean_h[b, :, :ns]) and (Mb[b, :, ns:] == 7.0).all()
        assert np.array_equal(Rb[b], c.run_h[b])
    img[n // 2] ^= 1
    bad = torch.empty(1, dtype=torch.int64, device="cuda")
    K8b, V8b, KSb, VSb, Mb2, Rb2 = fp8_sentinels(c)
    ra.kv_snapshot_verify(header, img, bad)
    ra.kv_snapshot_unpack_fp8(c.cfg, header, img, K8b, V8b, KSb, VSb, Mb2, Rb2, guard=bad)
    torch.cuda.synchronize()
    assert int(bad.item()) != -1
    assert (K8b == 0x11).all() and (KSb == 3.0).all() and (VSb == 4.0).all() and (Mb2 == 7.0).all()


def test_8bit_file_round_trip_then_decode_continues(tmp_path):
    """Summaries over the 8-bit cache, a decode step, save to a file, load into fresh buffers:
    the same decode step gives the same bits."""
    w = small("decode_1m", span_size=64, window=64, top_k=8, decode_len=6000)
    L = np.array([6000, 2501])
    c = Fp8SnapCase(w, L, capacity=6101)
    cfg = c.cfg
    zero = torch.zeros(2, dtype=torch.int64, device="cuda")
    Ld = torch.as_tensor(L).cuda()
    ra.span_summary_update_fp8(cfg, c.K8, c.KS, c.pipe.span_mean, c.pipe.run_sum, zero, Ld, int(L.max()))
    rows, _ = c.rows_for([0, 1], L - 1)
    p = c.pipe
    p.reserve(2, int(L.max()) - 1, ra.RA_OP_DECODE)

    def decode(K8, V8, KS, VS, M):
        ra.route_scores(cfg, rows, M, p.scores)
        ra.topk_spans(cfg, rows, p.scores, p.sel)
        ra.routed_attn_decode_fp8(cfg, rows, K8, V8, KS, VS, p.sel, p.out, p.workspace)
        torch.cuda.synchronize()
        return p.sel.clone(), p.out.clone()

    sel0, out0 = decode(c.K8, c.V8, c.KS, c.VS, p.span_mean)
    path = str(tmp_path / "session8.crsnap")
    root = ra.save_snapshot_fp8(path, cfg, c.K8, c.V8, c.KS, c.VS, p.span_mean, p.run_sum, L)
    with open(path, "rb") as f:
        on_disk = f.read()
    assert N.verify(on_disk) is None and on_disk[-32:].hex() == root
    assert N.parse_header(on_disk)["dtype"] == 2
    K8, V8, KS, VS, M, R = fp8_sentinels(c)
    got = ra.load_snapshot_fp8(path, cfg, K8, V8, KS, VS, M, R)
    assert list(got) == list(L)
    assert torch.equal(R, p.run_sum)
    sel1, out1 = decode(K8, V8, KS, VS, M)
    assert torch.equal(sel0, sel1) and torch.equal(out0, out1)
