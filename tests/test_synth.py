"""The seeded generator: determinism, position addressability, layouts and value recipe."""
import numpy as np

import synth
from synth import workloads as WL


def test_subrange_regenerates_identically():
    a = synth.fill(synth.BF16, 77, 2, 3, 0, 4, 100, 300, 128, 0, 64, 2.0)
    b = synth.fill(synth.BF16, 77, 2, 3, 1, 2, 250, 20, 128, 0, 64, 2.0)
    assert np.array_equal(a[1:3, 150:170], b)
    c = synth.fill(synth.F32, 77, 1, 0, 0, 8, 10, 5, 64, 1)
    d = synth.fill(synth.F32, 77, 1, 0, 0, 8, 10, 5, 64, 0)
    assert np.array_equal(c.transpose(1, 0, 2), d)


def test_normal_statistics_and_streams_differ():
    x = synth.fill(synth.F32, 5, 3, 0, 0, 1, 0, 20000, 64, 0).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.var() - 1) < 0.02
    y = synth.fill(synth.F32, 5, 2, 0, 0, 1, 0, 20000, 64, 0)
    assert not np.array_equal(x.astype(np.float32), y)


def test_span_offset_has_norm_two_and_is_constant_within_span():
    S = 32
    noisy = synth.fill(synth.F32, 9, 2, 0, 0, 2, 0, 4 * S, 128, 0, S, 2.0).astype(np.float64)
    plain = synth.fill(synth.F32, 9, 2, 0, 0, 2, 0, 4 * S, 128, 0, S, 0.0).astype(np.float64)
    off = noisy - plain
    for h in range(2):
        for j in range(4):
            blk = off[h, j * S:(j + 1) * S]
            assert np.allclose(blk, blk[0], atol=1e-5)
            assert abs(np.linalg.norm(blk[0]) - 2.0) < 1e-4
    assert not np.allclose(off[0, 0], off[0, S])


def test_bf16_is_rne_of_fp32():
    import torch
    f = synth.fill(synth.F32, 11, 3, 0, 0, 1, 0, 500, 64, 0)
    b = synth.fill(synth.BF16, 11, 3, 0, 0, 1, 0, 500, 64, 0)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def test_ragged_lengths_in_range_and_seeded():
    w = WL.WORKLOADS["ragged_decode_16"]
    a = w.seq_lengths()
    assert len(a) == 16 and a.min() >= 65536 and a.max() <= 524288
    assert np.array_equal(a, w.seq_lengths()) and len(set(a.tolist())) == 16
