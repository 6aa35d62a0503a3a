"""Pins for the cold-retrieval oracle (oracle/cold_retrieval.py): sign bits against torch's
signbit, the packing against a hand-packed example, Hamming distances against an element-by-element
sign comparison, the selection against the defining order checked over every pair on tiny inputs
with heavy ties, and the attention against torch's float64 scaled-dot-product attention in the
cases that reduce to dense causal attention (every cold token fetched, or none cold).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from oracle import cold_retrieval as C


def to_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


@pytest.mark.parametrize("bf16", [False, True])
def test_sign_bits_match_torch_signbit(bf16):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(5000), [0.0, -0.0, np.inf, -np.inf, 1e-40, -1e-40]]).astype(np.float32)
    stored = to_bits(x) if bf16 else x
    t = torch.from_numpy(x).to(torch.bfloat16) if bf16 else torch.from_numpy(x)
    assert np.array_equal(C.sign_bits(stored, bf16), torch.signbit(t).numpy().astype(np.uint8))


def test_signature_packing_by_hand():
    v = np.ones(16, dtype=np.float32)
    v[[0, 3, 9, 15]] = -2.0
    # byte 0: bits 0 and 3 -> 0b00001001; byte 1: bits 1 and 7 -> 0b10000010
    assert list(C.signatures(v, False)) == [9, 130]
    assert list(C.signatures(to_bits(v), True)) == [9, 130]


def test_hamming_counts_differing_signs():
    rng = np.random.default_rng(2)
    for d in (8, 64, 128):
        q = rng.standard_normal(d).astype(np.float32)
        k = rng.standard_normal((50, d)).astype(np.float32)
        k[0] = -q  # every sign differs
        k[1] = q * 3  # none differs
        ref = [sum(math.copysign(1, float(a)) != math.copysign(1, float(b)) for a, b in zip(q, row)) for row in k]
        got = C.hamming(C.signatures(q, False), C.signatures(k, False))
        assert list(got) == ref and got[0] == d and got[1] == 0


@pytest.mark.parametrize("kc", [1, 3, 7, 40])
def test_selection_is_the_smallest_by_distance_then_position(kc):
    rng = np.random.default_rng(3)
    d, H = 8, 5  # 8-bit signatures: distances collide constantly
    for trial in range(30):
        L = int(rng.integers(1, 60))
        keys = to_bits(rng.standard_normal((L, d)))
        q = to_bits(rng.standard_normal(d))
        sk = C.signatures(keys, True)
        sq = C.signatures(q, True)
        t = L - 1
        sel = C.select_cold(sq, sk, t, H, kc)
        n = max(0, t - H + 1)
        m = min(kc, n)
        chosen = [int(p) for p in sel if p >= 0]
        assert len(chosen) == m and list(sel[m:]) == [-1] * (kc - m) and chosen == sorted(chosen)
        dist = [sum(int(a) != int(b) for a, b in zip(C.sign_bits(q, True), C.sign_bits(keys[p], True)))
                for p in range(n)]
        rest = [p for p in range(n) if p not in chosen]
        for p in chosen:
            for r in rest:
                assert (dist[p], p) < (dist[r], r)


def _sdpa_f64(q, keys, values, upto):
    qt = torch.from_numpy(q)[None, None, None, :]
    kt = torch.from_numpy(keys[:upto + 1])[None, None]
    vt = torch.from_numpy(values[:upto + 1])[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, 0, 0].numpy()


@pytest.mark.parametrize("bf16", [False, True])
def test_all_cold_fetched_or_none_cold_is_dense_causal_attention(bf16):
    rng = np.random.default_rng(4)
    L, d, hkv, hq, H = 200, 16, 2, 4, 32
    keys = rng.standard_normal((hkv, L, d)).astype(np.float32)
    values = rng.standard_normal((hkv, L, d)).astype(np.float32)
    qs = rng.standard_normal((L, hq, d)).astype(np.float32)
    if bf16:
        keys, values, qs = to_bits(keys), to_bits(values), to_bits(qs)
    kd, vd, qd = O.widen(keys, bf16), O.widen(values, bf16), O.widen(qs, bf16)
    every = C.ColdProblem(keys, values, L, hq, H, L, bf16)  # top_k_cold >= any cold count
    few = C.ColdProblem(keys, values, L, hq, H, 3, bf16)
    for t in [0, 1, 17, 31, 32, 33, 100, 199]:
        for h in range(hq):
            ref = _sdpa_f64(qd[t, h], kd[h // 2], vd[h // 2], t)
            assert np.abs(every.row(qs[t, h], h, t)["out"] - ref).max() < 1e-12
            if t < H:  # no cold token at all
                assert np.abs(few.row(qs[t, h], h, t)["out"] - ref).max() < 1e-12


def test_attention_is_masked_attention_over_hot_and_fetched():
    rng = np.random.default_rng(5)
    L, d, H, kc = 300, 16, 40, 6
    keys = rng.standard_normal((1, L, d)).astype(np.float32)
    values = rng.standard_normal((1, L, d)).astype(np.float32)
    prob = C.ColdProblem(keys, values, L, 1, H, kc, False)
    for t in [50, 150, 299]:
        q = rng.standard_normal(d).astype(np.float32)
        res = prob.row(q, 0, t)
        mask = np.zeros(L, dtype=bool)
        mask[[p for p in res["sel"] if p >= 0]] = True
        mask[t - H + 1:t + 1] = True
        qt = torch.from_numpy(q.astype(np.float64))[None, None, None, :]
        kt = torch.from_numpy(keys[0].astype(np.float64))[None, None]
        vt = torch.from_numpy(values[0].astype(np.float64))[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask)[None, None, None])
        assert np.abs(res["out"] - ref[0, 0, 0].numpy()).max() < 1e-12
        assert res["n_attended"] == kc + H


def test_a_key_with_the_querys_signs_is_always_fetched():
    rng = np.random.default_rng(6)
    L, d, H, kc = 2000, 64, 256, 4
    keys = to_bits(rng.standard_normal((1, L, d)))
    q = to_bits(rng.standard_normal(d))
    qf = O.widen(q, True)
    keys[0, 777] = to_bits(np.abs(rng.standard_normal(d)) * np.sign(qf))  # same signs: distance 0
    keys[0, 5] = to_bits(-np.abs(rng.standard_normal(d)) * np.sign(qf))  # all signs differ: distance d
    prob = C.ColdProblem(keys, keys, L, 1, H, kc, True)
    sel = prob.row(q, 0, L - 1)["sel"]
    assert 777 in sel and 5 not in sel
    assert prob.distances(q, 0, L - 1)[777] == 0
