"""Pins of the oracle's decode step (one new query per head against the KV
cache; block selection from the query's stride softmax, the Top-tau prefix
plus the last block, then attention over the selected blocks). CPU only."""

import math

import numpy as np
import pytest
import torch

import oracle
from tests import brute


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def _brute_masses(q, k, S, B):
    """float64: full logits, stride means over each stride's tokens, softmax over strides, block sums."""
    q, k = q.astype(np.float64), k.astype(np.float64)
    Hq, d = q.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    ns, nb, r = -(-L // S), -(-L // B), B // S
    stride_of = np.arange(L) // S
    cnt = np.bincount(stride_of, minlength=ns).astype(np.float64)
    out = np.zeros((Hq, nb))
    for h in range(Hq):
        full = k[:, h // G, :] @ q[h] / math.sqrt(d)
        z = np.zeros(ns)
        np.add.at(z, stride_of, full)
        z /= cnt
        p = np.exp(z - z.max())
        p /= p.sum()
        np.add.at(out[h], np.arange(ns) // r, p)
    return out


CASES = [(512, 4, 2, 32, 8, 64), (203, 6, 2, 16, 4, 32), (1000, 2, 1, 64, 16, 128), (61, 2, 2, 16, 8, 32)]


@pytest.mark.parametrize("L,Hq,Hkv,d,S,B", CASES)
def test_decode_masses_match_brute_force(L, Hq, Hkv, d, S, B):
    q, k, v = _rand((Hq, d), 1 + L, 1.5), _rand((L, Hkv, d), 2 + L, 1.5), _rand((L, Hkv, d), 3 + L)
    res = oracle.decode(q, k, v, S=S, B=B, tau=0.9, round_bf16=False)
    np.testing.assert_allclose(res.mass, _brute_masses(q, k, S, B), rtol=2e-5, atol=2e-7)
    np.testing.assert_allclose(res.mass.sum(axis=1), 1.0, atol=2e-6)


def test_decode_tau_one_is_dense_attention():
    L, Hq, Hkv, d, S, B = 777, 4, 2, 32, 8, 64
    q, k, v = _rand((Hq, d), 11, 2.0), _rand((L, Hkv, d), 12), _rand((L, Hkv, d), 13)
    res = oracle.decode(q, k, v, S=S, B=B, tau=1.0, round_bf16=False)
    nb = -(-L // B)
    np.testing.assert_array_equal(res.row_count, nb)
    t = torch.from_numpy
    qq = t(q).double()[:, None, :]                                          # [Hq][1][d]
    kk = t(k).double().repeat_interleave(Hq // Hkv, dim=1).permute(1, 0, 2)  # [Hq][L][d]
    vv = t(v).double().repeat_interleave(Hq // Hkv, dim=1).permute(1, 0, 2)
    want = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[:, 0, :].numpy()
    np.testing.assert_allclose(res.out, want, rtol=1e-10, atol=1e-12)


def test_decode_equals_the_last_prefill_row_with_dense_lists():
    L, Hq, Hkv, d, B = 320, 4, 2, 16, 32
    Q, K, V = _rand((L, Hq, d), 21, 2.0), _rand((L, Hkv, d), 22), _rand((L, Hkv, d), 23)
    res = oracle.decode(Q[L - 1], K, V, S=4, B=B, tau=1.0, round_bf16=False)
    rc, ci = oracle.full_lists(L, Hq, B)
    pre = oracle.attention(Q, K, V, rc, ci, B=B, rows=np.array([[L - 1, h] for h in range(Hq)], np.int32))
    np.testing.assert_allclose(res.out, pre, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("tau", [0.3, 0.6, 0.9])
def test_decode_selection_is_min_cardinality_plus_last_block(tau):
    L, Hq, Hkv, d, S, B = 512, 4, 2, 32, 8, 64   # 8 blocks: exhaustive search is cheap
    q, k, v = _rand((Hq, d), 31, 3.0), _rand((L, Hkv, d), 32, 1.5), _rand((L, Hkv, d), 33)
    res = oracle.decode(q, k, v, S=S, B=B, tau=tau, round_bf16=False)
    nb = L // B
    for h in range(Hq):
        want, margin = brute.min_cardinality_set(res.mass[h].astype(np.float64), tau)
        want = sorted(want | {nb - 1})
        if margin > 1e-5:  # decisions fp32 can resolve
            np.testing.assert_array_equal(res.col_idx[h, : res.row_count[h]], want)
        assert res.col_idx[h, res.row_count[h] - 1] == nb - 1


def test_decode_attention_matches_masked_softmax():
    L, Hq, Hkv, d, S, B = 450, 4, 1, 16, 4, 32
    q, k, v = _rand((Hq, d), 41, 2.5), _rand((L, Hkv, d), 42, 1.5), _rand((L, Hkv, d), 43)
    res = oracle.decode(q, k, v, S=S, B=B, tau=0.5, round_bf16=False)
    nb = -(-L // B)
    for h in range(Hq):
        sel = np.zeros(nb, bool)
        sel[res.col_idx[h, : res.row_count[h]]] = True
        keys = np.nonzero(np.repeat(sel, B)[:L])[0]
        a = k[keys, 0, :].astype(np.float64) @ q[h].astype(np.float64) / math.sqrt(d)
        w = np.exp(a - a.max())
        want = w @ v[keys, 0, :].astype(np.float64) / w.sum()
        np.testing.assert_allclose(res.out[h], want, rtol=1e-10, atol=1e-12)
    # thresholds nest
    small = oracle.decode(q, k, v, S=S, B=B, tau=0.3, round_bf16=False)
    for h in range(Hq):
        assert set(small.col_idx[h, : small.row_count[h]]) <= set(res.col_idx[h, : res.row_count[h]])
