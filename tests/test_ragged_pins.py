"""Pins of the oracle on ragged inputs (sequence length not a multiple of the
block or the stride: a short last block and stride) and on a threshold per
query head. CPU only."""

import numpy as np
import pytest

import oracle
from tests import brute


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def test_pool_short_last_stride_is_the_mean_of_what_it_has():
    k = _rand((61, 3, 16), 1)  # strides of 8: 7 full and one of 5 tokens
    got = oracle.pool(k, S=8, round_bf16=False)
    assert got.shape == (8, 3, 16)
    kk = k.astype(np.float64)
    want = np.stack([kk[t * 8:min(61, t * 8 + 8)].mean(axis=0) for t in range(8)])
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-7)


RAGGED = [
    (200, 4, 2, 16, 8, 32, True),    # last block 8 tokens, strides full
    (203, 4, 2, 16, 8, 32, True),    # last block 11 tokens, last stride 3
    (130, 3, 1, 16, 4, 64, False),   # non-causal, last block 2 tokens
    (333, 8, 2, 32, 16, 64, True),
    (97, 2, 2, 8, 4, 16, False),
]


@pytest.mark.parametrize("L,Hq,Hkv,d,S,B,causal", RAGGED)
def test_ragged_block_mass_matches_brute_force(L, Hq, Hkv, d, S, B, causal):
    q = _rand((L, Hq, d), 10 + L, 1.5)
    k = _rand((L, Hkv, d), 20 + L, 1.5)
    res = oracle.search(q, k, S=S, B=B, tau=0.9, causal=causal, round_bf16=False)
    nb = -(-L // B)
    assert res.mass.shape == (Hq, nb, nb)
    want = brute.block_mass_ragged(q, k, S=S, B=B, causal=causal)
    np.testing.assert_allclose(res.mass, want, rtol=2e-5, atol=2e-7)
    np.testing.assert_allclose(res.mass[:, : nb - 1].sum(axis=2), 1.0, atol=2e-6)
    # the last (short) row keeps every candidate block
    np.testing.assert_array_equal(res.row_count[:, nb - 1], nb if not causal else nb)


def test_ragged_equals_regular_when_l_divides():
    # the ragged brute force reduces to the regular one on a multiple of B
    q, k = _rand((256, 4, 16), 5, 1.5), _rand((256, 2, 16), 6, 1.5)
    np.testing.assert_allclose(brute.block_mass_ragged(q, k, S=8, B=32),
                               brute.block_mass(q, k, S=8, B=32), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_ragged_attention_matches_masked_dense(causal):
    L, Hq, Hkv, d, B = 203, 4, 2, 16, 32
    q, k, v = _rand((L, Hq, d), 71, 2.0), _rand((L, Hkv, d), 72, 2.0), _rand((L, Hkv, d), 73)
    res = oracle.search(q, k, S=4, B=B, tau=0.6, causal=causal, round_bf16=False)
    got = oracle.attention(q, k, v, res.row_count, res.col_idx, B=B, causal=causal)
    want = brute.masked_attention_ragged(q, k, v, res.selected(), B=B, causal=causal)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)
    # dense lists on a ragged length equal plain softmax attention
    rc, ci = oracle.full_lists(L, Hq, B, causal)
    got = oracle.attention(q, k, v, rc, ci, B=B, causal=causal)
    want = brute.masked_attention_ragged(q, k, v, np.ones((Hq, -(-L // B), -(-L // B)), bool), B=B, causal=causal)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_ragged_recall_matches_brute_force():
    L, Hq, Hkv, d, B = 203, 4, 2, 16, 32
    q, k = _rand((L, Hq, d), 81, 2.0), _rand((L, Hkv, d), 82)
    res = oracle.search(q, k, S=4, B=B, tau=0.7, causal=True, round_bf16=False)
    got = oracle.mass_recall(q, k, res.row_count, res.col_idx, B=B)
    # dense float64 softmax under the element mask, averaged over the queries each block has
    elem = np.kron(res.selected().astype(np.int8), np.ones((B, B), np.int8)).astype(bool)[:, :L, :L]
    qq, kk = q.astype(np.float64), k.astype(np.float64)
    nb = -(-L // B)
    want = np.zeros((Hq, nb))
    for h in range(Hq):
        a = qq[:, h] @ kk[:, h // 2].T / np.sqrt(d)
        a = np.where(np.tril(np.ones((L, L), bool)), a, -np.inf)
        w = np.exp(a - a.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        per_q = (w * elem[h]).sum(axis=1)
        for i in range(nb):
            want[h, i] = per_q[i * B:min(L, (i + 1) * B)].mean()
    np.testing.assert_allclose(got, want, atol=1e-12)


def test_threshold_per_head_equals_separate_searches():
    L, Hq, Hkv, d, S, B = 512, 6, 2, 16, 8, 32
    q, k = _rand((L, Hq, d), 91, 2.0), _rand((L, Hkv, d), 92, 2.0)
    taus = np.array([0.5, 0.9, 0.75, 1.0, 0.3, 0.95], np.float32)
    got = oracle.search(q, k, S=S, B=B, tau=0.9, round_bf16=False, tau_per_head=taus)
    for h in range(Hq):
        one = oracle.search(q, k, S=S, B=B, tau=float(taus[h]), round_bf16=False)
        np.testing.assert_array_equal(got.row_count[h], one.row_count[h])
        np.testing.assert_array_equal(got.col_idx[h], one.col_idx[h])
