"""Pins of the CPU oracle to things other than itself (all CPU, no GPU).

Each test ties one step of the oracle to an independent fact: a hand-worked
example, a float64 brute force that takes a different route (tests/brute.py),
a library routine the step reduces to (torch's bfloat16 cast, torch SDPA), an
exhaustive subset search, or an invariant stated by the method (rows of
probabilities sum to one, the last query block is kept, query independence).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def _bf16(x):
    return torch.from_numpy(x).to(torch.bfloat16).float().numpy()


# ---------------------------------------------------------------- rounding / pooling

def test_round_bf16_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000).astype(np.float32),
        # exact halfway cases: ties go to the even bfloat16 neighbour
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130, 3.0e38, 0.0], np.float32),
    ]).astype(np.float32)
    k = x.reshape(-1, 1, 1)
    got = oracle.pool(k, S=1, round_bf16=True).reshape(-1)
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


def test_pool_is_stride_mean():
    k = _rand((64, 3, 16), 1)
    got = oracle.pool(k, S=8, round_bf16=False)
    want = k.astype(np.float64).reshape(8, 8, 3, 16).mean(axis=1)
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-7)


# ---------------------------------------------------------------- hand-worked example

def _hand_inputs():
    L, S = 24, 4
    a = [math.log(4), 0, 0, math.log(2), 0, 0]
    b = [0, 0, math.log(3), 0, 0, 0]
    k = np.zeros((L, 1, 4), np.float32)
    for t in range(L // S):
        k[t * S:(t + 1) * S, 0, 0] = a[t]
        k[t * S:(t + 1) * S, 0, 2] = b[t]
    q = np.zeros((L, 2, 4), np.float32)
    q[:, :, 0] = -50.0
    for s in range(L // S):
        q[s * S + 0, 0] = (2, 0, 0, 0)
        q[s * S + 1, 1] = (0, 0, 2, 0)
    return q, k


def test_hand_worked_example_figure2_config():
    spec = json.load(open(os.path.join(GOLDEN, "hand_worked_S4_B8.json")))
    exp = spec["expected"]
    q, k = _hand_inputs()
    for h in ("0", "1"):
        for tau, want in exp["selected_row1"][h].items():
            res = oracle.search(q, k, S=4, B=8, tau=float(tau), round_bf16=False)
            hh = int(h)
            np.testing.assert_allclose(res.mass[hh, 1, :2], exp["mass_row1"][h], rtol=2e-6)
            assert res.mass[hh, 1, 2] == 0.0
            assert list(res.col_idx[hh, 1, :res.row_count[hh, 1]]) == want
            assert list(res.col_idx[hh, 0, :res.row_count[hh, 0]]) == exp["selected_row0"]
            assert res.mass[hh, 0, 0] == pytest.approx(1.0, abs=1e-7)
            assert list(res.col_idx[hh, 2, :res.row_count[hh, 2]]) == exp["selected_row2"]
            assert not res.mass[hh, 2].any()


# ---------------------------------------------------------------- masses vs brute force

CASES = [
    # L, Hq, Hkv, d, S, B, causal
    (64, 2, 2, 8, 4, 16, True),
    (128, 4, 2, 16, 2, 8, True),
    (128, 8, 2, 16, 8, 32, True),
    (256, 7, 1, 16, 4, 32, True),
    (128, 4, 4, 8, 4, 16, False),
    (256, 4, 1, 32, 16, 64, True),
]


@pytest.mark.parametrize("L,Hq,Hkv,d,S,B,causal", CASES)
@pytest.mark.parametrize("bf16", [False, True])
def test_block_mass_matches_brute_force(L, Hq, Hkv, d, S, B, causal, bf16):
    q = _rand((L, Hq, d), 10 + L + Hq, 1.5)
    k = _rand((L, Hkv, d), 20 + L + Hq, 1.5)
    if bf16:
        q, k = _bf16(q), _bf16(k)
    res = oracle.search(q, k, S=S, B=B, tau=0.9, causal=causal, round_bf16=bf16)
    want = brute.block_mass(q, k, S=S, B=B, causal=causal, bf16_pool=bf16)
    np.testing.assert_allclose(res.mass, want, rtol=2e-5, atol=2e-7)


@pytest.mark.parametrize("L,Hq,Hkv,d,S,B,causal", CASES)
def test_block_mass_invariants(L, Hq, Hkv, d, S, B, causal):
    q = _rand((L, Hq, d), 3, 2.0)
    k = _rand((L, Hkv, d), 4, 2.0)
    res = oracle.search(q, k, S=S, B=B, tau=0.9, causal=causal, round_bf16=False)
    nb = L // B
    m = res.mass
    assert (m >= 0).all()
    np.testing.assert_allclose(m[:, : nb - 1].sum(axis=2), 1.0, atol=2e-6)
    assert not m[:, nb - 1].any()
    if causal:
        assert not np.triu(m, 1).any()


# ---------------------------------------------------------------- Top-tau selection

@pytest.mark.parametrize("tau", [0.5, 0.8, 0.9, 0.97])
def test_top_tau_is_minimum_cardinality_set(tau):
    L, Hq, S, B = 192, 6, 4, 16  # up to 11 candidate blocks per row
    q = _rand((L, Hq, 16), 7, 3.0)
    k = _rand((L, 2, 16), 8, 3.0)
    res = oracle.search(q, k, S=S, B=B, tau=tau, round_bf16=False)
    mass64 = brute.block_mass(q, k, S=S, B=B)
    nb = L // B
    checked = 0
    for h in range(Hq):
        for i in range(nb - 1):
            want, margin = brute.min_cardinality_set(mass64[h, i, : i + 1], tau)
            if margin < 1e-4:
                continue  # a float32 rounding could legitimately flip this row
            got = set(res.col_idx[h, i, : res.row_count[h, i]].tolist())
            assert got == want, (h, i)
            checked += 1
    assert checked > 20


def test_tau_one_keeps_every_causal_block_and_last_row_is_full():
    L, B = 256, 32
    q = _rand((L, 4, 16), 1, 2.0)
    k = _rand((L, 2, 16), 2, 2.0)
    for tau in (1.0, 0.3):
        res = oracle.search(q, k, S=8, B=B, tau=tau, round_bf16=False)
        nb = L // B
        for h in range(4):
            last = res.col_idx[h, nb - 1, : res.row_count[h, nb - 1]]
            assert list(last) == list(range(nb))
            if tau == 1.0:
                for i in range(nb):
                    assert list(res.col_idx[h, i, : res.row_count[h, i]]) == list(range(i + 1))


def test_selections_nest_across_tau_and_small_tau_is_argmax():
    L, B = 512, 32
    q = _rand((L, 4, 16), 5, 2.0)
    k = _rand((L, 4, 16), 6, 2.0)
    sel = [oracle.search(q, k, S=8, B=B, tau=t, round_bf16=False).selected() for t in (0.85, 0.9, 0.95)]
    assert (sel[0] <= sel[1]).all() and (sel[1] <= sel[2]).all()
    small = oracle.search(q, k, S=8, B=B, tau=1e-6, round_bf16=False)
    nb = L // B
    for h in range(4):
        for i in range(nb - 1):
            m = small.mass[h, i, : i + 1]
            assert small.row_count[h, i] == 1
            assert small.col_idx[h, i, 0] == int(np.argmax(m))


def test_selected_mass_reaches_tau_and_is_minimal():
    L, B, tau = 1024, 64, 0.9
    q = _rand((L, 4, 32), 11, 2.0)
    k = _rand((L, 2, 32), 12, 2.0)
    res = oracle.search(q, k, S=8, B=B, tau=tau, round_bf16=False)
    nb = L // B
    for h in range(4):
        for i in range(nb - 1):
            m = res.mass[h, i, : i + 1].astype(np.float64)
            sel = res.col_idx[h, i, : res.row_count[h, i]]
            T = m.sum()
            assert m[sel].sum() >= tau * T * (1 - 1e-6)
            # dropping the smallest selected block falls below tau
            if len(sel) > 1:
                assert m[sel].sum() - m[sel].min() < tau * T * (1 + 1e-6)
            # nothing unselected is heavier than something selected
            uns = np.setdiff1d(np.arange(i + 1), sel)
            if len(uns):
                assert m[uns].max() <= m[sel].min()


# ---------------------------------------------------------------- round robin and independence

def test_round_robin_offset_is_head_mod_stride():
    """Head h reads only the queries at offset h mod S of each stride."""
    L, Hq, S, B = 256, 16, 8, 32
    q = _rand((L, Hq, 16), 21, 2.0)
    k = _rand((L, 2, 16), 22, 2.0)
    base = oracle.search(q, k, S=S, B=B, tau=0.9, round_bf16=False).mass
    for h in (0, 3, 8, 13):
        off = h % S
        q2 = q.copy()
        other = [x for x in range(L) if x % S != off]
        q2[other, h, :] = _rand((len(other), 16), 23 + h, 5.0)
        m2 = oracle.search(q2, k, S=S, B=B, tau=0.9, round_bf16=False).mass
        np.testing.assert_array_equal(m2, base)       # other offsets are never read
        q3 = q.copy()
        own = [x for x in range(L) if x % S == off]
        q3[own, h, :] = _rand((len(own), 16), 40 + h, 5.0)
        m3 = oracle.search(q3, k, S=S, B=B, tau=0.9, round_bf16=False).mass
        assert not np.array_equal(m3[h], base[h])     # its own offset is
        np.testing.assert_array_equal(np.delete(m3, h, 0), np.delete(base, h, 0))
    # offsets of S consecutive heads cover every in-stride position once
    for h0 in range(2 * S):
        assert sorted((h % S) for h in range(h0, h0 + S)) == list(range(S))


def test_query_independence_and_causality():
    L, Hq, B, S = 512, 4, 32, 8
    q = _rand((L, Hq, 16), 31, 2.0)
    k = _rand((L, 2, 16), 32, 2.0)
    v = _rand((L, 2, 16), 33, 1.0)
    base = oracle.search(q, k, S=S, B=B, tau=0.9, round_bf16=False)
    i0 = 7
    cut = (i0 + 1) * B
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[cut:] = _rand(q2[cut:].shape, 34, 4.0)
    k2[cut:] = _rand(k2[cut:].shape, 35, 4.0)
    v2[cut:] = _rand(v2[cut:].shape, 36, 4.0)
    res = oracle.search(q2, k2, S=S, B=B, tau=0.9, round_bf16=False)
    np.testing.assert_array_equal(res.mass[:, : i0 + 1], base.mass[:, : i0 + 1])
    np.testing.assert_array_equal(res.col_idx[:, : i0 + 1], base.col_idx[:, : i0 + 1])
    o1 = oracle.attention(q, k, v, base.row_count, base.col_idx, B=B)
    o2 = oracle.attention(q2, k2, v2, base.row_count, base.col_idx, B=B)
    np.testing.assert_array_equal(o1[:cut], o2[:cut])


# ---------------------------------------------------------------- attention

@pytest.mark.parametrize("L,Hq,Hkv,d,B", [(128, 4, 4, 16, 16), (256, 8, 2, 32, 32), (192, 7, 1, 16, 64)])
def test_dense_lists_equal_causal_sdpa(L, Hq, Hkv, d, B):
    q = _rand((L, Hq, d), 51, 2.0)
    k = _rand((L, Hkv, d), 52, 2.0)
    v = _rand((L, Hkv, d), 53)
    rc, ci = oracle.full_lists(L, Hq, B)
    got = oracle.attention(q, k, v, rc, ci, B=B)
    G = Hq // Hkv
    qt = torch.from_numpy(q).double().permute(1, 0, 2)
    kt = torch.from_numpy(k).double().repeat_interleave(G, dim=1).permute(1, 0, 2)
    vt = torch.from_numpy(v).double().repeat_interleave(G, dim=1).permute(1, 0, 2)
    want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    np.testing.assert_allclose(got, want.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_dense_noncausal_equals_sdpa():
    L, Hq, d, B = 128, 2, 16, 32
    q = _rand((L, Hq, d), 61, 2.0)
    k = _rand((L, Hq, d), 62, 2.0)
    v = _rand((L, Hq, d), 63)
    rc, ci = oracle.full_lists(L, Hq, B, causal=False)
    got = oracle.attention(q, k, v, rc, ci, B=B, causal=False)
    t = lambda a: torch.from_numpy(a).double().permute(1, 0, 2)
    want = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))
    np.testing.assert_allclose(got, want.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_sparse_attention_matches_masked_dense(causal):
    L, Hq, Hkv, d, B = 256, 4, 2, 16, 32
    q = _rand((L, Hq, d), 71, 2.0)
    k = _rand((L, Hkv, d), 72, 2.0)
    v = _rand((L, Hkv, d), 73)
    res = oracle.search(q, k, S=4, B=B, tau=0.6, causal=causal, round_bf16=False)
    got = oracle.attention(q, k, v, res.row_count, res.col_idx, B=B, causal=causal)
    want = brute.masked_attention(q, k, v, res.selected(), B=B, causal=causal)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)
    # sampled-row interface gives the same rows
    rows = np.array([[5, 1], [200, 3], [255, 0], [64, 2]], np.int32)
    part = oracle.attention(q, k, v, res.row_count, res.col_idx, B=B, causal=causal, rows=rows)
    np.testing.assert_array_equal(part, got[rows[:, 0], rows[:, 1]])


def test_attention_rejects_bad_lists():
    L, B = 128, 32
    q = _rand((L, 2, 8), 1)
    k = _rand((L, 2, 8), 2)
    rc, ci = oracle.full_lists(L, 2, B)
    ci = ci.copy()
    ci[0, 1, :2] = [1, 0]  # not ascending
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, rc, ci, B=B)
    rc2, ci2 = oracle.full_lists(L, 2, B)
    ci2 = ci2.copy()
    ci2[1, 0, 0] = 2  # beyond the diagonal
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, rc2, ci2, B=B)


def test_identical_keys_give_running_mean_of_values():
    """Closed form: with every key equal, each causal row's softmax is uniform
    over its visible keys, so the output is the running mean of the values."""
    L, Hq, Hkv, d, B = 200, 4, 2, 16, 32
    q = _rand((L, Hq, d), 11, scale=3.0)
    k = np.broadcast_to(_rand((1, 1, d), 12), (L, Hkv, d)).copy()
    v = _rand((L, Hkv, d), 13)
    rc, ci = oracle.full_lists(L, Hq, B)
    got = oracle.attention(q, k, v, rc, ci, B=B)
    mean = np.cumsum(v.astype(np.float64), axis=0) / np.arange(1, L + 1)[:, None, None]
    for h in range(Hq):
        np.testing.assert_allclose(got[:, h, :], mean[:, h // (Hq // Hkv), :], rtol=0, atol=1e-12)
