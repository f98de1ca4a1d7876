"""Pins of the oracle's mass recall (the full-attention softmax mass inside the
selected blocks, the quantity behind the Figure 4 and 5 captions) to facts
other than itself. CPU only."""

import numpy as np
import pytest

import oracle
from synthetic.gen import Workload, make_inputs_f32
from tests import brute


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def _lists_from_mask(mask):
    Hq, nb, _ = mask.shape
    rc = mask.sum(axis=2).astype(np.int32)
    ci = np.full((Hq, nb, nb), -1, np.int32)
    for h in range(Hq):
        for i in range(nb):
            js = np.nonzero(mask[h, i])[0]
            ci[h, i, : len(js)] = js
    return rc, ci


def _random_mask(Hq, nb, seed, causal=True, p=0.5):
    rng = np.random.default_rng(seed)
    m = rng.random((Hq, nb, nb)) < p
    if causal:
        m &= np.tril(np.ones((nb, nb), bool))[None]
        # every row non-empty: keep one random admissible block where a row is empty
        for h in range(Hq):
            for i in range(nb):
                if not m[h, i].any():
                    m[h, i, rng.integers(0, i + 1)] = True
    else:
        for h in range(Hq):
            for i in range(nb):
                if not m[h, i].any():
                    m[h, i, rng.integers(0, nb)] = True
    return m


@pytest.mark.parametrize("causal", [True, False])
def test_recall_matches_dense_softmax_brute_force(causal):
    L, Hq, Hkv, d, B = 256, 4, 2, 32, 32
    q, k = _rand((L, Hq, d), 1), _rand((L, Hkv, d), 2)
    mask = _random_mask(Hq, L // B, 3, causal=causal)
    rc, ci = _lists_from_mask(mask)
    got = oracle.mass_recall(q, k, rc, ci, B=B, causal=causal)
    want = brute.mass_recall(q, k, mask, B=B, causal=causal)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_recall_of_all_blocks_is_one():
    L, Hq, Hkv, d, B = 512, 2, 1, 64, 64
    q, k = _rand((L, Hq, d), 4, 3.0), _rand((L, Hkv, d), 5)
    for causal in (True, False):
        rc, ci = oracle.full_lists(L, Hq, B, causal)
        np.testing.assert_allclose(oracle.mass_recall(q, k, rc, ci, B=B, causal=causal), 1.0, atol=1e-13)


def test_recall_of_complementary_selections_adds_to_one():
    L, Hq, Hkv, d, B = 384, 3, 3, 32, 32
    nb = L // B
    q, k = _rand((L, Hq, d), 6, 2.0), _rand((L, Hkv, d), 7)
    cand = np.tril(np.ones((nb, nb), bool))
    rng = np.random.default_rng(8)
    a = (rng.random((Hq, nb, nb)) < 0.5) & cand
    a[:, :, 0] = True                    # block 0 in A ...
    b = cand[None] & ~a
    b[:, np.arange(nb), np.arange(nb)] = True  # ... the diagonal in B
    a[:, np.arange(1, nb), np.arange(1, nb)] = False
    ra = oracle.mass_recall(q, k, *_lists_from_mask(a), B=B)
    rb = oracle.mass_recall(q, k, *_lists_from_mask(b), B=B)
    # row 0 has one candidate block, in both sets
    np.testing.assert_allclose(ra[:, 1:] + rb[:, 1:], 1.0, atol=1e-13)


def test_recall_closed_form_for_uniform_logits():
    # zero queries: every admissible key gets the same weight, so selecting only
    # block 0 gives r(x) = B / (x + 1) causally (all of it for x < B) and B / L otherwise
    L, Hq, Hkv, d, B = 512, 2, 1, 64, 64
    nb = L // B
    q = np.zeros((L, Hq, d), np.float32)
    k = _rand((L, Hkv, d), 9)
    mask = np.zeros((Hq, nb, nb), bool)
    mask[:, :, 0] = True
    rc, ci = _lists_from_mask(mask)
    got = oracle.mass_recall(q, k, rc, ci, B=B, causal=True)
    x = np.arange(L, dtype=np.float64)
    want = np.minimum(1.0, B / (x + 1)).reshape(nb, B).mean(axis=1)
    np.testing.assert_allclose(got, np.broadcast_to(want, (Hq, nb)), atol=1e-13)
    got_nc = oracle.mass_recall(q, k, rc, ci, B=B, causal=False)
    np.testing.assert_allclose(got_nc, B / L, atol=1e-13)


def test_recall_rows_subset_matches_full_table():
    L, Hq, Hkv, d, B = 256, 4, 2, 32, 64
    q, k = _rand((L, Hq, d), 10), _rand((L, Hkv, d), 11)
    mask = _random_mask(Hq, L // B, 12)
    rc, ci = _lists_from_mask(mask)
    full = oracle.mass_recall(q, k, rc, ci, B=B)
    rows = np.array([[3, 2], [0, 0], [1, 3]], np.int32)
    np.testing.assert_array_equal(oracle.mass_recall(q, k, rc, ci, B=B, rows=rows), full[rows[:, 0], rows[:, 1]])


def test_recall_grows_with_tau():
    # nested selections (sel(0.85) within sel(0.9) within sel(0.95)) can only gain mass
    w = Workload("nest", 1024, 4, 2, 64, "fp32", 64, 8, (0.9,), 13, "llm", 4)
    q, k, _ = make_inputs_f32(w)
    rec = []
    for tau in (0.85, 0.9, 0.95, 1.0):
        r = oracle.search(q, k, S=w.S, B=w.B, tau=tau, round_bf16=False, extras=False)
        rec.append(oracle.mass_recall(q, k, r.row_count, r.col_idx, B=w.B))
    for lo, hi in zip(rec, rec[1:]):
        assert np.all(hi >= lo - 1e-12)
    np.testing.assert_allclose(rec[-1], 1.0, atol=1e-12)
    # the last query block is kept whole at every tau
    for r_ in rec:
        np.testing.assert_allclose(r_[:, -1], 1.0, atol=1e-12)
