"""Shared mask per KV head (a variant of the per-head masks): the oracle's
union pinned on the CPU, the GPU's rr_share_group_lists compared with it
exactly, and attention / recall on the shared lists."""

import numpy as np
import pytest

import oracle
from synthetic.gen import Workload, make_inputs_f32, workload


def _mask(rc, ci):
    Hq, nb = rc.shape
    m = np.zeros((Hq, nb, nb), bool)
    for h in range(Hq):
        for i in range(nb):
            m[h, i, ci[h, i, : rc[h, i]]] = True
    return m


def _search(G=4, seed=21, tau=0.9):
    w = Workload("shared", 1024, 2 * G, 2, 64, "fp32", 64, 8, (tau,), seed, "llm", 4)
    q, k, _ = make_inputs_f32(w)
    return w, q, k, oracle.search(q, k, S=w.S, B=w.B, tau=tau, round_bf16=False, extras=False)


def test_union_is_the_or_of_the_group_masks():
    w, q, k, r = _search()
    G = w.G
    src = _mask(r.row_count, r.col_idx)
    rc, ci = oracle.share_group_lists(r.row_count, r.col_idx, G)
    got = _mask(rc, ci)
    want = np.repeat(src.reshape(w.Hkv, G, w.nb, w.nb).any(axis=1), G, axis=0)
    np.testing.assert_array_equal(got, want)
    for h in range(w.Hq):
        for i in range(w.nb):
            js = ci[h, i, : rc[h, i]]
            assert np.all(np.diff(js) > 0)          # ascending
            assert np.all(ci[h, i, rc[h, i]:] == -1)  # tail unused
    # every head's own selection is inside the shared one, and the group agrees
    assert np.all(got >= src)
    for g in range(w.Hkv):
        assert np.all(got[g * G:(g + 1) * G] == got[g * G])


def test_union_with_one_head_per_group_is_the_identity():
    w, q, k, r = _search()
    rc, ci = oracle.share_group_lists(r.row_count, r.col_idx, 1)
    np.testing.assert_array_equal(rc, r.row_count)
    np.testing.assert_array_equal(_mask(rc, ci), _mask(r.row_count, r.col_idx))


def test_shared_lists_hold_at_least_the_per_head_recall():
    w, q, k, r = _search()
    rc, ci = oracle.share_group_lists(r.row_count, r.col_idx, w.G)
    own = oracle.mass_recall(q, k, r.row_count, r.col_idx, B=w.B)
    shared = oracle.mass_recall(q, k, rc, ci, B=w.B)
    assert np.all(shared >= own - 1e-12)
    assert shared.mean() > own.mean()


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["llm_g4", "gauss_g7", "llama8b_L128k"])
def test_gpu_shared_lists_match_the_oracle(name):
    from tests.gpu_cases import DeviceCase, say
    if name == "llm_g4":
        w = Workload(name, 2048, 8, 2, 128, "bf16", 128, 16, (0.9,), 31, "llm", 8)
    elif name == "gauss_g7":
        w = Workload(name, 1024, 14, 2, 64, "bf16", 64, 8, (0.9,), 32, "gauss", 8)
    else:
        w = workload(name)
    import torch
    import dynamic_block_sparse_rr_amd as rr
    say(f"shared-mask case {name}")
    run = DeviceCase(w, 0.9)
    rc, ci, _ = run.search(export_mass=False)
    src_rc = torch.from_numpy(rc).cuda()
    src_ci = torch.from_numpy(ci).cuda()
    out_rc = torch.full_like(src_rc, -7)
    out_ci = torch.full_like(src_ci, -7)
    rr.rr_share_group_lists(run.p, src_rc, src_ci, out_rc, out_ci)
    torch.cuda.synchronize()
    grc, gci = out_rc.cpu().numpy(), out_ci.cpu().numpy()
    want = np.repeat(_mask(rc, ci).reshape(w.Hkv, w.G, w.nb, w.nb).any(axis=1), w.G, axis=0)
    np.testing.assert_array_equal(grc, want.sum(axis=2))
    for h in range(w.Hq):
        for i in range(w.nb):
            np.testing.assert_array_equal(gci[h, i, : grc[h, i]], np.nonzero(want[h, i])[0])
    if w.L <= 2048:
        orc, oci = oracle.share_group_lists(rc, ci, w.G)
        np.testing.assert_array_equal(grc, orc)
        # attention and recall on the shared lists
        out = run.attention(grc, gci)
        ref = oracle.attention(run.q, run.k, run.v, grc, gci, B=w.B, causal=w.causal)
        assert np.abs(out - ref).max() <= 2e-2 and np.abs(out - ref).mean() <= 2e-3
        got_r = run.recall(grc, gci)
        want_r = oracle.mass_recall(run.q, run.k, grc, gci, B=w.B, causal=w.causal)
        assert np.abs(got_r - want_r).max() <= 5e-4
    say(f"  keep per head {rc.sum() / rc.size / ((w.nb + 1) / 2):.4f}, shared {grc.sum() / grc.size / ((w.nb + 1) / 2):.4f}")
