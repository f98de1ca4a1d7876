"""GPU parity on ragged inputs: sequence lengths that are not a multiple of
the block (a short last block) or of the stride (a short last stride), a
threshold per query head, and a packed batch of variable-length sequences.

Same bars as the regular cases: block lists per tests/checker.py, exported
masses within 1e-4 relative, attention within max-abs 2e-2 / mean-abs 2e-3
(bf16) or 1e-4 / 1e-5 (fp32), recall within 5e-4.
"""

import numpy as np
import pytest
import torch

import dynamic_block_sparse_rr_amd as rr
import oracle
from synthetic.gen import Workload, make_inputs
from tests import checker
from tests.gpu_cases import DeviceCase, say

pytestmark = pytest.mark.gpu


def g(name, L, Hq, Hkv, d, S, B, dtype, causal=True, kind="gauss", seed=200):
    return Workload(name, L, Hq, Hkv, d, dtype, B, S, (0.9,), seed, kind, 8, causal)


RAGGED = [
    g("pair_tail80", 2000, 8, 2, 128, 16, 128, "bf16", kind="llm"),            # last block 80 keys
    g("pair_tail6_stride6", 1030, 8, 2, 128, 16, 128, "bf16", kind="llm"),     # last block and stride 6
    g("pair_noncausal_tail104", 1000, 4, 2, 128, 16, 128, "bf16", causal=False, kind="llm"),
    g("b64_tail39", 999, 4, 2, 64, 8, 64, "bf16"),                             # single-head kernel
    g("b64_noncausal_tail39", 999, 4, 2, 64, 8, 64, "bf16", causal=False),
    g("mha_b128_tail60", 700, 2, 2, 128, 16, 128, "bf16"),
    g("fp32_tail52", 500, 2, 1, 64, 8, 64, "fp32", kind="tiny"),
    g("fp32_noncausal_tail52", 500, 2, 1, 64, 8, 64, "fp32", causal=False),
    g("fp32_gqa_tail52", 500, 4, 2, 64, 8, 64, "fp32"),                        # KV head 1's rows end mid-tensor
    g("fp32_d128_b128_noncausal_tail44", 300, 4, 2, 128, 16, 128, "fp32", causal=False),  # 12-key last subtile
    g("fp32_seven_tokens", 7, 2, 2, 64, 8, 64, "fp32"),                        # one tile, one short subtile
    g("single_short_block", 50, 4, 2, 64, 8, 64, "bf16"),                      # nb = 1
    g("one_token", 1, 4, 2, 128, 16, 128, "bf16"),                              # L = 1: one key, one stride
    g("two_tokens_noncausal", 2, 4, 2, 128, 16, 128, "bf16", causal=False),
    g("seventeen_tokens", 17, 8, 2, 128, 16, 128, "bf16"),                      # one short block, a short stride
]


def tol(w):
    return (2e-2, 2e-3) if w.dtype == "bf16" else (1e-4, 1e-5)


@pytest.mark.parametrize("w", RAGGED, ids=[w.name for w in RAGGED])
def test_ragged_full_parity(w):
    say(f"ragged case {w.name} L={w.L} nb={w.nb} ns={w.ns}")
    run = DeviceCase(w, 0.9)
    rc, ci, mass = run.search(export_mass=True)
    orc = oracle.search(run.q, run.k, S=w.S, B=w.B, tau=0.9, causal=w.causal, round_bf16=w.dtype == "bf16")
    np.testing.assert_allclose(mass, orc.mass, rtol=1e-4, atol=1e-6)
    res = checker.classify(rc, ci, orc, 0.9, causal=w.causal)
    say(f"  masks exact={res['exact']} letter={res['letter']} near_tie={res['near_tie']} fail={res['fail']}")
    assert res["fail"] == 0, res["fail_rows"][:10]
    tmax, tmean = tol(w)
    want = oracle.attention(run.q, run.k, run.v, orc.row_count, orc.col_idx, B=w.B, causal=w.causal)
    got = run.attention(orc.row_count, orc.col_idx)
    mx, mean = checker.output_errors(got, want)
    say(f"  attention max-abs {mx:.3e} mean-abs {mean:.3e}")
    assert mx <= tmax and mean <= tmean
    out, rc2, ci2 = run.prefill()
    np.testing.assert_array_equal(rc2, rc)
    want2 = oracle.attention(run.q, run.k, run.v, rc2, ci2, B=w.B, causal=w.causal)
    mx2, mean2 = checker.output_errors(out, want2)
    assert mx2 <= tmax and mean2 <= tmean
    r = run.recall(rc, ci)
    rw = oracle.mass_recall(run.q, run.k, rc, ci, B=w.B, causal=w.causal)
    say(f"  recall max err {np.abs(r - rw).max():.2e}")
    assert np.abs(r - rw).max() <= 5e-4


def test_ragged_dense_equals_sdpa():
    # every block selected on a ragged length is plain causal attention
    w = g("dense_ragged", 1500, 4, 2, 128, 16, 128, "bf16", kind="llm")
    run = DeviceCase(w, 1.0)
    out, rc, ci = run.prefill()
    frc, _ = oracle.full_lists(w.L, w.Hq, w.B)
    np.testing.assert_array_equal(rc, frc)
    qq = run.q.float().permute(1, 0, 2)
    kk = run.k.float().repeat_interleave(w.G, dim=1).permute(1, 0, 2)
    vv = run.v.float().repeat_interleave(w.G, dim=1).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True).permute(1, 0, 2).numpy()
    mx, mean = checker.output_errors(out, ref)
    say(f"  dense ragged vs SDPA: max-abs {mx:.3e} mean-abs {mean:.3e}")
    assert mx <= 2e-2 and mean <= 2e-3


def test_threshold_per_head():
    w = g("per_head_tau", 2048, 8, 2, 128, 16, 128, "bf16", kind="llm")
    run = DeviceCase(w, 0.9)
    taus = np.array([0.5, 0.9, 0.75, 1.0, 0.3, 0.95, 0.85, 0.6], np.float32)
    td = torch.from_numpy(taus).cuda()
    rc = torch.empty((w.Hq, w.nb), dtype=torch.int32, device="cuda")
    ci = torch.empty((w.Hq, w.nb, w.nb), dtype=torch.int32, device="cuda")
    rr.rr_pattern_search_heads(run.p, run.qd, run.kd, td, rc, ci, None, run.pre.ws)
    torch.cuda.synchronize()
    rc, ci = rc.cpu().numpy(), ci.cpu().numpy()
    orc = oracle.search(run.q, run.k, S=w.S, B=w.B, tau=0.9, round_bf16=True, tau_per_head=taus)
    for h in range(w.Hq):
        one = checker.classify(rc[h:h + 1], ci[h:h + 1], _head(orc, h), float(taus[h]))
        assert one["fail"] == 0, (h, one["fail_rows"][:5])
    # values outside (0, 1] keep every candidate block
    bad = torch.tensor([float("nan"), 2.0, -1.0, 0.0, 0.9, 0.9, 0.9, 0.9], device="cuda")
    rc2 = torch.empty((w.Hq, w.nb), dtype=torch.int32, device="cuda")
    ci2 = torch.empty((w.Hq, w.nb, w.nb), dtype=torch.int32, device="cuda")
    rr.rr_pattern_search_heads(run.p, run.qd, run.kd, bad, rc2, ci2, None, run.pre.ws)
    torch.cuda.synchronize()
    frc, _ = oracle.full_lists(w.L, w.Hq, w.B)
    np.testing.assert_array_equal(rc2.cpu().numpy()[:4], frc[:4])


def _head(res, h):
    """The oracle result restricted to head h (shapes [1][...])."""
    return oracle.SearchResult(res.row_count[h:h + 1], res.col_idx[h:h + 1], res.mass[h:h + 1],
                               res.cminus[h:h + 1], res.cplus[h:h + 1], res.rank[h:h + 1],
                               res.total[h:h + 1], res.kbar)


def _varlen_case(lens, Hq, Hkv, seed, max_full_rows=20000):
    """A packed batch through rr_prefill_varlen against each sequence run alone
    (same kernels: lists and outputs bitwise equal) and against the oracle
    (every row where a sequence has at most max_full_rows (token, head) rows,
    else one row per (head, query block) plus 64 sampled rows)."""
    from synthetic.rows import sample_rows, work_item_rows

    ws_ = [Workload(f"seq{b}", L, Hq, Hkv, 128, "bf16", 128, 16, (0.9,), seed + b, "llm", 8)
           for b, L in enumerate(lens)]
    parts = [make_inputs(w_) for w_ in ws_]
    q = torch.cat([p_[0] for p_ in parts]).cuda()
    k = torch.cat([p_[1] for p_ in parts]).cuda()
    v = torch.cat([p_[2] for p_ in parts]).cuda()
    p = rr.problem(sum(lens), Hq, Hkv, 128, 16, 128, 0.9, True, "bf16")
    nbs = [-(-L // 128) for L in lens]
    rc = torch.full((sum(Hq * n for n in nbs),), -1, dtype=torch.int32, device="cuda")
    ci = torch.full((sum(Hq * n * n for n in nbs),), -1, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, float("nan"))
    ws = torch.empty(rr.rr_workspace_bytes_varlen(p, lens), dtype=torch.uint8, device="cuda")
    rr.rr_prefill_varlen(p, lens, q, k, v, out, rc, ci, ws)
    torch.cuda.synchronize()
    rc, ci, out = rc.cpu().numpy(), ci.cpu().numpy(), out.float().cpu().numpy()
    tok = roff = coff = 0
    for b, L in enumerate(lens):
        nb = nbs[b]
        one = DeviceCase(ws_[b], 0.9, inputs=parts[b])
        o1, rc1, ci1 = one.prefill()
        rcb = rc[roff:roff + Hq * nb].reshape(Hq, nb)
        cib = ci[coff:coff + Hq * nb * nb].reshape(Hq, nb, nb)
        np.testing.assert_array_equal(rcb, rc1)
        for h in range(Hq):
            for i in range(nb):
                np.testing.assert_array_equal(cib[h, i, :rcb[h, i]], ci1[h, i, :rc1[h, i]])
        np.testing.assert_array_equal(out[tok:tok + L], o1)  # same kernels, same inputs: bitwise
        # and against the oracle
        orc = oracle.search(parts[b][0], parts[b][1], S=16, B=128, tau=0.9, round_bf16=True)
        assert checker.classify(rcb, cib, orc, 0.9)["fail"] == 0
        if L * Hq <= max_full_rows:
            want = oracle.attention(parts[b][0], parts[b][1], parts[b][2], rcb, cib, B=128)
            mx, mean = checker.output_errors(out[tok:tok + L], want)
        else:
            rows = np.concatenate([work_item_rows(L, Hq, 128, seed=seed + b), sample_rows(L, Hq, 128, 64, seed=seed + b)])
            want = oracle.attention(parts[b][0], parts[b][1], parts[b][2], rcb, cib, B=128, rows=rows)
            mx, mean = checker.output_errors(out[tok:tok + L][rows[:, 0], rows[:, 1]], want)
        say(f"  varlen seq {b} L={L}: max-abs {mx:.3e} mean-abs {mean:.3e}")
        assert mx <= 2e-2 and mean <= 2e-3
        tok += L
        roff += Hq * nb
        coff += Hq * nb * nb


def test_varlen_batch_matches_single_sequences():
    _varlen_case([1000, 2048, 300, 1537], 8, 2, 300)


def test_varlen_batch_one_query_head_per_kv_head():
    """MHA (G = 1) and an odd group (G = 3) in the batched launches: every head
    of the first, and the last head of each KV head of the second, paired with
    itself over two adjacent query blocks (the 257-token sequence has an odd
    block count, so its lowest unit's lone head has no second block)."""
    _varlen_case([1000, 2048, 300, 1537], 4, 4, 320)
    _varlen_case([900, 1500, 257], 12, 4, 330)


def test_varlen_long_sequence_in_its_own_launch():
    """17,000 tokens at the 8B shape hold 16 * 133 = 2,128 work items, over 8
    per CU on 256 CUs: that sequence gets a launch of its own, the two short
    ones share one."""
    _varlen_case([17000, 3000, 999], 32, 8, 310)


def test_varlen_many_random_lengths_match_single_sequences():
    """40 sequences of seeded random lengths (1 to 3,000 tokens: one-block and
    one-token sequences, lengths off the block and the stride): two shared
    launch groups (32 + 8) for the search and the attention. Every sequence's
    lists and output equal the same sequence run alone, bit for bit; the lists
    of every sequence and the outputs of every fifth sequence against the oracle."""
    rng = np.random.default_rng(777)
    lens = [int(x) for x in rng.integers(1, 3001, 40)]
    lens[3], lens[17], lens[30] = 1, 128, 129  # one token, one whole block, one block and a token
    Hq, Hkv = 8, 2
    ws_ = [Workload(f"r{b}", L, Hq, Hkv, 128, "bf16", 128, 16, (0.9,), 900 + b, "llm" if L >= 64 else "gauss", 8)
           for b, L in enumerate(lens)]  # the 8B-shaped recipe needs more tokens than its 8 stripes
    parts = [make_inputs(w_) for w_ in ws_]
    q = torch.cat([p_[0] for p_ in parts]).cuda()
    k = torch.cat([p_[1] for p_ in parts]).cuda()
    v = torch.cat([p_[2] for p_ in parts]).cuda()
    p = rr.problem(sum(lens), Hq, Hkv, 128, 16, 128, 0.9, True, "bf16")
    nbs = [-(-L // 128) for L in lens]
    rc = torch.full((sum(Hq * n for n in nbs),), -1, dtype=torch.int32, device="cuda")
    ci = torch.full((sum(Hq * n * n for n in nbs),), -1, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, float("nan"))
    ws = torch.empty(rr.rr_workspace_bytes_varlen(p, lens), dtype=torch.uint8, device="cuda")
    rr.rr_prefill_varlen(p, lens, q, k, v, out, rc, ci, ws)
    torch.cuda.synchronize()
    rc, ci, out = rc.cpu().numpy(), ci.cpu().numpy(), out.float().cpu().numpy()
    tok = roff = coff = 0
    for b, L in enumerate(lens):
        nb = nbs[b]
        o1, rc1, ci1 = DeviceCase(ws_[b], 0.9, inputs=parts[b]).prefill()
        rcb = rc[roff:roff + Hq * nb].reshape(Hq, nb)
        cib = ci[coff:coff + Hq * nb * nb].reshape(Hq, nb, nb)
        np.testing.assert_array_equal(rcb, rc1)
        for h in range(Hq):
            for i in range(nb):
                np.testing.assert_array_equal(cib[h, i, :rcb[h, i]], ci1[h, i, :rc1[h, i]])
        np.testing.assert_array_equal(out[tok:tok + L], o1)
        orc = oracle.search(parts[b][0], parts[b][1], S=16, B=128, tau=0.9, round_bf16=True)
        assert checker.classify(rcb, cib, orc, 0.9)["fail"] == 0, b
        if b % 5 == 0:
            want = oracle.attention(parts[b][0], parts[b][1], parts[b][2], rcb, cib, B=128)
            mx, mean = checker.output_errors(out[tok:tok + L], want)
            assert mx <= 2e-2 and mean <= 2e-3, (b, mx, mean)
        tok += L
        roff += Hq * nb
        coff += Hq * nb * nb
    say(f"  varlen 40 random lengths ({min(lens)}..{max(lens)}): lists and outputs bitwise equal to single runs")
