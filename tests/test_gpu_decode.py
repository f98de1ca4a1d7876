"""GPU parity of rr_decode (one new query per head against the KV cache)
with the oracle's decode step.

Bars: block masses within 1e-4 relative + 1e-6 absolute; block lists equal
to the oracle's except blocks whose cumulative oracle mass (before or
including the block, relative to the row total) lies within 1e-4 of tau
(the same letter rule as prefill); outputs within max-abs 2e-2 / mean-abs
2e-3 (bf16) or 1e-4 / 1e-5 (fp32), against the oracle where the lists agree
and against a float64 softmax over the GPU's own list where they do not.
"""

import math

import numpy as np
import pytest
import torch

import dynamic_block_sparse_rr_amd as rr
import oracle
from synthetic.gen import Workload, make_inputs, workload
from tests.gpu_cases import say

pytestmark = pytest.mark.gpu


def run_decode(q, k, v, S, B, tau, dtype, pooled=False):
    L, Hkv, d = k.shape
    Hq = q.shape[0]
    p = rr.problem(L, Hq, Hkv, d, S, B, tau, True, dtype)
    nb = p.nb
    qd, kd, vd = q.contiguous().cuda(), k.contiguous().cuda(), v.contiguous().cuda()
    out = torch.empty_like(qd)
    rc = torch.empty((Hq,), dtype=torch.int32, device="cuda")
    ci = torch.full((Hq, nb), -1, dtype=torch.int32, device="cuda")
    mass = torch.empty((Hq, nb), dtype=torch.float32, device="cuda")
    ws = torch.empty(rr.rr_decode_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    kbar = None
    if pooled:  # pooled keys built beforehand, as a server would keep them
        kbar = torch.empty((p.ns, Hkv, d), dtype=kd.dtype, device="cuda")
        rr.rr_pool_keys(p, kd, kbar)
    rr.rr_decode(p, qd, kd, vd, out, rc, ci, mass, ws, kbar=kbar)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), rc.cpu().numpy(), ci.cpu().numpy(), mass.cpu().numpy()


def check(q, k, v, S, B, tau, dtype, name, pooled=False):
    out, rc, ci, mass = run_decode(q, k, v, S, B, tau, dtype, pooled)
    o = oracle.decode(q, k, v, S=S, B=B, tau=tau, round_bf16=dtype == "bf16")
    np.testing.assert_allclose(mass, o.mass, rtol=1e-4, atol=1e-6)
    Hq, nb = mass.shape
    tmax, tmean = (2e-2, 2e-3) if dtype == "bf16" else (1e-4, 1e-5)
    kf, vf, qf = k.float().numpy(), v.float().numpy(), q.float().numpy()
    G = Hq // k.shape[1]
    L, d = k.shape[0], k.shape[2]
    exact = letter = 0
    errs = []
    for h in range(Hq):
        got = list(ci[h, : rc[h]])
        want = list(o.col_idx[h, : o.row_count[h]])
        assert got[-1] == nb - 1 and np.all(np.diff(got) > 0)
        if got == want:
            exact += 1
            errs.append(np.abs(out[h] - o.out[h]))
            continue
        # letter rule on the oracle's masses
        m = o.mass[h].astype(np.float64)
        order = sorted(range(nb), key=lambda j: (-m[j], j))
        T = m.sum()
        cum = np.cumsum([m[j] for j in order])
        cminus = {j: (cum[i] - m[j]) / T for i, j in enumerate(order)}
        cplus = {j: cum[i] / T for i, j in enumerate(order)}
        for j in set(got) ^ set(want):
            assert j == nb - 1 or min(abs(cminus[j] - tau), abs(cplus[j] - tau)) <= 1e-4, (name, h, j)
        letter += 1
        keys = np.nonzero(np.repeat(np.isin(np.arange(nb), got), B)[:L])[0]
        a = kf[keys, h // G, :].astype(np.float64) @ qf[h].astype(np.float64) / math.sqrt(d)
        w = np.exp(a - a.max())
        errs.append(np.abs(out[h] - w @ vf[keys, h // G, :].astype(np.float64) / w.sum()))
    e = np.concatenate(errs)
    say(f"  decode {name}: lists exact={exact} letter={letter}; kept {rc.mean() / nb:.3f} of the blocks; "
        f"max-abs {e.max():.3e} mean-abs {e.mean():.3e}")
    assert e.max() <= tmax and e.mean() <= tmean
    return rc


@pytest.mark.parametrize("name,tau", [("llama8b_L128k", 0.9), ("llama8b_L32k", 0.85), ("video_L64k", 0.9)])
def test_decode_workload_last_token(name, tau):
    w = workload(name)
    q, k, v = make_inputs(w)
    say(f"decode case {name} tau={tau}")
    check(q[w.L - 1], k, v, w.S, w.B, tau, w.dtype, name)
    # with the pooled keys given: the same lists and output, bitwise
    a = run_decode(q[w.L - 1], k, v, w.S, w.B, tau, w.dtype)
    b = run_decode(q[w.L - 1], k, v, w.S, w.B, tau, w.dtype, pooled=True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_decode_ragged_cache_and_small_shapes():
    for (L, Hq, Hkv, d, S, B, dt, kind) in [(100001, 8, 2, 128, 16, 128, "bf16", "llm"), (5000, 4, 4, 64, 8, 64, "bf16", "gauss"),
                                             (777, 2, 1, 64, 8, 64, "fp32", "tiny"), (130, 4, 2, 128, 16, 128, "bf16", "gauss"),
                                             (1, 4, 2, 128, 16, 128, "bf16", "gauss"), (17, 8, 2, 128, 16, 128, "bf16", "gauss")]:
        w = Workload("dec", L, Hq, Hkv, d, dt, B, S, (0.9,), 7, kind, 8)
        q, k, v = make_inputs(w)
        check(q[L - 1], k, v, S, B, 0.9, dt, f"L{L}_d{d}_B{B}_{dt}")


def test_decode_group_shapes():
    # query heads per KV head 3, 5, 8 and 1 with 64 blocks per workgroup (the most), over every d x B,
    # and 10 (past the group kernels)
    for (L, Hq, Hkv, d, S, B, kind) in [(9000, 24, 3, 128, 16, 64, "llm"), (12345, 15, 3, 64, 8, 128, "gauss"),
                                         (3000, 6, 2, 128, 16, 128, "llm"), (32768, 64, 64, 64, 16, 64, "gauss"),
                                         (64, 8, 1, 128, 16, 128, "llm"),
                                         (5000, 20, 2, 128, 16, 128, "llm")]:  # G = 10: the per-head kernels in bf16
        w = Workload("dec", L, Hq, Hkv, d, "bf16", B, S, (0.9,), 11, kind, 8)
        q, k, v = make_inputs(w)
        say(f"decode group case L={L} Hq={Hq} Hkv={Hkv} d={d} B={B}")
        check(q[L - 1], k, v, S, B, 0.9, "bf16", f"L{L}_G{Hq // Hkv}_d{d}_B{B}")


def test_decode_equal_masses_keep_lowest_indices():
    # all keys zero: every whole block has the same mass, so the order among
    # them is by index alone and the cut must keep exactly the lowest ones
    for L, tau in [(32768 + 77, 0.9), (4096, 0.5)]:
        w = Workload("ties", L, 8, 2, 128, "bf16", 128, 16, (tau,), 13, "gauss", 8)
        q, k, v = make_inputs(w)
        k = torch.zeros_like(k)
        say(f"decode ties case L={L} tau={tau}")
        rc = check(q[L - 1], k, v, 16, 128, tau, "bf16", f"ties_L{L}")
        assert rc.min() > 1


def test_decode_attend_on_given_lists():
    # rr_decode_attend on rr_decode's own lists reproduces its output bitwise;
    # on caller lists (unordered, with entries outside [0, nb) and repeats) it
    # attends to exactly the listed blocks
    for (L, Hq, Hkv, d, B, dt) in [(40000, 16, 4, 128, 128, "bf16"), (3000, 6, 2, 64, 64, "bf16"),
                                   (2000, 4, 2, 64, 64, "fp32")]:
        w = Workload("att", L, Hq, Hkv, d, dt, B, 16 if d == 128 else 8, (0.9,), 17, "llm", 8)
        q, k, v = make_inputs(w)
        p = rr.problem(L, Hq, Hkv, d, w.S, B, 0.9, True, dt)
        nb = p.nb
        qd, kd, vd = q[L - 1].contiguous().cuda(), k.cuda(), v.cuda()
        ws = torch.empty(rr.rr_decode_workspace_bytes(p), dtype=torch.uint8, device="cuda")
        out1, out2 = torch.empty_like(qd), torch.empty_like(qd)
        rc = torch.empty((Hq,), dtype=torch.int32, device="cuda")
        ci = torch.full((Hq, nb), -1, dtype=torch.int32, device="cuda")
        rr.rr_decode(p, qd, kd, vd, out1, rc, ci, None, ws)
        rr.rr_decode_attend(p, qd, kd, vd, rc, ci, out2, ws)
        torch.cuda.synchronize()
        assert torch.equal(out1, out2)
        rng = np.random.default_rng(L)
        lists, counts = np.full((Hq, nb), -1, np.int32), np.zeros(Hq, np.int32)
        for h in range(Hq):
            pick = rng.permutation(nb)[: max(1, nb // 3)]
            extra = [nb + 5, -3, int(pick[0])] if h % 2 else []  # out of range, and a repeat
            row = np.concatenate([pick, extra]).astype(np.int32)
            lists[h, : len(row)], counts[h] = row, len(row)
        out3 = torch.empty_like(qd)
        rr.rr_decode_attend(p, qd, kd, vd, torch.from_numpy(counts).cuda(), torch.from_numpy(lists).cuda(), out3, ws)
        torch.cuda.synchronize()
        got = out3.float().cpu().numpy()
        kf, vf, qf = k.float().numpy(), v.float().numpy(), q[L - 1].float().numpy()
        G = Hq // Hkv
        err = []
        for h in range(Hq):
            blocks = [j for j in lists[h, : counts[h]] if 0 <= j < nb]
            keys = np.nonzero(np.repeat(np.isin(np.arange(nb), blocks), B)[:L])[0]
            a = kf[keys, h // G, :].astype(np.float64) @ qf[h].astype(np.float64) / math.sqrt(d)
            wgt = np.exp(a - a.max())
            err.append(np.abs(got[h] - wgt @ vf[keys, h // G, :].astype(np.float64) / wgt.sum()))
        e = np.concatenate(err)
        tmax, tmean = (2e-2, 2e-3) if dt == "bf16" else (1e-4, 1e-5)
        say(f"  decode_attend L={L} d={d} B={B} {dt}: caller lists max-abs {e.max():.3e} mean-abs {e.mean():.3e}")
        assert e.max() <= tmax and e.mean() <= tmean


def test_decode_tau_one_is_dense_sdpa():
    w = Workload("dense", 20000, 8, 2, 128, "bf16", 128, 16, (1.0,), 9, "llm", 8)
    q, k, v = make_inputs(w)
    out, rc, ci, _ = run_decode(q[-1], k, v, 16, 128, 1.0, "bf16")
    assert np.all(rc == w.nb)
    qq = q[-1].float()[:, None, :]
    kk = k.float().repeat_interleave(4, dim=1).permute(1, 0, 2)
    vv = v.float().repeat_interleave(4, dim=1).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[:, 0, :].numpy()
    say(f"  dense decode vs SDPA: max-abs {np.abs(out - ref).max():.3e}")
    assert np.abs(out - ref).max() <= 2e-2 and np.abs(out - ref).mean() <= 2e-3
