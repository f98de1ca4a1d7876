"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small shapes cover every kernel variant (dtype, d, B, r = B/S, GQA group size,
one or two sampled-query column tiles, causal or not, a single block, tau = 1)
and are compared in full. The five workload layers are compared on every
block-list row and every exported block mass; their attention output (the
prefill's, on the GPU's own lists) is compared in full at 1K tokens and
otherwise on one random query row of every (head, query block) work item
plus the block-edge rows. The output buffer starts as NaN, so a work item the
schedule never ran fails at any size. The oracle's searches of the large
layers are cached on disk (tests/oracle_cache.py).

Bars: block lists per tests/checker.py (no 'fail' rows); exported block masses
within 1e-4 relative + 1e-6 absolute; attention given the same lists within
max-abs 2e-2 and mean-abs 2e-3 for bf16, 1e-4 / 1e-5 for float32.
"""

import numpy as np
import pytest

import oracle
from synthetic.gen import Workload, workload
from tests import checker, oracle_cache, report
from tests.gpu_cases import DeviceCase, sample_rows, say, work_item_rows

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 2e-2, 2e-3
F32_MAX, F32_MEAN = 1e-4, 1e-5


def tol(w):
    return (BF16_MAX, BF16_MEAN) if w.dtype == "bf16" else (F32_MAX, F32_MEAN)


def g(name, L, Hq, Hkv, d, S, B, dtype, causal=True, kind="gauss", seed=100, n_stripes=8):
    return Workload(name, L, Hq, Hkv, d, dtype, B, S, (0.9,), seed, kind, n_stripes, causal)


SMALL = [
    (g("llm_g4_r8", 2048, 8, 2, 128, 16, 128, "bf16", kind="llm"), 0.9),
    (g("llm_g7_two_col_tiles", 1536, 14, 2, 128, 16, 128, "bf16", kind="llm"), 0.9),
    (g("gauss_r2_d64_b64", 1024, 4, 2, 64, 32, 64, "bf16"), 0.8),
    (g("gauss_r4", 1024, 8, 4, 128, 32, 128, "bf16"), 0.9),
    (g("gauss_r16", 2048, 4, 1, 128, 8, 128, "bf16"), 0.9),
    (g("gauss_r32_d64", 2048, 2, 1, 64, 4, 128, "bf16"), 0.9),
    (g("gauss_b64_d128", 1024, 4, 1, 128, 8, 64, "bf16"), 0.85),
    (g("noncausal", 1024, 4, 2, 128, 16, 128, "bf16", causal=False), 0.9),
    (g("mha_g1_b128", 1024, 3, 3, 128, 16, 128, "bf16"), 0.9),
    (g("llm_g8_d64", 2048, 16, 2, 64, 16, 128, "bf16", kind="llm"), 0.9),
    (g("gauss_g16", 1024, 32, 2, 128, 16, 128, "bf16"), 0.9),
    (g("single_block", 128, 2, 1, 128, 16, 128, "bf16"), 0.9),
    (g("tau_one", 1024, 4, 2, 128, 16, 128, "bf16"), 1.0),
    (g("fp32_d128", 512, 4, 2, 128, 16, 128, "fp32"), 0.9),
    (g("fp32_noncausal_b64", 512, 2, 2, 64, 8, 64, "fp32", causal=False), 0.9),
]


def oracle_search(w, tau, q, k, row_mask=None):
    return oracle.search(q, k, S=w.S, B=w.B, tau=tau, causal=w.causal,
                         round_bf16=w.dtype == "bf16", row_mask=row_mask)


def check_lists(w, tau, rc, ci, orc, rows=None):
    res = checker.classify(rc, ci, orc, tau, causal=w.causal, rows=rows)
    say(f"  masks {w.name} tau={tau}: exact={res['exact']} letter={res['letter']} "
        f"near_tie={res['near_tie']} fail={res['fail']} {res['fail_rows'][:5]}")
    assert res["fail"] == 0, res["fail_rows"][:10]
    return res


@pytest.mark.parametrize("w,tau", SMALL, ids=[c[0].name for c in SMALL])
def test_small_shapes_full_parity(w, tau):
    say(f"case {w.name} tau={tau}")
    run = DeviceCase(w, tau)
    rc, ci, mass = run.search(export_mass=True)
    orc = oracle_search(w, tau, run.q, run.k)
    np.testing.assert_allclose(mass, orc.mass, rtol=1e-4, atol=1e-6)
    check_lists(w, tau, rc, ci, orc)
    # attention on the oracle's lists, compared in full
    want = oracle.attention(run.q, run.k, run.v, orc.row_count, orc.col_idx, B=w.B, causal=w.causal)
    got = run.attention(orc.row_count, orc.col_idx)
    mx, mean = checker.output_errors(got, want)
    say(f"  attention {w.name}: max-abs {mx:.3e} mean-abs {mean:.3e}")
    tmax, tmean = tol(w)
    assert mx <= tmax and mean <= tmean
    # end to end, compared on the GPU's own lists
    out, rc2, ci2 = run.prefill()
    np.testing.assert_array_equal(rc2, rc)
    want2 = oracle.attention(run.q, run.k, run.v, rc2, ci2, B=w.B, causal=w.causal)
    mx2, mean2 = checker.output_errors(out, want2)
    assert mx2 <= tmax and mean2 <= tmean


def test_tau_one_equals_dense_attention():
    w = g("dense", 2048, 8, 2, 128, 16, 128, "bf16", kind="llm")
    run = DeviceCase(w, 1.0)
    out, rc, ci = run.prefill()
    frc, fci = oracle.full_lists(w.L, w.Hq, w.B)
    np.testing.assert_array_equal(rc, frc)
    for h in range(w.Hq):
        for i in range(w.nb):
            np.testing.assert_array_equal(ci[h, i, : rc[h, i]], np.arange(i + 1))
    want = oracle.attention(run.q, run.k, run.v, frc, fci, B=w.B)
    mx, mean = checker.output_errors(out, want)
    assert mx <= BF16_MAX and mean <= BF16_MEAN


def test_runs_are_bitwise_deterministic():
    w = g("det", 4096, 8, 2, 128, 16, 128, "bf16", kind="llm")
    run = DeviceCase(w, 0.9)
    a = run.prefill()
    b = run.prefill()
    np.testing.assert_array_equal(a[1], b[1])
    for h in range(w.Hq):
        for i in range(w.nb):
            np.testing.assert_array_equal(a[2][h, i, : a[1][h, i]], b[2][h, i, : b[1][h, i]])
    np.testing.assert_array_equal(a[0], b[0])


def test_query_independence_on_gpu():
    w = g("qi", 2048, 4, 2, 128, 16, 128, "bf16", kind="llm")
    run = DeviceCase(w, 0.9)
    rc, ci, _ = run.search(export_mass=False)
    q2 = run.q.clone()
    q2[(5 + 1) * w.B:] = -q2[(5 + 1) * w.B:]
    run2 = DeviceCase(w, 0.9, inputs=(q2, run.k, run.v))
    rc2, ci2, _ = run2.search(export_mass=False)
    np.testing.assert_array_equal(rc[:, :6], rc2[:, :6])
    for h in range(w.Hq):
        for i in range(6):
            np.testing.assert_array_equal(ci[h, i, : rc[h, i]], ci2[h, i, : rc2[h, i]])


# ------------------------------------------------------------------ workload shapes

def _workload_case(name, tau):
    w = workload(name)
    say(f"case {name} tau={tau} L={w.L}")
    run = DeviceCase(w, tau)
    rc, ci, mass = run.search(export_mass=True)
    orc = oracle_cache.search(w, tau, run.q, run.k, say=say)
    np.testing.assert_allclose(mass, orc.mass, rtol=1e-4, atol=1e-6)
    del mass
    res = check_lists(w, tau, rc, ci, orc)
    rows_checked = res["exact"] + res["letter"] + res["near_tie"] + res["fail"]
    say(f"  rows compared {rows_checked} of {w.Hq * w.nb}")
    line = (f"{name} tau={tau}: rows {rows_checked} of {w.Hq * w.nb}: exact {res['exact']} "
            f"letter {res['letter']} near_tie {res['near_tie']} fail {res['fail']}")
    assert rows_checked == w.Hq * w.nb
    keep = rc.sum() / (w.Hq * w.nb * (w.nb + 1) / 2)
    say(f"  keep fraction {keep:.4f}")
    del orc
    # attention end to end on the GPU's lists
    run.pre.out.fill_(float("nan"))
    out, rc2, ci2 = run.prefill()
    np.testing.assert_array_equal(rc2, rc)
    assert np.isfinite(out).all(), "some output rows were never written"

    tmax, tmean = tol(w)
    if w.L <= 1024:
        want = oracle.attention(run.q, run.k, run.v, rc2, ci2, B=w.B, causal=w.causal)
        mx, mean = checker.output_errors(out, want)
        say(f"  attention (all rows) max-abs {mx:.3e} mean-abs {mean:.3e}")
    else:
        srows = np.concatenate([work_item_rows(w.L, w.Hq, w.B, seed=w.seed),
                                sample_rows(w.L, w.Hq, w.B, 64, seed=w.seed)])
        say(f"  oracle attention on {len(srows)} rows (one per (head, query block) + edges) ...")
        want = oracle.attention(run.q, run.k, run.v, rc2, ci2, B=w.B, causal=w.causal, rows=srows)
        got = out[srows[:, 0], srows[:, 1]]
        mx, mean = checker.output_errors(got, want)
        say(f"  attention ({len(srows)} rows) max-abs {mx:.3e} mean-abs {mean:.3e}")
    nrows = w.L * w.Hq if w.L <= 1024 else len(srows)
    report.record(line + f"; attention {nrows} (token, head) rows max-abs {mx:.2e} mean-abs {mean:.2e}")
    assert mx <= tmax and mean <= tmean
    return res


def test_workload_tiny_fp32_L1k():
    _workload_case("tiny_fp32_L1k", 0.9)


def test_workload_llama8b_L16k():
    _workload_case("llama8b_L16k", 0.9)


@pytest.mark.parametrize("tau", [0.85, 0.9, 0.95])
def test_workload_llama8b_L32k(tau):
    _workload_case("llama8b_L32k", tau)


@pytest.mark.timeout(900)
def test_workload_video_L64k():
    _workload_case("video_L64k", 0.9)


@pytest.mark.timeout(900)
def test_workload_llama8b_L128k():
    _workload_case("llama8b_L128k", 0.9)
