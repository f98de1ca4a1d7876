"""GPU parity of rr_mass_recall (full-attention softmax mass inside the
selected blocks) against the oracle's float64 recall on the same lists.

Bar: absolute error <= 5e-4 per row. The GPU forms the scores in float32 from
exact bf16 products and sums up to L exponentials per query in float32 (one
running maximum for both sums, the same exponentials in both), so the ratio
carries a relative error of a few 1e-6 typically; 5e-4 leaves room for the
worst-case growth of the float32 sums at 128K keys. With every block
selected the two sums are the same float32 additions, so the recall is 1
exactly.
"""

import numpy as np
import pytest

import oracle
from synthetic.gen import Workload, workload
from tests.gpu_cases import DeviceCase, say

pytestmark = pytest.mark.gpu

ATOL = 5e-4


def g(name, L, Hq, Hkv, d, S, B, dtype, causal=True, kind="gauss", seed=100):
    return Workload(name, L, Hq, Hkv, d, dtype, B, S, (0.9,), seed, kind, 8, causal)


SMALL = [
    g("llm_b128_d128", 2048, 8, 2, 128, 16, 128, "bf16", kind="llm"),
    g("gauss_b64_d64", 1024, 4, 2, 64, 8, 64, "bf16"),
    g("gauss_b128_d64", 1024, 2, 1, 64, 16, 128, "bf16"),
    g("gauss_b64_d128_noncausal", 512, 3, 1, 128, 8, 64, "bf16", causal=False),
    g("llm_b64_d128_noncausal", 1024, 4, 2, 128, 8, 64, "bf16", causal=False, kind="llm"),
    g("fp32_b64_d64", 512, 4, 4, 64, 8, 64, "fp32", kind="tiny"),
    g("fp32_b128_d128_noncausal", 512, 2, 1, 128, 16, 128, "fp32", causal=False),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_recall_small_shapes_full(w):
    say(f"recall case {w.name}")
    run = DeviceCase(w, 0.9)
    rc, ci, _ = run.search(export_mass=False)
    got = run.recall(rc, ci)
    want = oracle.mass_recall(run.q, run.k, rc, ci, B=w.B, causal=w.causal)
    err = np.abs(got - want).max()
    say(f"  recall {w.name}: max-abs err {err:.2e}, mean recall {want.mean():.4f}, min {want.min():.4f}")
    assert err <= ATOL
    # every block selected: exactly one
    frc, fci = oracle.full_lists(w.L, w.Hq, w.B, w.causal)
    np.testing.assert_array_equal(run.recall(frc, fci), np.ones((w.Hq, w.nb), np.float32))


@pytest.mark.parametrize("name,rows_i", [
    ("llama8b_L16k", [0, 1, 5, 64, 100, 126, 127]),
    ("video_L64k", [0, 3, 255, 256, 400, 510, 511]),
    ("llama8b_L128k", [0, 2, 511, 900, 1022, 1023]),
])
def test_recall_workloads_sampled_rows(name, rows_i):
    w = workload(name)
    say(f"recall case {name}")
    run = DeviceCase(w, 0.9)
    rc, ci, _ = run.search(export_mass=False)
    got = run.recall(rc, ci)
    rng = np.random.default_rng(5)
    rows = np.array([[int(rng.integers(0, w.Hq)), i] for i in rows_i], np.int32)
    want = oracle.mass_recall(run.q, run.k, rc, ci, B=w.B, causal=w.causal, rows=rows)
    err = np.abs(got[rows[:, 0], rows[:, 1]] - want).max()
    say(f"  recall {name}: max-abs err {err:.2e} on {len(rows)} rows; GPU mean recall {got.mean():.4f}, "
        f"min {got.min():.4f}")
    assert err <= ATOL
    assert np.all(np.isfinite(got)) and got.min() > 0.0 and got.max() <= 1.0 + 1e-6
    np.testing.assert_array_equal(got[:, -1], 1.0)  # the last query block is kept whole
