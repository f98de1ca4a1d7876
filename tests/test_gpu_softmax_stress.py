"""GPU stress cases for the online softmax of the bf16 attention kernels.

Both bf16 kernels (the head-pair ping-pong kernel, and the one-head kernel
on the same problem with K/V repeated per query head) run on dense
causal lists (every block j <= i) against the oracle's attention, with scores
built to exercise the running maximum and the rescale:

  rising     scores grow with the key index, so the row maximum moves up in
             every block and O and the row sum are rescaled every block;
  falling    scores shrink with the key index: the first block holds the
             maximum and no later block rescales;
  underflow  scores of magnitude about 140 (base-e, after the 1/sqrt(d)
             scale): most probabilities underflow to zero in float32, the
             rest are dominated by a few keys;
  uniform    every key identical: each row is the plain mean of its visible
             values.

Bars as everywhere for bf16 outputs: max-abs 2e-2, mean-abs 2e-3 against the
float64 oracle on the same bf16 inputs.
"""

import numpy as np
import pytest
import torch

import oracle
from synthetic.gen import Workload
from tests import checker
from tests.gpu_cases import DeviceCase, say
from tests.test_gpu_attn_variants import VARIANTS, run_variant

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 2e-2, 2e-3
L, HQ, HKV, D, B = 1536, 4, 2, 128, 128


def inputs(case, seed=7):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(D).astype(np.float32)
    u /= np.linalg.norm(u)
    noise = lambda *s: 0.05 * rng.standard_normal(s).astype(np.float32)
    pos = (np.arange(L, dtype=np.float32) / L)[:, None, None]
    if case == "rising":
        q = 8.0 * u + noise(L, HQ, D)
        k = 64.0 * pos * u + noise(L, HKV, D)
    elif case == "falling":
        q = 8.0 * u + noise(L, HQ, D)
        k = 64.0 * (1.0 - pos) * u + noise(L, HKV, D)
    elif case == "underflow":
        q = 40.0 * u + noise(L, HQ, D)
        sign = np.where(rng.random((L, HKV, 1)) < 0.5, -1.0, 1.0).astype(np.float32)
        k = 40.0 * sign * u + noise(L, HKV, D)
    elif case == "uniform":
        q = rng.standard_normal((L, HQ, D)).astype(np.float32)
        k = np.broadcast_to(u, (L, HKV, D)).copy()
    else:
        raise ValueError(case)
    v = rng.standard_normal((L, HKV, D)).astype(np.float32)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return bf(q), bf(k), bf(v)


def dense_causal_lists(nb):
    rc = np.zeros((HQ, nb), np.int32)
    ci = np.zeros((HQ, nb, nb), np.int32)
    for i in range(nb):
        rc[:, i] = i + 1
        ci[:, i, : i + 1] = np.arange(i + 1)
    return rc, ci


@pytest.mark.parametrize("case", ["rising", "falling", "underflow", "uniform"])
def test_softmax_stress_all_kernels(case):
    say(f"case {case}")
    w = Workload(f"stress_{case}", L, HQ, HKV, D, "bf16", B, 16, (0.9,), 7, "gauss", 0, True)
    run = DeviceCase(w, 0.9, inputs=inputs(case))
    rc, ci = dense_causal_lists(w.nb)
    want = oracle.attention(run.q, run.k, run.v, rc, ci, B=B, causal=True)
    assert np.all(np.isfinite(want))
    for name in VARIANTS:
        got = run_variant(run, name, rc, ci)
        assert np.all(np.isfinite(got)), name
        mx, mean = checker.output_errors(got, want)
        say(f"  {name}: max-abs {mx:.3e} mean-abs {mean:.3e}")
        assert mx <= BF16_MAX and mean <= BF16_MEAN, name
    if case == "uniform":
        # each row is the mean of the values of keys 0..x of its KV head
        vf = run.v.float().numpy()
        csum = np.cumsum(vf, axis=0) / np.arange(1, L + 1, dtype=np.float32)[:, None, None]
        for h in range(HQ):
            np.testing.assert_allclose(want[:, h, :], csum[:, h // (HQ // HKV), :], atol=1e-5)
