"""GPU parity of the two bf16 attention kernels at B = 128 on the same lists.

The library picks its kernel from the problem alone: with two or more query
heads per KV head it launches the head-pair ping-pong kernel, with one it
launches the one-head-per-workgroup kernel. Both therefore run on the same
attention by posing it twice: once with the grouped K/V (ping-pong), once with
K/V repeated per query head (Hkv = Hq, so G = 1 and the one-head kernel). Each
is compared in full with the oracle's attention on the oracle's lists (bf16
bars: max-abs 2e-2, mean-abs 2e-3), and the two outputs with each other
within 1e-2 (the one-head kernel forms the row sums from the unrounded
probabilities, the ping-pong kernel from the bf16-rounded ones).

Shapes: odd groups (the last head of each KV head runs paired with itself
over two adjacent query blocks, one per slot; with an odd number of query
blocks the lowest block's lone head has no partner), causal and not, a
non-causal problem with a short last block, head dimension 64, and lists that
the search produced, so heads of one pair select different blocks.
"""

import dataclasses

import numpy as np
import pytest

import oracle
from synthetic.gen import Workload
from tests import checker
from tests.gpu_cases import DeviceCase, say

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 2e-2, 2e-3
VARIANTS = ["pingpong", "single_head"]


def g(name, L, Hq, Hkv, d, S, causal=True, kind="llm", seed=300):
    return Workload(name, L, Hq, Hkv, d, "bf16", 128, S, (0.9,), seed, kind, 8, causal)


CASES = [
    g("odd_group_g3", 1536, 6, 2, 128, 16),
    g("odd_group_g3_odd_nb", 1400, 3, 1, 128, 8),
    g("odd_group_g5_noncausal_d64", 1100, 10, 2, 64, 16, causal=False, kind="gauss"),
    g("noncausal_short_tail", 1000, 4, 2, 128, 16, causal=False, kind="gauss"),
    g("d64_g4", 1024, 8, 2, 64, 16),
]


def run_variant(run, name, rc, ci):
    """Attention of run's problem on the given lists through one kernel:
    'pingpong' as posed, 'single_head' with K/V repeated per query head."""
    if name == "pingpong":
        return run.attention(rc, ci)
    w = run.w
    G = w.Hq // w.Hkv
    wide = dataclasses.replace(w, name=w.name + "_g1", Hkv=w.Hq)
    k1 = run.k.repeat_interleave(G, dim=1).contiguous()
    v1 = run.v.repeat_interleave(G, dim=1).contiguous()
    return DeviceCase(wide, run.tau, inputs=(run.q, k1, v1)).attention(rc, ci)


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_attention_kernels_agree_with_oracle(w):
    say(f"case {w.name}")
    run = DeviceCase(w, 0.9)
    orc = oracle.search(run.q, run.k, S=w.S, B=w.B, tau=0.9, causal=w.causal, round_bf16=True)
    want = oracle.attention(run.q, run.k, run.v, orc.row_count, orc.col_idx, B=w.B, causal=w.causal)
    outs = {}
    for name in VARIANTS:
        got = run_variant(run, name, orc.row_count, orc.col_idx)
        mx, mean = checker.output_errors(got, want)
        say(f"  {name}: max-abs {mx:.3e} mean-abs {mean:.3e}")
        assert mx <= BF16_MAX and mean <= BF16_MEAN, name
        outs[name] = got
    d = np.abs(outs["single_head"] - outs["pingpong"])
    say(f"  single_head vs pingpong: max-abs {d.max():.3e}")
    assert d.max() <= 1e-2
