"""GPU parity of the three bf16 attention kernels at B = 128 on the same lists.

The library launches the head-pair ping-pong kernel by default when a KV head
has two or more query heads; RR_ATTN_PP=0 selects the head-pair kernel without
ping-pong and RR_ATTN_PAIR=0 the one-head-per-workgroup kernel. Both switches
are read at every launch. Each kernel is compared in full with the oracle's
attention on the oracle's lists (bf16 bars: max-abs 2e-2, mean-abs 2e-3), and
the three outputs with each other within 1e-2 (the two head-pair kernels sum
the same products in the same order; the one-head kernel forms the row sums
from the unrounded probabilities).

Shapes: odd groups (by default the last head of each KV head runs paired with
itself over two adjacent query blocks, one per slot; with an odd number of
query blocks the lowest block's lone head has no partner; the head-pair kernel
leaves half a workgroup idle instead), causal and not, a non-causal problem with
a short last block, head dimension 64, and lists that the search produced, so
heads of one pair select different blocks.
"""

import os

import numpy as np
import pytest

import oracle
from synthetic.gen import Workload
from tests import checker
from tests.gpu_cases import DeviceCase, say

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 2e-2, 2e-3
VARIANTS = [("pingpong", {}), ("pair", {"RR_ATTN_PP": "0"}), ("single_head", {"RR_ATTN_PAIR": "0"})]


def g(name, L, Hq, Hkv, d, S, causal=True, kind="llm", seed=300):
    return Workload(name, L, Hq, Hkv, d, "bf16", 128, S, (0.9,), seed, kind, 8, causal)


CASES = [
    g("odd_group_g3", 1536, 6, 2, 128, 16),
    g("odd_group_g3_odd_nb", 1400, 3, 1, 128, 8),
    g("odd_group_g5_noncausal_d64", 1100, 10, 2, 64, 16, causal=False, kind="gauss"),
    g("noncausal_short_tail", 1000, 4, 2, 128, 16, causal=False, kind="gauss"),
    g("d64_g4", 1024, 8, 2, 64, 16),
]


def run_variant(run, env, rc, ci):
    saved = {k: os.environ.get(k) for k in ("RR_ATTN_PP", "RR_ATTN_PAIR")}
    try:
        for k in saved:
            os.environ.pop(k, None)
        os.environ.update(env)
        return run.attention(rc, ci)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_attention_kernels_agree_with_oracle(w):
    say(f"case {w.name}")
    run = DeviceCase(w, 0.9)
    orc = oracle.search(run.q, run.k, S=w.S, B=w.B, tau=0.9, causal=w.causal, round_bf16=True)
    want = oracle.attention(run.q, run.k, run.v, orc.row_count, orc.col_idx, B=w.B, causal=w.causal)
    outs = {}
    for name, env in VARIANTS:
        got = run_variant(run, env, orc.row_count, orc.col_idx)
        mx, mean = checker.output_errors(got, want)
        say(f"  {name}: max-abs {mx:.3e} mean-abs {mean:.3e}")
        assert mx <= BF16_MAX and mean <= BF16_MEAN, name
        outs[name] = got
    for name in ("pair", "single_head"):
        d = np.abs(outs[name] - outs["pingpong"])
        say(f"  {name} vs pingpong: max-abs {d.max():.3e}")
        assert d.max() <= 1e-2, name
