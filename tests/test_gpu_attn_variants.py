"""GPU parity of the head-pair attention kernel's two forms at B = 128 on the
same lists.

The library picks its kernel from the problem alone: bf16 with B = 128 runs
the head-pair ping-pong kernel. Within a KV head it pairs two query heads;
with an odd count (one query head per KV head included) the last head is
paired with itself over two adjacent query blocks. Both forms therefore run
on the same attention by posing it twice: once with the grouped K/V (heads
paired), once with K/V repeated per query head (Hkv = Hq, so G = 1 and every
head self-paired). Each is compared in full with the oracle's attention on
the oracle's lists (bf16 bars: max-abs 2e-2, mean-abs 2e-3), and the two
outputs with each other within 1e-2 (each head walks its blocks in the same
order with the same softmax in both forms; on these cases their outputs
have in fact matched bit for bit). The one-head kernel (B = 64) meets the
oracle in the random problems below and in the ragged tests.

A second test poses random problems (length, heads, head dimension, block
size, causality, dtype) with random block lists, so that every kernel (head
pairs, one head, fp32) meets short and ragged layers, empty-looking tiles and
lists that skip the diagonal.

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
VARIANTS = ["paired", "self_paired"]


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
    """Attention of run's problem on the given lists in one form of the kernel:
    'paired' as posed, 'self_paired' with K/V repeated per query head."""
    if name == "paired":
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
    d = np.abs(outs["self_paired"] - outs["paired"])
    say(f"  self_paired vs paired: max-abs {d.max():.3e}")
    assert d.max() <= 1e-2


def random_lists(rng, Hq, nb, causal):
    """Random non-empty ascending block lists (causal ones within the row's
    diagonal; the diagonal itself is kept or left out at random)."""
    rc = np.zeros((Hq, nb), np.int32)
    ci = np.zeros((Hq, nb, nb), np.int32)
    for h in range(Hq):
        for i in range(nb):
            cand = np.arange(i + 1 if causal else nb)
            n = int(rng.integers(1, len(cand) + 1))
            sel = np.sort(rng.choice(cand, size=n, replace=False))
            rc[h, i] = n
            ci[h, i, :n] = sel
    return rc, ci


RANDOM_SEEDS = list(range(12))


@pytest.mark.parametrize("seed", RANDOM_SEEDS)
def test_attention_random_shapes_against_oracle(seed):
    rng = np.random.default_rng(9000 + seed)
    dtype = "fp32" if seed % 3 == 0 else "bf16"
    d = int(rng.choice([64, 128]))
    B = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 3, 4]))
    L = int(rng.integers(1, 6 * B + 1))
    causal = bool(rng.integers(0, 2))
    S = 16 if B == 128 else 8
    w = Workload(f"rand{seed}", L, Hkv * G, Hkv, d, dtype, B, S, (0.9,), 500 + seed, "gauss", 8, causal)
    say(f"case {w.name}: L={L} Hq={w.Hq} Hkv={Hkv} d={d} B={B} causal={causal} {dtype}")
    run = DeviceCase(w, 0.9)
    rc, ci = random_lists(rng, w.Hq, w.nb, causal)
    got = run.attention(rc, ci)
    want = oracle.attention(run.q, run.k, run.v, rc, ci, B=B, causal=causal)
    mx, mean = checker.output_errors(got, want)
    say(f"  max-abs {mx:.3e} mean-abs {mean:.3e}")
    tmax, tmean = (BF16_MAX, BF16_MEAN) if dtype == "bf16" else (1e-4, 1e-5)
    assert mx <= tmax and mean <= tmean
