"""Seeded choices of which output rows a check or a timing sample looks at.

Only random index selection lives here (no arithmetic of the attention
method): the GPU tests, the benchmark's CPU-baseline sample and the oracle
comparisons draw the same (token, head) pairs from the same seed.
"""

from __future__ import annotations

import numpy as np


def sample_rows(L: int, Hq: int, B: int, n: int, seed: int) -> np.ndarray:
    """(x, h) pairs: n random ones plus block edges and the first/last token."""
    rng = np.random.default_rng(seed)
    xs = list(rng.integers(0, L, n))
    xs += [0, 1, B - 1, B, L - 1, L - B, L - B - 1, L // 2]
    hs = list(rng.integers(0, Hq, len(xs)))
    return np.array(list(zip(xs, hs)), np.int32)


def work_item_rows(L: int, Hq: int, B: int, seed: int) -> np.ndarray:
    """(x, h) pairs, one per (query head h, query block i): a random query row
    of every block of every head (the last block may be short), so that each
    (head, query block) the attention's work schedule runs is looked at once.
    Ordered by head, then block."""
    rng = np.random.default_rng(seed)
    nb = -(-L // B)
    first = np.arange(nb, dtype=np.int64) * B
    size = np.minimum(B, L - first)
    out = np.empty((Hq * nb, 2), np.int32)
    for h in range(Hq):
        off = rng.integers(0, size)  # one draw per block, each below its block's size
        out[h * nb:(h + 1) * nb, 0] = first + off
        out[h * nb:(h + 1) * nb, 1] = h
    return out
