"""Float64 brute force for tiny inputs, written independently of the oracle.

It materialises the full L x L logit matrix and reaches the method's
quantities by a different route than the oracle does:
  * pooled scores as the stride mean of the full logits (q . mean(k) equals
    mean(q . k)), or, for bfloat16 inputs, from keys pooled in float64 and
    rounded to bfloat16 by torch;
  * Top-tau by exhaustive search over subsets (no sorting);
  * attention as a dense softmax under a materialised element mask.
"""

from __future__ import annotations

import itertools
import math

import numpy as np
import torch


def sampled_positions(L: int, Hq: int, S: int) -> np.ndarray:
    """[Hq][L/S] token index sampled by head h in stride s (offset h mod S)."""
    ns = L // S
    return np.array([[s * S + (h % S) for s in range(ns)] for h in range(Hq)], dtype=np.int64)


def block_mass(q, k, *, S, B, causal=True, bf16_pool=False) -> np.ndarray:
    """m[h][i][j] in float64 for rows i < nb-1 (last row left at 0)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    ns, nb, r = L // S, L // B, B // S
    pos = sampled_positions(L, Hq, S)
    out = np.zeros((Hq, nb, nb))
    if bf16_pool:
        kbar = torch.from_numpy(k.reshape(ns, S, Hkv, d).mean(axis=1)).to(torch.bfloat16).double().numpy()
    for h in range(Hq):
        g = h // G
        if bf16_pool:
            z = (q[pos[h], h, :] @ kbar[:, g, :].T) / math.sqrt(d)  # [ns][ns]
        else:
            full = (q[:, h, :] @ k[:, g, :].T) / math.sqrt(d)          # [L][L]
            z = full[pos[h]].reshape(ns, ns, S).mean(axis=2)            # stride mean
        if causal:
            z = np.where(np.tril(np.ones((ns, ns), bool)), z, -np.inf)
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        blk = p.reshape(nb, r, nb, r).sum(axis=3).mean(axis=1)         # [nb][nb]
        out[h, : nb - 1] = blk[: nb - 1]
    return out


def min_cardinality_set(m: np.ndarray, tau: float):
    """Smallest set of indices whose mass reaches tau * total, by enumeration.

    Returns (set, margin): among subsets of the minimal size it picks the one of
    largest mass; margin is how far the best subset of one fewer element falls
    short of the threshold (relative to the total), telling how robust the
    answer is to rounding.
    """
    n = len(m)
    total = float(np.sum(m))
    thr = tau * total
    best_prev = 0.0
    for size in range(1, n + 1):
        best, best_set = -1.0, None
        for c in itertools.combinations(range(n), size):
            s = float(sum(m[list(c)]))
            if s > best:
                best, best_set = s, c
        if best >= thr:
            return set(best_set), (thr - best_prev) / total
        best_prev = best
    return set(range(n)), 0.0


def masked_attention(q, k, v, mask_blocks: np.ndarray, *, B, causal=True) -> np.ndarray:
    """O [L][Hq][d], dense float64 softmax with the element mask built from block selections."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((L, Hq, d))
    elem = np.kron(mask_blocks.astype(np.int8), np.ones((B, B), np.int8)).astype(bool)  # [Hq][L][L]
    if causal:
        elem &= np.tril(np.ones((L, L), bool))[None]
    for h in range(Hq):
        g = h // G
        a = (q[:, h, :] @ k[:, g, :].T) / math.sqrt(d)
        a = np.where(elem[h], a, -np.inf)
        w = np.exp(a - a.max(axis=1, keepdims=True))
        out[:, h, :] = (w @ v[:, g, :]) / w.sum(axis=1, keepdims=True)
    return out


def mass_recall(q, k, mask_blocks: np.ndarray, *, B, causal=True) -> np.ndarray:
    """[Hq][nb] mean over each query block of the dense float64 softmax mass on the selected blocks.

    Materialises the full softmax matrix with torch (float64) and sums it under
    the block mask expanded to elements.
    """
    q = torch.from_numpy(np.asarray(q, np.float64))
    k = torch.from_numpy(np.asarray(k, np.float64))
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    nb = L // B
    elem = torch.from_numpy(np.kron(mask_blocks.astype(np.int8), np.ones((B, B), np.int8)).astype(bool))
    out = np.zeros((Hq, nb))
    for h in range(Hq):
        a = (q[:, h, :] @ k[:, h // G, :].T) / math.sqrt(d)
        if causal:
            a = a.masked_fill(~torch.ones(L, L, dtype=torch.bool).tril(), float("-inf"))
        w = torch.softmax(a, dim=1)
        per_query = (w * elem[h]).sum(dim=1)  # [L]
        out[h] = per_query.reshape(nb, B).mean(dim=1).numpy()
    return out


def block_mass_ragged(q, k, *, S, B, causal=True) -> np.ndarray:
    """block_mass for any L (float inputs): the last stride and block may be short.

    Pooled scores are the mean of the full logits over the tokens each stride
    has (q . mean(k) = mean(q . k)); key block j covers the strides
    t in [j*B/S, (j+1)*B/S) that exist. Rows i < nb-1 only (the last is 0).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    ns, nb, r = -(-L // S), -(-L // B), B // S
    out = np.zeros((Hq, nb, nb))
    stride_of = np.arange(L) // S
    cnt = np.bincount(stride_of, minlength=ns).astype(np.float64)
    for h in range(Hq):
        g = h // G
        pos = np.array([s * S + (h % S) for s in range((nb - 1) * r)], np.int64)
        full = (q[pos, h, :] @ k[:, g, :].T) / math.sqrt(d)        # [(nb-1) r][L]
        z = np.zeros((len(pos), ns))
        np.add.at(z, (slice(None), stride_of), full)               # sum over each stride's tokens
        z /= cnt[None, :]
        if causal:
            z = np.where(np.arange(ns)[None, :] <= np.arange(len(pos))[:, None], z, -np.inf)
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        blk = np.zeros((len(pos), nb))
        np.add.at(blk, (slice(None), np.arange(ns) // r), p)
        out[h, : nb - 1] = blk.reshape(nb - 1, r, nb).mean(axis=1)
    return out


def masked_attention_ragged(q, k, v, mask_blocks: np.ndarray, *, B, causal=True) -> np.ndarray:
    """masked_attention for any L: the block mask is expanded to nb*B elements and cut at L."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((L, Hq, d))
    elem = np.kron(mask_blocks.astype(np.int8), np.ones((B, B), np.int8)).astype(bool)[:, :L, :L]
    if causal:
        elem &= np.tril(np.ones((L, L), bool))[None]
    for h in range(Hq):
        g = h // G
        a = (q[:, h, :] @ k[:, g, :].T) / math.sqrt(d)
        a = np.where(elem[h], a, -np.inf)
        w = np.exp(a - a.max(axis=1, keepdims=True))
        out[:, h, :] = (w @ v[:, g, :]) / w.sum(axis=1, keepdims=True)
    return out
