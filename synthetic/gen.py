"""Seeded synthetic Q/K/V for causal prefill attention layers.

The RRAttention pages evaluate on long-context text (HELMET, LLaMA-3.1-8B-Instruct
at 16K-128K tokens) and on video (Video-MME with a video LMM); see the abstract
and the Figure 3 caption of "RRAttention: Dynamic Block Sparse Attention via
Per-Head Round-Robin Shifts for Long-Context Inference". Neither the data nor
the weights are used here. These generators stand in for those workloads with
random tensors of the same attention-layer shapes plus planted structure of the
kinds such layers show (an attention sink, a local window, vertical stripes,
per-frame clusters and cross-frame patch bands).

Every array is drawn in float32 from ``numpy.random.default_rng(seed)`` in the
order written below and then cast to the workload dtype (bfloat16 with
round-to-nearest-even through torch, or kept as float32). Layout is
``[L][H][d]`` (token-major, heads, head dim), batch 1.

Nothing in this module evaluates the attention method.
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import numpy as np
import torch

GENERATOR_VERSION = 1

# Amplitude of the planted structure in the 8B-shaped recipe: (local window,
# sink, stripes) logit boosts are LLM_ALPHA * (1.0, 1.0, 0.75). Found once by
# bisection so that the 32K-token layer at tau = 0.9 keeps about half of its
# causal blocks (tests/golden/calibrate_generator.py writes the record).
LLM_ALPHA = 10.62
# Logit boost between equal patch indices of different frames in the video
# recipe, found the same way on the 64K-token video layer at tau = 0.9.
VIDEO_BETA = 111.0


@dataclass(frozen=True)
class Workload:
    name: str
    L: int
    Hq: int
    Hkv: int
    d: int
    dtype: str  # "bf16" or "fp32"
    B: int
    S: int
    taus: tuple
    seed: int
    kind: str  # "tiny", "llm" or "video"
    n_stripes: int = 0
    causal: bool = True

    @property
    def nb(self) -> int:
        return -(-self.L // self.B)

    @property
    def ns(self) -> int:
        return -(-self.L // self.S)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def scaled(self, **kw) -> "Workload":
        """Same recipe with some fields replaced (smaller L for tests, another seed...)."""
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        # Tiny single layer, fp32: sink key x4, 3 stripe keys shifted along a
        # direction that every query also carries.
        Workload("tiny_fp32_L1k", 1024, 4, 4, 64, "fp32", 64, 8, (0.9,), 0, "tiny", 3),
        # LLaMA-3.1-8B-shaped layers (32 query heads, 8 KV heads, d = 128).
        Workload("llama8b_L16k", 16384, 32, 8, 128, "bf16", 128, 16, (0.9,), 1, "llm", 16),
        Workload("llama8b_L32k", 32768, 32, 8, 128, "bf16", 128, 16, (0.85, 0.9, 0.95), 2, "llm", 32),
        Workload("llama8b_L128k", 131072, 32, 8, 128, "bf16", 128, 16, (0.9,), 3, "llm", 64),
        # One GPU's share of the 128K layer split by KV head over 8 GPUs: 4 query
        # heads and their one KV head at full length (same recipe and seed).
        Workload("llama8b_L128k_tp8_share", 131072, 4, 1, 128, "bf16", 128, 16, (0.9,), 3, "llm", 64),
        # Video-LMM-shaped layer: 28 query heads, 4 KV heads.
        Workload("video_L64k", 65536, 28, 4, 128, "bf16", 128, 16, (0.9,), 4, "video"),
    ]
}


def workload(name: str) -> Workload:
    """A named layer above, or any other shape as
    `shape:L,Hq,Hkv,d,B,S[,dtype[,kind[,seed]]]` (defaults bf16, the LLaMA-like
    recipe "llm" with one stripe key per 2,048 tokens (at least 8), seed 11;
    tau 0.9; causal)."""
    if name.startswith("shape:"):
        f = name[len("shape:"):].split(",")
        if len(f) < 6:
            raise ValueError("shape:L,Hq,Hkv,d,B,S[,dtype[,kind[,seed]]] expected, got %r" % name)
        L, Hq, Hkv, d, B, S = (int(x) for x in f[:6])
        dtype = f[6] if len(f) > 6 else "bf16"
        kind = f[7] if len(f) > 7 else "llm"
        seed = int(f[8]) if len(f) > 8 else 11
        return Workload(name, L, Hq, Hkv, d, dtype, B, S, (0.9,), seed, kind, max(8, L // 2048))
    return WORKLOADS[name]


def to_dtype(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "fp32":
        return t.clone()
    raise ValueError(dtype)


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def _tiny(w: Workload, rng):
    q = _normal(rng, (w.L, w.Hq, w.d))
    k = _normal(rng, (w.L, w.Hkv, w.d))
    v = _normal(rng, (w.L, w.Hkv, w.d))
    u = _normal(rng, (w.d,))
    u /= np.linalg.norm(u)
    pos = rng.choice(np.arange(1, w.L), w.n_stripes, replace=False)
    k[0] *= 4.0
    k[pos] += 2.0 * u
    q += u
    return q, k, v


def _llm(w: Workload, rng, alpha: float):
    L, d = w.L, w.d
    assert d >= 64
    rs = np.float32(1.0 / math.sqrt(d))
    q = _normal(rng, (L, w.Hq, d))
    q *= rs
    k = _normal(rng, (L, w.Hkv, d))
    k *= rs
    v = _normal(rng, (L, w.Hkv, d))
    v *= rs
    # two directions on dims 32..d-1, made orthonormal (Gram-Schmidt)
    dirs = _normal(rng, (2, d - 32)).astype(np.float64)
    u_s = dirs[0] / np.linalg.norm(dirs[0])
    u_t = dirs[1] - (dirs[1] @ u_s) * u_s
    u_t /= np.linalg.norm(u_t)
    stripes = rng.choice(np.arange(1, L), w.n_stripes, replace=False)
    beta_l, beta_s, beta_t = alpha * 1.0, alpha * 1.0, alpha * 0.75
    # local window: 16 sinusoid pairs with wavelengths from 2*pi to 2*pi*512
    M, W = 16, 512.0
    omega = W ** (np.arange(M) / (M - 1) - 1.0)
    a_l = math.sqrt(beta_l * math.sqrt(d) / M)
    ang = np.outer(np.arange(L, dtype=np.float64), omega)
    rope = np.empty((L, 2 * M), dtype=np.float32)
    rope[:, 0::2] = a_l * np.cos(ang)
    rope[:, 1::2] = a_l * np.sin(ang)
    del ang
    q[:, :, : 2 * M] += rope[:, None, :]
    k[:, :, : 2 * M] += rope[:, None, :]
    del rope
    # sink on key 0
    q[:, :, 32:] += u_s.astype(np.float32)
    k[0, :, 32:] += np.float32(beta_s * math.sqrt(d)) * u_s.astype(np.float32)
    # vertical stripes
    q[:, :, 32:] += u_t.astype(np.float32)
    k[stripes, :, 32:] += np.float32(beta_t * math.sqrt(d)) * u_t.astype(np.float32)
    return q, k, v


def video_split(L: int):
    """(frames, visual tokens, text tokens): 256-token frames then trailing text."""
    n_text0 = L // 64
    frames = (L - n_text0) // 256
    nv = frames * 256
    return frames, nv, L - nv


def _video(w: Workload, rng, beta: float):
    L, d = w.L, w.d
    frames, nv, _ = video_split(L)
    rs = np.float32(1.0 / math.sqrt(d))
    q = _normal(rng, (L, w.Hq, d))
    k = _normal(rng, (L, w.Hkv, d))
    v = _normal(rng, (L, w.Hkv, d))
    q[:nv] *= rs
    k[:nv] *= rs
    v[:nv] *= rs
    mu = np.float32(0.5) * _normal(rng, (frames, w.Hkv, d))
    k[:nv].reshape(frames, 256, w.Hkv, d)[...] += mu[:, None, :, :]
    emb = _normal(rng, (256, d))
    emb /= np.linalg.norm(emb, axis=1, keepdims=True)
    a_v = np.float32(math.sqrt(beta * math.sqrt(d)))
    band = a_v * emb
    q[:nv].reshape(frames, 256, w.Hq, d)[...] += band[None, :, None, :]
    k[:nv].reshape(frames, 256, w.Hkv, d)[...] += band[None, :, None, :]
    return q, k, v


def make_inputs_f32(w: Workload, amplitude: float | None = None):
    """Float32 numpy arrays (q, k, v) before the cast to the workload dtype."""
    rng = np.random.default_rng(w.seed)
    if w.kind == "tiny":
        return _tiny(w, rng)
    if w.kind == "llm":
        return _llm(w, rng, LLM_ALPHA if amplitude is None else amplitude)
    if w.kind == "video":
        return _video(w, rng, VIDEO_BETA if amplitude is None else amplitude)
    if w.kind == "gauss":
        return (_normal(rng, (w.L, w.Hq, w.d)), _normal(rng, (w.L, w.Hkv, w.d)),
                _normal(rng, (w.L, w.Hkv, w.d)))
    raise ValueError(w.kind)


def make_inputs(w: Workload, amplitude: float | None = None):
    """CPU torch tensors (q, k, v) in the workload dtype, layout [L][H][d]."""
    q, k, v = make_inputs_f32(w, amplitude)
    return to_dtype(q, w.dtype), to_dtype(k, w.dtype), to_dtype(v, w.dtype)
