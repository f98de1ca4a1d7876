"""CPU oracle for RRAttention's prefill hot path -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
use this package. The GPU library neither imports nor links it, and the two
share no code. The arithmetic lives in ``rr_oracle.c`` (plain C, gcc); this
module only builds it and marshals numpy arrays.

Definition followed (the pages: "RRAttention: Dynamic Block Sparse Attention
via Per-Head Round-Robin Shifts for Long-Context Inference", abstract, TL;DR
and Figure 2 caption): stride-mean key pooling, head round-robin query
sampling at offset h mod S, stride-level softmax, block masses averaged over a
query block's samples, Top-tau cut on the (mass desc, index asc) order with the
last query block kept whole, then exact block-sparse attention. rr_oracle.c
states each step and the readings taken where the pages are silent.

Parity status: every function is pinned by tests/test_oracle_pins.py to an
independent float64 brute force, closed forms and library special cases; the
pages themselves print no worked numbers, so there is no pin to values printed
on the pages.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rr_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile rr_oracle.c with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("S", ctypes.c_int32), ("B", ctypes.c_int32),
                ("tau", ctypes.c_float), ("causal", ctypes.c_int32),
                ("round_bf16", ctypes.c_int32)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.rro_round_bf16.argtypes = [ctypes.c_float]
        lib.rro_round_bf16.restype = ctypes.c_float
        lib.rro_pool.argtypes = [ctypes.POINTER(_Problem), P, P]
        lib.rro_pool.restype = ctypes.c_int
        lib.rro_search.argtypes = [ctypes.POINTER(_Problem), P, P, P, P, P, P, P, P, P, P, P, P,
                                   ctypes.c_int]
        lib.rro_search.restype = ctypes.c_int
        lib.rro_attention.argtypes = [ctypes.POINTER(_Problem), P, P, P, P, P, P,
                                      ctypes.c_longlong, P, ctypes.c_int]
        lib.rro_attention.restype = ctypes.c_int
        lib.rro_recall.argtypes = [ctypes.POINTER(_Problem), P, P, P, P, P, ctypes.c_longlong, P,
                                   ctypes.c_int]
        lib.rro_recall.restype = ctypes.c_int
        lib.rro_decode.argtypes = [ctypes.POINTER(_Problem), P, P, P, P, P, P, P, ctypes.c_int]
        lib.rro_decode.restype = ctypes.c_int
        lib.rro_max_threads.argtypes = []
        lib.rro_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return _load().rro_max_threads()


def _f32(a) -> np.ndarray:
    """float32 contiguous numpy view of a numpy array or a CPU torch tensor."""
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").float().numpy()
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _problem(L, Hq, Hkv, d, S, B, tau, causal, round_bf16):
    return _Problem(L, Hq, Hkv, d, S, B, float(tau), int(bool(causal)), int(bool(round_bf16)))


def round_bf16(x: float) -> float:
    return _load().rro_round_bf16(float(x))


def pool(k, S: int, round_bf16: bool) -> np.ndarray:
    """Stride-mean pooled keys [L/S][Hkv][d] (float32 values)."""
    k = _f32(k)
    L, Hkv, d = k.shape
    out = np.empty((-(-L // S), Hkv, d), np.float32)
    p = _problem(L, Hkv, Hkv, d, S, S, 1.0, 1, round_bf16)
    rc = _load().rro_pool(ctypes.byref(p), _ptr(k), _ptr(out))
    if rc:
        raise ValueError("rro_pool failed (%d)" % rc)
    return out


@dataclass
class SearchResult:
    row_count: np.ndarray  # int32 [Hq][nb]
    col_idx: np.ndarray    # int32 [Hq][nb][nb], -1 padded
    mass: np.ndarray       # float32 [Hq][nb][nb]
    cminus: np.ndarray     # float32 [Hq][nb][nb]
    cplus: np.ndarray      # float32 [Hq][nb][nb]
    rank: np.ndarray       # int32 [Hq][nb][nb]
    total: np.ndarray      # float32 [Hq][nb]
    kbar: np.ndarray       # float32 [L/S][Hkv][d]

    def selected(self) -> np.ndarray:
        """Boolean block mask [Hq][nb][nb] from the lists."""
        Hq, nb = self.row_count.shape
        m = np.zeros((Hq, nb, nb), bool)
        for h in range(Hq):
            for i in range(nb):
                c = self.row_count[h, i]
                m[h, i, self.col_idx[h, i, :c]] = True
        return m


def search(q, k, *, S: int, B: int, tau: float, causal: bool = True, round_bf16: bool,
           nthreads: int = 0, extras: bool = True, row_mask=None, tau_per_head=None) -> SearchResult:
    """Round-robin pattern search with Top-tau selection (float32 arithmetic).

    row_mask: optional bool [Hq][nb]; only those rows are searched (the others
    get row_count 0), for spot checks of large layers.
    tau_per_head: optional [Hq] thresholds used in place of tau.
    L need not be a multiple of B or S: nb = ceil(L / B), and the last block
    and stride may be short.
    """
    q = _f32(q)
    k = _f32(k)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    nb = -(-L // B)
    p = _problem(L, Hq, Hkv, d, S, B, tau, causal, round_bf16)
    row_count = np.zeros((Hq, nb), np.int32)
    col_idx = np.zeros((Hq, nb, nb), np.int32)
    mass = np.zeros((Hq, nb, nb), np.float32)
    if extras:
        cminus = np.zeros((Hq, nb, nb), np.float32)
        cplus = np.zeros((Hq, nb, nb), np.float32)
        rank = np.zeros((Hq, nb, nb), np.int32)
        total = np.zeros((Hq, nb), np.float32)
        kbar = np.zeros((-(-L // S), Hkv, d), np.float32)
    else:
        cminus = cplus = rank = total = kbar = None
    rm = None if row_mask is None else np.ascontiguousarray(row_mask, dtype=np.uint8).reshape(Hq, nb)
    th = None if tau_per_head is None else np.ascontiguousarray(tau_per_head, dtype=np.float32).reshape(Hq)
    rc = _load().rro_search(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(row_count), _ptr(col_idx),
                            _ptr(mass), _ptr(cminus), _ptr(cplus), _ptr(rank), _ptr(total),
                            _ptr(kbar), _ptr(rm), _ptr(th), int(nthreads))
    if rc:
        raise ValueError("rro_search failed (%d)" % rc)
    return SearchResult(row_count, col_idx, mass, cminus, cplus, rank, total, kbar)


def attention(q, k, v, row_count, col_idx, *, B: int, causal: bool = True, rows=None,
              nthreads: int = 0) -> np.ndarray:
    """Block-sparse attention in float64.

    rows=None gives the full output [L][Hq][d]; otherwise rows is an int array
    of (x, h) pairs and the result is [len(rows)][d].
    """
    q = _f32(q)
    k = _f32(k)
    v = _f32(v)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    p = _problem(L, Hq, Hkv, d, 1, B, 1.0, causal, 0)
    rc_ = np.ascontiguousarray(row_count, np.int32)
    ci = np.ascontiguousarray(col_idx, np.int32)
    if rows is None:
        out = np.empty((L, Hq, d), np.float64)
        rp, n = None, 0
    else:
        rp = np.ascontiguousarray(rows, np.int32).reshape(-1, 2)
        n = rp.shape[0]
        out = np.empty((n, d), np.float64)
    rc = _load().rro_attention(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(rc_), _ptr(ci),
                               _ptr(rp), int(n), _ptr(out), int(nthreads))
    if rc == 3:
        raise ValueError("block lists are not ascending / in range / causal")
    if rc:
        raise ValueError("rro_attention failed (%d)" % rc)
    return out


def mass_recall(q, k, row_count, col_idx, *, B: int, causal: bool = True, rows=None,
                nthreads: int = 0) -> np.ndarray:
    """Full-attention softmax mass inside the selected blocks, float64.

    For each row (h, i): the mean over the B queries of query block i of the
    fraction of query x's full-attention softmax mass (over every admissible
    key) that falls on keys of the row's selected blocks. rows=None gives
    [Hq][nb]; otherwise rows is an int array of (h, i) pairs and the result is
    [len(rows)].
    """
    q = _f32(q)
    k = _f32(k)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    nb = -(-L // B)
    p = _problem(L, Hq, Hkv, d, 1, B, 1.0, causal, 0)
    rc_ = np.ascontiguousarray(row_count, np.int32)
    ci = np.ascontiguousarray(col_idx, np.int32)
    if rows is None:
        out = np.empty((Hq, nb), np.float64)
        rp, n = None, 0
    else:
        rp = np.ascontiguousarray(rows, np.int32).reshape(-1, 2)
        n = rp.shape[0]
        out = np.empty((n,), np.float64)
    rc = _load().rro_recall(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(rc_), _ptr(ci), _ptr(rp), int(n),
                            _ptr(out), int(nthreads))
    if rc == 3:
        raise ValueError("block lists are not ascending / in range / causal")
    if rc:
        raise ValueError("rro_recall failed (%d)" % rc)
    return out


def share_group_lists(row_count, col_idx, G: int):
    """Shared mask per KV head (a variant; the pages' masks are per query head).

    Row (h, i) of every head h of KV head g = h // G gets the ascending union of
    the blocks the G heads of g selected in row i. Returns (row_count,
    col_idx) in the same format, unused entries -1.
    """
    rc = np.asarray(row_count, np.int32)
    ci = np.asarray(col_idx, np.int32)
    Hq, nb = rc.shape
    out_rc = np.zeros_like(rc)
    out_ci = np.full_like(ci, -1)
    for g in range(Hq // G):
        for i in range(nb):
            u = set()
            for h in range(g * G, (g + 1) * G):
                u.update(int(j) for j in ci[h, i, : rc[h, i]])
            js = sorted(u)
            for h in range(g * G, (g + 1) * G):
                out_rc[h, i] = len(js)
                out_ci[h, i, : len(js)] = js
    return out_rc, out_ci


@dataclass
class DecodeResult:
    row_count: np.ndarray  # int32 [Hq]
    col_idx: np.ndarray    # int32 [Hq][nb], -1 padded
    mass: np.ndarray       # float32 [Hq][nb]
    out: np.ndarray        # float64 [Hq][d]


def decode(q, k, v, *, S: int, B: int, tau: float, round_bf16: bool, nthreads: int = 0) -> DecodeResult:
    """One decode step: the new query q [Hq][d] against the cache k, v [L][Hkv][d]
    (its own key and value at position L - 1). Block masses of the query's
    stride softmax, the Top-tau prefix plus the last block, then attention over
    the selected blocks in float64."""
    q = _f32(q)
    k = _f32(k)
    v = _f32(v)
    L, Hkv, d = k.shape
    Hq = q.shape[0]
    nb = -(-L // B)
    p = _problem(L, Hq, Hkv, d, S, B, tau, 1, round_bf16)
    rc = np.zeros((Hq,), np.int32)
    ci = np.zeros((Hq, nb), np.int32)
    mass = np.zeros((Hq, nb), np.float32)
    out = np.zeros((Hq, d), np.float64)
    st = _load().rro_decode(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(rc), _ptr(ci), _ptr(mass), _ptr(out),
                            int(nthreads))
    if st:
        raise ValueError("rro_decode failed (%d)" % st)
    return DecodeResult(rc, ci, mass, out)


def full_lists(L: int, Hq: int, B: int, causal: bool = True):
    """Lists that select every candidate block (the dense pattern)."""
    nb = -(-L // B)
    row_count = np.zeros((Hq, nb), np.int32)
    col_idx = np.full((Hq, nb, nb), -1, np.int32)
    for i in range(nb):
        n = i + 1 if causal else nb
        row_count[:, i] = n
        col_idx[:, i, :n] = np.arange(n)
    return row_count, col_idx
