"""Disk cache of oracle search results for the large workload layers.

The full oracle search of the 128K-token layer takes about a minute on 16
host threads; its result depends only on the workload's inputs (name, seed,
generator version), the threshold and the oracle's own source, so it is
stored once per machine and reused by later runs. The key holds all of them:
a changed oracle or generator recomputes. Location: $RR_ORACLE_CACHE, else
~/.cache/rr_oracle, else the temporary directory.
"""

from __future__ import annotations

import hashlib
import os
import tempfile

import numpy as np

import oracle
from synthetic.gen import GENERATOR_VERSION

_FIELDS = ("row_count", "col_idx", "mass", "cminus", "cplus", "rank", "total", "kbar")


def _oracle_sha() -> str:
    src = os.path.join(os.path.dirname(os.path.abspath(oracle.__file__)), "rr_oracle.c")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def cache_dir() -> str:
    d = os.environ.get("RR_ORACLE_CACHE")
    if not d:
        home = os.path.expanduser("~")
        d = os.path.join(home, ".cache", "rr_oracle") if os.access(home, os.W_OK) else ""
    if not d:
        d = os.path.join(tempfile.gettempdir(), "rr_oracle")
    os.makedirs(d, exist_ok=True)
    return d


def key(w, tau: float) -> str:
    return "%s_L%d_seed%d_gen%d_tau%.6f_oracle%s" % (w.name, w.L, w.seed, GENERATOR_VERSION, tau, _oracle_sha())


def search(w, tau: float, q, k, say=None) -> oracle.SearchResult:
    """oracle.search on the workload's own inputs (q, k), through the cache."""
    path = os.path.join(cache_dir(), key(w, tau) + ".npz")
    if os.path.exists(path):
        with np.load(path, allow_pickle=False) as z:
            res = oracle.SearchResult(*(z[f] for f in _FIELDS))
        if say:
            say(f"  oracle search from cache {os.path.basename(path)}")
        return res
    if say:
        say(f"  oracle search on {oracle.max_threads()} host threads ...")
    res = oracle.search(q, k, S=w.S, B=w.B, tau=tau, causal=w.causal, round_bf16=w.dtype == "bf16")
    tmp = path + ".tmp%d.npz" % os.getpid()
    try:
        np.savez(tmp, **{f: getattr(res, f) for f in _FIELDS})
        os.replace(tmp, path)
    except OSError:
        if os.path.exists(tmp):
            os.remove(tmp)
    return res
