"""Comparison of GPU block lists and outputs with the oracle.

Mask classes per searched row (h, i < nb-1):
  exact       same set of key blocks;
  letter      every mismatched block has a cumulative mass (before or
              including it, in the oracle's order, relative to the row total)
              within 1e-4 of tau -- such blocks sit on the cut, where float32
              summation order alone may move them;
  near_tie    otherwise, every remaining mismatched block has an oracle mass
              within 1e-5 (relative) of the oracle's last kept block, and the
              GPU's set still holds at least (tau - 1e-4) of the row's oracle
              mass: a valid Top-tau set under an ordering float32 cannot resolve;
  fail        anything else.
The unsearched last row must list every candidate block exactly.
"""

from __future__ import annotations

import numpy as np

LETTER_TOL = 1e-4
TIE_REL = 1e-5


def gpu_sets(row_count: np.ndarray, col_idx: np.ndarray, h: int, i: int) -> np.ndarray:
    return col_idx[h, i, : row_count[h, i]]


def classify(gpu_rc, gpu_ci, orc, tau: float, causal: bool = True, rows=None) -> dict:
    gpu_rc = np.asarray(gpu_rc)
    gpu_ci = np.asarray(gpu_ci)
    Hq, nb = gpu_rc.shape
    out = {"exact": 0, "letter": 0, "near_tie": 0, "fail": 0, "fail_rows": [], "list_errors": 0}
    it = rows if rows is not None else [(h, i) for h in range(Hq) for i in range(nb)]
    for h, i in it:
        ncand = i + 1 if causal else nb
        g = gpu_sets(gpu_rc, gpu_ci, h, i)
        if len(g) == 0 or np.any(np.diff(g) <= 0) or g.min() < 0 or g.max() >= ncand:
            out["list_errors"] += 1
            out["fail"] += 1
            out["fail_rows"].append((h, i, "bad list"))
            continue
        if i == nb - 1 or tau >= 1.0:
            if len(g) == ncand:
                out["exact"] += 1
            else:
                out["fail"] += 1
                out["fail_rows"].append((h, i, "not full"))
            continue
        o = orc.col_idx[h, i, : orc.row_count[h, i]]
        gs, os_ = set(g.tolist()), set(o.tolist())
        if gs == os_:
            out["exact"] += 1
            continue
        T = float(orc.total[h, i])
        m = orc.mass[h, i].astype(np.float64)
        m_cut = float(m[o].min())
        cls = "letter"
        for j in gs ^ os_:
            cm = float(orc.cminus[h, i, j]) / T
            cp = float(orc.cplus[h, i, j]) / T
            if abs(cm - tau) <= LETTER_TOL or abs(cp - tau) <= LETTER_TOL:
                continue
            if abs(m[j] - m_cut) <= TIE_REL * m_cut and m[list(gs)].sum() >= (tau - LETTER_TOL) * T:
                cls = "near_tie" if cls != "fail" else cls
                continue
            cls = "fail"
        out[cls] += 1
        if cls == "fail":
            out["fail_rows"].append((h, i, sorted(gs ^ os_)))
    return out


def output_errors(got: np.ndarray, want: np.ndarray) -> tuple[float, float]:
    d = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))
    return float(d.max()), float(d.mean())
