"""Find the planted-structure amplitudes of the synthetic generator (run by hand).

For the 8B-shaped recipe the amplitude alpha scales the sink, local-window and
stripe logit boosts; for the video recipe beta scales the cross-frame patch
band. Each is chosen by bisection so that the oracle's Top-tau search on the
reference layer (32K tokens for the 8B shape, 64K for the video shape) at
tau = 0.9 keeps half of the causal blocks, the regime the RRAttention pages
report (about half of the blocks, abstract and TL;DR). The result is
written to generator_calibration.json; the constants in synthetic/gen.py are
the rounded values from that record.

Usage: python tests/golden/calibrate_generator.py
"""

import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from synthetic.gen import GENERATOR_VERSION, make_inputs, workload  # noqa: E402

TARGET, TOL = 0.50, 0.01


def keep_fraction(w, amp, tau):
    q, k, _ = make_inputs(w, amp)
    res = oracle.search(q, k, S=w.S, B=w.B, tau=tau, round_bf16=w.dtype == "bf16", extras=False)
    nb = w.nb
    return float(res.row_count.sum()) / (w.Hq * nb * (nb + 1) / 2)


def bisect(w, lo, hi, iters=10):
    log = []
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        f = keep_fraction(w, mid, 0.9)
        log.append((mid, f))
        print(f"{w.name} amplitude {mid:.4f} keep {f:.4f}", flush=True)
        if abs(f - TARGET) <= TOL:
            break
        if f > TARGET:  # more structure -> fewer blocks
            lo = mid
        else:
            hi = mid
    return mid, log


def main():
    rec = {"generator_version": GENERATOR_VERSION, "target_keep": TARGET, "tolerance": TOL, "tau": 0.9}
    t0 = time.time()
    w = workload("llama8b_L32k")
    a, log = bisect(w, 8.0, 14.0)
    a = round(a, 2)
    rec["llm_alpha"] = a
    rec["llm_log"] = log
    rec["llm_keep_at_taus"] = {str(t): keep_fraction(w, a, t) for t in w.taus}
    wv = workload("video_L64k")
    b, logv = bisect(wv, 48.0, 160.0)
    b = round(b, 1)
    rec["video_beta"] = b
    rec["video_log"] = logv
    rec["video_keep"] = keep_fraction(wv, b, 0.9)
    rec["seconds"] = time.time() - t0
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "generator_calibration.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
