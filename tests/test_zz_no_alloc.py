"""rr_decode_noalloc (the decode step on the library's own device buffer, for
callers that cannot allocate) against rr_decode on a caller-owned workspace.

Two calls in a row on one process and stream, the second on a smaller cache,
each compared with rr_decode on the same inputs: block lists and block masses
must be identical (same kernels, same order of arithmetic), outputs within
the bf16 bar (max-abs 2e-2, mean-abs 2e-3; identical in practice). The first
call pools the cache's keys inside the call (the pooled keys then live in the
library's buffer too), the second takes them from the caller.
"""

import numpy as np
import pytest
import torch

import dynamic_block_sparse_rr_amd as rr
from synthetic.gen import Workload, make_inputs
from tests.gpu_cases import say

pytestmark = pytest.mark.gpu


def decode_both(L, seed, pooled):
    w = Workload("noalloc_decode_L%d" % L, L, 32, 8, 128, "bf16", 128, 16, (0.9,), seed, "llm", 16)
    Q, K, V = make_inputs(w)
    q = Q[L - 1].contiguous().cuda()
    k, v = K.cuda(), V.cuda()
    del Q
    p = rr.problem(L, 32, 8, 128, 16, 128, 0.9, True, "bf16")
    assert rr.rr_decode_workspace_bytes(p) <= rr.RR_DECODE_NOALLOC_MAX_WS
    kbar = None
    if pooled:
        kbar = torch.empty((p.ns, 8, 128), dtype=k.dtype, device="cuda")
        rr.rr_pool_keys(p, k, kbar)
    res = {}
    for mode in ("noalloc", "caller_ws"):
        out = torch.full_like(q, float("nan"))
        rc = torch.full((32,), -1, dtype=torch.int32, device="cuda")
        ci = torch.full((32, p.nb), -1, dtype=torch.int32, device="cuda")
        mass = torch.full((32, p.nb), float("nan"), dtype=torch.float32, device="cuda")
        if mode == "noalloc":
            rr.rr_decode_noalloc(p, q, k, v, out, rc, ci, mass, kbar=kbar)
        else:
            ws = torch.empty(rr.rr_decode_workspace_bytes(p), dtype=torch.uint8, device="cuda")
            rr.rr_decode(p, q, k, v, out, rc, ci, mass, ws, kbar=kbar)
        torch.cuda.synchronize()
        res[mode] = (out.float().cpu().numpy(), rc.cpu().numpy(), ci.cpu().numpy(), mass.cpu().numpy())
    return res


@pytest.mark.parametrize("L,seed,pooled", [(32768, 51, False), (8000, 52, True)])
def test_noalloc_decode_matches_caller_workspace(L, seed, pooled):
    say(f"case noalloc decode L={L} pooled_keys_given={pooled}")
    r = decode_both(L, seed, pooled)
    (o1, rc1, ci1, m1), (o2, rc2, ci2, m2) = r["noalloc"], r["caller_ws"]
    np.testing.assert_array_equal(rc1, rc2)
    for h in range(rc1.shape[0]):
        np.testing.assert_array_equal(ci1[h, : rc1[h]], ci2[h, : rc2[h]])
    np.testing.assert_array_equal(m1, m2)
    assert np.isfinite(o1).all()
    d = np.abs(o1.astype(np.float64) - o2)
    say(f"  lists equal, masses equal, output max-abs {d.max():.3e} mean-abs {d.mean():.3e}")
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
