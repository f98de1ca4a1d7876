"""Shared helpers of the GPU tests: run the library through its C ABI binding
and bring results back to the host for comparison with the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import dynamic_block_sparse_rr_amd as rr
from synthetic.gen import Workload, make_inputs
from synthetic.rows import sample_rows, work_item_rows  # noqa: F401


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_gpu(t):
    return t.contiguous().to("cuda")


def problem_of(w: Workload, tau: float) -> rr.Problem:
    return rr.problem(w.L, w.Hq, w.Hkv, w.d, w.S, w.B, tau, w.causal, w.dtype)


class DeviceCase:
    """Inputs of one workload resident on the GPU plus the library's workspace."""

    def __init__(self, w: Workload, tau: float, inputs=None):
        self.w = w
        self.tau = tau
        self.q, self.k, self.v = inputs if inputs is not None else make_inputs(w)
        self.qd, self.kd, self.vd = to_gpu(self.q), to_gpu(self.k), to_gpu(self.v)
        self.p = problem_of(w, tau)
        self.pre = rr.Prefill(self.p)

    def search(self, export_mass=True):
        nb = self.w.nb
        mass = torch.full((self.w.Hq, nb, nb), float("nan"), device="cuda") if export_mass else None
        self.pre.search(self.qd, self.kd, mass)
        torch.cuda.synchronize()
        rc = self.pre.row_count.cpu().numpy().copy()
        ci = self.pre.col_idx.cpu().numpy().copy()
        return rc, ci, (mass.cpu().numpy() if export_mass else None)

    def attention(self, row_count, col_idx):
        rc = torch.from_numpy(np.ascontiguousarray(row_count, np.int32)).cuda()
        ci = torch.from_numpy(np.ascontiguousarray(col_idx, np.int32)).cuda()
        self.pre.out.fill_(float("nan"))  # rows the kernel never writes stay NaN
        out = self.pre.attention(self.qd, self.kd, self.vd, rc, ci)
        torch.cuda.synchronize()
        return out.float().cpu().numpy()

    def recall(self, row_count, col_idx):
        """rr_mass_recall on the given lists: float [Hq][nb] on the host."""
        rc = torch.from_numpy(np.ascontiguousarray(row_count, np.int32)).cuda()
        ci = torch.from_numpy(np.ascontiguousarray(col_idx, np.int32)).cuda()
        out = torch.full((self.w.Hq, self.w.nb), float("nan"), device="cuda")
        rr.rr_mass_recall(self.p, self.qd, self.kd, rc, ci, out)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def prefill(self):
        out, rc, ci = self.pre(self.qd, self.kd, self.vd)
        torch.cuda.synchronize()
        return out.float().cpu().numpy(), rc.cpu().numpy().copy(), ci.cpu().numpy().copy()

