"""Seeded synthetic attention inputs shaped like the workloads of the RRAttention pages.

This module holds only random-number recipes and the workload table. It computes
nothing of the method itself (no pooling, scoring, softmax or selection), so the
GPU path and the oracle can both draw their inputs from it without sharing any
of the method's arithmetic.
"""

from .gen import WORKLOADS, Workload, make_inputs, workload, to_dtype  # noqa: F401
