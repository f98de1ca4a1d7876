"""Compile the gfx950 HIP library librr_attn.so in-tree with hipcc.

Usage: python -m dynamic_block_sparse_rr_amd.build
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "librr_attn.so")
SOURCES = ["rr_host.cpp", "search.hip", "attn.hip", "recall.hip", "decode.hip", "static_ws.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=" + ARCH,
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    """Always recompile (the caller wants a fresh build check)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed with status %d" % r.returncode)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
