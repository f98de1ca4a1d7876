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


# Extra flags per source. search.hip: its scoring kernel reads every MFMA
# result on the VALU (the softmax), so the accumulators stay in VGPRs rather
# than AGPRs (no v_accvgpr_read per score).
EXTRA_FLAGS = {"search.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False) -> str:
    """Always recompile (the caller wants a fresh build check): every source to
    an object (in parallel), then one link."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmd = [hipcc(), *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), *inc, "-c", os.path.join(CSRC, src), "-o", obj]
        cmd = [c for c in cmd if c != "-shared"]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    objs = []
    for src, obj, pr in procs:
        out, _ = pr.communicate()
        if pr.returncode != 0:
            sys.stderr.write(out)
            raise RuntimeError("hipcc failed with status %d (%s)" % (pr.returncode, src))
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc link failed with status %d" % r.returncode)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
