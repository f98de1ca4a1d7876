"""Python binding of the MI355X (gfx950) RRAttention prefill library.

Thin ctypes marshalling over the C ABI in include/rr_attn.h: every entry point
has the same name and arguments as there, every step of the computation runs
in the library's HIP kernels. PyTorch is used only to own device memory and to
name the stream. There is no CPU fallback: if librr_attn.so is missing, or a
tensor is not on a GPU, the call raises.

Method: "RRAttention: Dynamic Block Sparse Attention via Per-Head Round-Robin
Shifts for Long-Context Inference" (abstract, TL;DR, Figure 2 caption).
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "Problem", "RRError", "load", "problem", "rr_workspace_bytes", "rr_pattern_search",
    "rr_block_sparse_attn", "rr_prefill", "rr_status_string", "rr_version", "Prefill",
    "RR_OK", "RR_ERR_INVALID_ARG", "RR_ERR_UNSUPPORTED", "RR_ERR_WORKSPACE", "RR_ERR_HIP",
    "RR_BF16", "RR_FP32", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librr_attn.so")

RR_OK, RR_ERR_INVALID_ARG, RR_ERR_UNSUPPORTED, RR_ERR_WORKSPACE, RR_ERR_HIP = 0, 1, 2, 3, 4
RR_BF16, RR_FP32 = 0, 1
_DTYPES = {"bf16": RR_BF16, "fp32": RR_FP32}


class Problem(ctypes.Structure):
    """Mirror of rr_problem."""

    _fields_ = [("L", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("S", ctypes.c_int32), ("B", ctypes.c_int32),
                ("tau", ctypes.c_float), ("causal", ctypes.c_int32), ("dtype", ctypes.c_int32)]

    @property
    def nb(self) -> int:
        return -(-self.L // self.B)  # the last block may be short

    @property
    def ns(self) -> int:
        return -(-self.L // self.S)  # the last stride may be short

    def __repr__(self):
        return ("Problem(L=%d, Hq=%d, Hkv=%d, d=%d, S=%d, B=%d, tau=%g, causal=%d, dtype=%d)"
                % (self.L, self.Hq, self.Hkv, self.d, self.S, self.B, self.tau, self.causal, self.dtype))


class RRError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (fn, rr_status_string(status), status))


_lib = None


def load():
    """Load librr_attn.so (built by python -m dynamic_block_sparse_rr_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("librr_attn.so is not built; run `python -m dynamic_block_sparse_rr_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        PP = ctypes.POINTER(Problem)
        lib.rr_workspace_bytes.argtypes = [PP]
        lib.rr_workspace_bytes.restype = ctypes.c_size_t
        lib.rr_pattern_search.argtypes = [PP, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.rr_pattern_search.restype = ctypes.c_int
        lib.rr_block_sparse_attn.argtypes = [PP, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.rr_block_sparse_attn.restype = ctypes.c_int
        lib.rr_prefill.argtypes = [PP, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.rr_prefill.restype = ctypes.c_int
        lib.rr_mass_recall.argtypes = [PP, P, P, P, P, P, P]
        lib.rr_mass_recall.restype = ctypes.c_int
        lib.rr_share_group_lists.argtypes = [PP, P, P, P, P, P]
        lib.rr_share_group_lists.restype = ctypes.c_int
        lib.rr_pattern_search_heads.argtypes = [PP, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.rr_pattern_search_heads.restype = ctypes.c_int
        lib.rr_workspace_bytes_varlen.argtypes = [PP, ctypes.c_int32, P]
        lib.rr_workspace_bytes_varlen.restype = ctypes.c_size_t
        lib.rr_prefill_varlen.argtypes = [PP, ctypes.c_int32, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.rr_prefill_varlen.restype = ctypes.c_int
        lib.rr_decode_workspace_bytes.argtypes = [PP]
        lib.rr_decode_workspace_bytes.restype = ctypes.c_size_t
        lib.rr_decode.argtypes = [PP, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.rr_decode.restype = ctypes.c_int
        lib.rr_decode_noalloc.argtypes = [PP, P, P, P, P, P, P, P, P, P]
        lib.rr_decode_noalloc.restype = ctypes.c_int
        lib.rr_decode_attend.argtypes = [PP, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.rr_decode_attend.restype = ctypes.c_int
        lib.rr_pool_keys.argtypes = [PP, P, P, P]
        lib.rr_pool_keys.restype = ctypes.c_int
        lib.rr_status_string.argtypes = [ctypes.c_int]
        lib.rr_status_string.restype = ctypes.c_char_p
        lib.rr_version.argtypes = []
        lib.rr_version.restype = ctypes.c_int32
        _lib = lib
    return _lib


def problem(L, Hq, Hkv, d, S, B, tau, causal=True, dtype="bf16") -> Problem:
    dt = _DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    return Problem(int(L), int(Hq), int(Hkv), int(d), int(S), int(B), float(tau), int(bool(causal)), dt)


def _ptr(x):
    """Device address of a GPU tensor, an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if not x.is_cuda:
            raise ValueError("tensor arguments must live on the GPU (got %s)" % x.device)
        if not x.is_contiguous():
            raise ValueError("tensor arguments must be contiguous")
        return x.data_ptr()
    raise TypeError("expected a GPU tensor, an int device pointer or None, got %r" % type(x))


def _nbytes(ws, ws_bytes):
    if hasattr(ws, "numel"):
        have = ws.numel() * ws.element_size()
        if ws_bytes is not None and int(ws_bytes) > have:
            raise ValueError("ws_bytes (%d) exceeds the workspace tensor (%d bytes)" % (int(ws_bytes), have))
        return have if ws_bytes is None else int(ws_bytes)
    return 0 if ws_bytes is None else int(ws_bytes)


def _dt(p):
    """torch dtype of the problem's tensors."""
    import torch

    return torch.bfloat16 if p.dtype == RR_BF16 else torch.float32


def _want(x, name, dtype, numel):
    """Check a tensor argument against what the problem needs before its
    address reaches the library (which cannot check sizes or types); ints
    (raw device addresses) and None pass through unchecked."""
    if x is None or isinstance(x, int) or not hasattr(x, "dtype"):
        return
    if dtype is not None and x.dtype != dtype:
        raise ValueError("%s: expected dtype %s, got %s" % (name, dtype, x.dtype))
    if x.numel() < numel:
        raise ValueError("%s: expected at least %d elements, got %d" % (name, numel, x.numel()))


def _check_qkv(p, q=None, k=None, v=None, out=None):
    dt = _dt(p)
    _want(q, "q", dt, p.L * p.Hq * p.d)
    _want(k, "k", dt, p.L * p.Hkv * p.d)
    _want(v, "v", dt, p.L * p.Hkv * p.d)
    _want(out, "out", dt, p.L * p.Hq * p.d)


def _check_lists(p, row_count, col_idx, prefix=""):
    import torch

    _want(row_count, prefix + "row_count", torch.int32, p.Hq * p.nb)
    _want(col_idx, prefix + "col_idx", torch.int32, p.Hq * p.nb * p.nb)


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, status):
    if status != RR_OK:
        raise RRError(fn, status)


def rr_workspace_bytes(p: Problem) -> int:
    return int(load().rr_workspace_bytes(ctypes.byref(p)))


def rr_pattern_search(p, q, k, row_count, col_idx, block_mass, ws, ws_bytes=None, stream=None):
    nws = _nbytes(ws, ws_bytes)
    import torch

    _check_qkv(p, q, k)
    _check_lists(p, row_count, col_idx)
    _want(block_mass, "block_mass", torch.float32, p.Hq * p.nb * p.nb)
    _check("rr_pattern_search", load().rr_pattern_search(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(row_count), _ptr(col_idx), _ptr(block_mass),
        _ptr(ws), nws, _stream(stream)))


def rr_block_sparse_attn(p, q, k, v, row_count, col_idx, out, ws, ws_bytes=None, stream=None):
    nws = _nbytes(ws, ws_bytes)
    _check_qkv(p, q, k, v, out)
    _check_lists(p, row_count, col_idx)
    _check("rr_block_sparse_attn", load().rr_block_sparse_attn(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(row_count), _ptr(col_idx), _ptr(out),
        _ptr(ws), nws, _stream(stream)))


def rr_prefill(p, q, k, v, out, row_count, col_idx, ws, ws_bytes=None, stream=None):
    nws = _nbytes(ws, ws_bytes)
    _check_qkv(p, q, k, v, out)
    _check_lists(p, row_count, col_idx)
    _check("rr_prefill", load().rr_prefill(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(row_count), _ptr(col_idx),
        _ptr(ws), nws, _stream(stream)))


def rr_mass_recall(p, q, k, row_count, col_idx, recall, stream=None):
    import torch

    _check_qkv(p, q, k)
    _check_lists(p, row_count, col_idx)
    _want(recall, "recall", torch.float32, p.Hq * p.nb)
    _check("rr_mass_recall", load().rr_mass_recall(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(row_count), _ptr(col_idx), _ptr(recall), _stream(stream)))


def rr_share_group_lists(p, row_count, col_idx, shared_row_count, shared_col_idx, stream=None):
    _check_lists(p, row_count, col_idx)
    _check_lists(p, shared_row_count, shared_col_idx, "shared_")
    _check("rr_share_group_lists", load().rr_share_group_lists(
        ctypes.byref(p), _ptr(row_count), _ptr(col_idx), _ptr(shared_row_count), _ptr(shared_col_idx),
        _stream(stream)))


def rr_pattern_search_heads(p, q, k, tau_per_head, row_count, col_idx, block_mass, ws, ws_bytes=None,
                            stream=None):
    nws = _nbytes(ws, ws_bytes)
    import torch

    _check_qkv(p, q, k)
    _check_lists(p, row_count, col_idx)
    _want(tau_per_head, "tau_per_head", torch.float32, p.Hq)
    _want(block_mass, "block_mass", torch.float32, p.Hq * p.nb * p.nb)
    _check("rr_pattern_search_heads", load().rr_pattern_search_heads(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(tau_per_head), _ptr(row_count), _ptr(col_idx), _ptr(block_mass),
        _ptr(ws), nws, _stream(stream)))


def _lens(seq_lens):
    import numpy as np

    a = np.ascontiguousarray(seq_lens, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def rr_workspace_bytes_varlen(p: Problem, seq_lens) -> int:
    a, ptr = _lens(seq_lens)
    return int(load().rr_workspace_bytes_varlen(ctypes.byref(p), int(a.size), ptr))


def rr_prefill_varlen(p, seq_lens, q, k, v, out, row_count, col_idx, ws, ws_bytes=None, stream=None):
    nws = _nbytes(ws, ws_bytes)
    import torch

    a, ptr = _lens(seq_lens)
    _check_qkv(p, q, k, v, out)
    nbs = [-(-int(n) // p.B) for n in a]
    _want(row_count, "row_count", torch.int32, sum(p.Hq * n for n in nbs))
    _want(col_idx, "col_idx", torch.int32, sum(p.Hq * n * n for n in nbs))
    _check("rr_prefill_varlen", load().rr_prefill_varlen(
        ctypes.byref(p), int(a.size), ptr, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(row_count), _ptr(col_idx),
        _ptr(ws), nws, _stream(stream)))


def rr_decode_workspace_bytes(p: Problem) -> int:
    return int(load().rr_decode_workspace_bytes(ctypes.byref(p)))


def _check_decode(p, q, k, v, out, row_count, col_idx, block_mass=None, kbar=None):
    import torch

    dt = _dt(p)
    _want(q, "q", dt, p.Hq * p.d)
    _want(k, "k", dt, p.L * p.Hkv * p.d)
    _want(v, "v", dt, p.L * p.Hkv * p.d)
    _want(kbar, "kbar", dt, p.ns * p.Hkv * p.d)
    _want(out, "out", dt, p.Hq * p.d)
    _want(row_count, "row_count", torch.int32, p.Hq)
    _want(col_idx, "col_idx", torch.int32, p.Hq * p.nb)
    _want(block_mass, "block_mass", torch.float32, p.Hq * p.nb)


def rr_decode(p, q, k, v, out, row_count, col_idx, block_mass, ws, ws_bytes=None, stream=None, kbar=None):
    nws = _nbytes(ws, ws_bytes)
    _check_decode(p, q, k, v, out, row_count, col_idx, block_mass, kbar)
    _check("rr_decode", load().rr_decode(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(kbar), _ptr(out), _ptr(row_count), _ptr(col_idx),
        _ptr(block_mass), _ptr(ws), nws, _stream(stream)))


RR_DECODE_NOALLOC_MAX_WS = 32 << 20  # bytes of the library's own decode workspace per GPU


def rr_decode_noalloc(p, q, k, v, out, row_count, col_idx, block_mass=None, stream=None, kbar=None):
    """rr_decode with the library's own workspace: allocates nothing."""
    _check_decode(p, q, k, v, out, row_count, col_idx, block_mass, kbar)
    _check("rr_decode_noalloc", load().rr_decode_noalloc(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(kbar), _ptr(out), _ptr(row_count), _ptr(col_idx),
        _ptr(block_mass), _stream(stream)))


def rr_decode_attend(p, q, k, v, row_count, col_idx, out, ws, ws_bytes=None, stream=None):
    nws = _nbytes(ws, ws_bytes)
    _check_decode(p, q, k, v, out, row_count, col_idx)
    _check("rr_decode_attend", load().rr_decode_attend(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(row_count), _ptr(col_idx), _ptr(out), _ptr(ws),
        nws, _stream(stream)))


def rr_pool_keys(p, k, kbar, stream=None):
    dt = _dt(p)
    _want(k, "k", dt, p.L * p.Hkv * p.d)
    _want(kbar, "kbar", dt, p.ns * p.Hkv * p.d)
    _check("rr_pool_keys", load().rr_pool_keys(ctypes.byref(p), _ptr(k), _ptr(kbar), _stream(stream)))


def rr_status_string(status: int) -> str:
    return load().rr_status_string(int(status)).decode()


def rr_version() -> int:
    return int(load().rr_version())


class Prefill:
    """Owns the device workspace and outputs for one problem shape (torch allocations)."""

    def __init__(self, p: Problem, device="cuda"):
        import torch

        self.p = p
        self.device = torch.device(device)
        n = rr_workspace_bytes(p)
        if n == 0:
            raise RRError("rr_workspace_bytes", RR_ERR_UNSUPPORTED)
        self.ws = torch.empty(n, dtype=torch.uint8, device=self.device)
        nb = p.nb
        self.row_count = torch.empty((p.Hq, nb), dtype=torch.int32, device=self.device)
        self.col_idx = torch.empty((p.Hq, nb, nb), dtype=torch.int32, device=self.device)
        tdt = torch.bfloat16 if p.dtype == RR_BF16 else torch.float32
        self.out = torch.empty((p.L, p.Hq, p.d), dtype=tdt, device=self.device)

    def search(self, q, k, block_mass=None):
        rr_pattern_search(self.p, q, k, self.row_count, self.col_idx, block_mass, self.ws)
        return self.row_count, self.col_idx

    def attention(self, q, k, v, row_count=None, col_idx=None):
        rc = self.row_count if row_count is None else row_count
        ci = self.col_idx if col_idx is None else col_idx
        rr_block_sparse_attn(self.p, q, k, v, rc, ci, self.out, self.ws)
        return self.out

    def __call__(self, q, k, v):
        rr_prefill(self.p, q, k, v, self.out, self.row_count, self.col_idx, self.ws)
        return self.out, self.row_count, self.col_idx
