"""The C-ABI library on the CPU: it loads, exports what include/rr_attn.h
declares, and rejects invalid arguments on the host before any HIP call (so no
device is needed). No compute call is made here."""

import ctypes
import os
import re

import pytest

import dynamic_block_sparse_rr_amd as rr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(rr.LIB_PATH), reason="librr_attn.so not built")


def declared_functions():
    src = open(os.path.join(ROOT, "include", "rr_attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rr_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert names == sorted(["rr_workspace_bytes", "rr_pattern_search", "rr_block_sparse_attn",
                            "rr_prefill", "rr_mass_recall", "rr_share_group_lists", "rr_status_string",
                            "rr_version", "rr_pattern_search_heads", "rr_workspace_bytes_varlen",
                            "rr_prefill_varlen", "rr_decode_workspace_bytes", "rr_decode", "rr_decode_attend", "rr_pool_keys",
                            "rr_decode_noalloc"])
    lib = ctypes.CDLL(rr.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert rr.rr_version() >= 100
    for s in range(5):
        assert rr.rr_status_string(s)
    assert rr.rr_status_string(99) == "unknown status"


def base(**kw):
    args = dict(L=16384, Hq=32, Hkv=8, d=128, S=16, B=128, tau=0.9, causal=1, dtype=rr.RR_BF16)
    args.update(kw)
    return rr.Problem(**args)


def test_workspace_bytes():
    p = base()
    n = rr.rr_workspace_bytes(p)
    ns, nb = 16384 // 16, 16384 // 128
    # pooled keys + block masses + key-major V copy + work-queue counters, each 256-byte aligned
    assert n == ns * 8 * 128 * 2 + 32 * nb * nb * 4 + 16384 * 8 * 128 * 2 + 256
    assert rr.rr_workspace_bytes(base(dtype=rr.RR_FP32)) == ns * 8 * 128 * 4 + 32 * nb * nb * 4
    # a ragged length: ceil(L / B) blocks, ceil(L / S) strides, V copy padded to whole blocks
    n = rr.rr_workspace_bytes(base(L=1000))
    al = lambda x: -(-x // 256) * 256
    assert n == al(63 * 8 * 128 * 2) + al(32 * 8 * 8 * 4) + al(8 * 128 * 8 * 128 * 2) + 256

@pytest.mark.parametrize("kw,status", [
    (dict(L=0), rr.RR_ERR_INVALID_ARG),
    (dict(Hq=30), rr.RR_ERR_INVALID_ARG),           # not a multiple of Hkv
    (dict(S=48), rr.RR_ERR_INVALID_ARG),            # B not a multiple of S
    (dict(S=48), rr.RR_ERR_INVALID_ARG),            # B not a multiple of S
    (dict(tau=0.0), rr.RR_ERR_INVALID_ARG),
    (dict(tau=1.5), rr.RR_ERR_INVALID_ARG),
    (dict(tau=float("nan")), rr.RR_ERR_INVALID_ARG),
    (dict(causal=2), rr.RR_ERR_INVALID_ARG),
    (dict(dtype=7), rr.RR_ERR_INVALID_ARG),
    (dict(d=96), rr.RR_ERR_UNSUPPORTED),
    (dict(B=256, S=16), rr.RR_ERR_UNSUPPORTED),
    (dict(S=128), rr.RR_ERR_UNSUPPORTED),           # r = 1
    (dict(S=2), rr.RR_ERR_UNSUPPORTED),             # r = 64
    (dict(L=128 * 9000), rr.RR_ERR_UNSUPPORTED),    # nb above the select kernel's LDS capacity
])
def test_invalid_problems_rejected_on_host(kw, status):
    p = base(**kw)
    assert rr.rr_workspace_bytes(p) == 0
    lib = rr.load()
    fake = 1 << 20  # never dereferenced: validation fails first
    rc = lib.rr_pattern_search(ctypes.byref(p), fake, fake, fake, fake, None, fake, 1 << 40, 0)
    assert rc == status
    rc = lib.rr_block_sparse_attn(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, 1 << 40, 0)
    assert rc == status
    rc = lib.rr_prefill(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, 1 << 40, 0)
    assert rc == status
    rc = lib.rr_mass_recall(ctypes.byref(p), fake, fake, fake, fake, fake, 0)
    assert rc == status
    rc = lib.rr_share_group_lists(ctypes.byref(p), fake, fake, fake << 4, fake << 5, 0)
    assert rc == status


def test_pointer_and_workspace_checks():
    p = base()
    lib = rr.load()
    ok = 1 << 20
    need = rr.rr_workspace_bytes(p)
    # null input
    assert lib.rr_pattern_search(ctypes.byref(p), None, ok, ok, ok, None, ok, need, 0) == rr.RR_ERR_INVALID_ARG
    # misaligned input
    assert lib.rr_block_sparse_attn(ctypes.byref(p), ok + 2, ok, ok, ok, ok, ok, ok, need, 0) == rr.RR_ERR_INVALID_ARG
    # workspace missing / too small / misaligned
    assert lib.rr_prefill(ctypes.byref(p), ok, ok, ok, ok, ok, ok, None, need, 0) == rr.RR_ERR_WORKSPACE
    assert lib.rr_prefill(ctypes.byref(p), ok, ok, ok, ok, ok, ok, ok, need - 1, 0) == rr.RR_ERR_WORKSPACE
    assert lib.rr_pattern_search(ctypes.byref(p), ok, ok, ok, ok, None, ok + 8, need, 0) == rr.RR_ERR_WORKSPACE
    assert lib.rr_workspace_bytes(None) == 0
    # the recall harness: null / misaligned arguments, null problem
    assert lib.rr_mass_recall(ctypes.byref(p), ok, ok, ok, ok, None, 0) == rr.RR_ERR_INVALID_ARG
    assert lib.rr_mass_recall(ctypes.byref(p), ok, ok + 4, ok, ok, ok, 0) == rr.RR_ERR_INVALID_ARG
    assert lib.rr_mass_recall(None, ok, ok, ok, ok, ok, 0) == rr.RR_ERR_INVALID_ARG
    # shared lists: null, misaligned, and outputs overlapping the inputs
    far = 1 << 40
    assert lib.rr_share_group_lists(ctypes.byref(p), ok, ok, None, far, 0) == rr.RR_ERR_INVALID_ARG
    assert lib.rr_share_group_lists(ctypes.byref(p), ok, ok + 4, far, far << 1, 0) == rr.RR_ERR_INVALID_ARG
    assert lib.rr_share_group_lists(ctypes.byref(p), ok, far, ok + 1024, far << 1, 0) == rr.RR_ERR_INVALID_ARG
    assert lib.rr_share_group_lists(ctypes.byref(p), ok, far, far << 1, far + 4096, 0) == rr.RR_ERR_INVALID_ARG


def test_binding_refuses_cpu_tensors():
    import torch

    p = base(L=256, Hq=2, Hkv=1)
    q = torch.zeros((256, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        rr.rr_pattern_search(p, q, q, q, q, None, q, stream=0)


def test_varlen_and_per_head_checks_on_host():
    lib = rr.load()
    ok = 1 << 20
    p = base(L=300 + 1000 + 128)
    lens = (ctypes.c_int32 * 3)(300, 1000, 128)
    need = lib.rr_workspace_bytes_varlen(ctypes.byref(p), 3, lens)
    # the batched search holds every sequence's pooled keys and masses at once; the one attention launch
    # needs every sequence's V re-layout, then the queue counters
    al = lambda x: -(-x // 256) * 256
    vt = lambda L: al(-(-L // 128) * 128 * 8 * 128 * 2)
    srch = lambda L: al(-(-L // 16) * 8 * 128 * 2) + al(32 * (-(-L // 128)) ** 2 * 4)
    assert need == srch(300) + srch(1000) + srch(128) + vt(300) + vt(1000) + vt(128) + 256
    # fp32 (one attention launch per sequence): the largest single sequence decides
    pf = base(L=300 + 1000 + 128, dtype=rr.RR_FP32)
    assert lib.rr_workspace_bytes_varlen(ctypes.byref(pf), 3, lens) == rr.rr_workspace_bytes(base(L=1000, dtype=rr.RR_FP32))
    # lengths must add up to p->L, be positive, and be given
    bad = base(L=1427)
    assert lib.rr_workspace_bytes_varlen(ctypes.byref(bad), 3, lens) == 0
    assert lib.rr_prefill_varlen(ctypes.byref(bad), 3, lens, ok, ok, ok, ok, ok, ok, ok, need, 0) == rr.RR_ERR_INVALID_ARG
    zero = (ctypes.c_int32 * 2)(0, 1428)
    assert lib.rr_prefill_varlen(ctypes.byref(p), 2, zero, ok, ok, ok, ok, ok, ok, ok, need, 0) == rr.RR_ERR_INVALID_ARG
    assert lib.rr_prefill_varlen(ctypes.byref(p), 3, None, ok, ok, ok, ok, ok, ok, ok, need, 0) == rr.RR_ERR_INVALID_ARG
    assert lib.rr_prefill_varlen(ctypes.byref(p), 3, lens, ok, ok, ok, ok, ok, ok, ok, need - 1, 0) == rr.RR_ERR_WORKSPACE
    assert rr.rr_workspace_bytes_varlen(p, [300, 1000, 128]) == need
    # the next sequence's lists would start misaligned: Hq * nb * 4 bytes is not a multiple of 16
    small = rr.Problem(128, 2, 2, 64, 8, 64, 0.9, 1, rr.RR_BF16)
    two = (ctypes.c_int32 * 2)(64, 64)
    w2 = lib.rr_workspace_bytes_varlen(ctypes.byref(small), 2, two)
    assert w2 > 0
    assert lib.rr_prefill_varlen(ctypes.byref(small), 2, two, ok, ok, ok, ok, ok, ok, ok, w2, 0) == rr.RR_ERR_UNSUPPORTED
    # per-head thresholds: null array, misaligned array
    q = base()
    w = rr.rr_workspace_bytes(q)
    assert lib.rr_pattern_search_heads(ctypes.byref(q), ok, ok, None, ok, ok, None, ok, w, 0) == rr.RR_ERR_INVALID_ARG
    assert lib.rr_pattern_search_heads(ctypes.byref(q), ok, ok, ok + 2, ok, ok, None, ok, w, 0) == rr.RR_ERR_INVALID_ARG


def test_decode_checks_on_host():
    lib = rr.load()
    ok = 1 << 20
    p = base(L=131072)
    need = rr.rr_decode_workspace_bytes(p)
    al = lambda x: -(-x // 256) * 256
    ns, nb = 131072 // 16, 131072 // 128
    # pooled keys | block sums [Hq][nb] | chunk partials [Hq][ns/256][2] | masses [Hq][nb] | flags [Hq][nb] bytes |
    # split partials [Hq][nb/16][d+2] (16 blocks per workgroup: about 512 workgroups over nb * Hkv blocks)
    assert need == (al(ns * 8 * 128 * 2) + al(32 * nb * 4) + al(32 * (ns // 256) * 2 * 4) + al(32 * nb * 4)
                    + al(32 * nb) + al(32 * (nb // 16) * 130 * 4))
    assert lib.rr_decode(ctypes.byref(p), None, ok, ok, None, ok, ok, ok, None, ok, need, 0) == rr.RR_ERR_INVALID_ARG
    assert lib.rr_decode(ctypes.byref(p), ok, ok, ok, None, ok + 2, ok, ok, None, ok, need, 0) == rr.RR_ERR_INVALID_ARG
    assert lib.rr_decode(ctypes.byref(p), ok, ok, ok, ok + 8, ok, ok, ok, None, ok, need, 0) == rr.RR_ERR_INVALID_ARG
    assert lib.rr_decode(ctypes.byref(p), ok, ok, ok, None, ok, ok, ok, None, ok, need - 1, 0) == rr.RR_ERR_WORKSPACE
    assert lib.rr_decode(ctypes.byref(base(d=96)), ok, ok, ok, None, ok, ok, ok, None, ok, need, 0) == rr.RR_ERR_UNSUPPORTED
    assert lib.rr_decode_attend(ctypes.byref(p), ok, ok, ok, None, ok, ok, ok, need, 0) == rr.RR_ERR_INVALID_ARG
    assert lib.rr_decode_attend(ctypes.byref(p), ok, ok, ok, ok, ok + 4, ok, ok, need, 0) == rr.RR_ERR_INVALID_ARG
    assert lib.rr_decode_attend(ctypes.byref(p), ok, ok, ok, ok, ok, ok, ok, need - 1, 0) == rr.RR_ERR_WORKSPACE
    assert lib.rr_pool_keys(ctypes.byref(p), ok, None, 0) == rr.RR_ERR_INVALID_ARG
    assert lib.rr_pool_keys(ctypes.byref(base(S=48)), ok, ok, 0) == rr.RR_ERR_INVALID_ARG
    assert lib.rr_decode_workspace_bytes(None) == 0


class _NoLibrary:
    """Stands in for the loaded library: any use of it fails the test."""

    def __getattr__(self, name):
        raise AssertionError("the call reached the library (%s)" % name)


def test_binding_checks_tensors_before_the_library(monkeypatch):
    import torch

    monkeypatch.setattr(rr, "_lib", _NoLibrary())
    p = base(L=256, Hq=4, Hkv=2)
    bf = lambda *s: torch.zeros(s, dtype=torch.bfloat16)
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32)
    q, k, v, out = bf(256, 4, 128), bf(256, 2, 128), bf(256, 2, 128), bf(256, 4, 128)
    rc, ci = i32(4, 2), i32(4, 2, 2)
    ws = torch.zeros(16, dtype=torch.uint8)
    cases = [
        (lambda: rr.rr_pattern_search(p, q.float(), k, rc, ci, None, ws), "q: expected dtype"),
        (lambda: rr.rr_pattern_search(p, q, k[:100], rc, ci, None, ws), "k: expected at least"),
        (lambda: rr.rr_pattern_search(p, q, k, rc.long(), ci, None, ws), "row_count: expected dtype"),
        (lambda: rr.rr_pattern_search(p, q, k, rc, ci, bf(4, 2, 2), ws), "block_mass: expected dtype"),
        (lambda: rr.rr_block_sparse_attn(p, q, k, v, rc, ci[:1], out, ws), "col_idx: expected at least"),
        (lambda: rr.rr_block_sparse_attn(p, q, k, v, rc, ci, out[:10], ws), "out: expected at least"),
        (lambda: rr.rr_prefill(p, q, k, v.float(), out, rc, ci, ws), "v: expected dtype"),
        (lambda: rr.rr_mass_recall(p, q, k, rc, ci, torch.zeros(3)), "recall: expected at least"),
        (lambda: rr.rr_share_group_lists(p, rc, ci, rc, i32(3)), "shared_col_idx: expected at least"),
        (lambda: rr.rr_pattern_search_heads(p, q, k, torch.zeros(2), rc, ci, None, ws), "tau_per_head"),
        (lambda: rr.rr_prefill_varlen(p, [128, 128], q, k, v, out, i32(7), ci, ws), "row_count: expected at least"),
        (lambda: rr.rr_decode(p, bf(3, 128), k, v, bf(4, 128), i32(4), i32(4, 2), None, ws), "q: expected at least"),
        (lambda: rr.rr_decode_attend(p, bf(4, 128), k, v, i32(4), i32(4, 2), bf(4, 128).float(), ws),
         "out: expected dtype"),
        (lambda: rr.rr_pool_keys(p, k, bf(3, 2, 128)), "kbar: expected at least"),
        (lambda: rr.rr_pattern_search(p, q, k, rc, ci, None, ws, ws_bytes=17), "ws_bytes"),
    ]
    for call, msg in cases:
        with pytest.raises(ValueError, match=msg):
            call()


def test_valid_calls_without_a_device_return_hip_error():
    """Arguments that pass every host check reach the HIP runtime, which has
    no device here: the library returns RR_ERR_HIP instead of crashing. The
    addresses are fake, so this runs only where no GPU is visible."""
    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: fake device addresses must not reach a kernel")
    lib = rr.load()
    ok = 1 << 20
    p = base(L=1024, Hq=4, Hkv=2)
    need = rr.rr_workspace_bytes(p)
    dneed = rr.rr_decode_workspace_bytes(p)
    assert lib.rr_pattern_search(ctypes.byref(p), ok, ok, ok, ok, None, ok, need, None) == rr.RR_ERR_HIP
    assert lib.rr_block_sparse_attn(ctypes.byref(p), ok, ok, ok, ok, ok, ok, ok, need, None) == rr.RR_ERR_HIP
    assert lib.rr_prefill(ctypes.byref(p), ok, ok, ok, ok, ok, ok, ok, need, None) == rr.RR_ERR_HIP
    assert lib.rr_mass_recall(ctypes.byref(p), ok, ok, ok, ok, ok, None) == rr.RR_ERR_HIP
    assert lib.rr_decode(ctypes.byref(p), ok, ok, ok, None, ok, ok, ok, None, ok, dneed, None) == rr.RR_ERR_HIP
    assert lib.rr_pool_keys(ctypes.byref(p), ok, ok, None) == rr.RR_ERR_HIP


def test_noalloc_decode_checks_on_host():
    """rr_decode_noalloc validates like rr_decode and refuses problems whose
    workspace exceeds the library's own buffer, before any HIP call."""
    lib = rr.load()
    ok = 1 << 20
    assert rr.RR_DECODE_NOALLOC_MAX_WS == 32 << 20
    fits = base(L=131072)
    assert rr.rr_decode_workspace_bytes(fits) <= rr.RR_DECODE_NOALLOC_MAX_WS
    big = base(L=262144)  # pooled keys alone take 32 MiB
    assert rr.rr_decode_workspace_bytes(big) > rr.RR_DECODE_NOALLOC_MAX_WS
    assert lib.rr_decode_noalloc(ctypes.byref(big), ok, ok, ok, None, ok, ok, ok, None, 0) == rr.RR_ERR_WORKSPACE
    assert lib.rr_decode_noalloc(ctypes.byref(fits), None, ok, ok, None, ok, ok, ok, None, 0) == rr.RR_ERR_INVALID_ARG
    assert lib.rr_decode_noalloc(ctypes.byref(fits), ok, ok, ok, ok + 8, ok, ok, ok, None, 0) == rr.RR_ERR_INVALID_ARG
    assert lib.rr_decode_noalloc(ctypes.byref(base(d=96)), ok, ok, ok, None, ok, ok, ok, None, 0) == rr.RR_ERR_UNSUPPORTED
    assert lib.rr_decode_noalloc(None, ok, ok, ok, None, ok, ok, ok, None, 0) == rr.RR_ERR_INVALID_ARG
