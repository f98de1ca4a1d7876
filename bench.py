"""Benchmark of the RRAttention prefill hot path on one MI355X.

One step = one layer's causal prefill through the C ABI: the round-robin
pattern search (rr_pattern_search) followed by block-sparse attention over the
lists it produced (rr_block_sparse_attn), on seeded synthetic bf16 inputs that
are resident in HBM before timing starts. Default workload: the
LLaMA-3.1-8B-shaped layer at 131,072 tokens (32 query / 8 KV heads, d = 128,
B = 128, S = 16, tau = 0.9).

value = effective TFLOP/s of the whole step: F_comp / step time, where F_comp
counts 4*B*B*d FLOPs per computed off-diagonal block and 2*B*B*d per computed
diagonal block (the useful FLOPs of the blocks actually computed).

Prints one JSON line. Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse prefill attn ms + effective TFLOP/s per layer at 128K; % blocks computed"
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (published)
FP32_MATRIX_PEAK_TFLOPS = 157.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(workload_name: str, tau: float, record: str = "attn_bf16", source: str = "attn.hip"):
    """HBM bytes per attention call from the committed counter record, or None.

    The record (profiles/<record>_<workload>_traffic.json) holds FETCH_SIZE and
    WRITE_SIZE of the attention kernel scaled against a plain 1 GiB copy, and the
    sha256 of the kernel source they were taken on; a changed kernel reports None.
    """
    import hashlib

    path = os.path.join(ROOT, "profiles", "%s_%s_traffic.json" % (record, workload_name))
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(ROOT, "dynamic_block_sparse_rr_amd", "csrc", source)
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec.get("kernel_source_sha256"):
        return None
    if abs(float(rec.get("tau", -1)) - tau) > 1e-9:
        return None
    return float(rec["traffic_bytes"]), float(rec["algorithmic_bytes"])


def _pmc_rows(run_dir: str):
    """Per-dispatch counter sums of a rocprofv3 --pmc run (its counter_collection.csv):
    [(kernel name, duration ns, {counter: value})] in dispatch order."""
    import csv
    import glob

    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % run_dir)
    agg, meta = {}, {}
    for r in csv.DictReader(open(files[0])):
        k = int(r["Dispatch_Id"])
        agg.setdefault(k, {})
        agg[k][r["Counter_Name"]] = agg[k].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        meta[k] = (r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return [(meta[k][0], meta[k][1], agg[k]) for k in sorted(agg)]


def write_traffic_record(args):
    """profiles/attn_bf16_<workload>_traffic.json from three rocprofv3 --pmc runs of
    `bench.py --steps 1 --warmup 0 --calib-copy ...` (FETCH_SIZE, WRITE_SIZE, and the
    SQ/GRBM counters): the attention kernel's counters scaled by what the same counters
    read for the plain 1 GiB copy that runs first, plus its clock and MFMA busy."""
    import hashlib

    from synthetic.gen import workload

    w = workload(args.workload)
    tau = args.tau if args.tau is not None else w.taus[len(w.taus) // 2]
    dirs = args.traffic_record
    runs = [_pmc_rows(d) for d in dirs]

    def pick(rows, key):
        return [r for r in rows if key in r[0]]

    copy_f = pick(runs[0], "copyBuffer")[0][2]["FETCH_SIZE"]
    copy_w = pick(runs[1], "copyBuffer")[0][2]["WRITE_SIZE"]
    att_f = [r[2]["FETCH_SIZE"] for r in pick(runs[0], "attn_bf16_pp_kernel")]
    att_w = [r[2]["WRITE_SIZE"] for r in pick(runs[1], "attn_bf16_pp_kernel")]
    gib_kib = float(1 << 20)
    fs, ws_ = gib_kib / copy_f, gib_kib / copy_w
    f = float(np.median(att_f)) * 1024 * fs
    wr = float(np.median(att_w)) * 1024 * ws_
    alg = 2 * (w.L * w.Hq * w.d * 2) + 2 * (w.L * w.Hkv * w.d * 2)  # Q, O and K, V once each
    src = os.path.join(ROOT, "dynamic_block_sparse_rr_amd", "csrc", "attn.hip")
    rec = {
        "kernel": "attn_bf16_pp_kernel<%d,%d>" % (w.d, w.B), "workload": w.name, "tau": tau,
        "kernel_source_sha256": hashlib.sha256(open(src, "rb").read()).hexdigest(),
        "fetch_size_kib": float(np.median(att_f)), "write_size_kib": float(np.median(att_w)),
        "copy_1GiB_fetch_size_kib": copy_f, "copy_1GiB_write_size_kib": copy_w,
        "fetch_scale": fs, "write_scale": ws_, "hbm_fetch_bytes": f, "hbm_write_bytes": wr,
        "traffic_bytes": f + wr, "algorithmic_bytes": alg,
    }
    if len(runs) > 2:
        att = pick(runs[2], "attn_bf16_pp_kernel")[0]
        cp = pick(runs[2], "copyBuffer")[0]
        rec["sq"] = {k: att[2][k] for k in sorted(att[2])}
        if "GRBM_GUI_ACTIVE" in att[2]:  # summed over the 8 XCDs
            rec["core_clock_ghz_during_attention"] = att[2]["GRBM_GUI_ACTIVE"] / 8 / att[1]
            rec["core_clock_ghz_during_copy"] = cp[2]["GRBM_GUI_ACTIVE"] / 8 / cp[1]
            if "SQ_VALU_MFMA_BUSY_CYCLES" in att[2]:
                ncu = 256
                rec["mfma_busy"] = att[2]["SQ_VALU_MFMA_BUSY_CYCLES"] / (att[2]["GRBM_GUI_ACTIVE"] / 8 * ncu * 4)
    path = os.path.join(ROOT, "profiles", "attn_bf16_%s_traffic.json" % w.name)
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps({k: rec[k] for k in ("workload", "traffic_bytes", "algorithmic_bytes")}), flush=True)


def computed_flops(rc: np.ndarray, ci: np.ndarray, B: int, d: int, causal: bool):
    """(F_comp, blocks computed, diagonal blocks computed) from the block lists."""
    Hq, nb = rc.shape
    total = int(rc.sum())
    if causal:
        last = ci[np.arange(Hq)[:, None], np.arange(nb)[None, :], np.maximum(rc - 1, 0)]
        ndiag = int((last == np.arange(nb)[None, :]).sum())
    else:
        ndiag = 0
    f = 4.0 * B * B * d * (total - ndiag) + 2.0 * B * B * d * ndiag
    return f, total, ndiag


def search_logits(w, rows=None) -> int:
    """Sampled logits the search evaluates (rows: query-block indices, all heads)."""
    r = w.B // w.S
    it = range(w.nb - 1) if rows is None else rows
    n = 0
    for i in it:
        if i >= w.nb - 1:
            continue
        for a in range(r):
            s = i * r + a
            n += (s + 1) if w.causal else w.ns
    return n * w.Hq


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or 'unknown'."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _row_flops(w, rc, ci, rows) -> float:
    """Computed FLOPs (QK and PV) of the given (token, head) output rows on these lists."""
    f = 0.0
    for x, h in rows:
        i = x // w.B
        js = ci[h, i, : rc[h, i]]
        keys = int(sum(min(w.B, x - j * w.B + 1) if (w.causal and j == i) else min(w.B, w.L - j * w.B)
                       for j in js))
        f += 4.0 * w.d * keys
    return f


def cpu_baseline(w, q, k, v, rc, ci, f_comp, tau, n_attn_rows=8192, full=False):
    """The oracle on the host cores: the whole search, and attention on a
    bounded sample of (token, head) rows scaled to the whole step by FLOPs.
    full: the whole attention up to 32K tokens; beyond, every row of four
    heads spread over the KV heads, scaled by the FLOPs of their lists."""
    import oracle
    from synthetic.rows import sample_rows

    cores = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.search(q, k, S=w.S, B=w.B, tau=tau, causal=w.causal, round_bf16=w.dtype == "bf16", extras=False)
    t_search = time.perf_counter() - t0

    log("  oracle search %.2fs on %d threads" % (t_search, cores))
    if full and w.L > 32768:
        heads = [j * (w.Hq // 4) for j in range(4)]
        f_sub = 0.0
        t_attn = 0.0
        for h in heads:  # one head at a time, a progress line after each
            f_sub += computed_flops(rc[h:h + 1], ci[h:h + 1], w.B, w.d, w.causal)[0]
            rows = np.array([(x, h) for x in range(w.L)], np.int32)
            t0 = time.perf_counter()
            oracle.attention(q, k, v, rc, ci, B=w.B, causal=w.causal, rows=rows)
            t_attn += time.perf_counter() - t0
            log("  oracle attention, head %d: %.1fs" % (h, t_attn))
        est = t_search + t_attn * (f_comp / f_sub)
        return {
            "value": f_comp / est / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": ("the whole search (%.2fs) + attention of every row of heads %s (%.2fs, x%.2f to the whole "
                       "attention by computed FLOPs); full step %.0f s with the attention extrapolated"
                       % (t_search, heads, t_attn, f_comp / f_sub, est)),
            "search_s": round(t_search, 3), "attn_heads_s": round(t_attn, 3), "step_s_est": round(est, 1),
        }
    if full or w.L * w.Hq <= n_attn_rows:  # the whole attention, nothing extrapolated
        t_attn = 0.0
        for h in range(w.Hq):  # one head at a time, a progress line after each
            rows = np.array([(x, h) for x in range(w.L)], np.int32)
            t0 = time.perf_counter()
            oracle.attention(q, k, v, rc, ci, B=w.B, causal=w.causal, rows=rows)
            t_attn += time.perf_counter() - t0
            if w.L > 4096:
                log("  oracle attention, head %d: %.1fs" % (h, t_attn))
        est = t_search + t_attn
        return {
            "value": f_comp / est / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "the whole step: search (%.3fs) and attention (%.3fs) in full" % (t_search, t_attn),
            "search_s": round(t_search, 4), "attn_s": round(t_attn, 4),
        }
    srows = sample_rows(w.L, w.Hq, w.B, n_attn_rows, seed=11)
    f_sample = _row_flops(w, rc, ci, srows)
    t0 = time.perf_counter()
    oracle.attention(q, k, v, rc, ci, B=w.B, causal=w.causal, rows=srows)
    t_attn = time.perf_counter() - t0
    est = t_search + t_attn * (f_comp / f_sample)
    return {
        "value": f_comp / est / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": ("the whole search (%.2fs) + attention of %d sampled (token, head) rows on the GPU's block "
                   "lists (%.2fs, x%.0f to the whole attention by computed FLOPs); full step %.0f s with the "
                   "attention extrapolated" % (t_search, len(srows), t_attn, f_comp / f_sample, est)),
        "search_s": round(t_search, 3),
        "attn_sample_s": round(t_attn, 3),
    }


def measured_peaks():
    """Run ./peak (peak.hip: MFMA and HBM rates measured on this GPU) in a child
    process and return its summary dict, or None if it is not built or fails."""
    import subprocess

    exe = os.path.join(ROOT, "peak")
    if not os.path.exists(exe):
        log("peak is not built (python -c 'import __graft_entry__ as g; g.build()'): measured peaks omitted")
        return None
    r = subprocess.run([exe, "all"], capture_output=True, text=True, timeout=120)
    if r.returncode != 0:
        log("peak failed (%d): %s" % (r.returncode, r.stderr.strip()[-300:]))
        return None
    for line in r.stdout.splitlines():
        if line.startswith('{"summary"'):
            return json.loads(line)["summary"]
    return None


# ragged sequence lengths of the packed batch (none a multiple of B = 128), 131,072 tokens in all
VARLEN_LENS = [40000, 23456, 17000, 16383, 12800, 9999, 6000, 5434]


def bench_varlen(args):
    """Packed batch of sequences (rr_prefill_varlen); one JSON line like the single-sequence bench."""
    import torch

    import dynamic_block_sparse_rr_amd as rr
    from synthetic.gen import Workload, make_inputs

    lens = VARLEN_LENS
    if args.varlen_lens:  # "a,b,c" or "LxN" (N sequences of L tokens)
        if "x" in args.varlen_lens:
            L_, n_ = args.varlen_lens.split("x")
            lens = [int(L_)] * int(n_)
        else:
            lens = [int(t) for t in args.varlen_lens.split(",")]
    tau = args.tau if args.tau is not None else 0.9
    parts = [make_inputs(Workload("llama8b_seq%d" % b, L, 32, 8, 128, "bf16", 128, 16, (tau,), 40 + b, "llm", 64))
             for b, L in enumerate(lens)]
    q = torch.cat([x[0] for x in parts]).cuda()
    k = torch.cat([x[1] for x in parts]).cuda()
    v = torch.cat([x[2] for x in parts]).cuda()
    del parts
    p = rr.problem(sum(lens), 32, 8, 128, 16, 128, tau, True, "bf16")
    nbs = [-(-L // 128) for L in lens]
    rc = torch.empty((sum(32 * n for n in nbs),), dtype=torch.int32, device="cuda")
    ci = torch.empty((sum(32 * n * n for n in nbs),), dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ws = torch.empty(rr.rr_workspace_bytes_varlen(p, lens), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        rr.rr_prefill_varlen(p, lens, q, k, v, out, rc, ci, ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        ev[s_][0].record(stream)
        step()
        ev[s_][1].record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ev_ms = [e[0].elapsed_time(e[1]) for e in ev]
    rcn, cin = rc.cpu().numpy(), ci.cpu().numpy()
    f_comp = 0.0
    blocks = cand = 0
    roff = coff = 0
    for L, nb in zip(lens, nbs):
        rcb = rcn[roff:roff + 32 * nb].reshape(32, nb)
        cib = cin[coff:coff + 32 * nb * nb].reshape(32, nb, nb)
        f, nblk, _ = computed_flops(rcb, cib, 128, 128, True)
        f_comp += f
        blocks += nblk
        cand += 32 * nb * (nb + 1) // 2
        roff += 32 * nb
        coff += 32 * nb * nb
    value = f_comp / (ms * 1e-3) / 1e12

    # beside it, untimed in the line's value: the same sequences, one rr_prefill call each
    offs = np.cumsum([0] + lens)
    ps = [rr.problem(L, 32, 8, 128, 16, 128, tau, True, "bf16") for L in lens]
    rcs = [torch.empty((32 * n,), dtype=torch.int32, device="cuda") for n in nbs]
    cis = [torch.empty((32 * n * n,), dtype=torch.int32, device="cuda") for n in nbs]
    ws1 = torch.empty(max(rr.rr_workspace_bytes(x) for x in ps), dtype=torch.uint8, device="cuda")

    def step_each():
        for b, L in enumerate(lens):
            a, e = int(offs[b]), int(offs[b + 1])
            rr.rr_prefill(ps[b], q[a:e], k[a:e], v[a:e], out[a:e], rcs[b], cis[b], ws1, stream=stream)

    for _ in range(args.warmup):
        step_each()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step_each()
    torch.cuda.synchronize()
    ms_each = (time.perf_counter() - t0) * 1e3 / args.steps
    del ws1
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama8b_varlen_batch_%dk" % (sum(lens) // 1024), "seq_lens": lens, "Hq": 32, "Hkv": 8, "d": 128,
                   "B": 128, "S": 16, "tau": tau, "causal": True},
        "step_ms_median_events": round(float(np.median(ev_ms)), 3),
        "blocks_computed_pct": round(100.0 * blocks / cand, 2),
        "note": ("rr_prefill_varlen: the searches one after the other; the attention of each sequence long enough to "
                 "fill the GPU alone in a launch of its own, the others in one shared launch"),
        "per_sequence_calls_ms": round(ms_each, 3),
        "per_sequence_calls_tflops": round(f_comp / (ms_each * 1e-3) / 1e12, 2),
    }
    print(json.dumps(line), flush=True)


def bench_decode(args):
    """One decode step of the 128K layer: the last token's queries against the whole cache."""
    import torch

    import dynamic_block_sparse_rr_amd as rr
    from synthetic.gen import make_inputs, workload

    w = workload(args.workload)
    tau = args.tau if args.tau is not None else w.taus[len(w.taus) // 2]
    Q, K, V = make_inputs(w)
    q = Q[w.L - 1].contiguous().cuda()
    k, v = K.cuda(), V.cuda()
    del Q
    stream = torch.cuda.current_stream()
    res = {}
    for t in (tau, 1.0):
        p = rr.problem(w.L, w.Hq, w.Hkv, w.d, w.S, w.B, t, True, w.dtype)
        kbar = torch.empty((p.ns, w.Hkv, w.d), dtype=k.dtype, device="cuda")
        out = torch.empty_like(q)
        rc = torch.empty((w.Hq,), dtype=torch.int32, device="cuda")
        ci = torch.empty((w.Hq, w.nb), dtype=torch.int32, device="cuda")
        ws = torch.empty(rr.rr_decode_workspace_bytes(p), dtype=torch.uint8, device="cuda")
        e = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        rr.rr_pool_keys(p, k, kbar, stream=stream)  # first launch loads the code object
        e[0].record(stream)
        rr.rr_pool_keys(p, k, kbar, stream=stream)
        e[1].record(stream)
        for _ in range(max(3, args.warmup)):
            rr.rr_decode(p, q, k, v, out, rc, ci, None, ws, stream=stream, kbar=kbar)
        n = max(20, 10 * args.steps)
        e[2].record(stream)
        for _ in range(n):
            rr.rr_decode(p, q, k, v, out, rc, ci, None, ws, stream=stream, kbar=kbar)
        e[3].record(stream)
        # the attention stage alone on the same lists (lists to flags, split-K attention, combine)
        out2 = torch.empty_like(q)
        rr.rr_decode_attend(p, q, k, v, rc, ci, out2, ws, stream=stream)
        e[4].record(stream)
        for _ in range(n):
            rr.rr_decode_attend(p, q, k, v, rc, ci, out2, ws, stream=stream)
        e[5].record(stream)
        torch.cuda.synchronize()
        us = e[2].elapsed_time(e[3]) * 1e3 / n
        att_us = e[4].elapsed_time(e[5]) * 1e3 / n
        rcn, cin = rc.cpu().numpy(), ci.cpu().numpy()
        # algorithmic bytes: K and V of the blocks each KV head's query heads selected (their union),
        # the pooled keys once, the queries and outputs
        tile = 2 * w.B * w.d * 2
        union = 0
        for g in range(w.Hkv):
            sel = set()
            for h in range(g * w.G, (g + 1) * w.G):
                sel.update(int(j) for j in cin[h, : rcn[h]])
            union += len(sel)
        esz = 2 if w.dtype == "bf16" else 4
        att_bytes = union * tile + 2 * w.Hq * w.d * esz
        nbytes = att_bytes + p.ns * w.Hkv * w.d * esz
        res[t] = {"us": us, "att_us": att_us, "pool_us": e[0].elapsed_time(e[1]) * 1e3,
                  "kept": float(rcn.mean() / w.nb), "union": union / (w.Hkv * w.nb),
                  "bytes": nbytes, "tbps": nbytes / (us * 1e-6) / 1e12,
                  "att_bytes": att_bytes, "att_tbps": att_bytes / (att_us * 1e-6) / 1e12}
    r, d_ = res[tau], res[1.0]
    line = {
        "metric": "decode step us per layer at 128K (one new token, pooled keys kept with the cache)",
        "value": round(r["us"], 2), "unit": "us", "n_gpus": 1, "steps": max(20, 10 * args.steps),
        "warmup": max(3, args.warmup), "ms_per_step": round(r["us"] / 1e3, 4), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name + "_decode", "L": w.L, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "B": w.B,
                   "S": w.S, "tau": tau},
        "blocks_kept": round(r["kept"], 4), "blocks_read_per_kv_head": round(r["union"], 4),
        # dominant stage: the split-K attention (HIP events around rr_decode_attend, which also runs the
        # small list-to-flag and combine kernels); bytes = K and V of the union of each KV head's
        # selected blocks, plus the queries and outputs
        "roofline": {"bound": "hbm", "achieved": round(r["att_tbps"] * 1e3, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(r["att_tbps"] / 8.0, 4), "traffic": None,
                     "algorithmic_bytes": r["att_bytes"], "stage_us": round(r["att_us"], 2)},
        "step_GBps": round(r["tbps"] * 1e3, 1), "step_algorithmic_bytes": r["bytes"],
        "dense_decode_us": round(d_["us"], 2), "dense_decode_GBps": round(d_["tbps"] * 1e3, 1),
        "speedup_vs_dense": round(d_["us"] / r["us"], 3),
        "pool_keys_us_whole_cache": round(r["pool_us"], 1),
    }
    tr = measured_traffic(w.name, tau, record="decode_attn_bf16", source="decode.hip")
    if tr is not None:
        line["roofline"]["traffic"] = tr[0]
        line["roofline"]["traffic_unit"] = "bytes per attention kernel launch (HBM, FETCH_SIZE + WRITE_SIZE)"
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama8b_L128k",
                    help="a named layer (synthetic.gen.WORKLOADS) or shape:L,Hq,Hkv,d,B,S[,dtype[,kind[,seed]]]")
    ap.add_argument("--tau", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline-full", action="store_true",
                    help="time the oracle's whole step (up to 32K tokens) or every row of four heads (longer "
                         "layers) instead of a bounded sample: minutes at 64K and 128K")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--recall", action="store_true",
                    help="also run rr_mass_recall on the produced lists: the full-attention softmax mass the "
                         "selection holds per (head, query block), its statistics and its kernel time")
    ap.add_argument("--shared-mask", action="store_true",
                    help="variant: every head of a KV head attends over the union of the group's selections "
                         "(rr_share_group_lists runs inside the step, after the search)")
    ap.add_argument("--varlen", action="store_true",
                    help="a packed batch of LLaMA-8B-shaped sequences of ragged lengths (about 128K tokens in "
                         "all) through rr_prefill_varlen instead of one sequence")
    ap.add_argument("--varlen-lens", default=None,
                    help="with --varlen: the sequence lengths, as a,b,c or LxN (N sequences of L tokens)")
    ap.add_argument("--decode", action="store_true",
                    help="one decode step against the 128K cache (rr_decode, pooled keys given) instead of prefill")
    ap.add_argument("--cold", action="store_true",
                    help="also time steps that each follow a 1 GiB buffer write (flushes the 256 MiB MALL); "
                         "reported as cold_* fields, events only")
    ap.add_argument("--hbm-ceiling", action="store_true",
                    help="run peak.hip's cache probe: plain and block-walk reads of a K/V cache of the workload's "
                         "shape, the practical read ceiling of the decode attention")
    ap.add_argument("--no-peak", action="store_true",
                    help="skip the measured MFMA/HBM peaks (peak.hip) that the roofline also divides by")
    ap.add_argument("--traffic-record", nargs="+", default=None, metavar="PMC_DIR",
                    help="write profiles/attn_bf16_<workload>_traffic.json from the output directories of "
                         "rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE, optionally the SQ/GRBM counters) of "
                         "this script with --calib-copy; runs nothing on the GPU")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run a plain 1 GiB device-to-device copy, the reference kernel for "
                         "scaling HBM byte counters")
    args = ap.parse_args()
    if args.traffic_record:
        return write_traffic_record(args)
    if args.hbm_ceiling:  # a child process of its own, before this one touches the GPU
        import subprocess

        from synthetic.gen import workload as wl

        w = wl(args.workload)
        probe = os.path.join(ROOT, "peak")
        if not os.path.exists(probe):
            raise SystemExit("peak is not built: run python -c 'import __graft_entry__ as g; g.build()'")
        sys.exit(subprocess.run([probe, "cache", str(w.L), str(w.Hkv)]).returncode)
    if args.gpus != 1:
        print("bench.py measures one GPU only: the operator runs on a single device "
              "(sharding it across GPUs is a design note, not implemented).", file=sys.stderr)
        sys.exit(2)

    peaks = None
    if not (args.no_peak or args.varlen or args.decode):
        peaks = measured_peaks()  # a child process, before this one touches the GPU
        if peaks:
            log("measured peaks: " + json.dumps(peaks))

    import torch

    import dynamic_block_sparse_rr_amd as rr
    from synthetic.gen import make_inputs, workload

    if args.calib_copy:  # a plain 1 GiB device copy first: the reference for HBM byte counters
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.varlen:
        return bench_varlen(args)
    if args.decode:
        return bench_decode(args)
    w = workload(args.workload)
    tau = args.tau if args.tau is not None else w.taus[len(w.taus) // 2]
    log(f"workload {w.name}: L={w.L} Hq={w.Hq} Hkv={w.Hkv} d={w.d} B={w.B} S={w.S} tau={tau}")
    t0 = time.perf_counter()
    q, k, v = make_inputs(w)
    log(f"inputs generated in {time.perf_counter() - t0:.1f}s")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    p = rr.problem(w.L, w.Hq, w.Hkv, w.d, w.S, w.B, tau, w.causal, w.dtype)
    pre = rr.Prefill(p)
    stream = torch.cuda.current_stream()

    # the lists the attention reads: the search's own, or their union per KV head
    if args.shared_mask:
        arc, aci = torch.empty_like(pre.row_count), torch.empty_like(pre.col_idx)
    else:
        arc, aci = pre.row_count, pre.col_idx

    def search():
        rr.rr_pattern_search(p, qd, kd, pre.row_count, pre.col_idx, None, pre.ws, stream=stream)
        if args.shared_mask:
            rr.rr_share_group_lists(p, pre.row_count, pre.col_idx, arc, aci, stream=stream)

    def attend():
        rr.rr_block_sparse_attn(p, qd, kd, vd, arc, aci, pre.out, pre.ws, stream=stream)

    def step():
        search()
        attend()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        search()
        ev[s][1].record(stream)
        attend()
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    search_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    attn_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    ms_per_step = wall * 1e3 / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step (search {search_ms:.3f} ms, attention {attn_ms:.3f} ms)")

    step_ms = [e[0].elapsed_time(e[2]) for e in ev]
    cold = {}
    if args.cold:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        cs, ca = [], []
        for _ in range(max(3, args.steps)):
            flush.fill_(1)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            search()
            e[1].record(stream)
            attend()
            e[2].record(stream)
            torch.cuda.synchronize()
            cs.append(e[0].elapsed_time(e[1]))
            ca.append(e[1].elapsed_time(e[2]))
        del flush
        cold = {"cold_search_ms_median": round(float(np.median(cs)), 3),
                "cold_attn_ms_median": round(float(np.median(ca)), 3),
                "cold_step_ms_median": round(float(np.median(np.add(cs, ca))), 3)}
        log(f"cold steps (after a 1 GiB write): search {np.median(cs):.3f} ms, attention {np.median(ca):.3f} ms")

    rc = arc.cpu().numpy()
    ci = aci.cpu().numpy()
    f_comp, nblocks, ndiag = computed_flops(rc, ci, w.B, w.d, w.causal)
    causal_blocks = w.Hq * w.nb * (w.nb + 1) // 2 if w.causal else w.Hq * w.nb * w.nb
    pct = 100.0 * nblocks / causal_blocks
    attn_tflops = f_comp / (attn_ms * 1e-3) / 1e12
    value = f_comp / (ms_per_step * 1e-3) / 1e12
    peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_MATRIX_PEAK_TFLOPS

    extra = {}
    if not args.no_dense:
        # dense baseline: the same attention kernel with every causal block listed
        dp = rr.problem(w.L, w.Hq, w.Hkv, w.d, w.S, w.B, 1.0, w.causal, w.dtype)
        drc = torch.empty_like(pre.row_count)
        dci = torch.empty_like(pre.col_idx)
        rr.rr_pattern_search(dp, qd, kd, drc, dci, None, pre.ws, stream=stream)
        # as many warm-up and timed calls as the sparse step had (at least 1 and 2), so that
        # short layers are timed at the same settled clock as the sparse step
        for _ in range(max(1, args.warmup)):
            rr.rr_block_sparse_attn(dp, qd, kd, vd, drc, dci, pre.out, pre.ws, stream=stream)
        ndense = max(2, args.steps)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(ndense):
            rr.rr_block_sparse_attn(dp, qd, kd, vd, drc, dci, pre.out, pre.ws, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / ndense
        f_dense, _, _ = computed_flops(drc.cpu().numpy(), dci.cpu().numpy(), w.B, w.d, w.causal)
        extra = {"dense_attn_ms": round(dense_ms, 3),
                 "dense_attn_tflops": round(f_dense / (dense_ms * 1e-3) / 1e12, 1),
                 "speedup_vs_dense": round(dense_ms / ms_per_step, 3)}
        del drc, dci
        log(f"dense attention {dense_ms:.3f} ms")

    if args.recall:
        rec = torch.empty((w.Hq, w.nb), dtype=torch.float32, device="cuda")
        rr.rr_mass_recall(p, qd, kd, arc, aci, rec, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(3):
            rr.rr_mass_recall(p, qd, kd, arc, aci, rec, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        rec_ms = e0.elapsed_time(e1) / 3
        r = rec.cpu().numpy()
        cand = w.nb * (w.nb + 1) // 2 if w.causal else w.nb * w.nb
        f_qk = 2.0 * w.B * w.B * w.d * cand * w.Hq  # scores of every candidate block
        extra["mass_recall"] = {
            "mean": round(float(r.mean()), 5), "min": round(float(r.min()), 5),
            "p10": round(float(np.percentile(r, 10)), 5), "p50": round(float(np.percentile(r, 50)), 5),
            "rows_below_0.5": int((r < 0.5).sum()), "rows": int(r.size),
            "kernel_ms": round(rec_ms, 3), "score_tflops": round(f_qk / (rec_ms * 1e-3) / 1e12, 1)}
        log(f"mass recall: mean {r.mean():.4f} min {r.min():.4f} ({rec_ms:.3f} ms)")

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "L": w.L, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "B": w.B,
                   "S": w.S, "tau": tau, "causal": w.causal, "seed": w.seed, "batch": 1,
                   **({"mask": "shared per KV head (union of the group's selections)"} if args.shared_mask else {})},
        "step_ms_median_events": round(float(np.median(step_ms)), 3),
        **cold,
        "search_ms": round(search_ms, 3),
        "attn_ms": round(attn_ms, 3),
        "search_share": round(search_ms / (search_ms + attn_ms), 4),
        "blocks_computed_pct": round(pct, 2),
        "attn_effective_tflops": round(attn_tflops, 1),
        **extra,
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 1), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / peak, 4), "traffic": None,
                     "kernel": ("bf16 block-sparse attention (timed with the V re-layout pass of the same call)"
                                if w.dtype == "bf16" else "fp32 block-sparse attention on the fp32 MFMA")},
    }
    if peaks:
        key = "mfma_bf16_reg_2w_TFLOPs" if w.dtype == "bf16" else "mfma_f32_reg_2w_TFLOPs"
        mp = float(peaks[key])
        line["roofline"]["peak_measured"] = mp
        line["roofline"]["frac_measured"] = round(attn_tflops / mp, 4) if mp > 0 else None
        line["roofline"]["peak_measured_kind"] = (
            "peak.hip on this GPU: %s MFMA with register operands, two waves per SIMD" %
            ("32x32x16 bf16" if w.dtype == "bf16" else "32x32x2 fp32"))
        if w.dtype == "bf16":
            line["roofline"]["peak_lds_fed_measured"] = float(peaks["mfma_bf16_lds_2w_TFLOPs"])
            # the same MFMA stream on pseudo-random operands: the rate the chip sustains when every
            # multiplier bit toggles as in real activations (its clock drops under that load)
            mr = float(peaks.get("mfma_bf16_reg_2w_random_TFLOPs", 0.0))
            if mr > 0:
                line["roofline"]["peak_measured_random_operands"] = mr
                line["roofline"]["frac_measured_random_operands"] = round(attn_tflops / mr, 4)
            # ... and fed like the attention: one LDS operand per MFMA, pseudo-random data
            ml = float(peaks.get("mfma_bf16_lds_2w_random_TFLOPs", 0.0))
            if ml > 0:
                line["roofline"]["peak_lds_fed_random_operands"] = ml
                line["roofline"]["frac_lds_fed_random_operands"] = round(attn_tflops / ml, 4)
            # ... and with a softmax-like VALU stream on the same SIMDs, as much VALU work per MFMA as the
            # attention issues (peak.hip coexec): the rate a kernel doing both can reach on this GPU
            mv = float(peaks.get("mfma_bf16_lds_random_with_softmax_valu_TFLOPs", 0.0))
            if mv > 0:
                line["roofline"]["peak_lds_fed_with_softmax_valu"] = mv
                line["roofline"]["frac_lds_fed_with_softmax_valu"] = round(attn_tflops / mv, 4)
        line["measured_peaks"] = peaks
    tr = measured_traffic(w.name, tau)
    if tr is not None:
        line["roofline"]["traffic"] = tr[0]
        line["roofline"]["traffic_unit"] = "bytes per attention call (HBM, FETCH_SIZE + WRITE_SIZE)"
        line["roofline"]["algorithmic_bytes"] = tr[1]
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline(w, q, k, v, rc, ci, f_comp, tau, full=args.cpu_baseline_full)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
