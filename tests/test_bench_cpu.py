"""bench.py's host-side contract (no GPU): one GPU only, and the traffic record
is used only for the kernel source it was measured on."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_record_only_for_its_own_kernel_source(tmp_path, monkeypatch):
    import bench

    prof = tmp_path / "profiles"
    prof.mkdir()
    src_dir = tmp_path / "dynamic_block_sparse_rr_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (src_dir / "attn.hip").write_bytes(b"kernel source A")
    import hashlib

    sha = hashlib.sha256(b"kernel source A").hexdigest()
    rec = {"kernel_source_sha256": sha, "tau": 0.9, "traffic_bytes": 123.0, "algorithmic_bytes": 45.0}
    (prof / "attn_bf16_wl_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("wl", 0.9) == (123.0, 45.0)
    assert bench.measured_traffic("wl", 0.85) is None  # another tau
    assert bench.measured_traffic("other", 0.9) is None  # no record
    (src_dir / "attn.hip").write_bytes(b"kernel source B")
    assert bench.measured_traffic("wl", 0.9) is None  # the kernel changed since the counters were taken


def _pmc_csv(path, rows):
    """A counter_collection.csv like rocprofv3 --output-format csv writes: (dispatch, kernel, counter, value,
    start, end) per row."""
    path.mkdir(parents=True, exist_ok=True)
    hdr = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id","Grid_Size","Kernel_Id",'
           '"Kernel_Name","Workgroup_Size","LDS_Block_Size","Scratch_Size","VGPR_Count","Accum_VGPR_Count",'
           '"SGPR_Count","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"')
    lines = [hdr]
    for d, name, counter, value, t0, t1 in rows:
        lines.append('%d,%d,"Agent 1",1,1,1,1,1,"%s",256,0,0,8,0,32,"%s",%f,%d,%d' % (d, d, name, counter, value, t0, t1))
    (path / "pmc_counter_collection.csv").write_text("\n".join(lines) + "\n")


def test_traffic_record_written_from_counter_runs(tmp_path, monkeypatch):
    """bench.py --traffic-record: the attention kernel's FETCH_SIZE and WRITE_SIZE scaled by what the same
    counters read for the 1 GiB copy, the clock from GRBM_GUI_ACTIVE summed over 8 XCDs, the kernel
    source's sha256, and the algorithmic bytes Q + K + V + O of the workload."""
    import hashlib

    import bench

    attn = "void rr::attn_bf16_pp_kernel<128, 128, false, false>(...)"
    copy = "__amd_rocclr_copyBuffer"
    gib = float(1 << 20)
    _pmc_csv(tmp_path / "pf", [(1, copy, "FETCH_SIZE", gib / 2, 0, 100), (2, attn, "FETCH_SIZE", 1000.0, 0, 10)])
    _pmc_csv(tmp_path / "pw", [(1, copy, "WRITE_SIZE", gib, 0, 100), (2, attn, "WRITE_SIZE", 300.0, 0, 10)])
    _pmc_csv(tmp_path / "ps", [(1, copy, "GRBM_GUI_ACTIVE", 8 * 240.0, 0, 100),
                               (2, attn, "GRBM_GUI_ACTIVE", 8 * 16.5, 0, 10),
                               (2, attn, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 16.5 * 256 * 4, 0, 10)])
    src_dir = tmp_path / "dynamic_block_sparse_rr_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (src_dir / "attn.hip").write_bytes(b"kernel source")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(sys, "argv", ["bench.py", "--traffic-record", str(tmp_path / "pf"), str(tmp_path / "pw"),
                                      str(tmp_path / "ps"), "--workload", "llama8b_L16k", "--tau", "0.9"])
    bench.main()
    rec = json.loads((tmp_path / "profiles" / "attn_bf16_llama8b_L16k_traffic.json").read_text())
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["hbm_fetch_bytes"] == 1000.0 * 1024 * 2 and rec["hbm_write_bytes"] == 300.0 * 1024
    assert rec["traffic_bytes"] == rec["hbm_fetch_bytes"] + rec["hbm_write_bytes"]
    L, Hq, Hkv, d = 16384, 32, 8, 128
    assert rec["algorithmic_bytes"] == 2 * L * Hq * d * 2 + 2 * L * Hkv * d * 2
    assert rec["kernel_source_sha256"] == hashlib.sha256(b"kernel source").hexdigest()
    assert abs(rec["core_clock_ghz_during_attention"] - 1.65) < 1e-9
    assert abs(rec["core_clock_ghz_during_copy"] - 2.4) < 1e-9
    assert abs(rec["mfma_busy"] - 0.5) < 1e-9
    # and bench reads it back while the source matches
    assert bench.measured_traffic("llama8b_L16k", 0.9) == (rec["traffic_bytes"], float(rec["algorithmic_bytes"]))


def test_shape_workloads_parse():
    """`--workload shape:L,Hq,Hkv,d,B,S[,dtype[,kind[,seed]]]` names any layer."""
    from synthetic.gen import make_inputs, workload

    w = workload("shape:4096,32,32,128,128,16")
    assert (w.L, w.Hq, w.Hkv, w.d, w.B, w.S, w.dtype, w.kind, w.causal) == (4096, 32, 32, 128, 128, 16, "bf16",
                                                                           "llm", True)
    assert w.G == 1 and w.nb == 32 and w.taus == (0.9,)
    w2 = workload("shape:300,4,2,64,64,8,fp32,gauss,5")
    assert (w2.dtype, w2.kind, w2.seed, w2.nb) == ("fp32", "gauss", 5, 5)
    q, k, v = make_inputs(w2)
    assert tuple(q.shape) == (300, 4, 64) and tuple(k.shape) == (300, 2, 64) and str(q.dtype) == "torch.float32"
    import pytest

    with pytest.raises(ValueError):
        workload("shape:4096,32,32")
