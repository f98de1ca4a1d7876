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
