"""bench.py's host logic, without a GPU: the one-GPU rule, and the traffic
figure's tie to the kernel source it was measured on."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


def test_traffic_is_reported_only_for_the_kernel_it_was_measured_on(tmp_path, monkeypatch):
    rec = {"workload": "w", "kernel_sha": bench.kernel_hash(), "hbm_bytes_per_launch": 123.0}
    path = tmp_path / "attn_fwd_w_traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "{prefix}_{workload}_traffic.json"))
    assert bench.read_traffic("w") == 123.0
    rec["kernel_sha"] = "0" * 16
    path.write_text(json.dumps(rec))
    assert bench.read_traffic("w") is None
    assert bench.read_traffic("missing") is None


def test_committed_traffic_files_name_their_kernel():
    prof = os.path.join(ROOT, "profiles")
    files = [f for f in os.listdir(prof) if f.endswith("_traffic.json")]
    assert files
    for f in files:
        rec = json.load(open(os.path.join(prof, f)))
        assert len(rec["kernel_sha"]) == 16
        assert rec["hbm_bytes_per_launch"] > 0
        # The read-back agrees with the hash check, whichever way it goes.
        w = rec["workload"]
        got = bench.read_traffic(w)
        assert (got is not None) == (rec["kernel_sha"] == bench.kernel_hash(bench.kernel_kind(w)))
