"""Host-side behaviour of bench.py that needs no GPU: the one-GPU guard, the
workload choice, and the gate that reports HBM traffic only for the kernel
source the counters were taken on."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_unknown_workload_is_rejected():
    r = _run("--workload", "no_such_workload")
    assert r.returncode == 2
    assert "--workload must be one of" in r.stderr


def test_source_hash_covers_the_shared_headers():
    alone = bench.src_hash("fa_fwd.hip")
    with_headers = bench.src_hash("fa_fwd.hip", "fa_device.h", "fa_internal.h")
    assert alone != with_headers and len(with_headers) == 16


def test_traffic_is_reported_only_for_the_profiled_source(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "fwd_bf16_llama_n8192_traffic.json").write_text(
        json.dumps({"kernel_src_sha": "abc123", "traffic_bytes_per_launch": 12345}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profile("abc123") == 12345
    assert bench.traffic_from_profile("other") is None


def test_committed_traffic_summary_is_well_formed():
    path = os.path.join(ROOT, "profiles", "fwd_bf16_llama_n8192_traffic.json")
    t = json.load(open(path))
    assert t["traffic_bytes_per_launch"] > t["algorithmic_bytes_per_launch"] > 0
    assert len(t["kernel_src_sha"]) == 16
