"""Host-side logic of bench.py (no GPU): the committed HBM-traffic lookup that feeds the
roofline's `traffic` field is used only while its kernel-source hash matches."""

import json
import os

import bench


def _tree(tmp_path, source: bytes, sha: str, workload: str, traffic: int):
    csrc = tmp_path / "mixture_experts_ffn_02_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "moe_gemm.hip").write_bytes(source)
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"moe_gemm_sha": sha, workload: {"traffic_bytes_per_launch": traffic}}
    (prof / "gate_up_gemm_traffic.json").write_text(json.dumps(rec))


def test_traffic_used_when_the_kernel_source_matches(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    src = b"// kernel source A\n"
    import hashlib

    _tree(tmp_path, src, hashlib.sha256(src).hexdigest()[:16], "decode_w", 123)
    assert bench.committed_traffic("decode_w") == 123
    assert bench.committed_traffic("other_workload") is None


def test_traffic_null_once_the_kernel_source_changed(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _tree(tmp_path, b"// kernel source B\n", "0" * 16, "decode_w", 123)
    assert bench.committed_traffic("decode_w") is None


def test_committed_traffic_file_names_its_kernel_source():
    p = os.path.join(bench.ROOT, "profiles", "gate_up_gemm_traffic.json")
    d = json.load(open(p))
    assert len(d["moe_gemm_sha"]) == 16
    recs = {k: v for k, v in d.items() if k != "moe_gemm_sha"}
    assert recs and all(v["traffic_bytes_per_launch"] > 0 for v in recs.values())


def test_more_than_one_gpu_is_refused_with_a_message():
    """--gpus N > 1 exits (status 2) with a message before any GPU work: the layer runs on one
    GPU's share of the experts."""
    import subprocess
    import sys

    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""
