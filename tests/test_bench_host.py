"""CPU tests of bench.py's host logic: the committed counter records are tied to the kernel
sources they were taken with, the vector-ALU roofline arithmetic, and the one-GPU refusal."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _record(tmp_path, sha=None, **extra):
    src = tmp_path / "k.hip"
    src.write_bytes(b"kernel source\n")
    rec = {"kernel_sources": [os.path.relpath(src, ROOT)],
           "kernel_sources_sha256": sha or hashlib.sha256(src.read_bytes()).hexdigest()}
    rec.update(extra)
    path = tmp_path / "rec.json"
    path.write_text(json.dumps(rec))
    return str(path), src


def test_record_is_current_only_for_the_sources_it_hashes(tmp_path):
    path, src = _record(tmp_path, traffic_bytes_per_launch=123)
    assert bench.kernel_record(path)["traffic_bytes_per_launch"] == 123
    assert bench.measured_traffic(path) == 123
    src.write_bytes(b"kernel source, edited\n")
    assert bench.kernel_record(path) is None
    assert bench.measured_traffic(path) is None


def test_record_with_a_wrong_hash_or_missing_file_is_ignored(tmp_path):
    path, _ = _record(tmp_path, sha="0" * 64, traffic_bytes_per_launch=1)
    assert bench.measured_traffic(path) is None
    assert bench.kernel_record(str(tmp_path / "absent.json")) is None


def test_committed_records_name_existing_sources():
    for path in (bench.TRAFFIC_FILE, bench.PREFILL_TRAFFIC_FILE):
        with open(path) as f:
            rec = json.load(f)
        assert rec["kernel_sources"], path
        for s in rec["kernel_sources"]:
            assert os.path.isfile(os.path.join(ROOT, s)), s
        assert rec["traffic_bytes_per_launch"] == \
            rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"]


def test_alu_roofline_arithmetic(monkeypatch):
    monkeypatch.setattr(bench, "kernel_record", lambda path=None: {"valu_per_weight": 2.0})
    r = bench.alu_roofline(weights_per_launch=1e9, launch_s=1e-3)
    peak = 256 * 4 * 16 * 2.4e9 / 2.0 / 1e9  # G weights/s
    assert r["peak"] == pytest.approx(peak, rel=1e-6)
    assert r["achieved"] == pytest.approx(1000.0)
    assert r["frac"] == pytest.approx(1000.0 / peak, abs=1e-4)
    assert r["bound"] == "alu"
    monkeypatch.setattr(bench, "kernel_record", lambda path=None: None)
    assert bench.alu_roofline(1e9, 1e-3) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout
