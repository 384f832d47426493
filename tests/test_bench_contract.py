"""bench.py's contract pieces that need no GPU: the multi-GPU refusal, the
FLOP accounting of the roofline and the source-hash gate on measured traffic."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_status_2():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_flops_per_family():
    S, Hq, D = 1024, 4, 128
    pairs = S * S / 2
    assert bench.algorithmic_flops("fwd", S, Hq, D, True) == 4 * D * pairs * Hq
    assert bench.algorithmic_flops("dkdv", S, Hq, D, True) == 8 * D * pairs * Hq
    assert bench.algorithmic_flops("dq", S, Hq, D, True) == 6 * D * pairs * Hq
    assert bench.algorithmic_flops("dq", S, Hq, D, False) == 6 * D * S * S * Hq
    assert bench.algorithmic_flops("pack", S, Hq, D, True) == 0.0


def _write_traffic(tmp_path, family, sha):
    prof = tmp_path / "profiles"
    prof.mkdir(exist_ok=True)
    rec = {"source_sha256": sha, "fetch_bytes_per_launch": 1000, "write_bytes_per_launch": 24}
    (prof / f"traffic_{family}_S1_hc1.md").write_text("# t\n\ntraffic_json: " + json.dumps(rec) + "\n")
    return prof


def test_traffic_is_reported_only_for_the_profiled_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES_DIR", str(tmp_path / "profiles"))
    _write_traffic(tmp_path, "dkdv", bench.kernel_source_hash("dkdv"))
    assert bench.measured_traffic("dkdv", "S1", 1) == 1024
    _write_traffic(tmp_path, "dkdv", "0" * 64)
    assert bench.measured_traffic("dkdv", "S1", 1) is None
    assert bench.measured_traffic("fwd", "S1", 1) is None  # no file


def test_kernel_source_hash_tracks_the_family_sources():
    assert bench.kernel_source_hash("dkdv") == bench.kernel_source_hash("dq")  # same file
    assert bench.kernel_source_hash("fwd") != bench.kernel_source_hash("dkdv")
