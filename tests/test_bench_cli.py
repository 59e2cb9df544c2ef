"""bench.py's command-line contract on the host (no GPU): it refuses more
than one GPU with a message, and the stored HBM traffic of the chain is
read only while its kernel-source hash matches."""

import os
import subprocess
import sys

from conftest import ROOT


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_stored_traffic_requires_matching_source_hash(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    sha = bench.kernel_source_sha()
    assert len(sha) == 16
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "t_ok.txt").write_text(f"kernel_source_sha = {sha}\ntraffic_bytes_per_launch = 123\n")
    (prof / "t_old.txt").write_text("kernel_source_sha = 0000000000000000\n"
                                    "traffic_bytes_per_launch = 123\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: sha)
    assert bench.load_traffic("t_ok") == 123.0
    assert bench.load_traffic("t_old") is None
    assert bench.load_traffic("t_missing") is None
