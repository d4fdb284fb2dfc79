"""The benchmark's command-line contract on the CPU: one GPU only (a
request for more exits with a message and status 2), and the traffic
figures are read from the committed counter summary only when it was taken
on the current kernel sources."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_summary_needs_the_current_sources(tmp_path, monkeypatch):
    good = (f"# header\nkernel_sources_sha256 {bench.kernel_sources_sha256()}\n"
            "traffic k_decode fetch=1.5e+09 write=2.0e+09 total=3.5e+09\n")
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "t.txt").write_text(good)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", "profiles/t.txt")
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda: good.split()[3])
    assert bench.measured_traffic() == {"k_decode": {"fetch": 1.5e9, "write": 2.0e9, "total": 3.5e9}}
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda: "0" * 64)
    assert bench.measured_traffic() == {}
