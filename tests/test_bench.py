"""Host logic of bench.py (CPU only)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_source_hash_is_sha256_hex():
    h = bench.kernel_source_hash()
    assert len(h) == 64 and int(h, 16) >= 0


def _summary(path, sha, fetch=1000.0, fscale=2.0, write=10.0, wscale=1.0):
    with open(path, "w") as f:
        f.write("# summary\n\n")
        f.write(f"- kernel_source_sha256: {sha}\n- fetch_kib_per_dispatch: {fetch}\n")
        f.write(f"- fetch_scale: {fscale}\n- write_kib_per_dispatch: {write}\n- write_scale: {wscale}\n")


def test_measured_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    path = tmp_path / f"{bench.KERNEL}_decode_hbm_counters.md"
    assert bench.measured_traffic("decode") is None          # no summary
    _summary(path, bench.kernel_source_hash())
    assert bench.measured_traffic("decode") == (1000.0 * 2.0 + 10.0 * 1.0) * 1024.0
    _summary(path, "0" * 64)                                  # other sources
    assert bench.measured_traffic("decode") is None
