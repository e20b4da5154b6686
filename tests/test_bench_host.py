"""Host-side checks of bench.py's contract pieces that need no GPU: the refusal of more than one
GPU, and the reading of HBM traffic from a rocprofv3 counter summary keyed by the kernel sources."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def _summary(path, sha, hbm):
    path.write_text("# HBM traffic and counters: k, workload w\n\n"
                    f"kernel_source_sha256_16: {sha}\nfetch_kib_per_dispatch: 1.0\nhbm_bytes_per_launch: {hbm}\n")


def test_traffic_is_read_when_the_summary_matches_the_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    for src in bench.KERNEL_SOURCES:          # same relative source paths, same contents
        dst = tmp_path / src
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(ROOT, src), "rb").read())
    _summary(prof / "attn_fwd_wl_hbm_counters.txt", bench.kernel_source_hash(), 12345)
    assert bench.read_traffic("attn_fwd", "wl") == 12345.0


def test_traffic_is_null_for_a_stale_or_missing_summary(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    for src in bench.KERNEL_SOURCES:
        dst = tmp_path / src
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(ROOT, src), "rb").read())
    _summary(prof / "attn_fwd_wl_hbm_counters.txt", "0000000000000000", 12345)
    assert bench.read_traffic("attn_fwd", "wl") is None
    assert bench.read_traffic("attn_bwd_dq", "wl") is None
