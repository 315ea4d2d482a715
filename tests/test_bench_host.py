"""bench.py's host logic without a GPU: the one-GPU guard, and the rule that a committed HBM
counter summary is used only for the kernel sources it was taken on."""

import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_summary_follows_the_source_hash(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    f.write_text("# a comment = not a field\nsource_hash = abc123\nhbm_bytes_per_call = 4096\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.read_traffic("abc123") == 4096.0
    assert bench.read_traffic("def456") is None          # other kernel sources: not used
    f.write_text("source_hash = abc123\n")                # no byte count: not used
    assert bench.read_traffic("abc123") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.read_traffic("abc123") is None


def test_committed_traffic_summary():
    """The committed counter summary carries both fields; when it was taken on other decode
    sources bench.py reports traffic as null, and this says so."""
    fields = {}
    with open(bench.TRAFFIC_FILE) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                fields[k.strip()] = v.strip()
    assert len(fields.get("source_hash", "")) == 16
    assert float(fields["hbm_bytes_per_call"]) > 1e9
    if bench.read_traffic(bench.kernel_source_hash(*bench.DECODE_SOURCES)) is None:
        pytest.skip("the counter summary predates the current decode sources")


def test_source_hash_covers_the_named_sources_only():
    all_h = bench.kernel_source_hash()
    dec_h = bench.kernel_source_hash(*bench.DECODE_SOURCES)
    mq_h = bench.kernel_source_hash("pa_mq.hip")
    assert len({all_h, dec_h, mq_h}) == 3
    assert dec_h == bench.kernel_source_hash(*bench.DECODE_SOURCES)  # deterministic
