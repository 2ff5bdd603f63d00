"""Host-side checks of bench.py: the one-GPU contract and the bookkeeping that
decides whether the committed HBM-traffic record still describes the kernel."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_source_digest_ignores_comments_and_layout_only(tmp_path):
    a = tmp_path / "a.hpp"
    b = tmp_path / "b.hpp"
    c = tmp_path / "c.hpp"
    a.write_text("// header\nint f(int x) { return x + 1; }  /* trailing */\n")
    b.write_text("/* another\n   comment */\nint f(int x)\n{\n  return x + 1;\n}\n")
    c.write_text("int f(int x) { return x + 2; }\n")
    da, db, dc = (bench.source_digest([str(p)]) for p in (a, b, c))
    assert da == db
    assert da != dc


def test_measured_traffic_follows_the_record_digest(tmp_path, monkeypatch):
    rec = json.load(open(bench.TRAFFIC_RECORD))
    current = bench.source_digest(rec["sources"]) == rec["source_digest"]
    expected = int(rec["read_bytes"] + rec["write_bytes"]) if current else None
    assert bench.measured_traffic() == expected
    # a record whose digest no longer matches its sources yields no traffic figure
    stale = dict(rec, source_digest="0" * 64)
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(stale))
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(path))
    assert bench.measured_traffic() is None


def test_measured_counters_follow_the_record_digest(tmp_path, monkeypatch):
    rec = json.load(open(bench.TRAFFIC_RECORD))
    current = bench.source_digest(rec["sources"]) == rec["source_digest"]
    got = bench.measured_counters()
    if current:
        assert got["lds_bank_conflict_cycles"] == 0
        assert 0 < got["mfma_busy_under_profiler"] <= 1
        # every MFMA op is bf16: 2 * 4096^3 flop at 512 flop per op
        assert got["mfma_mops_bf16"] * 512 == 2 * 4096 ** 3
    else:
        assert got is None
    stale = dict(rec, source_digest="0" * 64)
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(stale))
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(path))
    assert bench.measured_counters() is None


def test_unknown_extra_workload_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--extra", "gemm_sizes,nonesuch"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "nonesuch" in r.stderr and "gemm_sizes" not in r.stderr.split("choose from")[0]
    assert r.stdout == ""
