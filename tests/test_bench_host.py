"""Host-side checks of bench.py: the one-GPU contract, and the bookkeeping that
writes the committed counter record and decides whether it still describes
the kernel in the built library."""
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


def test_headline_kernel_is_found_in_the_built_library():
    """The record is keyed on the headline kernel's machine code: exactly one
    kernel of the built library matches its symbol, and the digest is stable."""
    from mma_fragment_layouts_amd import codeobj, library_path
    name, d = codeobj.kernel_digest(library_path(), bench.HEADLINE_SYMBOL)
    assert "gemm_fast_kernel" in name and len(d) == 64
    assert bench.headline_digest() == d
    # every instantiation of the fast kernel is a separate, distinct kernel
    ks = codeobj.kernels(library_path())
    fast = {n: v for n, v in ks.items() if "gemm_fast_kernel" in n}
    assert len(fast) >= 8 and len(set(fast.values())) == len(fast)


def test_counter_record_follows_the_code_digest(tmp_path, monkeypatch):
    rec = json.load(open(bench.TRAFFIC_RECORD))
    current = rec.get("code_digest") == bench.headline_digest()
    got = bench.counter_record()
    assert (got is not None) == current
    if current:
        c = bench.measured_counters(got)
        assert c["lds_bank_conflict_cycles"] == 0
        assert 0 < c["mfma_busy_under_profiler"] <= 1
        # every MFMA op is bf16: 2 * 4096^3 flop at 512 flop per op
        assert c["mfma_mops_bf16"] * 512 == 2 * 4096 ** 3
        assert bench.measured_traffic(got) == int(rec["read_bytes"] + rec["write_bytes"])
    # a record taken on other machine code yields neither counters nor traffic
    stale = dict(rec, code_digest="0" * 64)
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(stale))
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(path))
    assert bench.counter_record() is None
    assert bench.measured_counters(None) is None and bench.measured_traffic(None) is None


def _fake_run(directory, kernel_rows):
    """A rocprofv3 counter_collection.csv with the given (kernel, dispatch,
    counter, value) rows (kernel names contain commas, as the profiler's do)."""
    import csv
    directory.mkdir(parents=True)
    cols = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
            "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
            "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(directory / "p_counter_collection.csv", "w", newline="") as fh:
        w = csv.writer(fh, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(cols)
        for kern, disp, name, val in kernel_rows:
            w.writerow([disp, disp, "Agent 1", 1, 1, 1, 1, 1, kern, 256, 0, 0, 8, 0, 32, name, val, 0, 1])


def test_record_counters_from_profiler_runs(tmp_path, monkeypatch):
    """The record is computed from the profiler's CSV: the last N dispatches of
    the headline kernel averaged, byte counters scaled by the copies' reads."""
    gemm = "void mfl::" + bench.HEADLINE_PROFILED + "(unsigned short const*, unsigned short const*, float*, ...)"
    copy = "__amd_rocclr_copyBuffer"
    a_rows, f_rows, w_rows = [], [], []
    for d in range(10):   # dispatches 0..9; the first three (pre-warm) differ
        early = d < 3
        for name, val in (("SQ_VALU_MFMA_BUSY_CYCLES", 134217728), ("GRBM_GUI_ACTIVE", 8 * (300000 if early else 200000)),
                          ("SQ_LDS_IDX_ACTIVE", 16777216), ("SQ_LDS_BANK_CONFLICT", 0), ("SQ_INSTS_LDS", 4194304),
                          ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 268435456)):
            a_rows.append((gemm, d, name, val))
        f_rows.append((gemm, d, "FETCH_SIZE", 98304.0))
        w_rows.append((gemm, d, "WRITE_SIZE", 65536.0))
    for d in range(10, 13):
        f_rows.append((copy, d, "FETCH_SIZE", 131072.0))   # reads 256 MiB, counter shows half
        w_rows.append((copy, d, "WRITE_SIZE", 262144.0))
    _fake_run(tmp_path / "A", a_rows)
    _fake_run(tmp_path / "F", f_rows)
    _fake_run(tmp_path / "W", w_rows)
    out = tmp_path / "record.json"
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(out))
    bench.record_counters(str(tmp_path / "A"), str(tmp_path / "F"), str(tmp_path / "W"), last=7, commands="x")
    rec = json.load(open(out))
    assert rec["code_digest"] == bench.headline_digest()
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["read_bytes"] == 98304 * 1024 * 2 and rec["write_bytes"] == 64 << 20
    c = rec["counters"]
    assert c["gui_active_cycles_per_xcd"] == 200000
    assert abs(c["mfma_busy_under_profiler"] - 134217728 / (200000 * 1024)) < 1e-4
    assert bench.counter_record() == rec


def test_unknown_extra_workload_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--extra", "gemm_sizes,nonesuch"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "nonesuch" in r.stderr and "gemm_sizes" not in r.stderr.split("choose from")[0]
    assert r.stdout == ""
