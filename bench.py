#!/usr/bin/env python3
"""Benchmark of the MFMA fragment-layout GEMM library on one MI355X.

Headline workload: dense GEMM M = N = K = 4096, bf16 operands (A row-major,
B column-major, leading dimension 4096 + 64 with NaN padding), fp32
accumulation and fp32 output (ldc = 4096).  One step = one gemm_tile_mma call
(global -> swizzled LDS -> MFMA with register accumulators -> one store per
output element).  Operands are rounded to bf16 by the library before timing,
as the workload specifies bf16 inputs.

Timing: prewarm_ms (default 100) of untimed back-to-back steps — the GPU takes
about 200 launches to settle after a cold start — then W untimed warm-up steps,
then exactly K timed steps between two synchronisations.

Prints ONE JSON line with the metric, a roofline object for the GEMM kernel
(flops per launch / mean launch time from HIP events on the launch stream),
the CPU oracle's throughput on the host cores, and per-workload figures for
the other workloads (single 256^3 GEMM, the 4096^3 GEMM in every operand
order, block-repeat tiles, split fp32 GEMM with 1/2/3 chains, attention pair),
each timed as 3 warm-up launches (and at least 30 ms of settling launches) then
the best of 3 rounds of 20 back-to-back launches.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--prewarm-ms T] [--no-extra]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense fp16/bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk/CU
PEAK_HBM_GBS = 8000.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def event_time_ms(fn, n, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(n):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end)


def settle(fn, ms):
    """Launch fn back to back, untimed, for at least ms milliseconds: after host
    work the GPU has idled and its clocks take tens of milliseconds of load to
    settle again."""
    import torch
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(5):
            fn()
        torch.cuda.synchronize()


def best_of(fn, stream, warm=3, rounds=3, per=20, settle_ms=30.0):
    """Timing protocol of the Warp spike: 3 warm-up launches, then the best of
    3 rounds of 20 back-to-back launches; returns ms per launch.  The warm-up
    also runs for at least settle_ms (clock settling)."""
    for _ in range(warm):
        fn()
    settle(fn, settle_ms)
    return min(event_time_ms(fn, per, stream) for _ in range(rounds)) / per


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "gemm_4096_bf16_traffic.json")
# The headline kernel: mangled name in the code object, and as the profiler names it.
HEADLINE_SYMBOL = "gemm_fast_kernelILi256ELi256ELi4ELi4ELi0ELi1ELi2ELb0ELb0ELb0ELi2E"
HEADLINE_PROFILED = "gemm_fast_kernel<256, 256, 4, 4, 0, 1, 2, false, false, false, 2>"


def headline_digest():
    """sha256 of the headline kernel's gfx950 instructions and descriptor in the
    library that is built now (None if the library cannot be read)."""
    from mma_fragment_layouts_amd import codeobj, library_path
    try:
        return codeobj.kernel_digest(library_path(), HEADLINE_SYMBOL)[1]
    except Exception:
        return None


def counter_record():
    """The committed rocprofv3 record of the headline kernel, or None when it
    was taken on other machine code than the library built now (the record
    stores the digest of the kernel it measured; nothing re-keys it by hand)."""
    try:
        rec = json.load(open(TRAFFIC_RECORD))
    except Exception:
        return None
    d = headline_digest()
    return rec if d is not None and rec.get("code_digest") == d else None


def measured_counters(rec):
    """MFMA-busy and LDS counters per GEMM launch from the record."""
    if rec is None:
        return None
    c = dict(rec["counters"])
    c.pop("note", None)
    c["source"] = "profiles/gemm_4096_bf16_counters.md"
    return c


def measured_traffic(rec):
    """HBM bytes per GEMM launch (FETCH_SIZE and WRITE_SIZE scaled by a plain copy)."""
    return None if rec is None else int(rec["read_bytes"] + rec["write_bytes"])


def _counter_rows(directory):
    """{kernel name: {dispatch id: {counter: value}}} from a rocprofv3 --pmc run."""
    import csv
    import glob
    rows = {}
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            rows.setdefault(r["Kernel_Name"], {}).setdefault(int(r["Dispatch_Id"]), {})[r["Counter_Name"]] = \
                float(r["Counter_Value"])
    return rows


def record_counters(dir_a, dir_f, dir_w, last, commands):
    """Write the counter record of the headline kernel from three rocprofv3
    --pmc runs of this benchmark (group A: MFMA busy, LDS; FETCH_SIZE; WRITE_SIZE,
    the last two with --copy-calibration).  Per-dispatch values are averaged
    over the last `last` dispatches of the kernel (warm-up and timed steps);
    the byte counters are scaled by what they read for the 256 MiB copies.
    The record carries the digest of the kernel in the library built now, which
    must be the library the runs used."""
    def per_dispatch(directory, kernel, counters, n):
        rows = [v for k, v in _counter_rows(directory).items() if kernel in k]
        disp = sorted((i, c) for r in rows for i, c in r.items())
        if len(disp) < n:
            raise SystemExit(f"{directory}: {len(disp)} dispatches of {kernel}, need {n}")
        take = [c for _, c in disp[-n:]]
        return {name: sum(c[name] for c in take) / n for name in counters}

    a = per_dispatch(dir_a, HEADLINE_PROFILED, ["SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE",
                                                "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS",
                                                "SQ_INSTS_VALU_MFMA_MOPS_BF16"], last)
    f = per_dispatch(dir_f, HEADLINE_PROFILED, ["FETCH_SIZE"], last)["FETCH_SIZE"]
    w = per_dispatch(dir_w, HEADLINE_PROFILED, ["WRITE_SIZE"], last)["WRITE_SIZE"]
    cf = per_dispatch(dir_f, "copyBuffer", ["FETCH_SIZE"], 3)["FETCH_SIZE"]
    cw = per_dispatch(dir_w, "copyBuffer", ["WRITE_SIZE"], 3)["WRITE_SIZE"]
    copy_bytes = 256 << 20
    ff, fw = copy_bytes / 1024 / cf, copy_bytes / 1024 / cw
    gui_per_xcd = a["GRBM_GUI_ACTIVE"] / 8
    digest = headline_digest()
    if digest is None:
        raise SystemExit("cannot read the headline kernel from the built library")
    rec = {
        "kernel": HEADLINE_PROFILED,
        "kernel_symbol": HEADLINE_SYMBOL,
        "workload": "M=N=K=4096 bf16, lda=ldb=4160, ldc=4096",
        "code_digest": digest,
        "digest": "sha256 of the kernel's gfx950 instructions and descriptor in lib/libmfl.so "
                  "(mma_fragment_layouts_amd/codeobj.py)",
        "commands": commands,
        "dispatches_averaged": last,
        "fetch_size_kib_raw": round(f, 2), "write_size_kib_raw": round(w, 2),
        "copy_fetch_kib_raw": round(cf, 2), "copy_write_kib_raw": round(cw, 2), "copy_bytes": copy_bytes,
        "fetch_scale": round(ff, 4), "write_scale": round(fw, 4),
        "read_bytes": int(round(f * 1024 * ff)), "write_bytes": int(round(w * 1024 * fw)),
        "counters": {
            "mfma_busy_under_profiler": round(a["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui_per_xcd * 1024), 4),
            "lds_bank_conflict_cycles": int(a["SQ_LDS_BANK_CONFLICT"]),
            "lds_active_cycles": int(a["SQ_LDS_IDX_ACTIVE"]),
            "mfma_mops_bf16": int(a["SQ_INSTS_VALU_MFMA_MOPS_BF16"]),
            "lds_instructions": int(a["SQ_INSTS_LDS"]),
            "gui_active_cycles_per_xcd": int(gui_per_xcd),
            "note": "per dispatch; under the profiler every dispatch is serialised with a counter read-out, "
                    "so MFMA busy is below the timed run's"},
    }
    with open(TRAFFIC_RECORD, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec, indent=1))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(a, bt, budget_s=10.0, max_runs=20):
    """The oracle as it stands (numpy fp64 on the quantised inputs), timed on the
    host's cores over the full 4096^3 problem, repeated for about budget_s
    seconds; the median run is reported."""
    from oracle import reference as R
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"),
                      default=1)
    except Exception:
        threads = os.cpu_count() or 1
    runs = []
    start = time.perf_counter()
    while len(runs) < max_runs and (not runs or time.perf_counter() - start < budget_s):
        t0 = time.perf_counter()
        R.gemm_ref(a[:, :4096], bt[:, :4096], "bf16")
        runs.append(time.perf_counter() - t0)
    dt = float(np.median(runs))
    return {"value": 2 * 4096 ** 3 / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"full 4096^3 bf16 GEMM (RNE quantisation of A and B plus the fp64 matmul), median of "
                      f"{len(runs)} runs in {time.perf_counter() - start:.1f} s",
            "seconds": round(dt, 3), "cpu_model": cpu_model(), "nproc": os.cpu_count()}


def sclk_under_load(step, torch, seconds=1.0):
    """SCLK (MHz) read by rocm-smi, run as a child process, while the GEMM runs
    back to back; None if the tool or its output is unavailable."""
    import re
    import subprocess
    import threading
    found = {}

    def probe():
        time.sleep(seconds / 2)
        try:
            out = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                                 timeout=30).stdout
            for card in json.loads(out).values():
                for key, val in card.items():
                    if key.lower().startswith("sclk"):
                        m = re.search(r"(\d+)\s*mhz", str(val), re.I)
                        if m:
                            found["mhz"] = int(m.group(1))
        except Exception:
            pass

    th = threading.Thread(target=probe)
    th.start()
    t0 = time.perf_counter()
    while th.is_alive() and time.perf_counter() - t0 < 60:
        for _ in range(50):
            step()
        torch.cuda.synchronize()
    th.join()
    return found.get("mhz")


def mfma_ceiling(torch, mfl, stream, iters=512):
    """What the matrix cores sustain with nothing else running: the library's
    mfma_rate_probe (16 independent bf16 16x16x32 chains per wave, hashed operand
    values, no memory or LDS traffic), timed like the other workloads."""
    dev = torch.device("cuda:0")
    out = torch.empty((mfl.RATE_PROBE_OUTPUTS,), device=dev)
    ms = best_of(lambda: mfl.mfma_rate_probe(mfl.BF16, iters, 0x9E3779B9, out, stream), stream, per=10)
    tf = mfl.mfma_rate_flops(iters) / ms / 1e9
    return {"tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "probe": f"mfma_rate_probe: {mfl.RATE_PROBE_OUTPUTS // 64} waves x {iters} x 16 bf16 16x16x32 MFMA, "
                     "no memory traffic"}


EXTRA = ("gemm_256", "gemm_orders", "block_repeat", "split", "attention")
# opt-in legs (not run by default)
EXTRA_OPTIONAL = ("gemm_sizes", "attention_fused")


def extra_workloads(torch, mfl, inputs, stream, which=EXTRA):
    dev = torch.device("cuda:0")
    out = {}

    def q16(x, dt):
        src = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        o = torch.empty(src.shape, dtype=torch.int16, device=dev)
        mfl.quantize_fp32(dt, src, o, src.numel(), stream)
        return o

    if "gemm_256" in which:
        gemm_256(torch, mfl, inputs, stream, dev, q16, out)
    if "gemm_orders" in which:
        gemm_orders(torch, mfl, inputs, stream, dev, q16, out)
    if "block_repeat" in which:
        block_repeat(torch, mfl, inputs, stream, dev, q16, out)
    if "split" in which:
        split(torch, mfl, inputs, stream, dev, out)
    if "attention" in which:
        attention(torch, mfl, inputs, stream, dev, out)
    if "gemm_sizes" in which:
        gemm_sizes(torch, mfl, inputs, stream, dev, q16, out)
    if "attention_fused" in which:
        attention_fused(torch, mfl, inputs, stream, dev, out)
    return out


def gemm_256(torch, mfl, inputs, stream, dev, q16, out):
    """Single 256^3 fp16 GEMM (latency)."""
    a, bt = inputs.gemm_small()
    da, db = q16(a, mfl.F16), q16(bt, mfl.F16)
    c = torch.empty((256, 256), device=dev)
    call = lambda st: mfl.gemm_tile_mma(mfl.F16, 256, 256, 256, da, 256, 0, db, 256, 1, c, 256, 0, st)
    ms = best_of(lambda: call(stream), stream)
    # The same 20 back-to-back launches captured in one HIP graph: a replay has
    # no per-call host work, so it shows the launches' own latency.
    per = 20
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.graph(graph, stream=side):
        for _ in range(per):
            call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g_ms = best_of(graph.replay, stream, per=1) / per
    out["gemm_256_f16"] = {"us": round(ms * 1e3, 2), "tflops": round(2 * 256 ** 3 / ms / 1e9, 2),
                           "graph_us": round(g_ms * 1e3, 2), "bound": "latency (64 workgroups of 32 x 32)",
                           "frac_mfma_peak": round(2 * 256 ** 3 / ms / 1e9 / PEAK_BF16_TFLOPS, 5)}



def gemm_orders(torch, mfl, inputs, stream, dev, q16, out):
    """The 4096^3 bf16 GEMM in each operand order (ld 4160, NaN padding).  A
    column-major or B row-major operand is staged as k-major LDS slabs and read
    with the transpose read.  Also the K-contiguous order with fp16 operands and
    with the 32x32x16 instruction."""
    a, bt = inputs.gemm_dense()
    n = 4096

    def padded(x):
        s = np.full((n, 4160), np.nan, np.float32)
        s[:, :n] = x
        return s

    store_a = {mfl.ROW_MAJOR: a, mfl.COL_MAJOR: padded(a[:, :n].T)}
    store_b = {mfl.COL_MAJOR: bt, mfl.ROW_MAJOR: padded(bt[:, :n].T)}
    name = {mfl.ROW_MAJOR: "row", mfl.COL_MAJOR: "col"}
    c = torch.empty((n, n), device=dev)
    res = {}
    for oa in (mfl.ROW_MAJOR, mfl.COL_MAJOR):
        for ob in (mfl.COL_MAJOR, mfl.ROW_MAJOR):
            da, db = q16(store_a[oa], mfl.BF16), q16(store_b[ob], mfl.BF16)
            # both instructions: a k-major operand moves the same LDS bytes per
            # flop with either, but the reads differ in count and phase pattern
            for shape, suffix in ((0, ""), (1, "_32x32x16")):
                ms = best_of(lambda: mfl.gemm_tile_mma_shape(shape, mfl.BF16, n, n, n, da, 4160, oa, db, 4160, ob, c, n,
                                                             0, stream), stream)
                tf = 2 * n ** 3 / ms / 1e9
                res[f"A_{name[oa]}_B_{name[ob]}{suffix}"] = {"us": round(ms * 1e3, 1), "tflops": round(tf, 1),
                                                             "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
            del da, db
    out["gemm_4096_bf16_orders"] = res
    # The K-contiguous order with fp16 operands, and with the 32x32x16 instruction.
    var = {}
    for label, dt, shape in (("f16_16x16x32", mfl.F16, 0), ("bf16_32x32x16", mfl.BF16, 1)):
        da, db = q16(a, dt), q16(bt, dt)
        ms = best_of(lambda: mfl.gemm_tile_mma_shape(shape, dt, n, n, n, da, 4160, mfl.ROW_MAJOR, db, 4160,
                                                     mfl.COL_MAJOR, c, n, 0, stream), stream)
        tf = 2 * n ** 3 / ms / 1e9
        var[label] = {"us": round(ms * 1e3, 1), "tflops": round(tf, 1), "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        del da, db
    out["gemm_4096_variants"] = var


def gemm_sizes(torch, mfl, inputs, stream, dev, q16, out):
    """The bf16 GEMM (A row-major, B column-major, fp32 C, ld = n + 64) at square
    sizes from 1024 to 8192.  The fast path covers C with 256 x 256 tiles, one
    workgroup each: 4096^3 is one tile per compute unit, so every unit stores its
    fp32 tile at the same moment; at 8192^3 (four tiles per unit) a tile's store
    can overlap other units' K loops."""
    res = {}
    for n in (1024, 2048, 3072, 4096, 6144, 8192):
        a, bt = inputs.gemm_dense(n, n, n)
        ld = a.shape[1]
        da, db = q16(a, mfl.BF16), q16(bt, mfl.BF16)
        del a, bt
        c = torch.empty((n, n), device=dev)
        ms = best_of(lambda: mfl.gemm_tile_mma(mfl.BF16, n, n, n, da, ld, mfl.ROW_MAJOR, db, ld, mfl.COL_MAJOR, c, n,
                                               0, stream), stream)
        tf = 2 * n ** 3 / ms / 1e9
        tiles = ((n + 255) // 256) ** 2
        res[str(n)] = {"us": round(ms * 1e3, 1), "tflops": round(tf, 1), "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                       "tiles_256_per_cu": round(tiles / 256, 3)}
        log(f"gemm {n}^3: {ms * 1e3:.1f} us, {tf:.1f} TFLOP/s")
        del da, db, c
    out["gemm_bf16_sizes"] = res


def block_repeat(torch, mfl, inputs, stream, dev, q16, out):
    """2048^2 output, 64 repeats; both arms of the Warp spike's comparison: the
    register accumulator with swizzled LDS and the shared-memory API (plain LDS
    tiles, C through LDS on every repeat)."""
    rep = {}
    for tm, tn, tk, th in [(64, 64, 64, 64), (64, 64, 64, 128), (64, 64, 64, 256), (32, 32, 32, 128),
                           (128, 128, 32, 128), (128, 128, 32, 256)]:
        for name, dt in (("f16", mfl.F16), ("bf16", mfl.BF16)):
            a, bt = inputs.block_repeat(tm, tn, tk)
            da, db = q16(a, dt), q16(bt, dt)
            c = torch.empty((2048, 2048), device=dev)
            ms = best_of(lambda: mfl.gemm_block_repeat(dt, tm, tn, tk, th, 64, 2048, 2048, da, db, c, stream), stream)
            ms_lds = best_of(lambda: mfl.gemm_block_repeat_lds_api(dt, tm, tn, tk, th, 64, 2048, 2048, da, db, c,
                                                                   stream), stream)
            tf = 2 * 2048 * 2048 * tk * 64 / ms / 1e9
            tf_lds = 2 * 2048 * 2048 * tk * 64 / ms_lds / 1e9
            rep[f"{tm}x{tn}x{tk}/{th}/{name}"] = {"tflops": round(tf, 1), "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                                                 "lds_api_tflops": round(tf_lds, 1),
                                                 "register_over_lds_api": round(tf / tf_lds, 2)}
    out["block_repeat"] = rep


def split(torch, mfl, inputs, stream, dev, out):
    """Split fp32 GEMM 4096^3, bf16 pieces: the planes path (each operand split
    once into hi / lo planes, the split pass included in the time) and the
    split-on-load kernel."""
    a, bt = inputs.gemm_split()
    da = torch.from_numpy(a).to(dev)
    db = torch.from_numpy(bt).to(dev)
    c = torch.empty((4096, 4096), device=dev)
    wsb = mfl.gemm_split_fp32_workspace_bytes(4096, 4096, 4096, 4096, 0, 1, 4096, 1, 1, 4096)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    sp = {}
    for chains, lolo in ((1, 0), (2, 0), (3, 0), (3, 1)):
        ms = best_of(lambda: mfl.gemm_split_fp32_ws(mfl.BF16, 4096, 4096, 4096, da, 4096, 0, 1, db, 4096, 1, 1, chains,
                                                    lolo, c, 4096, 0, ws, wsb, stream), stream, rounds=2, per=5)
        ms_load = best_of(lambda: mfl.gemm_split_fp32(mfl.BF16, 4096, 4096, 4096, da, 4096, 0, 1, db, 4096, 1, 1, chains,
                                                      lolo, c, 4096, 0, stream), stream, rounds=2, per=5)
        nprod = 3 + lolo
        mf = nprod * 2 * 4096 ** 3 / ms / 1e9
        sp[f"chains{chains}{'+lolo' if lolo else ''}"] = {
            "us": round(ms * 1e3, 1), "useful_tflops": round(2 * 4096 ** 3 / ms / 1e9, 1),
            "mfma_tflops": round(mf, 1), "frac_mfma_peak": round(mf / PEAK_BF16_TFLOPS, 4),
            "split_on_load_us": round(ms_load * 1e3, 1)}
    # 3 chains with A column-major and B row-major (k-major planes, transpose reads)
    dat = torch.from_numpy(np.ascontiguousarray(a.T)).to(dev)
    dbt = torch.from_numpy(np.ascontiguousarray(bt.T)).to(dev)
    ms = best_of(lambda: mfl.gemm_split_fp32_ws(mfl.BF16, 4096, 4096, 4096, dat, 4096, 1, 1, dbt, 4096, 0, 1, 3, 0, c,
                                                4096, 0, ws, wsb, stream), stream, rounds=2, per=5)
    mf = 3 * 2 * 4096 ** 3 / ms / 1e9
    sp["chains3_A_col_B_row"] = {"us": round(ms * 1e3, 1), "useful_tflops": round(2 * 4096 ** 3 / ms / 1e9, 1),
                                 "mfma_tflops": round(mf, 1), "frac_mfma_peak": round(mf / PEAK_BF16_TFLOPS, 4)}
    out["split_4096"] = sp
    del da, db, dat, dbt, c, ws


def attention(torch, mfl, inputs, stream, dev, out):
    """Attention pair 2048 x nk x 128, all three algorithms, 1 and 2 chains, at the
    workload's 32,768 keys; and the fused and materialised algorithms at the
    other contexts of Strata PR #800's "Numbers" table, 8,192 and 131,072 keys."""
    for nk, algos, key in ((32768, ((mfl.ATTN_MATERIALISED, "materialised"), (mfl.ATTN_FUSED, "fused"),
                                     (mfl.ATTN_FUSED_SPLIT_KV, "fused_split_kv")), "attention_2048x32768"),
                           (8192, ((mfl.ATTN_MATERIALISED, "materialised"), (mfl.ATTN_FUSED, "fused")),
                            "attention_2048x8192"),
                           (131072, ((mfl.ATTN_MATERIALISED, "materialised"), (mfl.ATTN_FUSED, "fused")),
                            "attention_2048x131072")):
        q, k, v = inputs.attention(2048, nk)
        dq, dk, dv = (torch.from_numpy(x).to(dev) for x in (q, k, v))
        o = torch.empty((2048, 128), device=dev)
        att = {}
        for algo, aname in algos:
            wsb = mfl.attention_workspace_bytes(2048, nk, 128, algo)
            ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
            nprod = 3 if algo == mfl.ATTN_FUSED_SPLIT_KV else 2   # products per GEMM: hh, hl (, lh)
            for chains in (1, 2):
                ms = best_of(lambda: mfl.attention_split_fp32(2048, nk, 128, dq, dk, dv, chains, algo, o, ws, wsb,
                                                              stream), stream, rounds=2, per=5)
                mf = 2 * nprod * 2 * 2048 * nk * 128 / ms / 1e9   # 2 GEMMs x nprod products
                att[f"{aname}_chains{chains}"] = {"ms": round(ms, 4), "mfma_tflops": round(mf, 1),
                                                  "frac_mfma_peak": round(mf / PEAK_BF16_TFLOPS, 4)}
            del ws
        out[key] = att
        del dq, dk, dv, o


def attention_fused(torch, mfl, inputs, stream, dev, out):
    """The fused algorithm alone at 2048 x 32768 x 128 with 2 chains: the only
    attention launches of the run, so that a counter or trace run of this leg
    sees that kernel at that size and nothing else of its kind."""
    q, k, v = inputs.attention(2048, 32768)
    dq, dk, dv = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    o = torch.empty((2048, 128), device=dev)
    wsb = mfl.attention_workspace_bytes(2048, 32768, 128, mfl.ATTN_FUSED)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    ms = best_of(lambda: mfl.attention_split_fp32(2048, 32768, 128, dq, dk, dv, 2, mfl.ATTN_FUSED, o, ws, wsb, stream),
                 stream, rounds=2, per=5)
    mf = 2 * 2 * 2 * 2048 * 32768 * 128 / ms / 1e9
    out["attention_2048x32768_fused"] = {"ms": round(ms, 4), "mfma_tflops": round(mf, 1),
                                         "frac_mfma_peak": round(mf / PEAK_BF16_TFLOPS, 4)}
    del dq, dk, dv, o, ws


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--shape", type=int, default=0, help="MFMA shape of the GEMM fast path (0: 16x16x32, 1: 32x32x16)")
    p.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    p.add_argument("--extra", default=",".join(EXTRA),
                   help="comma list of the other workloads to run (" + ", ".join(EXTRA) + "; opt-in: " +
                   ", ".join(EXTRA_OPTIONAL) + ")")
    p.add_argument("--prewarm-ms", type=float, default=100.0,
                   help="untimed back-to-back GEMM launches before the warm-up steps, in ms (clock settling)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-clock", action="store_true", help="skip the SCLK reading under load")
    p.add_argument("--no-ceiling", action="store_true", help="skip the MFMA-rate ceiling measurement")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run 3 plain device copies of 256 MiB (reference for the HBM byte counters)")
    p.add_argument("--record-counters", nargs=3, metavar=("PMC_A_DIR", "FETCH_DIR", "WRITE_DIR"),
                   help="no GPU work: write profiles/gemm_4096_bf16_traffic.json from three rocprofv3 --pmc runs "
                        "of this benchmark (see profiles/gemm_4096_bf16_counters.md) and exit")
    p.add_argument("--record-last", type=int, default=7, help="dispatches averaged by --record-counters")
    p.add_argument("--record-commands", default="", help="the rocprofv3 commands, stored in the record")
    args = p.parse_args()
    if args.record_counters:
        record_counters(*args.record_counters, last=args.record_last, commands=args.record_commands)
        return
    which = tuple(w for w in args.extra.split(",") if w)
    unknown = [w for w in which if w not in EXTRA + EXTRA_OPTIONAL]
    if unknown:
        print(f"unknown --extra workloads {unknown}; choose from {EXTRA + EXTRA_OPTIONAL}", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the GEMM shards by output "
              "blocks with no exchange, so N GPUs would run N independent copies.", file=sys.stderr)
        sys.exit(2)

    import torch
    import mma_fragment_layouts_amd as mfl
    from mma_fragment_layouts_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mfl.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    M = N = K = 4096
    LD = 4096 + 64
    log("generating inputs")
    a, bt = inputs.gemm_dense()
    da32 = torch.from_numpy(a).to(dev)
    db32 = torch.from_numpy(bt).to(dev)
    da = torch.empty(da32.shape, dtype=torch.int16, device=dev)
    db = torch.empty(db32.shape, dtype=torch.int16, device=dev)
    mfl.quantize_fp32(mfl.BF16, da32, da, da32.numel(), stream)
    mfl.quantize_fp32(mfl.BF16, db32, db, db32.numel(), stream)
    del da32, db32
    c = torch.empty((M, N), device=dev)

    def step():
        mfl.gemm_tile_mma_shape(args.shape, mfl.BF16, M, N, K, da, LD, mfl.ROW_MAJOR, db, LD, mfl.COL_MAJOR, c, N, 0,
                                stream)

    # The GPU takes about 200 back-to-back launches (~25 ms) to settle after a
    # cold start (launches 100-199 measured 4-7 % slower than the steady state);
    # run the same step untimed for prewarm_ms before the warm-up steps.
    log("prewarm", args.prewarm_ms, "ms")
    settle(step, args.prewarm_ms)
    log("warmup", args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("timing", args.steps, "steps")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps
    flops = 2.0 * M * N * K
    ms_per_step = wall * 1e3 / args.steps
    value = flops * args.steps / wall / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    log(f"{value:.1f} TFLOP/s wall, {achieved:.1f} TFLOP/s by events, {kernel_ms * 1e3:.1f} us/launch")
    rec = counter_record() if args.shape == 0 else None

    result = {
        "metric": "GEMM TFLOP/s (bf16/fp16->fp32, 4096^3) and % of MI355X MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "dense GEMM M=N=K=4096, bf16 A row-major / B col-major, lda=ldb=4160 (NaN pad), "
                               "fp32 accumulate, fp32 C ldc=4096",
                   "m": M, "n": N, "k": K, "lda": LD, "ldb": LD, "ldc": N,
                   "mfma": "16x16x32" if args.shape == 0 else "32x32x16", "tile": "256x256x64, 16 waves (64x64 each)",
                   "prewarm_ms": args.prewarm_ms},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(rec),
                     "kernel_us": round(kernel_ms * 1e3, 2)},
        # MFMA busy and LDS bank conflicts of this kernel from the committed counter run
        "counters": measured_counters(rec) if args.shape == 0 else None,
    }
    if not args.no_clock:
        log("clock under load")
        mhz = sclk_under_load(step, torch)
        result["roofline"]["sclk_mhz_under_load"] = mhz
        if mhz:
            # the same 4096 flop/clock/CU at the clock the chip held under this load
            at_clk = 256 * 4096 * mhz * 1e6 / 1e12
            result["roofline"]["peak_at_sclk"] = round(at_clk, 1)
            result["roofline"]["frac_at_sclk"] = round(achieved / at_clk, 4)
    if not args.no_ceiling:
        log("mfma ceiling")
        ceil = mfma_ceiling(torch, mfl, stream)
        result["roofline"]["mfma_ceiling"] = ceil
        result["roofline"]["frac_of_ceiling"] = round(achieved / ceil["tflops"], 4)
    if args.copy_calibration:
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_extra:
        log("other workloads")
        result["workloads"] = extra_workloads(torch, mfl, inputs, stream, which)
    if not args.no_cpu:
        log("cpu oracle baseline")
        result["cpu_baseline"] = cpu_baseline(a, bt)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
