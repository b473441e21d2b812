#!/usr/bin/env python3
"""Benchmark of the BitLinear W1.58A8 hot path on one MI355X.

Headline (one JSON line on stdout): decode at model width, M=1 -- one pass of
the BitLinear FFN chain
    absmax-quant(x) -> up 2560->6912 (+ReLU^2) -> subln RMSNorm + requant
    -> down 6912->2560
on the decode workload's synthetic inputs (seed 1).  `value` is packed
ternary weight bytes streamed per second (8,847,360 bytes per step).  Weights
rotate over enough packed copies that every step reads them from HBM, not
from the 256 MB Infinity Cache.  A second figure times the same chain at
M=4096 (prefill, seed 3) and reports int8 TOPS of the two GEMMs.

Cold cache: the steps rotate over 64 packed copies of the step's weights
(566 MB), and right before the timed replay one pass over all copies is run
in the order the replay reads them, so every copy the timed steps read was
last read 63 copies (557 MB, over twice the 256 MB Infinity Cache) earlier,
whatever the step count: its weight bytes come from HBM, as in steady-state
decode where the other layers' weights are read in between.

Steps are launched from HIP graphs (one graph holds the K timed steps), so
the host does not limit the measured rate.  Weight packing is an offline step
(packed weights are the deployment format) and is timed separately.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0         # MI355X dense int8 MFMA, TOPS
MALL_BYTES = 256 * 1024 * 1024  # Infinity Cache
FLUSH_BYTES = 1 << 30           # read between the warm-up and a timed replay
ROOFLINE_COPIES = 128           # up-matrix copies the roofline loop rotates (566 MB)
H, F = 2560, 6912
PACKED_BYTES_MATRIX = H * F // 4              # 4,423,680
PACKED_BYTES_STEP = 2 * PACKED_BYTES_MATRIX  # 8,847,360
METRIC = "BitLinear W1.58A8 GB/s (M=1) & int8 TOPS (M=4096), % of MI355X roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def src_hash(*names):
    """Hash of the kernel sources and of the compiler flags they are built
    with (include paths left out: they differ between checkouts)."""
    from bit_gemm_absmax_amd import build as _build
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "bit_gemm_absmax_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    h.update(" ".join(f for f in _build.FLAGS if not f.startswith("-I")).encode())
    return h.hexdigest()[:16]


# Kernels whose rocprofv3 kernel-trace durations bench.py reports beside its
# own event timings: key -> (kernel name prefix, workgroups, sources)
DURATION_KERNELS = {
    "decode_up_m1": ("k_decode<4, 4, false, 3>", 432, ("gemv.hip", "bl_device.h")),
    "decode_down_m1": ("k_decode<8, 4, false, 4>", 160, ("gemv.hip", "bl_device.h")),
    "gemm_up_m4096": ("k_gemm_pipe<256, 256, 2, 4, 4, 1, ", 432, ("gemm.hip", "bl_device.h")),
    "gemm_down_m4096": ("k_gemm_pipe<256, 160, 4, 2, 4, 1, ", 256, ("gemm.hip", "bl_device.h")),
}


PROFILE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d {dir} -o bench -- python3 bench.py "
               "--steps 300 --warmup 20 --no-cpu --no-shapes")


def durations_from(trace_dir):
    """profiles/kernel_durations.json and a markdown table from a rocprofv3
    --kernel-trace run of bench.py: per kernel of DURATION_KERNELS, the
    average and median of its dispatch durations (GPU timestamps)."""
    import csv
    import glob
    import statistics
    def clean(name):
        name = name.replace("bl::(anonymous namespace)::", "")
        return name[5:] if name.startswith("void ") else name

    table = {}
    f = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    db = glob.glob(os.path.join(trace_dir, "**", "*results.db"), recursive=True)
    if f:
        for r in csv.DictReader(open(f[0])):
            wgs = int(r["Grid_Size_X"] if "Grid_Size_X" in r else r["Grid_Size"]) // \
                int(r["Workgroup_Size_X"] if "Workgroup_Size_X" in r else r["Workgroup_Size"])
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            table.setdefault((clean(r["Kernel_Name"]), wgs), []).append(dur)
    elif db:  # rocprofv3's default SQLite (rocpd) output
        import sqlite3
        con = sqlite3.connect(db[0])
        for name, gx, wx, t0, t1 in con.execute("select name, grid_x, workgroup_x, start, end from kernels"):
            table.setdefault((clean(name), gx // wx), []).append((t1 - t0) / 1e3)
    else:
        raise SystemExit(f"no kernel_trace.csv or results.db under {trace_dir}")
    rec = {"command": PROFILE_CMD.format(dir=trace_dir)}
    rows = []
    for key, (prefix, wgs, srcs) in DURATION_KERNELS.items():
        vals = [x for (n, w), v in table.items() if n.startswith(prefix) and w == wgs for x in v]
        if not vals:
            raise SystemExit(f"kernel {prefix} ({wgs} WGs) not in the trace")
        rec[key] = {"kernel": prefix, "workgroups": wgs, "calls": len(vals),
                    "avg_us": round(statistics.mean(vals), 3), "median_us": round(statistics.median(vals), 3),
                    "min_us": round(min(vals), 3), "source_hash": src_hash(*srcs)}
        rows.append(f"| {key} | `{prefix}` | {wgs} | {len(vals)} | {statistics.mean(vals):.3f} | "
                    f"{statistics.median(vals):.3f} | {min(vals):.3f} |")
    with open(os.path.join(ROOT, "profiles", "kernel_durations.json"), "w") as fo:
        json.dump(rec, fo, indent=1)
    print("| key | kernel | WGs | calls | avg us | median us | min us |")
    print("|---|---|---|---|---|---|---|")
    print("\n".join(rows))


def rocprof_figures(key, units_per_launch, peak):
    """The dominant kernel's rate from the committed rocprofv3 trace
    (profiles/kernel_durations.json), while its sources are unchanged."""
    try:
        with open(os.path.join(ROOT, "profiles", "kernel_durations.json")) as f:
            rec = json.load(f).get(key)
    except (OSError, ValueError):
        rec = None
    if not rec or rec.get("source_hash") != src_hash(*DURATION_KERNELS[key][2]):
        return {"rocprof_us_per_launch": None, "frac_rocprof": None}
    rate = units_per_launch / (rec["avg_us"] * 1e-6)
    return {"rocprof_us_per_launch": rec["avg_us"], "rocprof_median_us": rec["median_us"],
            "frac_rocprof": round(rate / peak, 4)}


def traffic_from_profile(kernel_key, sources):
    """HBM bytes per launch from committed PMC counters, only while the
    kernel's sources are unchanged since they were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != src_hash(*sources):
        return None
    return rec.get("bytes_per_launch")


# Kernels whose HBM traffic is taken from rocprofv3 counters: key -> (kernel
# name prefix in the trace, workgroups, sources whose hash the figures belong to)
TRAFFIC_KERNELS = {
    "decode_up_m1": ("k_decode<4, 4, false, 3>", 432, ("gemv.hip", "bl_device.h")),
    "gemm_up_m4096": ("k_gemm_pipe<256, 256, 2, 4, 4, 1, ", 432, ("gemm.hip", "bl_device.h")),
    "gemm_down_m4096": ("k_gemm_pipe<256, 160, 4, 2, 4, 1, ", 256, ("gemm.hip", "bl_device.h")),
    "batch_gate_m64": ("k_batch<4, 2, 2, 3, false, false>", 216, ("gemv.hip", "bl_device.h")),
    "batch_down_m64": ("k_batch<4, 1, 2, 7, false, false>", 160, ("gemv.hip", "bl_device.h")),
    "decode_tall_m1": ("k_decode_stream<4, 3, 1>", None, ("gemv.hip", "bl_device.h")),
}
CALIB_BYTES = 256 << 20   # the calibration kernel reads and writes 256 MiB
GEMM_BATCH = 10           # prefill GEMM launches per timed graph
# The three commands behind profiles/traffic.json ({fetch} and {write} are the
# counter output directories, the two arguments of --traffic-from).
PMC_CMDS = [
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch} -o p -- python3 bench.py --pmc-drive",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write} -o p -- python3 bench.py --pmc-drive",
    "python3 bench.py --traffic-from {fetch} {write}",
]


def pmc_drive():
    """The launches the traffic counters are read from: the decode up kernel
    over 128 weight copies (566 MB, over twice the Infinity Cache, so its
    weight bytes come from HBM), a plain
    elementwise pass over 256 MiB (x -> -x: reads and writes 256 MiB, the
    counters' calibration), the two prefill GEMMs, and the batched decode
    gate and down BitLinears at M=64 over 8 weight copies each."""
    import numpy as np
    import torch

    from bit_gemm_absmax_amd import bitlinear as bl
    from bit_gemm_absmax_amd import synth
    bl.load()
    dev = torch.device("cuda:0")
    d = synth.decode_gemv()
    pu, su = bl.pack_weights(torch.from_numpy(d["W_up"]).to(dev))
    ups = [bl.QuantForward(pu.clone(), su, 1, relu2=True) for _ in range(ROOFLINE_COPIES)]
    x = torch.from_numpy(d["X_up"]).to(dev)
    y = torch.empty((1, F), dtype=torch.float32, device=dev)
    for _ in range(3):
        for q in ups:
            q(x, y_out=y)
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst, ups
    p = synth.prefill()
    X = torch.from_numpy(p["X"]).to(dev)
    pu4, su4 = bl.pack_weights(torch.from_numpy(p["W_up"]).to(dev))
    pd4, sd4 = bl.pack_weights(torch.from_numpy(p["W_down"]).to(dev))
    xq, xs, rs = bl.quant_act(X)
    up = bl.forward(xq, xs, pu4, su4, x_rowsum=rs, relu2=True, subln=True)
    yu = torch.empty((X.shape[0], F), dtype=torch.float32, device=dev)
    yd = torch.empty((X.shape[0], H), dtype=torch.float32, device=dev)
    for _ in range(3):
        bl.forward(xq, xs, pu4, su4, x_rowsum=rs, relu2=True, y_out=yu)
        bl.forward(up["q"], up["q_scale"], pd4, sd4, x_rowsum=up["q_rowsum"], y_out=yd)
    torch.cuda.synchronize()
    del X, xq, up, yu, yd
    b = synth.batched_decode()
    pg, sg = bl.pack_weights(torch.from_numpy(b["W_gate"]).to(dev))
    pdb, sdb = bl.pack_weights(torch.from_numpy(b["W_down"]).to(dev))
    gates = [pg.clone() for _ in range(8)]
    downs = [pdb.clone() for _ in range(8)]
    x64 = torch.from_numpy(b["X64"]).to(dev)
    q64, s64, r64 = bl.quant_act(x64)
    h64 = torch.from_numpy(synth.activations(np.random.default_rng(7), 64, F)).to(dev)
    q2, s2, r2 = bl.quant_act(h64)
    yg = torch.empty((64, F), dtype=torch.float32, device=dev)
    yb = torch.empty((64, H), dtype=torch.float32, device=dev)
    for _ in range(3):
        for w in gates:
            bl.forward(q64, s64, w, sg, x_rowsum=r64, y_out=yg)
        for w in downs:
            bl.forward(q2, s2, w, sdb, x_rowsum=r2, y_out=yb)
    torch.cuda.synchronize()
    del gates, downs
    # the tall decode (2560 -> 131,328, persistent streaming launch) over 3
    # copies of its 84 MB matrix
    tall = pu.repeat(19, 1)
    talls = [tall] + [tall.clone() for _ in range(2)]
    qts = [bl.QuantForward(c, su, 1, relu2=True) for c in talls]
    yt = torch.empty((1, tall.shape[0]), dtype=torch.float32, device=dev)
    for _ in range(3):
        for q in qts:
            q(x, y_out=yt)
    torch.cuda.synchronize()
    log("pmc-drive done")


def traffic_from(fetch_dir, write_dir):
    """profiles/traffic.json and a markdown table from two rocprofv3 --pmc
    runs of --pmc-drive (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch).
    Each counter is scaled by what it reads for the calibration pass, whose
    true traffic is known (256 MiB each way)."""
    import csv
    import glob
    import statistics

    def per_kernel(d, counter):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not f:
            raise SystemExit(f"no counter_collection.csv under {d}")
        out = {}
        for r in csv.DictReader(open(f[0])):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"].replace("bl::(anonymous namespace)::", "")
            if name.startswith("void "):
                name = name[5:]
            wgs = int(r["Grid_Size"]) // int(r["Workgroup_Size"])
            out.setdefault((name, wgs), []).append(float(r["Counter_Value"]) * 1024.0)
        return out

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")

    def find(table, prefix, wgs):
        vals = [v for (n, w), v in table.items() if n.startswith(prefix) and (wgs is None or w == wgs)]
        if not vals:
            raise SystemExit(f"kernel {prefix} ({wgs} WGs) not in the counters")
        return statistics.median([x for v in vals for x in v])

    def calib(table):
        vals = [x for (n, w), v in table.items() if "neg_kernel" in n for x in v]
        if not vals:
            raise SystemExit("calibration pass (neg kernel) not in the counters")
        return CALIB_BYTES / statistics.median(vals)

    ff, fw = calib(fetch), calib(write)
    rec = {"calibration": {"pass": "torch.neg over 256 MiB fp32 (reads and writes 268,435,456 B)",
                           "fetch_factor": round(ff, 4), "write_factor": round(fw, 4)},
           "commands": [c.format(fetch=fetch_dir, write=write_dir) for c in PMC_CMDS]}
    rows = []
    for key, (prefix, wgs, srcs) in TRAFFIC_KERNELS.items():
        fb = find(fetch, prefix, wgs) * ff
        wb = find(write, prefix, wgs) * fw
        rec[key] = {"kernel": prefix, "workgroups": wgs, "fetch_bytes": round(fb), "write_bytes": round(wb),
                    "bytes_per_launch": round(fb + wb), "source_hash": src_hash(*srcs)}
        rows.append(f"| {key} | `{prefix}` | {wgs} | {fb / 1e6:.2f} | {wb / 1e6:.2f} | {(fb + wb) / 1e6:.2f} |")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print("| key | kernel | WGs | fetch MB | write MB | total MB |")
    print("|---|---|---|---|---|---|")
    print("\n".join(rows))
    print(f"\nCalibration: FETCH_SIZE x {ff:.4f}, WRITE_SIZE x {fw:.4f} "
          "(torch.neg over 256 MiB fp32 reads and writes 268,435,456 B).")


def flush_reader(torch, dev):
    """A callable that reads FLUSH_BYTES (torch's sum: plain loads, which
    allocate in the Infinity Cache) so that no weight copy stays there."""
    buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    def flush():
        buf.sum()
    return flush


def time_graph(torch, fn, reps=1):
    """Capture fn() into a HIP graph, replay once to warm, then time `reps`
    replays with events on the launch stream.  Returns seconds per replay."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # eager warm-up on the side stream (allocations settle)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / reps, g


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(budget_s=10.0):
    """The scalar oracle on this host: the decode step (M=1, seed 1) repeated
    for about budget_s seconds on one core (liboracle.so) and then on every
    core this process may use (liboracle_mt.so, the same per-element code with
    the outer loops split over threads, identical results); and a bounded
    sample of the prefill chain (64 of the 4096 rows, seed 3) on every core."""
    import numpy as np

    import oracle
    from bit_gemm_absmax_amd import synth
    d = synth.decode_gemv()
    qu, gu = oracle.quantize_weights(d["W_up"])
    qd, gd = oracle.quantize_weights(d["W_down"])
    x = d["X_up"]

    def steps(budget):
        n = 0
        t0 = time.perf_counter()
        while True:
            oracle.ffn_layer(x, qu, gu, qd, gd, pre_gain=None, residual=False)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return n, el

    with oracle.parallel(1):
        n1, el1 = steps(budget_s * 0.6)
    nthreads = oracle.default_threads()
    with oracle.parallel(nthreads) as used:
        nm, elm = steps(budget_s * 0.4)
        p = synth.prefill()
        qpu, gpu_ = oracle.quantize_weights(p["W_up"])
        qpd, gpd = oracle.quantize_weights(p["W_down"])
        rows = p["X"][:64]
        t0 = time.perf_counter()
        oracle.ffn_layer(rows, qpu, gpu_, qpd, gpd, pre_gain=None, residual=False)
        elp = time.perf_counter() - t0
    per1, perm = el1 / n1, elm / nm
    ops_p = 2.0 * 2 * 64 * H * F
    return {"value": round(PACKED_BYTES_STEP / perm / 1e9, 4), "unit": "GB/s", "cores": used,
            "kind": "oracle", "cpu_model": cpu_model(), "ms_per_step": round(perm * 1e3, 3),
            "sample": f"{nm} decode steps (M=1, up 2560->6912 + ReLU^2 + subln requant + down 6912->2560, "
                      f"seed 1) by the scalar C oracle's OpenMP build on {used} threads, {elm:.1f} s",
            "one_core": {"value": round(PACKED_BYTES_STEP / per1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                         "ms_per_step": round(per1 * 1e3, 3),
                         "sample": f"{n1} decode steps by the one-core build, {el1:.1f} s"},
            "prefill_rows": {"value": round(ops_p / elp / 1e12, 5), "unit": "TOPS", "cores": used,
                             "s": round(elp, 3),
                             "sample": "64 of the 4096 prefill rows (seed 3) through quant, up + ReLU^2, subln "
                                       "requant, down, on the OpenMP build"}}


def bench_batched(torch, bl, synth, dev, log):
    """Batched decode, M = 8, 32, 64 (seed 2): one layer's BitLinear set --
    quantise x, o 2560->2560, gate 2560->6912, up 2560->6912 (+ReLU^2, subln
    RMSNorm and int8 requant), down 6912->2560 -- over rotating packed copies
    (cold: more than twice the Infinity Cache).  o, gate and up read the same
    quantised rows, so the set runs them as one grouped launch
    (bitlinear_forward_grouped); each BitLinear alone is timed as well."""
    d = synth.batched_decode()
    names = ("o", "gate", "up", "down")
    packed = {}
    for n in names:
        W = torch.from_numpy(d[f"W_{n}"]).to(dev)
        packed[n] = bl.pack_weights(W)
        del W
    set_bytes = sum(packed[n][0].numel() for n in names)
    C = -(-(2 * MALL_BYTES) // set_bytes) + 1
    copies = [{n: packed[n][0].clone() for n in names} for _ in range(C)]
    scale = {n: packed[n][1] for n in names}
    out = []
    for M in (8, 32, 64):
        X = torch.from_numpy(d[f"X{M}"]).to(dev)
        xq, xs, rs = bl.quant_act(X)
        u0 = bl.forward(xq, xs, copies[0]["up"], scale["up"], x_rowsum=rs, relu2=True, subln=True)
        yo = torch.empty((M, H), dtype=torch.float32, device=dev)
        yg = torch.empty((M, F), dtype=torch.float32, device=dev)
        yu = torch.empty((M, F), dtype=torch.float32, device=dev)
        yd = torch.empty((M, H), dtype=torch.float32, device=dev)

        def one(n, c):
            if n == "o":
                bl.forward(xq, xs, c["o"], scale["o"], x_rowsum=rs, y_out=yo)
            elif n == "gate":
                bl.forward(xq, xs, c["gate"], scale["gate"], x_rowsum=rs, y_out=yg)
            elif n == "up":
                bl.forward(xq, xs, c["up"], scale["up"], x_rowsum=rs, relu2=True, subln=True, y_out=yu)
            else:
                bl.forward(u0["q"], u0["q_scale"], c["down"], scale["down"], x_rowsum=u0["q_rowsum"], y_out=yd)

        per = {}
        for n in names:
            t, gg = time_graph(torch, lambda n=n: [one(n, c) for c in copies], reps=3)
            del gg
            t /= C
            nb = copies[0][n].numel()
            per[n] = {"us": round(t * 1e6, 3), "GB_per_s": round(nb / t / 1e9, 1)}

        def grouped(c, a, b, r):
            return bl.forward_grouped(a, b, r, [
                {"packed": c["o"], "w_scale": scale["o"], "y_out": yo},
                {"packed": c["gate"], "w_scale": scale["gate"], "y_out": yg},
                {"packed": c["up"], "w_scale": scale["up"], "relu2": True, "subln": True, "y_out": yu}])

        qws = torch.empty(max(1, bl.load().bitlinear_quant_forward_grouped_workspace_bytes(M, H)), dtype=torch.uint8,
                          device=dev)

        def layer_set():
            # quantise x inside the grouped launch (a few tokens) or before it
            for c in copies:
                u = bl.quant_forward_grouped(X, [
                    {"packed": c["o"], "w_scale": scale["o"], "y_out": yo},
                    {"packed": c["gate"], "w_scale": scale["gate"], "y_out": yg},
                    {"packed": c["up"], "w_scale": scale["up"], "relu2": True, "subln": True, "y_out": yu}],
                    ws=qws)[2]
                bl.forward(u["q"], u["q_scale"], c["down"], scale["down"], x_rowsum=u["q_rowsum"], y_out=yd)

        def layer_set_two_step():
            for c in copies:
                a, b, r = bl.quant_act(X)
                u = grouped(c, a, b, r)[2]
                bl.forward(u["q"], u["q_scale"], c["down"], scale["down"], x_rowsum=u["q_rowsum"], y_out=yd)

        t, gg = time_graph(torch, layer_set, reps=3)
        del gg
        t /= C
        t2, gg = time_graph(torch, layer_set_two_step, reps=3)
        del gg
        t2 /= C
        tg, gg = time_graph(torch, lambda: [grouped(c, xq, xs, rs) for c in copies], reps=3)
        del gg
        tg /= C
        per["grouped_o_gate_up"] = {"us": round(tg * 1e6, 3),
                                    "GB_per_s": round(sum(copies[0][n].numel() for n in ("o", "gate", "up")) / tg / 1e9, 1),
                                    "note": "one launch for the three contractions, then the subln requant of up"}
        ops = 2.0 * M * set_bytes * 4
        floor = max(set_bytes / (HBM_PEAK_GBS * 1e9), ops / (INT8_PEAK_TOPS * 1e12))
        rec = {"M": M, "set_us": round(t * 1e6, 3), "set_two_step_us": round(t2 * 1e6, 3),
               "set_GB_per_s": round(set_bytes / t / 1e9, 1),
               "set_TOPS": round(ops / t / 1e12, 2), "roofline_frac": round(floor / t, 4), "kernels": per}
        out.append(rec)
        log(f"batched decode M={M}: set {t * 1e6:.2f} us -> {set_bytes / t / 1e9:.0f} GB/s "
            f"(quantiser as its own launch: {t2 * 1e6:.2f} us); "
            + ", ".join(f"{n} {per[n]['us']:.2f} us" for n in list(names) + ["grouped_o_gate_up"]))
    return {"workload": "batched decode, one layer's BitLinear set (quant, o 2560->2560, gate and up "
                        "2560->6912 as one grouped launch that quantises x itself up to 8 tokens, ReLU^2 + subln "
                        "requant, down 6912->2560), seed 2",
            "packed_bytes_per_set": int(set_bytes), "weight_copies": C,
            "roofline": "max(packed bytes / 8 TB/s, int8 ops / 5 POPS) over the measured time", "runs": out}


def bench_ffn_layers(torch, bl, synth, dev, log):
    """Context: one FFN layer through bitnet_ffn_forward at M = 8, 32, 64
    (pre-norm, residual), plain (up, down) and gated (gate and up in one
    launch, then down), over rotating copies that exceed twice the Infinity
    Cache; GB/s counts the packed bytes of the layer's matrices."""
    import numpy as np
    rng = np.random.default_rng(8)
    packs = {}
    for name, (n, k) in (("gate", (F, H)), ("up", (F, H)), ("down", (H, F))):
        Wt = torch.from_numpy(synth.weights(rng, n, k)).to(dev)
        packs[name] = bl.pack_weights(Wt)
        del Wt
    out = []
    for gated in (False, True):
        nb = (3 if gated else 2) * PACKED_BYTES_MATRIX
        R = max(2, -(-(2 * MALL_BYTES) // nb))
        layers = []
        for _ in range(R):
            L = {"up": packs["up"][0].clone(), "up_scale": packs["up"][1],
                 "down": packs["down"][0].clone(), "down_scale": packs["down"][1]}
            if gated:
                L.update(gate=packs["gate"][0].clone(), gate_scale=packs["gate"][1])
            layers.append(L)
        for M in (8, 32, 64):
            stacks = [bl.FFNStack([L], H, F, M, dev) for L in layers]
            h = torch.from_numpy(synth.activations(rng, M, H)).to(dev)

            def run():
                for st in stacks:
                    st(h)

            t, gg = time_graph(torch, run, reps=3)
            del gg
            t /= R
            log(f"FFN layer {'gated' if gated else 'plain'} M={M}: {t * 1e6:.2f} us -> {nb / t / 1e9:.0f} GB/s")
            out.append({"gated": gated, "M": M, "us": round(t * 1e6, 2), "packed_bytes": nb,
                        "GB_per_s": round(nb / t / 1e9, 1)})
            del stacks
        del layers
        torch.cuda.empty_cache()
    return {"workload": "one FFN layer (pre-norm, residual), hidden 2560, intermediate 6912, seed 8",
            "copies_rotated": "packed bytes over twice the Infinity Cache", "runs": out}


def bench_stack(torch, bl, synth, dev, log, passes=8):
    """The 30-layer FFN stack (seed 4) with pre-norm and residual, at M=1 and
    M=32, all layers' packed weights resident; the timed passes rotate over
    three copies of the stack so each pass reads its weights from HBM."""
    import numpy as np
    layers = []
    rng = None
    t0 = time.perf_counter()
    for rng, l, Wu, Wd in synth.ffn_stack_weights():
        pu, su = bl.pack_weights(torch.from_numpy(Wu).to(dev))
        pd, sd = bl.pack_weights(torch.from_numpy(Wd).to(dev))
        layers.append({"up": pu, "up_scale": su, "down": pd, "down_scale": sd})
    h0 = synth.ffn_stack_hidden(rng)
    log(f"stack weights generated and packed in {time.perf_counter() - t0:.1f} s")
    nbytes = sum(L["up"].numel() + L["down"].numel() for L in layers)
    R = max(2, -(-(2 * MALL_BYTES) // nbytes) + 1)
    sets = [layers] + [[{k: (v.clone() if k in ("up", "down") else v) for k, v in L.items()} for L in layers]
                       for _ in range(R - 1)]
    out = []
    for M in (1, 32):
        stacks = [bl.FFNStack(ls, H, F, M, dev) for ls in sets]
        h = torch.from_numpy(np.ascontiguousarray(h0[:M])).to(dev)

        def run():
            for i in range(passes):
                stacks[i % R](h)

        t, gg = time_graph(torch, run, reps=2)
        del gg
        t /= passes
        ops = 2.0 * M * nbytes * 4
        rec = {"M": M, "us_per_pass": round(t * 1e6, 2), "us_per_layer": round(t * 1e6 / len(layers), 3),
               "GB_per_s": round(nbytes / t / 1e9, 1), "TOPS": round(ops / t / 1e12, 3),
               "frac_hbm": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}
        out.append(rec)
        log(f"stack M={M}: {t * 1e6:.1f} us per 30-layer pass -> {nbytes / t / 1e9:.0f} GB/s")
        del stacks
        if M == 1:
            # the same pass as one persistent launch (BL_FFN_PERSISTENT)
            pst = [bl.FFNStack(ls, H, F, 1, dev, persistent=True) for ls in sets]

            def run_p():
                for i in range(passes):
                    pst[i % R](h)

            tp, gg = time_graph(torch, run_p, reps=2)
            del gg, pst
            tp /= passes
            rec["persistent_us_per_pass"] = round(tp * 1e6, 2)
            rec["persistent_us_per_layer"] = round(tp * 1e6 / len(layers), 3)
            rec["persistent_GB_per_s"] = round(nbytes / tp / 1e9, 1)
            log(f"stack M=1 persistent: {tp * 1e6:.1f} us per 30-layer pass -> {nbytes / tp / 1e9:.0f} GB/s")
    return {"workload": "30-layer FFN stack (RMSNorm, quant, up 2560->6912, ReLU^2, subln requant, down "
                        "6912->2560, residual add), seed 4",
            "layers": len(layers), "packed_bytes_per_pass": int(nbytes), "weight_copies": R,
            "launch": "HIP graph of the timed passes", "runs": out}


def tall_decode(torch, bl, d, pu, su, dev, log):
    """Context only: the M=1 decode kernel (fused quantisation + BitLinear +
    ReLU^2, K=2560) on a tall matrix, the seed-1 up weights repeated 19 times
    along N (131,328 rows, 84 MB packed), rotating over 7 such copies (588 MB,
    over twice the Infinity Cache): the kernel's streaming rate once one
    launch moves far more than its fixed latency."""
    reps = 19
    tall = pu.repeat(reps, 1)
    N = tall.shape[0]
    nb = tall.numel()
    copies = [tall] + [tall.clone() for _ in range(6)]
    qfs = [bl.QuantForward(c, su, 1, relu2=True) for c in copies]
    x = torch.from_numpy(d["X_up"]).to(dev)
    y = torch.empty((1, N), dtype=torch.float32, device=dev)

    def run():
        for q in qfs:
            q(x, y_out=y)

    t, gg = time_graph(torch, run, reps=3)
    del gg, copies, qfs, tall
    t /= 7
    log(f"decode M=1 2560->{N} (tall, {nb / 1e6:.0f} MB): {t * 1e6:.2f} us -> {nb / t / 1e9:.0f} GB/s")
    return {"K": 2560, "N": N, "packed_bytes": nb, "us_per_launch": round(t * 1e6, 2),
            "GB_per_s": round(nb / t / 1e9, 1), "frac_hbm": round(nb / t / 1e9 / HBM_PEAK_GBS, 4),
            "kernel": "k_decode_stream<4,3,1> (persistent: rows quantised once per workgroup, tiles streamed)",
            "traffic": traffic_from_profile("decode_tall_m1", ("gemv.hip", "bl_device.h")),
            "weights": "seed-1 up matrix repeated 19x along N; 7 copies rotated"}


def bench_latent(torch, bl, synth, dev, log):
    """Context: BitLinear from latent weights (ternarised inside the call, the
    training-time forward) at the up shape K=2560, N=6912, fp32 and bf16
    weights, M = 1 and 4096, rotating copies that exceed twice the Infinity
    Cache.  The packer reads the latent matrix twice (absmean, then
    ternarise + pack); GB/s counts one read of the latent bytes."""
    import numpy as np
    rng = np.random.default_rng(7)
    W = torch.from_numpy(synth.weights(rng, F, H)).to(dev)
    out = []
    for dtype, name in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        Wd = W.to(dtype)
        nb = Wd.numel() * Wd.element_size()
        copies = [Wd] + [Wd.clone() for _ in range(max(1, -(-(2 * MALL_BYTES) // nb)) - 1)]
        for M in (1, 4096):
            X = torch.from_numpy(synth.activations(rng, M, H)).to(dev)
            y = torch.empty((M, F), dtype=torch.float32, device=dev)

            def run():
                for c in copies:
                    bl.latent_forward(X, c, relu2=True, y_out=y)

            t, gg = time_graph(torch, run, reps=3)
            del gg
            t /= len(copies)
            log(f"latent forward {name} M={M}: {t * 1e6:.1f} us ({nb / t / 1e9:.0f} GB/s of latent weights)")
            out.append({"dtype": name, "M": M, "us": round(t * 1e6, 2), "latent_bytes": nb,
                        "GB_per_s": round(nb / t / 1e9, 1), "copies": len(copies)})
        del copies, Wd
        torch.cuda.empty_cache()
    return {"workload": "BitLinear from latent weights, K=2560, N=6912, +ReLU^2 (seed 7)", "runs": out}


def stream_read(torch, dev, log):
    """Context only: the read-bandwidth reference.  A plain streaming read of
    1 GiB (libblbench.so: 16-byte non-temporal loads, 8192 workgroups, every
    byte read once), and torch's sum over the same bytes for comparison."""
    import ctypes
    from bit_gemm_absmax_amd import build as blbuild
    if not os.path.exists(blbuild.BENCH_LIB):
        raise RuntimeError(f"{blbuild.BENCH_LIB} is not built (python -m bit_gemm_absmax_amd.build)")
    lib = ctypes.CDLL(blbuild.BENCH_LIB)
    lib.blbench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
    lib.blbench_stream_read.restype = ctypes.c_int
    nbytes = 1 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)

    def run():
        rc = lib.blbench_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"blbench_stream_read returned {rc}")

    t, gg = time_graph(torch, run, reps=20)
    del gg
    ts, gg = time_graph(torch, lambda: buf.sum(), reps=20)
    del gg, buf, sink
    gbs, gbs_sum = nbytes / t / 1e9, nbytes / ts / 1e9
    log(f"streaming read, 1 GiB: {gbs:.0f} GB/s (nt-load read kernel); torch.sum {gbs_sum:.0f} GB/s")
    return {"GB_per_s": round(gbs, 1), "torch_sum_GB_per_s": round(gbs_sum, 1),
            "kernel": "k_stream_read: 8192 x 256 threads, 8 x 16-byte nt loads in flight per thread"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--copies", type=int, default=64, help="packed weight copies rotated per step")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-shapes", action="store_true", help="skip the per-shape M=1 decode sweep")
    ap.add_argument("--no-batched", action="store_true", help="skip the batched decode (M = 8, 32, 64)")
    ap.add_argument("--no-stack", action="store_true", help="skip the 30-layer stack (M = 1, 32)")
    ap.add_argument("--no-latent", action="store_true", help="skip the latent-weight forward (M = 1, 4096)")
    ap.add_argument("--pmc-drive", action="store_true",
                    help="only run the launches the HBM traffic counters are read from")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc runs of --pmc-drive")
    ap.add_argument("--durations-from", metavar="TRACE_DIR",
                    help="write profiles/kernel_durations.json from a rocprofv3 --kernel-trace run of bench.py")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.durations_from:
        durations_from(args.durations_from)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the BitLinear path here has no multi-GPU "
              "(sharded) implementation; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.pmc_drive:
        pmc_drive()
        return

    import numpy as np
    import torch

    from bit_gemm_absmax_amd import bitlinear as bl
    from bit_gemm_absmax_amd import synth
    bl.load()  # raises if the HIP library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---------------------------------------------------------------- decode, M=1
    d = synth.decode_gemv()
    t0 = time.perf_counter()
    Wu = torch.from_numpy(d["W_up"]).to(dev)
    Wd = torch.from_numpy(d["W_down"]).to(dev)
    pu, su = bl.pack_weights(Wu)
    pd, sd = bl.pack_weights(Wd)
    torch.cuda.synchronize()
    pack_t, _ = time_graph(torch, lambda: (bl.pack_weights(Wu), bl.pack_weights(Wd)), reps=5)
    log(f"pack (offline) up+down: {pack_t * 1e3:.3f} ms")
    del Wu, Wd

    R = max(1, args.copies)
    reuse = (R - 1) * PACKED_BYTES_STEP  # other weight bytes read between two reads of one copy
    cold = reuse >= 2 * MALL_BYTES
    if not cold:
        log(f"warning: {R} copies ({R * PACKED_BYTES_STEP / 1e6:.0f} MB) fit the Infinity Cache; numbers are warm")
    layers = [{"up": pu.clone(), "up_scale": su, "down": pd.clone(), "down_scale": sd} for _ in range(R)]
    stacks = [bl.FFNStack([L], H, F, 1, dev, pre_norm=False, residual=False) for L in layers]
    x0 = torch.from_numpy(d["X_up"]).to(dev)
    h = x0.clone()

    def steps(n, start=0):
        for i in range(n):
            stacks[(start + i) % R](h)

    # warm-up (eager) then the timed K steps from one graph
    steps(args.warmup)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps(args.steps)
    g.replay()  # graph warm-up replay
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed_replay():
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / args.steps

    # the warm-up replay just read the copies the timed replay reads: one pass
    # over all copies in replay order, so each timed copy was last read R - 1
    # copies earlier
    steps(R)
    step_s = timed_replay()
    value = PACKED_BYTES_STEP / step_s / 1e9
    # context: the same replay after 1 GiB of unrelated reads (Infinity Cache
    # and address-translation caches cold)
    flush = flush_reader(torch, dev)
    flush()
    flushed_s = timed_replay()
    del flush
    log(f"decode step (graph): {step_s * 1e6:.2f} us -> {value:.1f} GB/s")

    # eager rate for context
    torch.cuda.synchronize()
    t = time.perf_counter()
    steps(200)
    torch.cuda.synchronize()
    eager_s = (time.perf_counter() - t) / 200
    del g

    # gated variant of the same step (context): ReLU^2(gate) * up, one
    # launch streaming gate and up, then the down launch; 3 matrices per step
    gate_w = torch.from_numpy(synth.weights(np.random.default_rng(6), F, H)).to(dev)
    pg, sg = bl.pack_weights(gate_w)
    del gate_w
    gstacks = [bl.FFNStack([dict(L, gate=pg.clone(), gate_scale=sg)], H, F, 1, dev, pre_norm=False,
                           residual=False) for L in layers[:max(8, R * 2 // 3)]]
    RG = len(gstacks)

    def gsteps(n):
        for i in range(n):
            gstacks[i % RG](h)

    gsteps(50)
    gated_s, gg = time_graph(torch, lambda: gsteps(4 * RG), reps=2)
    del gg
    gated_s /= 4 * RG
    log(f"gated decode step (graph): {gated_s * 1e6:.2f} us -> {1.5 * PACKED_BYTES_STEP / gated_s / 1e9:.1f} GB/s")

    # dominant kernel: the step's up kernel (fused absmax quant + up BitLinear
    # + ReLU^2 at M=1), back to back over ROOFLINE_COPIES weight copies (566 MB,
    # so each launch reads its weights from HBM); then the down one
    del layers, stacks, gstacks
    torch.cuda.empty_cache()
    RC = ROOFLINE_COPIES
    L_launch = 2 * RC
    pool_u = torch.empty((RC, PACKED_BYTES_MATRIX), dtype=torch.uint8, device=dev)
    pool_u.copy_(pu.reshape(1, -1).expand(RC, -1))
    pool_d = torch.empty((RC, PACKED_BYTES_MATRIX), dtype=torch.uint8, device=dev)
    pool_d.copy_(pd.reshape(1, -1).expand(RC, -1))
    ups = [bl.QuantForward(pool_u[i].view(F, H // 4), su, 1, relu2=True) for i in range(RC)]
    dns = [bl.QuantForward(pool_d[i].view(H, F // 4), sd, 1, rmsnorm=True) for i in range(RC)]
    y = torch.empty((1, F), dtype=torch.float32, device=dev)
    y2 = torch.empty((1, H), dtype=torch.float32, device=dev)
    xd = torch.from_numpy(d["X_down"]).to(dev)

    def up_run():
        for i in range(L_launch):
            ups[i % RC](x0, y_out=y)

    def dn_run():
        for i in range(L_launch):
            dns[i % RC](xd, y_out=y2)

    gemv_s, gg = time_graph(torch, up_run, reps=3)
    gemv_s /= L_launch
    del gg
    gemv_dn_s, gg = time_graph(torch, dn_run, reps=3)
    gemv_dn_s /= L_launch
    del gg
    achieved = PACKED_BYTES_MATRIX / gemv_s / 1e9
    log(f"up kernel M=1: {gemv_s * 1e6:.2f} us/launch -> {achieved:.1f} GB/s; "
        f"down: {gemv_dn_s * 1e6:.2f} us -> {PACKED_BYTES_MATRIX / gemv_dn_s / 1e9:.1f} GB/s")
    traffic = traffic_from_profile("decode_up_m1", ["gemv.hip", "bl_device.h"])
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "k_decode<4,4,false,3> (absmax quant + up BitLinear + ReLU^2, M=1, K=2560, N=6912)",
                "bytes_per_launch": PACKED_BYTES_MATRIX, "us_per_launch": round(gemv_s * 1e6, 3),
                "timing": f"HIP events around a graph of {L_launch} back-to-back launches over {RC} weight "
                          f"copies ({RC * PACKED_BYTES_MATRIX / 1e6:.0f} MB)",
                "down_us_per_launch": round(gemv_dn_s * 1e6, 3)}
    roofline.update(rocprof_figures("decode_up_m1", PACKED_BYTES_MATRIX / 1e9, HBM_PEAK_GBS))
    del ups, dns, pool_u, pool_d
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------- decode, M=1, per BitLinear shape
    # Fused quantise + BitLinear at M=1 for the block's shapes (attention:
    # q/o 2560->2560, k/v 2560->640, a 2560->3840 layer; FFN: up, down),
    # rotating over >= 512 MB of packed copies so every launch reads HBM.
    shapes = []
    if not args.no_shapes:
        rng = np.random.default_rng(5)
        for K, N, what in ((2560, 2560, "q/o"), (2560, 640, "k/v"), (2560, 3840, "q+k+v size"),
                           (2560, 6912, "up"), (6912, 2560, "down")):
            Wt = torch.from_numpy(synth.weights(rng, N, K)).to(dev)
            pk, sk = bl.pack_weights(Wt)
            nb = N * K // 4
            ncp = max(16, -(-(2 * MALL_BYTES) // nb))
            pool = torch.empty((ncp, nb), dtype=torch.uint8, device=dev)
            pool.copy_(pk.reshape(1, nb).expand(ncp, nb))
            qfs = [bl.QuantForward(pool[i].view(N, K // 4), sk, 1) for i in range(ncp)]
            xs1 = torch.from_numpy(synth.activations(rng, 1, K, outliers=True)).to(dev)
            ys1 = torch.empty((1, N), dtype=torch.float32, device=dev)

            def shape_run():
                for q in qfs:
                    q(xs1, y_out=ys1)

            t, gg = time_graph(torch, shape_run, reps=3)
            del gg
            t /= ncp
            shapes.append({"K": K, "N": N, "layer": what, "us_per_launch": round(t * 1e6, 3),
                           "GB_per_s": round(nb / t / 1e9, 1), "weight_copies": ncp})
            log(f"decode M=1 {K}->{N} ({what}): {t * 1e6:.2f} us -> {nb / t / 1e9:.0f} GB/s")
            del pool, qfs, Wt
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- prefill, M=4096
    prefill = None
    if not args.no_prefill:
        p = synth.prefill()
        X = torch.from_numpy(p["X"]).to(dev)
        pu4, su4 = bl.pack_weights(torch.from_numpy(p["W_up"]).to(dev))
        pd4, sd4 = bl.pack_weights(torch.from_numpy(p["W_down"]).to(dev))
        M = X.shape[0]
        xq4, xs4, rs4 = bl.quant_act(X)
        up = bl.forward(xq4, xs4, pu4, su4, x_rowsum=rs4, relu2=True, subln=True)
        torch.cuda.synchronize()

        def chain():
            a, b, c = bl.quant_act(X)
            u = bl.forward(a, b, pu4, su4, x_rowsum=c, relu2=True, subln=True)
            bl.forward(u["q"], u["q_scale"], pd4, sd4, x_rowsum=u["q_rowsum"])

        chain_s, gg = time_graph(torch, chain, reps=args.prefill_steps)
        del gg
        yu = torch.empty((M, F), dtype=torch.float32, device=dev)
        yd = torch.empty((M, H), dtype=torch.float32, device=dev)
        # each GEMM alone: GEMM_BATCH back-to-back launches in one graph, so a
        # graph launch's own gap (a few us) is not charged to every GEMM
        up_s, gg = time_graph(torch, lambda: [bl.forward(xq4, xs4, pu4, su4, x_rowsum=rs4, relu2=True, y_out=yu)
                                              for _ in range(GEMM_BATCH)], reps=args.prefill_steps)
        del gg
        up_s /= GEMM_BATCH
        dn_s, gg = time_graph(torch, lambda: [bl.forward(up["q"], up["q_scale"], pd4, sd4, x_rowsum=up["q_rowsum"],
                                                         y_out=yd) for _ in range(GEMM_BATCH)],
                              reps=args.prefill_steps)
        del gg
        dn_s /= GEMM_BATCH
        ops = 2.0 * M * H * F
        tops_up = ops / up_s / 1e12
        tops_dn = ops / dn_s / 1e12
        tops = 2 * ops / (up_s + dn_s) / 1e12
        log(f"prefill chain {chain_s * 1e3:.3f} ms; up GEMM {up_s * 1e6:.1f} us ({tops_up:.0f} TOPS); "
            f"down GEMM {dn_s * 1e6:.1f} us ({tops_dn:.0f} TOPS)")
        prefill = {"metric": "int8 TOPS of the two FFN GEMMs at M=4096", "value": round(tops, 2),
                   "unit": "TOPS", "ms_per_chain": round(chain_s * 1e3, 4),
                   "config": {"workload": "prefill chain M=4096: quant, up 2560->6912 +ReLU^2, subln "
                                          "requant, down 6912->2560 (seed 3)",
                              "cache": "warm: the replays reuse one copy of each matrix (the GEMMs are bound "
                                       "by the matrix cores; their operands are re-read from L2 by many tiles)"},
                   "roofline": {"bound": "mfma", "achieved": round(tops_up, 2), "peak": INT8_PEAK_TOPS,
                                "unit": "TOPS", "frac": round(tops_up / INT8_PEAK_TOPS, 4),
                                "traffic": traffic_from_profile("gemm_up_m4096", ["gemm.hip", "bl_device.h"]),
                                "kernel": "k_gemm_pipe<256,256,2,4,4,1,ReLU^2> (M=4096, K=2560, N=6912)",
                                "ops_per_launch": int(ops), "us_per_launch": round(up_s * 1e6, 2),
                                "timing": f"HIP events around a graph of {GEMM_BATCH} back-to-back launches, "
                                          f"{args.prefill_steps} replays",
                                "down_us_per_launch": round(dn_s * 1e6, 2),
                                "down_tops": round(tops_dn, 2),
                                **rocprof_figures("gemm_up_m4096", ops / 1e12, INT8_PEAK_TOPS)}}

    batched = None if args.no_batched else bench_batched(torch, bl, synth, dev, log)
    torch.cuda.empty_cache()
    stack = None if args.no_stack else bench_stack(torch, bl, synth, dev, log)
    torch.cuda.empty_cache()
    ffn_layers = None if args.no_batched else bench_ffn_layers(torch, bl, synth, dev, log)
    torch.cuda.empty_cache()
    latent = None if args.no_latent else bench_latent(torch, bl, synth, dev, log)
    torch.cuda.empty_cache()
    read = stream_read(torch, dev, log)
    roofline["read_peak_measured_GB_per_s"] = read["GB_per_s"]
    roofline["frac_of_read_peak"] = round(roofline["achieved"] / read["GB_per_s"], 4)
    tall = tall_decode(torch, bl, d, pu, su, dev, log)

    cpu = None if args.no_cpu else cpu_baseline(args.cpu_seconds)
    out = {"metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 6), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "i8", "data": "synthetic",
           "config": {"workload": "decode FFN chain at model width, M=1: quant, up 2560->6912 +ReLU^2, "
                                  "subln requant, down 6912->2560 (seed 1)",
                      "M": 1, "hidden": H, "ffn": F, "packed_bytes_per_step": PACKED_BYTES_STEP,
                      "weight_copies": R,
                      "cache": ("cold: every weight copy a timed step reads was last read cold_bytes_touched "
                                "bytes of other weight copies earlier (over twice the 256 MB Infinity Cache)"
                                if cold else "warm: the rotated copies fit twice the Infinity Cache"),
                      "cold_bytes_touched": reuse,
                      "timed_weight_bytes_distinct": min(args.steps, R) * PACKED_BYTES_STEP,
                      "after_1GiB_flush_us_per_step": round(flushed_s * 1e6, 3),
                      "launch": "HIP graph of the K steps", "eager_us_per_step": round(eager_s * 1e6, 2),
                      "pack_ms_up_plus_down": round(pack_t * 1e3, 4),
                      "gated_step_us": round(gated_s * 1e6, 3),
                      "gated_step_GB_per_s": round(1.5 * PACKED_BYTES_STEP / gated_s / 1e9, 1)},
           "roofline": roofline, "cpu_baseline": cpu, "prefill": prefill, "decode_shapes": shapes,
           "batched_decode": batched, "stack": stack, "ffn_layer_batched": ffn_layers, "latent_forward": latent, "stream_read": read,
           "decode_tall": tall}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
