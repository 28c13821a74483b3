#!/usr/bin/env python3
"""Benchmark of the float8 MoE quantization hot path on one MI355X (gfx950).

One step is one pass of the whole path over one batch of synthetic MoE-shaped
input, every kernel from libmxq:
  1. mxq_quantize_mx    dispatch payload X (65536, 5120) bf16 -> e4m3 (65536, 5120)
                        + e8m0 (65536, 160): the two all-to-all send buffers
  2. mxq_dequantize_mx  those two buffers -> bf16 (65536, 5120)
  3. mxq_group_scale_fp8  tokens (16640, 5120) bf16, 16 Zipf(1.1) expert groups,
                        row-major e4m3 + (16, 5120) fp32 scales
  4. mxq_group_scale_fp8  the same token shape, 128 groups, column-major e4m3
  5. mxq_transpose_u8   that column-major output -> row-major
Sources: "[mxfp8 MoE training] Support mxfp8 all to all in expert parallel"
(Summary; Performance: seq 8192 x local batch 8 tokens, dim 5120, 16 experts)
and "[moe training] fix uncoalesced global accesses in per group rowwise scaling
kernel" (Summary; Performance tables at (16640, 5120), 16..128 groups).

The metric is achieved HBM bandwidth: algorithmic bytes (each input read once,
each output written once) over time.  The step's bytes are those of the method:
the transform in call 5 is overhead (it moves 2 more bytes per element), so it
is timed inside the step but its bytes are reported apart, not counted.  Inputs are resident in device memory
before timing starts; several independent buffer sets are rotated so that no
step finds the previous step's data in the 256 MB last-level cache.

The JSON line also carries, under "grouped_mm", the next row of the path timed
on its own (it is not part of the step or of `value`): the MXFP8 scaled grouped
GEMM of the MoE configuration -- tokens (16640, 5120) routed to 16 experts
(Zipf 1.1), expert weights (16, 8192, 5120) ~ N(0, 0.02^2), both quantized with
mxq_quantize_mx, Y_g = X_g W_g^T on the scaled-fp8 MFMA, bf16 out -- with its
own roofline against the dense fp8 matrix peak (5.0 PFLOP/s).  Sources:
"[float8] add float8 rowwise MoE prototype" (Summary) and "[mxfp8 MoE training]
Support mxfp8 all to all in expert parallel" (Performance: MXFP8 grouped GEMMs).

Prints ONE JSON line (see the keys below).  --gpus N > 1 is refused: this path
runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
METRIC = "achieved HBM GB/s (and % of peak) for MXFP8 quant+dequant and group scaling"
HBM_PEAK_GBPS = 8000.0                     # MI355X HBM3E, 8 TB/s
DISPATCH = (65536, 5120)
TOKENS = (16640, 5120)
G_ROW, G_COL = 16, 128
WGRAD_N = 8192                     # expert feature width of the output gradient dY (the wgrad operand)
EXPERTS = (16, 8192, 5120)                 # (G, N, K) of the grouped GEMM
MFMA_FP8_PEAK_TFLOPS = 5000.0              # MI355X dense fp8 matrix peak
PROFILES = os.path.join(HERE, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic_counters.json")


def mx_bytes(M, K):                # read bf16, write e4m3 + e8m0 (or the reverse)
    return M * K * 2 + M * K + M * K // 32


def group_bytes(M, K, G):          # read bf16, write e4m3 + fp32 (G, K) scales
    return M * K * 3 + 4 * G * K


def transpose_bytes(M, K):         # read and write one byte per element
    return 2 * M * K


def kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(HERE, "float8_quantization_moe_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--rotate", type=int, default=4, help="independent buffer sets cycled through")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-gemm", action="store_true", help="skip the grouped GEMM leg (same as leaving gemm out of --legs)")
    p.add_argument("--legs", default=",".join(LEGS),
                   help="comma-separated measurement legs run beside the timed step: " + ", ".join(LEGS))
    p.add_argument("--seed", type=int, default=0, help="offset added to the seed of every synthetic input")
    p.add_argument("--cpu-mx-rows", type=int, default=49152, help="dispatch rows in the CPU sample")
    p.add_argument("--cpu-group-rows", type=int, default=16640, help="token rows in the CPU sample")
    p.add_argument("--ingest-counters", nargs="+", metavar="CSV",
                   help="turn rocprofv3 outputs of this script (kernel stats, FETCH_SIZE and WRITE_SIZE "
                        "counter collections) into the summaries under profiles/ and exit")
    p.add_argument("--profile-commands", default="", help="text recorded with --ingest-counters")
    return p.parse_args()


COUNTER_SOURCES = ["mx_codec.hip", "mx_dim0.hip", "device_common.hpp"]
# Legs beside the step: NEXT-row variants, the group-scaling sweep over 16-128
# groups, the MX codec at the token shape, group scaling beside streaming copies,
# and the grouped GEMM.
LEGS = ("variants", "sweep", "tokens", "concurrency", "gemm")
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30       # the 1 GiB device copies of the streaming-ceiling leg


def _cdiv(a, b):
    return -(-a // b)


# Launch grids (work-items) of the kernels the bench runs, from the launch
# configurations in csrc/: they tell apart dispatches of one kernel at different
# sizes in the profiler's per-dispatch records.
def grid_mx(M, K):                 # flat codec: 1024 16-byte chunks per 256-thread workgroup
    return min(_cdiv(M * K // 8, 1024), 1 << 22) * 256


def grid_dim0(M, K):               # 32 rows x 1024 columns per 256-thread workgroup
    return (M // 32) * _cdiv(K, 1024) * 256


def grid_transpose(R, C):          # 128 x 128-byte tiles, 256 threads
    return _cdiv(R, 128) * _cdiv(C, 128) * 256


def grid_hold(M, K, G):            # (128-row chunks + G + 1 slots) x 256-column strips, 256 threads
    return (_cdiv(M, 128) + G + 1) * _cdiv(K, 256) * 256


def grid_finalize(K, G):           # (group, 256-column strip), 256 threads
    return G * _cdiv(K, 256) * 256


def grid_col_blocks(M, K):         # 128-row blocks x 256-column strips, 256 threads
    return _cdiv(M, 128) * _cdiv(K, 256) * 256


def grid_split_amax(M, K):         # 128-row blocks x 256-column tiles, 256 threads
    return _cdiv(M, 128) * _cdiv(K, 256) * 256


def grid_split_quant(M, K):        # 128-row blocks x 128-column tiles, 256 threads
    return _cdiv(M, 128) * _cdiv(K, 128) * 256


def ingest_counters(stats_csv, fetch_csv, write_csv, sq_csv=None, commands=""):
    """Summaries for profiles/: per-kernel durations and HBM bytes per dispatch
    from FETCH_SIZE / WRITE_SIZE (KiB), each scaled by what the counter reads for
    the 1 GiB device copies of known size; optionally vector memory / LDS
    instruction counts and LDS bank conflicts per dispatch.  Dispatches are kept
    apart by kernel and grid size (one kernel runs at several sizes); durations
    come from the per-dispatch kernel trace next to `stats_csv`."""
    import csv
    import collections
    import statistics

    def norm(name):                               # "void mxq::k<false>(...)" -> "mxq::k<false>"
        name = name.replace("(anonymous namespace)::", "").split("(")[0]
        return name[5:] if name.startswith("void ") else name

    def per_dispatch_counter(path, counter=None):
        agg = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            if counter is None or r["Counter_Name"] == counter:
                agg[(norm(r["Kernel_Name"]), int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
        return agg

    fetch, write = per_dispatch_counter(fetch_csv), per_dispatch_counter(write_csv)
    copies_f = [v for (k, _), vs in fetch.items() if k == COPY_KERNEL for v in vs]
    copies_w = [v for (k, _), vs in write.items() if k == COPY_KERNEL for v in vs]
    f_copy, w_copy = max(copies_f) * 1024.0, max(copies_w) * 1024.0      # the 1 GiB copies are the largest
    f_scale, w_scale = COPY_BYTES / f_copy, COPY_BYTES / w_copy
    n_cal = sum(1 for v in copies_f if v * 1024.0 > 0.99 * f_copy)
    durations = collections.defaultdict(list)
    trace_csv = stats_csv.replace("_kernel_stats.csv", "_kernel_trace.csv")
    for r in csv.DictReader(open(trace_csv)):
        g = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        durations[(norm(r["Kernel_Name"]), g)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)

    D, T = DISPATCH, TOKENS
    known = {   # (kernel, grid) -> (workload, algorithmic bytes per dispatch)
        ("mxq::mx_quantize_kernel<false>", grid_mx(*D)): ("(65536, 5120)", mx_bytes(*D)),
        ("mxq::mx_quantize_kernel<false>", grid_mx(*T)): ("(16640, 5120)", mx_bytes(*T)),
        ("mxq::mx_quantize_kernel<true>", grid_mx(*D)): ("(65536, 5120) RCEIL", mx_bytes(*D)),
        ("mxq::mx_dequantize_kernel", grid_mx(*D)): ("(65536, 5120)", mx_bytes(*D)),
        ("mxq::mx_dequantize_kernel", grid_mx(*T)): ("(16640, 5120)", mx_bytes(*T)),
        ("mxq::mx_quantize_dim0_kernel<false>", grid_dim0(*D)): ("(65536, 5120) dim 0", mx_bytes(*D)),
        ("mxq::mx_quantize_dim0_kernel<true>", grid_dim0(*D)): ("(65536, 5120) dim 0 RCEIL", mx_bytes(*D)),
        ("mxq::mx_dequantize_dim0_kernel", grid_dim0(*D)): ("(65536, 5120) dim 0", mx_bytes(*D)),
        ("mxq::mx_dispatch_pack_kernel", D[0] * 256): ("(65536, 5120) top-1", mx_bytes(*D) + 4 * D[0]),
        ("mxq::transpose_u8_kernel", grid_transpose(T[1], T[0])): ("5120 x 16640", transpose_bytes(*T)),
    }
    for G in (16, 32, 64, 128):
        known[("mxq::group_hold_kernel<0>", grid_hold(*T, G))] = (f"(16640, 5120) G={G} row", None)
    for G in (32, 64, 128):
        known[("mxq::group_amax_kernel<1, true>", grid_hold(*T, G))] = (f"(16640, 5120) G={G} col", None)
        known[("mxq::group_finalize_kernel", grid_finalize(T[1], G))] = (f"G={G}", None)
    known[("mxq::group_hold_kernel<1>", grid_hold(*T, 16))] = ("(16640, 5120) G=16 col", None)
    known[("mxq::group_hold_kernel<1>", grid_hold(T[0], 8192, 16))] = ("(16640, 8192) dY G=16 col", None)
    known[("mxq::group_quant_col_blocks_kernel", grid_col_blocks(*T))] = ("(16640, 5120) col", None)
    known[("mxq::group_split_amax_kernel<256>", grid_split_amax(*T))] = ("(16640, 5120), forced", None)
    known[("mxq::group_split_quant_kernel<0>", grid_split_quant(*T))] = ("(16640, 5120) row, forced", None)
    known[("mxq::group_amax_kernel<0, false>", grid_hold(*T, 16))] = ("(16640, 5120) G=16 row, forced", None)
    known[("mxq::group_quant_kernel<0>", grid_hold(*T, 16))] = ("(16640, 5120) G=16 row, forced", None)
    known[("mxq::group_finalize_kernel", grid_finalize(T[1], 16))] = ("G=16, forced", None)

    lines = ["# HBM traffic per dispatch, hot-path step (dispatch payload 65536x5120, tokens 16640x5120)", "",
             "Commands (from the repository root):", "", "```", commands.strip(), "```", "",
             f"Calibration: the {n_cal} {COPY_KERNEL} copies of 1 GiB read {f_copy / 1024:.1f} KiB by FETCH_SIZE "
             f"and write {w_copy / 1024:.1f} KiB by WRITE_SIZE; scale factors {f_scale:.4f} (fetch) and "
             f"{w_scale:.4f} (write).", "",
             "Rows are per kernel and launch grid (work-items); the workload is named where the bench runs that "
             "kernel at that grid.", "",
             "| kernel | workload | grid | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled HBM bytes / dispatch | "
             "algorithmic bytes | ratio | average us (trace) |", "|---|---|---|---|---|---|---|---|---|---|"]
    out = {"source_files": COUNTER_SOURCES, "fetch_scale": f_scale, "write_scale": w_scale, "kernels": {}}
    src_hash = kernel_source_hash(COUNTER_SOURCES)

    def hbm(key):
        if key not in fetch or key not in write:
            return None
        return statistics.mean(fetch[key]) * 1024 * f_scale + statistics.mean(write[key]) * 1024 * w_scale

    for key in sorted(fetch):
        k, grid = key
        if k == COPY_KERNEL or key not in write:
            continue
        what, a = known.get(key, ("", None))
        h = hbm(key)
        dur = f"{statistics.mean(durations[key]):.2f}" if durations.get(key) else "-"
        lines.append(f"| {k} | {what or '-'} | {grid} | {len(fetch[key])} | {statistics.mean(fetch[key]):.1f} | "
                     f"{statistics.mean(write[key]):.1f} | {h:,.0f} | {a if a else '-'} | "
                     f"{h / a if a else float('nan'):.4f} | {dur} |")
        if a and what.startswith("(65536, 5120)"):
            out["kernels"][k.split("::")[-1]] = {"hbm_bytes_per_launch": round(h), "algorithmic_bytes": a,
                                                 "source_sha256": src_hash}

    # whole calls: the kernels each call launches at that call's grid (the
    # plan kernels are shared by several calls and counted at their mean)
    def any_grid(k):
        keys = [key for key in fetch if key[0] == k]
        if not keys or any(key not in write for key in keys):
            return None
        return statistics.mean(hbm(key) for key in keys)

    calls = [("group scaling G=16 row-major, hold (plan + hold)",
              [("mxq::group_plan_kernel<128>", None), ("mxq::group_hold_kernel<0>", grid_hold(*T, 16))],
              group_bytes(T[0], T[1], 16)),
             ("group scaling G=128 column-major, two-pass (amax with the tables + finalize + quantize)",
              [("mxq::group_amax_kernel<1, true>", grid_hold(*T, 128)),
               ("mxq::group_finalize_kernel", grid_finalize(T[1], 128)),
               ("mxq::group_quant_col_blocks_kernel", grid_col_blocks(*T))], group_bytes(T[0], T[1], 128)),
             ("group scaling G=16 row-major, split forced (amax + quantize)",
              [("mxq::group_split_amax_kernel<256>", grid_split_amax(*T)),
               ("mxq::group_split_quant_kernel<0>", grid_split_quant(*T))], group_bytes(T[0], T[1], 16)),
             ("dispatch pack, top-1 over 16 experts (count + place with the scan folded in + pack)",
              [("mxq::dp_count_kernel", None), ("mxq::dp_place_scan_kernel", None),
               ("mxq::mx_dispatch_pack_kernel", D[0] * 256)], mx_bytes(*D) + 8 * D[0])]
    lines += ["", "Whole calls (sum of the kernels each call launches):", "",
              "| call | scaled HBM bytes | algorithmic bytes | ratio |", "|---|---|---|---|"]
    for name, ks, a in calls:
        parts = [any_grid(k) if g is None else hbm((k, g)) for k, g in ks]
        if any(x is None for x in parts):
            continue
        lines.append(f"| {name} | {sum(parts):,.0f} | {a} | {sum(parts) / a:.4f} |")
    if sq_csv:
        sq = collections.defaultdict(lambda: collections.defaultdict(list))
        for r in csv.DictReader(open(sq_csv)):
            sq[(norm(r["Kernel_Name"]), int(r["Grid_Size"]))][r["Counter_Name"]].append(float(r["Counter_Value"]))
        names = sorted({c for k in sq.values() for c in k})
        lines += ["", "Vector memory, LDS and wave counts per dispatch (means):", "",
                  "| kernel | grid | " + " | ".join(names) + " |", "|---" * (len(names) + 2) + "|"]
        for key in sorted(sq):
            if key[0] == COPY_KERNEL or key[0].startswith("at::"):
                continue
            lines.append(f"| {key[0]} | {key[1]} | " + " | ".join(
                f"{statistics.mean(sq[key][c]):,.0f}" if sq[key][c] else "-" for c in names) + " |")
    lines += ["", "Kernel durations (rocprofv3 --kernel-trace --stats, all grids of a kernel together):", "",
              "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in csv.DictReader(open(stats_csv)):
        k = norm(r["Name"])
        if k.startswith("at::"):
            continue
        lines.append(f"| {k} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} |")
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, "hbm_traffic_hot_path_step.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print("\n".join(lines))


def launch_stats(torch, stream, fn, reps):
    """Per-launch durations (us) of fn(i), i = 0..reps-1, each bracketed by its own
    events on `stream`: mean, median, min and p90."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        evs[i][0].record(stream)
        fn(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    t = sorted(e[0].elapsed_time(e[1]) * 1e3 for e in evs)
    return {"avg_us": round(sum(t) / len(t), 2), "median_us": round(t[len(t) // 2], 2), "min_us": round(t[0], 2),
            "p90_us": round(t[min(len(t) - 1, int(0.9 * len(t)))], 2)}


def rate(nbytes, us):
    return {"algorithmic_bytes": nbytes, "GBps": round(nbytes / (us * 1e3), 1),
            "frac_of_peak": round(nbytes / (us * 1e3) / HBM_PEAK_GBPS, 4)}


def device_facts(torch):
    """Name, CUs, L2, clocks and memory bus of device 0, from torch's properties and
    hipDeviceGetAttribute of the HIP runtime torch has loaded (attribute numbers of
    hip_runtime_api.h's hipDeviceAttribute_t; checked against the CU count)."""
    import ctypes
    props = torch.cuda.get_device_properties(0)
    out = {"name": props.name, "arch": getattr(props, "gcnArchName", ""), "cus": props.multi_processor_count,
           "l2_bytes_per_xcd": getattr(props, "L2_cache_size", None), "hbm_bytes": props.total_memory}
    try:
        path = next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64.so" in l)
        hip = ctypes.CDLL(path)
        def attr(a):
            v = ctypes.c_int(0)
            return v.value if hip.hipDeviceGetAttribute(ctypes.byref(v), a, 0) == 0 else None
        if attr(63) == props.multi_processor_count:          # hipDeviceAttributeMultiprocessorCount
            out.update({"peak_sclk_mhz": attr(5) / 1000, "peak_mclk_mhz": attr(60) / 1000,
                        "memory_bus_bits": attr(59), "l2_bytes_per_xcd": attr(19)})
    except (StopIteration, OSError, TypeError):
        pass
    return out


def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count()
    return model, n


def bench_grouped_mm(args, dev, stream, x_host, ends, W, mxq, np, torch):
    """Quantize tokens and expert weights with libmxq, then time the scaled grouped
    GEMM alone (two token buffer sets alternate; the 671 MB of fp8 weights exceed
    the last-level cache by themselves)."""
    G, N, K = EXPERTS
    M = x_host.shape[0]
    offs = torch.from_numpy(ends).to(dev)
    w_host = W.expert_weights(G, N, K, seed=2 + args.seed)
    w_dev = w_host.to(dev).view(G * N, K)
    del w_host
    wq = torch.empty((G * N, K), dtype=torch.uint8, device=dev)
    wsc = torch.empty((G * N, K // 32), dtype=torch.uint8, device=dev)
    x_dev = x_host.to(dev)
    xsets = []
    for _ in range(2):
        xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
        xs = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
        mxq.mxq_quantize_mx(x_dev, xq, xs, stream)
        xsets.append((xq, xs))
    # time the weight quantization too (context: it runs once per weight update)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    mxq.mxq_quantize_mx(w_dev, wq, wsc, stream)
    e0.record(stream)
    mxq.mxq_quantize_mx(w_dev, wq, wsc, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wquant_us = e0.elapsed_time(e1) * 1e3
    del w_dev, x_dev
    wq3 = wq.view(G, N, K)
    ws3 = wsc.view(G, N, K // 32)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    wsp = torch.empty(max(mxq.mxq_grouped_mm_workspace_bytes(M, N, K, G), 16), dtype=torch.uint8, device=dev)

    def call(i):
        xq, xs = xsets[i % 2]
        mxq.mxq_scaled_grouped_mm(xq, xs, wq3, ws3, offs, y, wsp, stream)

    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    reps = max(10, args.steps // 2)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        evs[i][0].record(stream)
        call(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    times = sorted(e[0].elapsed_time(e[1]) * 1e3 for e in evs)
    med = times[len(times) // 2]

    # the same product on the packed dispatch payload (tokens routed top-1 by the
    # Zipf draw whose group sizes these are), packed by mxq_dispatch_pack_mx
    x_dev = x_host.to(dev)
    ids = torch.from_numpy(W.routed_expert_ids(M, G, topk=1, seed=1 + args.seed)).to(dev)
    packed = torch.empty((M, K + K // 32), dtype=torch.uint8, device=dev)
    pends = torch.empty(G, dtype=torch.int32, device=dev)
    src = torch.empty(M, dtype=torch.int32, device=dev)
    dws = torch.empty(mxq.mxq_dispatch_pack_workspace_bytes(M, K, 1, G), dtype=torch.uint8, device=dev)
    mxq.mxq_dispatch_pack_mx(x_dev, ids, G, packed, pends, src, dws, stream)
    torch.cuda.synchronize()
    del x_dev
    same_groups = bool(np.array_equal(pends.cpu().numpy(), ends))
    for i in range(2):
        mxq.mxq_scaled_grouped_mm_packed(packed, wq3, ws3, pends, y, wsp, stream)
    torch.cuda.synchronize()
    pevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        pevs[i][0].record(stream)
        mxq.mxq_scaled_grouped_mm_packed(packed, wq3, ws3, pends, y, wsp, stream)
        pevs[i][1].record(stream)
    torch.cuda.synchronize()
    ptimes = sorted(e[0].elapsed_time(e[1]) * 1e3 for e in pevs)
    pmed = ptimes[len(ptimes) // 2]
    del packed, src, dws, ids
    rows = int(ends[-1])                                  # routed rows (all of them here)
    flops = 2.0 * rows * N * K
    tflops = flops / (med * 1e6)
    return {
        "workload": (f"MXFP8 scaled grouped GEMM: tokens ({M}, {K}) in {G} Zipf(1.1) groups x expert "
                     f"weights ({G}, {N}, {K}), bf16 out; operands quantized with mxq_quantize_mx"),
        "avg_us": round(float(np.mean(times)), 1), "median_us": round(med, 1), "min_us": round(times[0], 1),
        "TFLOPs": round(tflops, 1),
        "roofline": {"bound": "mfma", "kernel": "mm_tile_kernel", "achieved": round(tflops, 1),
                     "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / MFMA_FP8_PEAK_TFLOPS, 4),
                     "flops_per_launch": flops, "timed": "median of per-launch events (plan + tile kernels)"},
        "packed_payload": {"median_us": round(pmed, 1), "TFLOPs": round(2.0 * rows * N * K / (pmed * 1e6), 1),
                           "frac": round(2.0 * rows * N * K / (pmed * 1e6) / MFMA_FP8_PEAK_TFLOPS, 4),
                           "same_groups_as_above": same_groups,
                           "what": "mxq_scaled_grouped_mm_packed on the mxq_dispatch_pack_mx rows"},
        "weight_quantize_us": round(wquant_us, 1),
        "operand_bytes": M * K * (1 + 1 / 32) + G * N * K * (1 + 1 / 32) + 2 * M * N,
    }


def main():
    args = parse_args()
    if args.ingest_counters:
        if len(args.ingest_counters) not in (3, 4):
            raise SystemExit("--ingest-counters STATS_CSV FETCH_CSV WRITE_CSV [SQ_CSV]")
        ingest_counters(*args.ingest_counters, commands=args.profile_commands)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported.  The quantization kernels shard by token rows with no exchange of their own; "
              "the all-to-all that would carry their buffers between GPUs is not part of this path.", file=sys.stderr)
        sys.exit(2)
    legs = {l.strip() for l in args.legs.split(",") if l.strip()}
    unknown = legs - set(LEGS)
    if unknown:
        raise SystemExit(f"--legs: unknown {sorted(unknown)}; choose from {', '.join(LEGS)}")
    if args.no_gemm:
        legs.discard("gemm")

    import numpy as np
    import torch

    import workloads as W
    from float8_quantization_moe_amd import mxq

    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    mxq.lib()                                     # fails loudly if libmxq.so is missing
    dev = torch.device("cuda:0")
    ROW, COL = mxq.MXQ_LAYOUT_ROW, mxq.MXQ_LAYOUT_COL

    # ------------------------------------------------------ synthetic inputs --
    M1, K1 = DISPATCH
    M2, K2 = TOKENS
    x1_host = W.dispatch_payload(M1, K1, seed=args.seed)
    x2_host = W.moe_tokens(M2, K2, seed=args.seed)
    ends16 = W.zipf_group_ends(M2, G_ROW, seed=1 + args.seed)
    ends128 = W.zipf_group_ends(M2, G_COL, seed=1 + args.seed)
    x1_dev = x1_host.to(dev)
    x2_dev = x2_host.to(dev)
    offs16 = torch.from_numpy(ends16).to(dev)
    offs128 = torch.from_numpy(ends128).to(dev)

    class BufferSet:
        def __init__(self):
            self.x1 = x1_dev.clone()
            self.q1 = torch.empty((M1, K1), dtype=torch.uint8, device=dev)
            self.s1 = torch.empty((M1, K1 // 32), dtype=torch.uint8, device=dev)
            self.y1 = torch.empty((M1, K1), dtype=torch.bfloat16, device=dev)
            self.x2 = x2_dev.clone()
            self.x3 = x2_dev.clone()              # the 128-group pass reads its own copy
            self.q2 = torch.empty((M2, K2), dtype=torch.uint8, device=dev)
            self.sc2 = torch.empty((G_ROW, K2), dtype=torch.float32, device=dev)
            self.q3 = torch.empty((K2, M2), dtype=torch.uint8, device=dev)
            self.sc3 = torch.empty((G_COL, K2), dtype=torch.float32, device=dev)
            self.q3t = torch.empty((M2, K2), dtype=torch.uint8, device=dev)

    sets = [BufferSet() for _ in range(max(1, args.rotate))]
    ws = torch.empty(max(mxq.mxq_group_scale_workspace_bytes(M2, K2, G_ROW),
                         mxq.mxq_group_scale_workspace_bytes(M2, K2, G_COL)), dtype=torch.uint8, device=dev)
    del x1_dev, x2_dev
    torch.cuda.synchronize()

    calls = ["mx_quantize", "mx_dequantize", "group_scale_g16_row", "group_scale_g128_col", "transpose_col_to_row"]
    call_bytes = {
        "mx_quantize": mx_bytes(M1, K1),
        "mx_dequantize": mx_bytes(M1, K1),
        "group_scale_g16_row": group_bytes(M2, K2, G_ROW),
        "group_scale_g128_col": group_bytes(M2, K2, G_COL),
        "transpose_col_to_row": transpose_bytes(M2, K2),
    }
    # the method's bytes: the transform (call 5) is overhead, timed but not counted
    step_bytes = sum(v for c, v in call_bytes.items() if c != "transpose_col_to_row")
    transform_bytes = call_bytes["transpose_col_to_row"]
    stream = torch.cuda.current_stream()

    def call_fns(b):
        return [
            lambda: mxq.mxq_quantize_mx(b.x1, b.q1, b.s1, stream),
            lambda: mxq.mxq_dequantize_mx(b.q1, b.s1, b.y1, stream),
            lambda: mxq.mxq_group_scale_fp8(b.x2, offs16, ROW, b.q2, b.sc2, ws, stream),
            lambda: mxq.mxq_group_scale_fp8(b.x3, offs128, COL, b.q3, b.sc3, ws, stream),
            lambda: mxq.mxq_transpose_u8(b.q3, b.q3t, stream),
        ]

    fns_per_set = [call_fns(b) for b in sets]

    def step(i, dom=None, ev=None):
        for j, fn in enumerate(fns_per_set[i % len(sets)]):
            if j == dom:
                ev[0].record(stream)
            fn()
            if j == dom:
                ev[1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Per-call durations: each call alone, back to back over the rotated buffer
    # sets, between two events (no event between launches, which would add a gap).
    reps = max(10, args.steps // 2)
    per_call_us = {}
    for j, c in enumerate(calls):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fns_per_set[0][j]()
        torch.cuda.synchronize()
        e0.record(stream)
        for r in range(reps):
            fns_per_set[r % len(sets)][j]()
        e1.record(stream)
        torch.cuda.synchronize()
        per_call_us[c] = e0.elapsed_time(e1) * 1e3 / reps
    per_call_dist = {c: launch_stats(torch, stream, lambda r, j=j: fns_per_set[r % len(sets)][j](), reps)
                     for j, c in enumerate(calls)}
    variants = {}
    if "variants" in legs:
        # Variants of the path's calls (the NEXT rows), each alone on the same rotated
        # buffers and shapes; reported beside the step, not part of `value`.
        FLOOR, RCEIL = mxq.MXQ_SCALE_FLOOR, mxq.MXQ_SCALE_RCEIL
        POW2, INV = mxq.MXQ_GROUP_POW2_SCALE, mxq.MXQ_GROUP_INVERSE_SCALE
        s_dim0 = lambda b: b.s1.view(M1 // 32, K1)      # (M/32, K) scales: the same byte count as (M, K/32)
        variant_calls = [
            ("mx_quantize_rows_rceil", mx_bytes(M1, K1), lambda b: mxq.mxq_quantize_mx_ex(b.x1, 1, RCEIL, b.q1, b.s1, stream)),
            ("mx_quantize_cols_floor", mx_bytes(M1, K1), lambda b: mxq.mxq_quantize_mx_ex(b.x1, 0, FLOOR, b.q1, s_dim0(b), stream)),
            ("mx_quantize_cols_rceil", mx_bytes(M1, K1), lambda b: mxq.mxq_quantize_mx_ex(b.x1, 0, RCEIL, b.q1, s_dim0(b), stream)),
            ("mx_dequantize_cols", mx_bytes(M1, K1), lambda b: mxq.mxq_dequantize_mx_ex(b.q1, s_dim0(b), 0, b.y1, stream)),
            ("group_scale_g16_row_pow2_inverse", group_bytes(M2, K2, G_ROW),
             lambda b: mxq.mxq_group_scale_fp8_ex(b.x2, offs16, ROW, POW2 | INV, b.q2, b.sc2, ws, stream)),
            ("group_scale_g128_col_pow2_inverse", group_bytes(M2, K2, G_COL),
             lambda b: mxq.mxq_group_scale_fp8_ex(b.x3, offs128, COL, POW2 | INV, b.q3, b.sc3, ws, stream)),
        ]
        variants = {}
        for name, nbytes, fn in variant_calls:
            for b in sets:
                fn(b)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for r in range(reps):
                fn(sets[r % len(sets)])
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            variants[name] = {"avg_us": round(us, 2), "algorithmic_bytes": nbytes, "GBps": round(nbytes / (us * 1e3), 1),
                              "frac_of_peak": round(nbytes / (us * 1e3) / HBM_PEAK_GBPS, 4),
                              "shape": [M1, K1] if name.startswith("mx_") else [M2, K2]}
        # the fused dispatch pack at the dispatch shape: (65536, 5120) routed top-1 over 16 Zipf experts
        ids1 = torch.from_numpy(W.routed_expert_ids(M1, G_ROW, topk=1, seed=1 + args.seed)).to(dev)
        pk1 = torch.empty((M1, K1 + K1 // 32), dtype=torch.uint8, device=dev)
        pe1 = torch.empty(G_ROW, dtype=torch.int32, device=dev)
        ps1 = torch.empty(M1, dtype=torch.int32, device=dev)
        pw1 = torch.empty(mxq.mxq_dispatch_pack_workspace_bytes(M1, K1, 1, G_ROW), dtype=torch.uint8, device=dev)
        fn = lambda i: mxq.mxq_dispatch_pack_mx(sets[i % len(sets)].x1, ids1, G_ROW, pk1, pe1, ps1, pw1, stream)
        for i in range(2):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for r in range(reps):
            fn(r)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        nb = mx_bytes(M1, K1) + M1 * 4 * 2               # + the ids read and the source indices written
        variants["dispatch_pack_top1_e16"] = {"avg_us": round(us, 2), "algorithmic_bytes": nb,
                                              "GBps": round(nb / (us * 1e3), 1),
                                              "frac_of_peak": round(nb / (us * 1e3) / HBM_PEAK_GBPS, 4),
                                              "shape": [M1, K1], "what": "sort by expert + gather + MX quantize + pack"}
        del ids1, pk1, pe1, ps1, pw1
        # the other operand of the weight-gradient GEMM: dY (16640, 8192), 16 groups, column-major
        dy = [torch.empty((M2, WGRAD_N), dtype=torch.bfloat16, device=dev).normal_() for _ in range(min(2, len(sets)))]
        qdy = torch.empty((WGRAD_N, M2), dtype=torch.uint8, device=dev)
        sdy = torch.empty((G_ROW, WGRAD_N), dtype=torch.float32, device=dev)
        wsdy = torch.empty(mxq.mxq_group_scale_workspace_bytes(M2, WGRAD_N, G_ROW), dtype=torch.uint8, device=dev)
        fn = lambda i: mxq.mxq_group_scale_fp8(dy[i % len(dy)], offs16, COL, qdy, sdy, wsdy, stream)
        for i in range(2):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for r in range(reps):
            fn(r)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        nb = group_bytes(M2, WGRAD_N, G_ROW)
        variants["group_scale_wgrad_dy_g16_col"] = {"avg_us": round(us, 2), "algorithmic_bytes": nb,
                                                    "GBps": round(nb / (us * 1e3), 1),
                                                    "frac_of_peak": round(nb / (us * 1e3) / HBM_PEAK_GBPS, 4),
                                                    "shape": [M2, WGRAD_N]}
        del dy, qdy, sdy, wsdy
    group_sweep = {}
    if "sweep" in legs:
        # ---------------------------------------------- (16640, 5120) sweeps ---
        # Per-group scaling over the pages' sweep (16 to 128 groups) in both layouts,
        # and the column-major route followed by the transform back, timed as one
        # unit (its bytes: the method's; the transform's are overhead).  Each call
        # bracketed by its own events; medians reported.
        group_sweep = {}
        qsets = [torch.empty((M2, K2), dtype=torch.uint8, device=dev) for _ in range(2)]
        qt = torch.empty((M2, K2), dtype=torch.uint8, device=dev)
        for G in (16, 32, 64, 128):
            offs = torch.from_numpy(W.zipf_group_ends(M2, G, seed=1 + args.seed)).to(dev)
            sc = torch.empty((G, K2), dtype=torch.float32, device=dev)
            wsg = torch.empty(mxq.mxq_group_scale_workspace_bytes(M2, K2, G), dtype=torch.uint8, device=dev)
            nb = group_bytes(M2, K2, G)
            fns = {
                "row": lambda i: mxq.mxq_group_scale_fp8(sets[i % len(sets)].x2, offs, ROW, qsets[i % 2], sc, wsg, stream),
                "col": lambda i: mxq.mxq_group_scale_fp8(sets[i % len(sets)].x2, offs, COL, qsets[i % 2], sc, wsg, stream),
                "col_then_transform_to_row": lambda i: (
                    mxq.mxq_group_scale_fp8(sets[i % len(sets)].x2, offs, COL, qsets[i % 2], sc, wsg, stream),
                    mxq.mxq_transpose_u8(qsets[i % 2].view(K2, M2), qt, stream)),
            }
            for name, fn in fns.items():
                for i in range(2):
                    fn(i)
                st = launch_stats(torch, stream, fn, reps)
                group_sweep[f"g{G}_{name}"] = {**st, **rate(nb, st["median_us"])}
            del offs, sc, wsg
        del qsets, qt
    mx_tokens = {}
    if "tokens" in legs:
        # MX quantize / dequantize at the token shape (the target names both shapes)
        xq_t = torch.empty((M2, K2), dtype=torch.uint8, device=dev)
        xs_t = torch.empty((M2, K2 // 32), dtype=torch.uint8, device=dev)
        y_t = torch.empty((M2, K2), dtype=torch.bfloat16, device=dev)
        mx_tokens = {}
        for name, fn in (("mx_quantize", lambda i: mxq.mxq_quantize_mx(sets[i % len(sets)].x2, xq_t, xs_t, stream)),
                         ("mx_dequantize", lambda i: mxq.mxq_dequantize_mx(xq_t, xs_t, y_t, stream))):
            for i in range(2):
                fn(i)
            st = launch_stats(torch, stream, fn, reps)
            mx_tokens[name] = {**st, **rate(mx_bytes(M2, K2), st["median_us"]), "shape": [M2, K2]}
        del xq_t, xs_t, y_t
    concurrency = {}
    if "concurrency" in legs:
        # Group scaling (16 groups, row-major) while streaming copies of 1 GiB run
        # on a second stream of the same GPU, against the same call alone: the hold
        # method (the default; it keeps a group's tiles resident together, so other
        # work on the device can make its waits run out), with its route counters,
        # and the two methods that never wait, forced through the tuning hook.
        side = torch.cuda.Stream()
        big_src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        big_dst = torch.empty_like(big_src)
        g16 = lambda i: mxq.mxq_group_scale_fp8(sets[i % len(sets)].x2, offs16, ROW, sets[0].q2, sets[0].sc2, ws, stream)
        concurrency = {"what": ("group scaling (16640, 5120), 16 groups, row-major, while 1 GiB device copies run "
                                "on a second stream; per-launch events on the call's stream")}
        for method in ("hold", "split", "twopass"):
            with mxq.group_scale_knobs(method=method):
                for i in range(2):
                    g16(i)
                alone = launch_stats(torch, stream, g16, 10)
                torch.cuda.synchronize()
                with torch.cuda.stream(side):
                    for _ in range(8):
                        big_dst.copy_(big_src)                # about 8 x 0.4 ms of copying queued on the side stream
                beside = launch_stats(torch, stream, g16, 10)     # issued at once, overlapping the copies
                entry = {"alone": alone, "beside_streaming_copy": beside}
                if method == "hold":
                    t_out, reread = mxq.mxq_group_scale_route_counters(ws, M2, K2, len(ends16), ROW, stream)
                    entry["last_call_route_counters"] = {"timed_out_tiles": t_out, "tiles_reread_from_x": reread}
                torch.cuda.synchronize()
            concurrency[method] = entry
        del big_src, big_dst, side
    for i in range(2):
        step(i)
    torch.cuda.synchronize()

    # The dominant kernel: the longest single-kernel call.  Its launches are
    # bracketed by events inside the timed region, on the stream it runs on.
    dom = max(("mx_quantize", "mx_dequantize"), key=lambda c: per_call_us[c])
    dom_idx = calls.index(dom)

    # ------------------------------------------------------------ timed run --
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i, dom_idx, ev[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    h1 = time.perf_counter()
    host_ms = (h1 - h0) * 1e3 / args.steps
    dev_ms = t_start.elapsed_time(t_end) / args.steps
    ms_per_step = max(host_ms, dev_ms)
    dom_us = 1e3 * float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    kernels = {c: {"avg_us": round(per_call_us[c], 2), **rate(call_bytes[c], per_call_us[c]),
                   "per_launch": per_call_dist[c]} for c in calls}
    kernels["transpose_col_to_row"]["note"] = "overhead of the column-major route: not in step_algorithmic_bytes"
    value = step_bytes / (ms_per_step * 1e6)          # GB/s

    # streaming ceiling for context: a device-to-device copy of 1 GiB
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * (1 << 30) * 10 / (e0.elapsed_time(e1) * 1e6)
    del src, dst

    # --------------------------------------------------- dominant kernel ---
    # the single-kernel call that takes the longest; its launch is bracketed by
    # events on the stream it runs on
    dom_kernel = {"mx_quantize": "mx_quantize_kernel<false>", "mx_dequantize": "mx_dequantize_kernel"}[dom]
    achieved = call_bytes[dom] / (dom_us * 1e3)
    traffic = None
    traffic_note = "no counter file"
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        entry = tr.get("kernels", {}).get(dom_kernel)
        if entry and entry.get("source_sha256") == kernel_source_hash(COUNTER_SOURCES):
            traffic = int(entry["hbm_bytes_per_launch"])
            traffic_note = "rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated"
        elif entry:
            traffic_note = "kernel changed since the counters were taken"
    roofline = {"bound": "hbm", "kernel": dom_kernel, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "traffic_note": traffic_note, "algorithmic_bytes_per_launch": call_bytes[dom],
                "avg_launch_us": round(dom_us, 2)}

    # ------------------------------------------------------ grouped GEMM --
    grouped_mm = None if "gemm" not in legs else bench_grouped_mm(args, dev, stream, x2_host, ends16, W, mxq, np, torch)

    # --------------------------------------------------------- CPU baseline --
    cpu_baseline = None
    if not args.no_cpu_baseline:
        import oracle
        model, ncpu = cpu_info()
        r1 = min(args.cpu_mx_rows, M1)
        r2 = min(args.cpu_group_rows, M2)
        xb1 = np.ascontiguousarray(W.bf16_bits(x1_host)[:r1])
        xb2 = np.ascontiguousarray(W.bf16_bits(x2_host)[:r2])
        e16 = np.minimum(ends16, r2).astype(np.int32)
        e128 = np.minimum(ends128, r2).astype(np.int32)
        t0 = time.perf_counter()
        q, s = oracle.mx_quantize(xb1)
        y = oracle.mx_dequantize(q, s)
        g16, sc16 = oracle.group_scale(xb2, e16, oracle.LAYOUT_ROW)
        g128, sc128 = oracle.group_scale(xb2, e128, oracle.LAYOUT_COL)
        g128t = oracle.transpose_u8(g128)
        t1 = time.perf_counter()
        sample_bytes = (2 * mx_bytes(r1, K1) + group_bytes(r2, K2, G_ROW) + group_bytes(r2, K2, G_COL)
                        + transpose_bytes(r2, K2))
        # the sample's rows were also computed by the GPU in the last step: same bytes?
        b = sets[(args.warmup + args.steps - 1) % len(sets)]
        same_mx = (np.array_equal(b.q1[:r1].cpu().numpy(), q) and np.array_equal(b.s1[:r1].cpu().numpy(), s)
                   and np.array_equal(W.bf16_bits(b.y1[:r1].cpu()), y))
        # the same oracle calls on all available host threads, rows split statically
        # (the oracle's C code releases the GIL inside each call); group scaling is
        # split by columns, which keeps every group's rows together
        from concurrent.futures import ThreadPoolExecutor
        nthr = max(1, min(ncpu or 1, 16))
        def rows_of(n):
            step = -(-n // nthr)
            return [(a, min(n, a + step)) for a in range(0, n, step)]
        def cols_of(n):
            step = max(8, -(-n // nthr) // 8 * 8)
            return [(a, min(n, a + step)) for a in range(0, n, step)]
        def mx_part(ab):
            qq, ss = oracle.mx_quantize(np.ascontiguousarray(xb1[ab[0]:ab[1]]))
            oracle.mx_dequantize(qq, ss)
        def grp_part(ab):
            xs_ = np.ascontiguousarray(xb2[:, ab[0]:ab[1]])
            oracle.group_scale(xs_, e16, oracle.LAYOUT_ROW)
            gq, _ = oracle.group_scale(xs_, e128, oracle.LAYOUT_COL)
            oracle.transpose_u8(gq)
        t2 = time.perf_counter()
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(mx_part, rows_of(r1)))
            list(ex.map(grp_part, cols_of(K2)))
        t3 = time.perf_counter()
        cpu_baseline = {
            "value": round(sample_bytes / ((t1 - t0) * 1e9), 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "seconds": round(t1 - t0, 2),
            "sample": (f"same five calls on the first {r1} of {M1} dispatch rows and "
                       + (f"all {M2} token rows" if r2 == M2 else
                          f"the first {r2} of {M2} token rows (group offsets cut at {r2})")
                       + "; one thread; algorithmic bytes of the sample over wall time"),
            "cpu_model": model, "host_cpus_available": ncpu,
            "mx_sample_matches_gpu": bool(same_mx),
            "all_cores": {"value": round(sample_bytes / ((t3 - t2) * 1e9), 3), "unit": "GB/s", "cores": nthr,
                          "seconds": round(t3 - t2, 2),
                          "split": "MX rows, group-scaling columns, statically over the threads"},
        }

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16->e4m3",
        "data": "synthetic",
        "config": {
            "workload": ("MoE float8 quantization step: MXFP8 quantize+dequantize of a (65536, 5120) bf16 "
                         "dispatch payload, per-group fp8 scaling of (16640, 5120) bf16 tokens with 16 Zipf "
                         "groups row-major and 128 groups column-major + transform to row-major"),
            "dispatch_shape": list(DISPATCH), "tokens_shape": list(TOKENS),
            "groups_row": G_ROW, "groups_col": G_COL, "rotated_buffer_sets": len(sets),
            "step_algorithmic_bytes": step_bytes,
            "transform_overhead_bytes": transform_bytes,
            "seed": args.seed, "legs": sorted(legs),
        },
        "frac_of_peak": round(value / HBM_PEAK_GBPS, 4),
        "roofline": roofline,
        "cpu_baseline": cpu_baseline,
        "kernels": kernels,
        "group_sweep": group_sweep,
        "mx_tokens_shape": mx_tokens,
        "group_scale_concurrency": concurrency,
        "variants": variants,
        "grouped_mm": grouped_mm,
        "kernels_method": "each call alone, back to back over the rotated buffer sets, events at both ends",
        "copy_ceiling_GBps": round(copy_gbps, 1),
        "device": device_facts(torch),
        "host_ms_per_step": round(host_ms, 4), "device_ms_per_step": round(dev_ms, 4),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
