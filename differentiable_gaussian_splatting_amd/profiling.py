"""rocprofv3 output -> the short text summaries kept under profiles/, and the HBM traffic record bench.py reads.

    python -m differentiable_gaussian_splatting_amd.profiling trace STATS_CSV --title T --cmd CMD [--timed-range R]
    python -m differentiable_gaussian_splatting_amd.profiling pmc --dir D --cmd CMD --workload W > profiles/y.md

`trace` turns a `rocprofv3 --kernel-trace --stats` kernel_stats.csv into a table of per-kernel calls and durations;
with `--timed-range` (and `--marker-trace` in the rocprofv3 run) it first tabulates the dispatches inside that
ROCTx range, which bench.py opens around its timed steps.
`pmc` reads the counter_collection.csv files of the passes under D (subdirectories valu, flops, fetch, write,
calib_fetch, calib_write; each made by one `rocprofv3 --pmc` run) and writes per-kernel counter averages per
dispatch. HBM bytes per launch are FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled so that the same counters
read exactly the known traffic of a plain device copy (`bench.py --calib-copy`: 256 MiB read + 256 MiB written per
copy). The summary ends with a JSON block: per kernel the scaled bytes and a hash of the sources the kernel is built
from, so that bench.py reports the traffic only while the kernel is unchanged.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# sources each reported kernel is compiled from (its file, the headers it includes, the build flags)
KERNEL_SOURCES = {
    "k_forward": ["raster_fwd.hip", "raster_common.hpp", "gsr_internal.hpp"],
    "k_backward": ["raster_bwd.hip", "raster_common.hpp", "gsr_internal.hpp"],
    "k_backward_det": ["raster_bwd.hip", "raster_common.hpp", "gsr_internal.hpp"],
    "k_backward_splat": ["raster_bwd.hip", "raster_common.hpp", "gsr_internal.hpp"],
    "k_adam": ["adam.hip", "gsr_internal.hpp"],
    "k_project_forward": ["project.hip", "gsr_internal.hpp"],
    "k_project_backward": ["project.hip", "gsr_internal.hpp"],
    "k_ssim_maps": ["loss.hip", "gsr_internal.hpp"],
    "k_ssim_grad": ["loss.hip", "gsr_internal.hpp"],
    "k_upsweep": ["sort.hip", "scan_common.hpp", "gsr_internal.hpp"],
    "k_scan_rows": ["sort.hip", "scan_common.hpp", "gsr_internal.hpp"],
    "k_scatter": ["sort.hip", "scan_common.hpp", "gsr_internal.hpp"],
    "k_prep_rows": ["bin.hip", "scan_common.hpp", "gsr_internal.hpp"],
    "k_tile_cols": ["bin.hip", "scan_common.hpp", "gsr_internal.hpp"],
    "k_tile_starts": ["bin.hip", "scan_common.hpp", "gsr_internal.hpp"],
    "k_tile_scatter": ["bin.hip", "scan_common.hpp", "gsr_internal.hpp"],
    "k_tile_depth": ["tile_depth.hip", "scan_common.hpp", "gsr_internal.hpp"],
    "k_super_order": ["tile_depth.hip", "scan_common.hpp", "gsr_internal.hpp"],
}
# bench.py stage -> the kernel instance its default configuration launches (template arguments as rocprofv3
# prints them: the raster kernels with the skips on, the exact forward exponential, the dense Adam)
STAGE_KERNEL = {"forward": "k_forward<true,true>", "forward_fast_exp": "k_forward<true,false>",
                "backward": "k_backward<true>",
                "backward_deterministic": "k_backward_det<true>", "backward_per_splat": "k_backward_splat<true,false>",
                "adam": "k_adam<false>",
                "adam_visible": "k_adam<true>", "project_forward": "k_project_forward",
                "project_backward": "k_project_backward", "loss_l1_ssim": ("k_ssim_maps", "k_ssim_grad")}


def sort_kernels(passes: dict) -> tuple:
    """The kernel instances of the binning's two radix sorts in the default configuration (presort scheme: 4 passes
    of 8-bit digits over the depth keys, then the tile passes of 6-bit digits over packed keys), one entry per
    launch, for traffic_for."""
    depth = ("k_upsweep<uint32,4u,8u>", "k_scan_rows", "k_scatter<uint32,4u,8u,false,false>") * passes["depth"]
    t = passes["tile"]
    tile = ("k_upsweep<uint32,16u,6u>", "k_scan_rows") * t + ("k_scatter<uint32,16u,6u,false,true>",) * (t - 1) + \
        ("k_scatter<uint32,16u,6u,true,true>",)
    return depth + tile


# the tile-first scheme's sort under the box rule: the count table's column scan, the tile starts, the scatter and
# the per-tile order, one launch each
TILE_FIRST_SORT_KERNELS = ("k_tile_cols", "k_tile_starts", "k_tile_scatter", "k_super_order")

CALIB_BYTES = 256 * 1024 * 1024  # read and written by each copy of bench.py --calib-copy
TRAFFIC_BEGIN, TRAFFIC_END = "<!-- traffic-json", "traffic-json -->"


def source_hash(kernel: str) -> str:
    """Hash of the sources and build flags of a kernel (any instance of it: the name before '<' is looked up)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel.split("<")[0]]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    with open(os.path.join(HERE, "build.py"), "rb") as f:
        flags = re.search(rb"FLAGS = \[.*?\]", f.read(), re.S)
    h.update(flags.group(0) if flags else b"")
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "")
    n = n.split("(")[0]
    return n.replace("void ", "").replace("gsr::", "").strip()


def base_kernel(name: str) -> str:
    """k_backward<true> -> k_backward."""
    return short_name(name).split("<")[0]


def _range_windows(marker_csv: str, name: str) -> list:
    """(start, end) timestamps of every ROCTx range `name` in a rocprofv3 marker trace (bench.py opens one per
    timed repeat)."""
    try:
        rows = list(csv.DictReader(open(marker_csv)))
    except OSError:
        return []
    return [(int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows if name in r.values()]


def timed_table(kernel_csv: str, windows) -> list:
    """Per-kernel calls and durations of the dispatches that ran inside any of `windows`, longest total first."""
    acc = collections.defaultdict(list)
    for r in csv.DictReader(open(kernel_csv)):
        t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        if any(t0 >= w0 and t1 <= w1 for w0, w1 in windows):
            acc[short_name(r["Kernel_Name"])].append(t1 - t0)
    total = sum(sum(v) for v in acc.values()) or 1
    out = ["| kernel | calls | avg µs | min µs | max µs | total ms | % |", "|---|---|---|---|---|---|---|"]
    for k, v in sorted(acc.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| `{k[:90]}` | {len(v)} | {sum(v) / len(v) / 1e3:.2f} | {min(v) / 1e3:.2f} | "
                   f"{max(v) / 1e3:.2f} | {sum(v) / 1e6:.3f} | {100 * sum(v) / total:.2f} |")
    return out


def trace_md(stats_csv: str, title: str, cmd: str, timed_range: str | None = None) -> str:
    """The kernel summary of a trace; with `timed_range`, first a table of the dispatches inside that ROCTx range
    (read from the kernel and marker traces written next to the stats file)."""
    rows = list(csv.DictReader(open(stats_csv)))
    out = [f"# {title}", "", "Command (run from the repository root):", "", "```", cmd, "```", ""]
    if timed_range:
        stem = stats_csv[:-len("kernel_stats.csv")]
        windows = _range_windows(stem + "marker_api_trace.csv", timed_range)
        if windows:
            span = sum(w1 - w0 for w0, w1 in windows) / 1e6
            out += [f"Dispatches inside the {len(windows)} ROCTx ranges \"{timed_range}\" ({span:.3f} ms in all):", ""]
            out += timed_table(stem + "kernel_trace.csv", windows) + ["", "Every dispatch of the run:", ""]
    out += ["| kernel | calls | avg µs | min µs | max µs | total ms | % |", "|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{short_name(r['Name'])[:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out) + "\n"


def _counters(path: str, first: int | None = None):
    """{kernel short name: {counter: mean value per dispatch}}; the mean duration in ns is under '_ns'. With
    `first`, only each kernel's first `first` dispatches count (bench.py runs its step before anything else)."""
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    seen = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        k = short_name(r["Kernel_Name"])
        d = r["Dispatch_Id"]
        if d not in seen[k]:
            seen[k].append(d)
        if first is not None and seen[k].index(d) >= first:
            continue
        acc[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        acc[k]["_ns"].append(float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}, None


def _find_csv(d: str):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith("counter_collection.csv"):
                return os.path.join(root, f)
    return None


def pmc_md(base: str, cmd: str, workload: str, first: int | None = None) -> str:
    passes = {}
    for p in ("valu", "flops", "fetch", "write", "calib_fetch", "calib_write"):
        path = _find_csv(os.path.join(base, p))
        if path:
            passes[p] = _counters(path, None if p.startswith("calib") else first)
    # calibration: the copy kernel's counter reading for CALIB_BYTES each way
    scale = {}
    for cnt, p in (("FETCH_SIZE", "calib_fetch"), ("WRITE_SIZE", "calib_write")):
        if p in passes:
            vals = [v[cnt] for k, v in passes[p][0].items() if cnt in v and "copy" in k.lower()]
            if vals:
                scale[cnt] = CALIB_BYTES / (max(vals) * 1024.0)
    kernels = sorted({k for p in passes.values() for k in p[0]})
    lines = [f"# Hardware counters, {workload}", "", "Commands (run from the repository root; one `rocprofv3 --pmc` "
             "run per pass):", "", "```", cmd, "```", ""]
    if scale:
        lines += ["Calibration (`bench.py --calib-copy`, 256 MiB read + 256 MiB written per copy): bytes = "
                  f"FETCH_SIZE KiB x 1024 x {scale.get('FETCH_SIZE', float('nan')):.4f}, "
                  f"WRITE_SIZE KiB x 1024 x {scale.get('WRITE_SIZE', float('nan')):.4f}.", ""]
    cols = [("valu", "_ns"), ("valu", "SQ_INSTS_VALU"), ("valu", "SQ_INSTS_SALU"), ("valu", "SQ_INSTS_LDS"),
            ("valu", "SQ_INSTS_MFMA"), ("valu", "SQ_VALU_MFMA_BUSY_CYCLES"),
            ("flops", "SQ_INSTS_VALU_FLOPS_FP32"), ("flops", "SQ_INSTS_VALU_FLOPS_FP64"),
            ("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")]
    lines += [("Per dispatch (mean over each kernel's first %d dispatches: the step's warmup and timed launches "
               "come before\nthe other blocks of bench.py, which run some of the same kernels on other inputs). "
               % first if first else "Per dispatch (mean over the profiled dispatches). ") +
              "`_ns` is the dispatch duration in the valu pass;",
              "VALU issue = (SQ_INSTS_VALU - SQ_INSTS_MFMA) x 4 cycles (a wave64 instruction on a 16-lane SIMD) /",
              "(1024 SIMDs x duration x 2.4 GHz), MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 x duration x 2.4 GHz)",
              "(fp32 MFMA and VALU do not overlap on one SIMD, so their sum is the SIMDs' busy share); the FLOPS",
              "counters count per wave instruction (an FMA counts 2), so counted TFLOP/s = 64 lanes x (FLOPS_FP32 +",
              "FLOPS_FP64) / duration, an upper bound (inactive lanes count).", "",
              "| kernel | " + " | ".join(c for _, c in cols) + " | VALU issue | MFMA busy | counted TFLOP/s | "
              "HBM MB (scaled) |",
              "|---|" + "---|" * (len(cols) + 4)]
    record = {}
    for k in kernels:
        vals = []
        for p, c in cols:
            v = passes.get(p, ({}, {}))[0].get(k, {}).get(c)
            vals.append("" if v is None else f"{v:.4g}")
        fetch = passes.get("fetch", ({}, {}))[0].get(k, {}).get("FETCH_SIZE")
        write = passes.get("write", ({}, {}))[0].get(k, {}).get("WRITE_SIZE")
        v = passes.get("valu", ({}, {}))[0].get(k, {})
        f = passes.get("flops", ({}, {}))[0].get(k, {})
        ns = v.get("_ns")
        mfma = v.get("SQ_INSTS_MFMA", 0.0)
        issue = (v["SQ_INSTS_VALU"] - mfma) * 4 / (1024 * ns * 2.4) if ns and "SQ_INSTS_VALU" in v else None
        mbusy = v["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * ns * 2.4) if ns and "SQ_VALU_MFMA_BUSY_CYCLES" in v else None
        hbm = None
        if fetch is not None and write is not None and len(scale) == 2:
            hbm = fetch * 1024 * scale["FETCH_SIZE"] + write * 1024 * scale["WRITE_SIZE"]
            if base_kernel(k) in KERNEL_SOURCES:  # one record per instance (k_adam<false> and <true> differ)
                inst = (short_name(k).replace(", ", ",").replace("unsigned int", "uint32")
                        .replace("unsigned long", "uint64"))
                counted = (64 * (f.get("SQ_INSTS_VALU_FLOPS_FP32", 0) + f.get("SQ_INSTS_VALU_FLOPS_FP64", 0))
                           if "SQ_INSTS_VALU_FLOPS_FP32" in f else None)
                record[inst] = {"hbm_bytes": hbm, "fetch_kib": fetch, "write_kib": write, "valu_issue": issue,
                                "valu_insts": None if "SQ_INSTS_VALU" not in v else v["SQ_INSTS_VALU"] - mfma,
                                "mfma_insts": mfma, "mfma_busy_cycles": v.get("SQ_VALU_MFMA_BUSY_CYCLES"),
                                "counted_flops": counted, "sources": source_hash(inst)}
        tf = (64 * (f.get("SQ_INSTS_VALU_FLOPS_FP32", 0) + f.get("SQ_INSTS_VALU_FLOPS_FP64", 0)) / (f["_ns"] * 1e3)
              if f.get("_ns") else None)
        lines.append(f"| `{k[:60]}` | " + " | ".join(vals) + f" | {'' if issue is None else f'{issue:.3f}'} | "
                     f"{'' if mbusy is None else f'{mbusy:.3f}'} | "
                     f"{'' if tf is None else f'{tf:.2f}'} | {'' if hbm is None else f'{hbm / 1e6:.1f}'} |")
    lines += ["", TRAFFIC_BEGIN, json.dumps({"workload": workload, "scale": scale, "kernels": record}, indent=1),
              TRAFFIC_END, ""]
    return "\n".join(lines)


def read_traffic(md_path: str):
    """The JSON record of a pmc summary, or None."""
    try:
        text = open(md_path).read()
    except OSError:
        return None
    a, b = text.find(TRAFFIC_BEGIN), text.find(TRAFFIC_END)
    if a < 0 or b < 0:
        return None
    return json.loads(text[a + len(TRAFFIC_BEGIN):b])


def traffic_for(kernel: str, md_path: str):
    """Recorded HBM bytes per launch of the kernel instance `kernel` (e.g. "k_adam<false>"; a tuple of instances
    gives their sum), or None when unrecorded or its sources changed since."""
    if isinstance(kernel, (tuple, list)):  # a stage of several kernels: their sum
        parts = [traffic_for(k, md_path) for k in kernel]
        return None if any(p is None for p in parts) else sum(parts)
    rec = read_traffic(md_path)
    if not rec or kernel not in rec.get("kernels", {}):
        return None
    k = rec["kernels"][kernel]
    return k["hbm_bytes"] if k.get("sources") == source_hash(kernel) else None


def valu_issue_for(kernel, md_path: str):
    """Recorded fraction of the chip's VALU issue slots the kernel instance used (SQ_INSTS_VALU x 4 cycles over
    1024 SIMDs x duration x 2.4 GHz), or None when unrecorded or its sources changed since."""
    rec = read_traffic(md_path)
    if not rec or kernel not in rec.get("kernels", {}):
        return None
    k = rec["kernels"][kernel]
    return k.get("valu_issue") if k.get("sources") == source_hash(kernel) else None


def mfma_busy_for(kernel, md_path: str):
    """Recorded SIMD cycles per launch spent in MFMA instructions (SQ_VALU_MFMA_BUSY_CYCLES) of the kernel instance,
    or None when unrecorded or its sources changed since."""
    rec = read_traffic(md_path)
    if not rec or kernel not in rec.get("kernels", {}):
        return None
    k = rec["kernels"][kernel]
    return k.get("mfma_busy_cycles") if k.get("sources") == source_hash(kernel) else None


def valu_insts_for(kernel, md_path: str):
    """Recorded VALU wave instructions per launch (SQ_INSTS_VALU) of the kernel instance, or None when unrecorded or
    its sources changed since: with the kernel's live duration it gives the share of the chip's VALU issue slots
    the kernel used, SQ_INSTS_VALU x 4 cycles / (1024 SIMDs x duration x 2.4 GHz)."""
    rec = read_traffic(md_path)
    if not rec or kernel not in rec.get("kernels", {}):
        return None
    k = rec["kernels"][kernel]
    return k.get("valu_insts") if k.get("sources") == source_hash(kernel) else None


def counted_flops_for(kernel, md_path: str):
    """Recorded vector flops per launch of the kernel instance from the FLOPS counters, 64 lanes x
    (SQ_INSTS_VALU_FLOPS_FP32 + SQ_INSTS_VALU_FLOPS_FP64): an upper bound on the vector work, since inactive lanes
    count; MFMA flops are not in these counters. None when unrecorded or its sources changed since."""
    rec = read_traffic(md_path)
    if not rec or kernel not in rec.get("kernels", {}):
        return None
    k = rec["kernels"][kernel]
    return k.get("counted_flops") if k.get("sources") == source_hash(kernel) else None


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("--title", required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--timed-range", default=None, help="ROCTx range whose dispatches get a table of their own")
    p = sub.add_parser("pmc")
    p.add_argument("--dir", required=True)
    p.add_argument("--cmd", required=True)
    p.add_argument("--workload", required=True)
    p.add_argument("--first", type=int, default=None, help="count only each kernel's first N dispatches")
    a = ap.parse_args(argv)
    if a.what == "trace":
        sys.stdout.write(trace_md(a.stats_csv, a.title, a.cmd, a.timed_range))
    else:
        sys.stdout.write(pmc_md(a.dir, a.cmd, a.workload, a.first))


if __name__ == "__main__":
    main()
