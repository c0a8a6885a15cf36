"""rocprofv3 output -> the short text summaries kept under profiles/, and the HBM traffic record bench.py reads.

    python -m differentiable_gaussian_splatting_amd.profiling trace STATS_CSV --title T --cmd CMD > profiles/x.md
    python -m differentiable_gaussian_splatting_amd.profiling pmc --dir D --cmd CMD --workload W > profiles/y.md

`trace` turns a `rocprofv3 --kernel-trace --stats` kernel_stats.csv into a table of per-kernel calls and durations.
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
    "k_adam": ["adam.hip", "gsr_internal.hpp"],
    "k_project_forward": ["project.hip", "gsr_internal.hpp"],
    "k_project_backward": ["project.hip", "gsr_internal.hpp"],
    "k_ssim_maps": ["loss.hip", "gsr_internal.hpp"],
    "k_ssim_grad": ["loss.hip", "gsr_internal.hpp"],
}
# bench.py stage -> kernel
STAGE_KERNEL = {"forward": "k_forward", "backward": "k_backward", "backward_deterministic": "k_backward_det",
                "adam": "k_adam",
                "project_forward": "k_project_forward", "project_backward": "k_project_backward",
                "loss_l1_ssim": "k_ssim_maps"}
CALIB_BYTES = 256 * 1024 * 1024  # read and written by each copy of bench.py --calib-copy
TRAFFIC_BEGIN, TRAFFIC_END = "<!-- traffic-json", "traffic-json -->"


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
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


def trace_md(stats_csv: str, title: str, cmd: str) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    out = [f"# {title}", "", "Command (repository root on the GPU box):", "", "```", cmd, "```", "",
           "| kernel | calls | avg µs | min µs | max µs | total ms | % |", "|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{short_name(r['Name'])[:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out) + "\n"


def _counters(path: str):
    """{kernel short name: {counter: mean value per dispatch}}; the mean duration in ns is under '_ns'."""
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(path)):
        k = short_name(r["Kernel_Name"])
        acc[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        acc[k]["_ns"].append(float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}, None


def _find_csv(d: str):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith("counter_collection.csv"):
                return os.path.join(root, f)
    return None


def pmc_md(base: str, cmd: str, workload: str) -> str:
    passes = {}
    for p in ("valu", "flops", "fetch", "write", "calib_fetch", "calib_write"):
        path = _find_csv(os.path.join(base, p))
        if path:
            passes[p] = _counters(path)
    # calibration: the copy kernel's counter reading for CALIB_BYTES each way
    scale = {}
    for cnt, p in (("FETCH_SIZE", "calib_fetch"), ("WRITE_SIZE", "calib_write")):
        if p in passes:
            vals = [v[cnt] for k, v in passes[p][0].items() if cnt in v and "copy" in k.lower()]
            if vals:
                scale[cnt] = CALIB_BYTES / (max(vals) * 1024.0)
    kernels = sorted({k for p in passes.values() for k in p[0]})
    lines = [f"# Hardware counters, {workload}", "", "Commands (repository root on the GPU box; one `rocprofv3 --pmc` "
             "run per pass):", "", "```", cmd, "```", ""]
    if scale:
        lines += ["Calibration (`bench.py --calib-copy`, 256 MiB read + 256 MiB written per copy): bytes = "
                  f"FETCH_SIZE KiB x 1024 x {scale.get('FETCH_SIZE', float('nan')):.4f}, "
                  f"WRITE_SIZE KiB x 1024 x {scale.get('WRITE_SIZE', float('nan')):.4f}.", ""]
    cols = [("valu", "_ns"), ("valu", "SQ_INSTS_VALU"), ("valu", "SQ_INSTS_SALU"), ("valu", "SQ_INSTS_LDS"),
            ("flops", "SQ_INSTS_VALU_FLOPS_FP32"), ("flops", "SQ_INSTS_VALU_FLOPS_FP64"),
            ("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")]
    lines += ["Per dispatch (mean over the profiled dispatches). `_ns` is the dispatch duration in the valu pass;",
              "VALU issue = SQ_INSTS_VALU x 4 cycles (a wave64 instruction on a 16-lane SIMD) / (1024 SIMDs x",
              "duration x 2.4 GHz); the FLOPS counters count per wave instruction (an FMA counts 2), so counted",
              "TFLOP/s = 64 lanes x (FLOPS_FP32 + FLOPS_FP64) / duration, an upper bound (inactive lanes count).", "",
              "| kernel | " + " | ".join(c for _, c in cols) + " | VALU issue | counted TFLOP/s | HBM MB (scaled) |",
              "|---|" + "---|" * (len(cols) + 3)]
    record = {}
    for k in kernels:
        vals = []
        for p, c in cols:
            v = passes.get(p, ({}, {}))[0].get(k, {}).get(c)
            vals.append("" if v is None else f"{v:.4g}")
        fetch = passes.get("fetch", ({}, {}))[0].get(k, {}).get("FETCH_SIZE")
        write = passes.get("write", ({}, {}))[0].get(k, {}).get("WRITE_SIZE")
        hbm = None
        if fetch is not None and write is not None and len(scale) == 2:
            hbm = fetch * 1024 * scale["FETCH_SIZE"] + write * 1024 * scale["WRITE_SIZE"]
            bk = base_kernel(k)
            if bk in KERNEL_SOURCES:
                record[bk] = {"hbm_bytes": hbm, "fetch_kib": fetch, "write_kib": write,
                              "sources": source_hash(bk), "instance": k}
        v = passes.get("valu", ({}, {}))[0].get(k, {})
        f = passes.get("flops", ({}, {}))[0].get(k, {})
        ns = v.get("_ns")
        issue = v["SQ_INSTS_VALU"] * 4 / (1024 * ns * 2.4) if ns and "SQ_INSTS_VALU" in v else None
        tf = (64 * (f.get("SQ_INSTS_VALU_FLOPS_FP32", 0) + f.get("SQ_INSTS_VALU_FLOPS_FP64", 0)) / (f["_ns"] * 1e3)
              if f.get("_ns") else None)
        lines.append(f"| `{k[:60]}` | " + " | ".join(vals) + f" | {'' if issue is None else f'{issue:.3f}'} | "
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
    """Recorded HBM bytes per launch of `kernel`, or None when unrecorded or its sources changed since."""
    rec = read_traffic(md_path)
    if not rec or kernel not in rec.get("kernels", {}):
        return None
    k = rec["kernels"][kernel]
    return k["hbm_bytes"] if k.get("sources") == source_hash(kernel) else None


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("--title", required=True)
    t.add_argument("--cmd", required=True)
    p = sub.add_parser("pmc")
    p.add_argument("--dir", required=True)
    p.add_argument("--cmd", required=True)
    p.add_argument("--workload", required=True)
    a = ap.parse_args(argv)
    if a.what == "trace":
        sys.stdout.write(trace_md(a.stats_csv, a.title, a.cmd))
    else:
        sys.stdout.write(pmc_md(a.dir, a.cmd, a.workload))


if __name__ == "__main__":
    main()
