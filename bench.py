"""Benchmark of the splat rasterizer hot path on one MI355X.

A step is one pass of the whole path over the 800x800, 410k-splat workload: bin (the (tile, depth) order of the
pairs and the tile ranges), render_forward, render_backward, then the fused Adam step over 59 float32 parameters per
splat (5 groups). Inputs are seeded synthetic data resident in device memory before the timed region; the arena is
pre-grown. Defaults: W = 10 warmup steps, then 3 repeats of K = 50 timed steps (the median repeat is reported).

Prints one JSON line: the metric is splat-pixel evaluations per second over whole steps, where the evaluations of a
step are E_fwd (list entries the forward examines, up to and including each pixel's stopping splat) plus E_bwd
(entries the backward replays, the sum of last_contrib), both counted exactly by the CPU oracle on the same input.
A "projection" block beside it times the steps on either side of the path on their own: the projection of 410k 3D
Gaussians and its backward pass, the L1 + SSIM loss, and a whole training iteration chaining them with the path and
Adam.

    python bench.py [--steps K] [--warmup W] [--workload iter410k] [--no-cpu-baseline]
    python bench.py --calib-copy      # a plain 256 MiB device copy, to scale HBM byte counters
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd+bwd raster ms/iter @800×800, 410k splats; splat-pixel evals/s"
UNIT = "splat-pixel evals/s"
TIMED_RANGE = "timed steps"  # ROCTx range around the timed steps
MEASURED_RANGE = "measured steps"  # ROCTx range around the steps that carry HIP events
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
ALU_PEAK_TFLOPS = 157.3  # MI355X's published fp32 vector peak (it counts packed dual-fp32 FMA)
# fp32 vector rate without packed dual-fp32 instructions (which this build does not use): 256 CUs x 64 lanes x 2
# flops (FMA) x 2.4 GHz, reported beside the published peak
ALU_NONPACKED_TFLOPS = 256 * 64 * 2 * 2.4e9 / 1e12
# VALU issue: a wave64 instruction occupies a 16-lane SIMD for 4 cycles; 1024 SIMDs at 2.4 GHz
VALU_ISSUE_PER_S = 1024 * 2.4e9 / 4

# Algorithmic operation counts per evaluation (each add, sub, mul, min, exp counts 1; comparisons and negations 0):
#   sigma       dx, dy, (a dx) dx, (c dy) dy, (b dx) dy, two sums, x0.5                        = 11
#   alpha       exp, o G, min                                                                  = 3
#   stop test   1 - alpha, T (1 - alpha)                                                       = 2
#   composite   alpha T, rgb w (3), C += (3)                                                   = 7
#   backward, per composited entry (73): the replay 11 + 3 + 1; w = alpha T; w g (3); mine (3);
#               after = (C - acc) - mine (6); rgb T, after / (1 - alpha), their difference, times g (12) and the
#               sum (2); dL/dalpha G, dL/dsigma (2); dx^2/2, dx dy, dy^2/2 (5); conic terms (3); a dx + b dy,
#               b dx + c dy (6) and their products (2); acc += mine (3); T update (1); 9 accumulations
FWD_OPS = {"sigma_skip": 11, "alpha_reject": 14, "stop": 16, "contrib": 23}
BWD_OPS = {"sigma_skip": 11, "alpha_reject": 14, "contrib": 73}
# L1 + SSIM per pixel and channel: the products x^2, y^2, x y (3); 5 quantities x 11 taps x 2 passes as FMA (220);
# variances, covariance and S with its three derivatives (25); 3 derivative maps x 11 taps x 2 passes (132); the
# gradient's combination with the L1 sign (6)
LOSS_OPS = 3 + 220 + 25 + 132 + 6


def scene_label(spec) -> str:
    """The generator's parameters of a workload, e.g. '70% s in 0.3-4 px, 30% s in 4-40 px, color_a =
    sigmoid(N(-2, 1.5))'."""
    tot = sum(c[0] for c in spec.size_classes)
    sizes = ", ".join(f"{round(100 * c[0] / tot)}% s in {c[1]:g}-{c[2]:g} px" for c in spec.size_classes)
    return f"{sizes}, color_a = sigmoid(N({spec.opacity_mu:g}, {spec.opacity_sd:g}))"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="iter410k")
    ap.add_argument("--bin-scheme", choices=["tile_depth", "presort", "key64"], default="tile_depth")
    ap.add_argument("--raster-skip", type=int, choices=[0, 1], default=1)
    ap.add_argument("--bin-rule", choices=["box", "ellipse"], default="box")
    ap.add_argument("--repeats", type=int, default=3, help="timed repeats of K steps (median and spread reported)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bin-stress", action="store_true", help="skip the binning leg on the 1M-splat scene")
    ap.add_argument("--no-views", action="store_true", help="skip the changing-views leg")
    ap.add_argument("--bin-stress-only", action="store_true",
                    help="run only the binning leg on the 1M-splat scene (for its counter profile)")
    ap.add_argument("--calib-copy", action="store_true")
    return ap.parse_args()


def calib_copy():
    """Copies 256 MiB device to device ten times: rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE on this run give the
    counters' reading for a known traffic of 256 MiB read + 256 MiB written per copy."""
    import torch
    n = 64 * 1024 * 1024
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_read": 4 * n, "calib_copy_bytes_written": 4 * n, "copies": 10}))


def device_stream_gbs(torch) -> dict:
    """Bytes moved per second (read + written) by two of torch's streaming kernels on 512 MiB vectors, each the
    median of ten event-timed launches: a copy (one read, one write) and an addition (two reads, one write). They
    show the HBM rate plain streaming kernels reach on this GPU, beside the published 8 TB/s."""
    import numpy as np
    n = 128 * 1024 * 1024
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.ones_like(a)
    c = torch.empty_like(a)

    def rate(f, nbytes):
        f()
        ts = []
        for _ in range(10):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            f()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return nbytes / (float(np.median(ts)) * 1e-3) / 1e9

    out = {"copy": rate(lambda: c.copy_(a), 8 * n), "add": rate(lambda: torch.add(a, b, out=c), 12 * n)}
    del a, b, c
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def run_oracle(sc, adam_groups, hp, bc, bin_rule="box"):
    """CPU baseline leg: the plain single-threaded oracle over one whole step of the same workload; also the exact
    evaluation counts used by the GPU figure and the flop model."""
    import numpy as np

    import oracle
    t = {}
    t0 = time.perf_counter()
    ob = oracle.bin(sc.splats, sc.depths, sc.width, sc.height, rule=bin_rule)
    t["bin"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    out, ft, lc, fst = oracle.render_forward(sc.splats, ob, sc.width, sc.height)
    t["forward"] = time.perf_counter() - t0
    bst = {}
    t0 = time.perf_counter()
    oracle.render_backward(sc.splats, ob, sc.width, sc.height, out, ft, lc, sc.v_out, stats=bst)
    t["backward"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    for _, p, g, m, v in adam_groups:
        oracle.adam_step(p, g, m, v, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], *bc)
    t["adam"] = time.perf_counter() - t0
    # the same step with the forward and backward spread over the host's cores by bands of tile rows (binning's
    # stable sort and Adam stay single-threaded)
    threads = max(1, min(16, os.cpu_count() or 1))
    tm = {"bin": t["bin"], "adam": t["adam"]}
    t0 = time.perf_counter()
    oracle.render_forward_mt(sc.splats, ob, sc.width, sc.height, threads)
    tm["forward"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.render_backward_mt(sc.splats, ob, sc.width, sc.height, out, ft, lc, sc.v_out, threads)
    tm["backward"] = time.perf_counter() - t0
    return {"times": t, "times_mt": tm, "threads": threads, "fwd_stats": fst, "bwd_stats": bst,
            "num_pairs": ob.num_pairs, "out": out, "lc": lc, "ranges": ob.ranges,
            "super_pairs": super_pairs(ob.keys, ob.vals, sc.width)}


def super_pairs(keys, vals, width):
    """(splat, super-tile) pairs of the bins: the distinct 2 x 2-tile squares among each splat's tiles."""
    import numpy as np
    tx_n = (width + 15) // 16
    tiles = (keys >> np.uint64(32)).astype(np.int64)
    sup = (tiles // tx_n // 2) * ((tx_n + 1) // 2) + (tiles % tx_n) // 2
    return int(np.unique(vals.astype(np.int64) * (1 << 32) + sup).size)


def roctx():
    """The ROCTx marker library (its ranges cost nothing unless a profiler records them), or None."""
    import ctypes
    for name in ("librocprofiler-sdk-roctx.so.1", "libroctx64.so.4"):
        try:
            lib = ctypes.CDLL(name)
        except OSError:
            continue
        lib.roctxRangePushA.argtypes = [ctypes.c_char_p]
        return lib
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported (the tile-sharded multi-GPU "
              "path is design-only)", file=sys.stderr)
        sys.exit(2)
    if args.calib_copy:
        calib_copy()
        return

    import numpy as np
    import torch

    from differentiable_gaussian_splatting_amd import gsr, scenes

    if args.bin_stress_only:
        ctx = gsr.Context(0)
        print(json.dumps({"bin_stress": bench_bin_stress(args, ctx, gsr, scenes, torch, np)}), flush=True)
        ctx.close()
        return

    print(f"[bench] workload {args.workload}: generating inputs", file=sys.stderr, flush=True)
    sc = scenes.make_scene(args.workload)
    W, H, N = sc.width, sc.height, sc.spec.n
    hp = scenes.ADAM_HPARAMS
    bc = scenes.adam_bias_corrections(hp["beta1"], hp["beta2"], hp["step"])
    adam_host = scenes.make_adam_groups(N, seed=sc.spec.seed)

    ctx = gsr.Context(0)
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_BIN_SCHEME, scheme_opt(gsr, args.bin_scheme))
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_RASTER_SKIP, args.raster_skip)
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_BIN_RULE, gsr.GSR_BIN_ELLIPSE if args.bin_rule == "ellipse" else gsr.GSR_BIN_BOX)
    splats = torch.from_numpy(sc.splats).cuda()
    depths = torch.from_numpy(sc.depths).cuda()
    v_out = torch.from_numpy(sc.v_out).cuda()
    out_rgba = torch.empty((H, W, 4), dtype=torch.float32, device="cuda")
    final_T = torch.empty((H, W), dtype=torch.float32, device="cuda")
    last_contrib = torch.empty((H, W), dtype=torch.int32, device="cuda")
    grad = torch.empty((N, 9), dtype=torch.float32, device="cuda")
    groups = [tuple(torch.from_numpy(a).cuda() for a in g[1:]) + (hp["lr"],) for g in adam_host]
    adam_elems = sum(g[0].numel() for g in groups)

    # pre-grow the arena (first-touch and allocation stay out of the timed region)
    bins = gsr.gsr_bin(ctx, splats, depths, W, H)
    gsr.gsr_reserve(ctx, int(bins.num_pairs * 1.05) + 1024, N)

    stream = torch.cuda.current_stream()
    names = ["bin", "forward", "backward", "adam"]

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        b = gsr.gsr_bin(ctx, splats, depths, W, H)
        if ev:
            ev[1].record(stream)
        gsr.gsr_render_forward(ctx, splats, b, W, H, out_rgba, final_T, last_contrib)
        if ev:
            ev[2].record(stream)
        gsr.gsr_render_backward(ctx, splats, b, W, H, out_rgba, final_T, last_contrib, v_out, grad)
        if ev:
            ev[3].record(stream)
        gsr.gsr_adam_step(ctx, groups, hp["beta1"], hp["beta2"], hp["eps"], *bc)
        if ev:
            ev[4].record(stream)
        return b

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, synchronized on both sides, with nothing else on the stream (HIP events
    # between the kernels cost about 50 us of launch gaps per step, so they are taken in the steps after it); the
    # region is run `repeats` times and the median repeat is reported, with the spread
    rx = roctx()  # the timed region as a ROCTx range, so that a kernel trace can single out its dispatches
    walls = []
    for rep in range(args.repeats):
        print(f"[bench] timing {args.steps} steps (repeat {rep + 1} of {args.repeats})", file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        if rx:
            rx.roctxRangePushA(TIMED_RANGE.encode())
        t0 = time.perf_counter()
        for _ in range(args.steps):
            b = step()
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
        if rx:
            rx.roctxRangePop()
    wall = float(np.median(walls))
    ms_per_step = wall * 1e3 / args.steps

    # K more steps per repeat with HIP events on the library's stream: torch's around each stage (its launches and
    # small kernels included), the library's around each stage's main kernel (GSR_OPT_KERNEL_TIMING); the kernels'
    # own durations are the ones the rooflines use. Per repeat the mean over its K steps; reported: the median of
    # the repeats and their standard deviation.
    kernel_stage = {"bin": gsr.GSR_STAGE_BIN, "forward": gsr.GSR_STAGE_FORWARD, "backward": gsr.GSR_STAGE_BACKWARD,
                    "adam": gsr.GSR_STAGE_ADAM, "depth_sort": gsr.GSR_STAGE_DEPTH_SORT,
                    "tile_sort": gsr.GSR_STAGE_TILE_SORT, "tile_scan": gsr.GSR_STAGE_TILE_SCAN,
                    "tile_depth": gsr.GSR_STAGE_TILE_DEPTH}
    # the binning's inner stages a scheme does not run record nothing (0 ms)
    optional = {"depth_sort", "tile_scan", "tile_depth"}
    stage_reps = {nm: [] for nm in names}
    kernel_reps = {nm: [] for nm in kernel_stage}
    for rep in range(args.repeats):
        print(f"[bench] {args.steps} steps with per-stage and per-kernel events (repeat {rep + 1})", file=sys.stderr,
              flush=True)
        gsr.gsr_set_option(ctx, gsr.GSR_OPT_KERNEL_TIMING, args.steps)
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        if rx:
            rx.roctxRangePushA(MEASURED_RANGE.encode())
        for k in range(args.steps):
            b = step(events[k])
        torch.cuda.synchronize()
        if rx:
            rx.roctxRangePop()
        for i, nm in enumerate(names):
            stage_reps[nm].append(float(np.mean([events[k][i].elapsed_time(events[k][i + 1])
                                                 for k in range(args.steps)])))
        for nm, stg in kernel_stage.items():
            t = gsr.gsr_kernel_times(ctx, stg)
            assert len(t) == args.steps or (nm in optional and not t), f"{nm}: {len(t)} launches recorded"
            kernel_reps[nm].append(float(np.mean(t)) if t else 0.0)
        gsr.gsr_set_option(ctx, gsr.GSR_OPT_KERNEL_TIMING, 0)
    stage_ms = {nm: float(np.median(v)) for nm, v in stage_reps.items()}
    kernel_ms = {nm: float(np.median(v)) for nm, v in kernel_reps.items()}
    spread = {"ms_per_step": {"repeats": [w * 1e3 / args.steps for w in walls],
                              "sigma": float(np.std([w * 1e3 / args.steps for w in walls]))},
              "stage_ms": {nm: {"repeats": v, "sigma": float(np.std(v))} for nm, v in stage_reps.items()},
              "kernel_ms": {nm: {"repeats": v, "sigma": float(np.std(v))} for nm, v in kernel_reps.items()}}
    P = b.num_pairs
    e_bwd_gpu = int(last_contrib.to(torch.int64).sum().item())
    sync_free = bench_sync_free(args, ctx, gsr, torch, np, step, b, walls)
    fast_exp = bench_fast_exp_forward(args, ctx, gsr, torch, np, splats, b, W, H, out_rgba, final_T, last_contrib)
    det = bench_deterministic_backward(args, ctx, gsr, torch, np, stream, splats, b, W, H, out_rgba, final_T,
                                       last_contrib, v_out, grad)
    per_splat = bench_per_splat_backward(args, ctx, gsr, torch, np, splats, b, W, H, out_rgba, final_T,
                                         last_contrib, v_out, grad)

    # CPU baseline leg (rank 0, N = 1): the oracle on one whole step of the same input; its exact counts
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline: oracle over one step", file=sys.stderr, flush=True)
        cpu = run_oracle(sc, adam_host, hp, bc, args.bin_rule)
        assert cpu["num_pairs"] == P, "pair count differs from the oracle"
        assert int(cpu["lc"].astype(np.int64).sum()) == e_bwd_gpu, "last_contrib sum differs from the oracle"

    result = {"metric": METRIC, "unit": UNIT, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": "f32", "data": "synthetic",
              "config": {"workload": f"{args.workload}: {W}x{H} image, {N} splats ({scene_label(sc.spec)}), "
                                     "bin + forward + backward + fused Adam over 59 fp32 params per splat",
                         "image": [W, H], "splats": N, "pairs": P, "adam_elements": adam_elems,
                         "bin_scheme": args.bin_scheme, "bin_rule": args.bin_rule,
                         "raster_skip": args.raster_skip}}
    result["repeats"] = args.repeats
    result["stage_ms"] = stage_ms
    result["kernel_ms"] = kernel_ms  # the main kernel(s) of each stage alone (GSR_OPT_KERNEL_TIMING)
    result["spread"] = spread
    result["timing"] = ("value and ms_per_step: wall clock of K timed steps, which carry no events, the median of "
                        f"{args.repeats} repeats; stage_ms and kernel_ms: HIP events in K further steps per repeat "
                        "(torch's around each stage, the library's around each stage's main kernel on its stream), "
                        "the median of the repeats' means; spread: each repeat and the standard deviation")
    result["fwd_bwd_ms"] = stage_ms["forward"] + stage_ms["backward"]
    det["ratio_to_default"] = det["ms"] / stage_ms["backward"]
    det["kernel_ratio_to_default"] = det["kernel_ms"] / kernel_ms["backward"]
    result["deterministic_backward"] = det
    result["sync_free_bin"] = sync_free
    fast_exp["kernel_ratio_to_exact"] = fast_exp["kernel_ms"] / kernel_ms["forward"]
    result["forward_fast_exp"] = fast_exp
    per_splat["kernel_ratio_to_default"] = per_splat["kernel_ms"] / kernel_ms["backward"]
    result["per_splat_backward"] = per_splat
    if cpu is not None:
        fs, bs = cpu["fwd_stats"], cpu["bwd_stats"]
        e_fwd, e_bwd = fs["visited"], bs["visited"]
        evals = e_fwd + e_bwd
        result["value"] = evals * args.steps / wall
        result["evals_per_step"] = {"E_fwd": e_fwd, "E_bwd": e_bwd,
                                    "E_nom": int((cpu["ranges"][:, 1].astype(np.int64) -
                                                  cpu["ranges"][:, 0]).sum() * 256)}
        result["fwd_bwd_evals_per_s"] = evals / (result["fwd_bwd_ms"] * 1e-3)
        # algorithmic operations per launch
        fwd_ops = (FWD_OPS["sigma_skip"] * (fs["sigma_neg"] + fs["sigma_ge_skip"]) +
                   FWD_OPS["alpha_reject"] * (fs["alpha_reject"] - fs["sigma_ge_skip"]) +
                   FWD_OPS["stop"] * fs["stopped"] + FWD_OPS["contrib"] * fs["contrib"])
        bwd_ops = (BWD_OPS["sigma_skip"] * (bs["sigma_neg"] + bs["sigma_ge_skip"]) +
                   BWD_OPS["alpha_reject"] * (bs["alpha_reject"] - bs["sigma_ge_skip"]) +
                   BWD_OPS["contrib"] * bs["contrib"])
        adam_bytes = 28 * adam_elems
        eff = ("effective rate: the method's own operations per launch (the oracle's exact evaluation counts times "
               "the per-evaluation operation model above) over the kernel's time; peak: the published fp32 vector "
               "figure")
        roofs = {
            "forward": {"bound": "alu", "achieved": fwd_ops / (kernel_ms["forward"] * 1e-3) / 1e12,
                        "peak": ALU_PEAK_TFLOPS, "unit": "TFLOP/s", "work_per_launch": fwd_ops, "achieved_kind": eff},
            "backward": {"bound": "alu", "achieved": bwd_ops / (kernel_ms["backward"] * 1e-3) / 1e12,
                         "peak": ALU_PEAK_TFLOPS, "unit": "TFLOP/s", "work_per_launch": bwd_ops,
                         "achieved_kind": eff},
            "adam": {"bound": "hbm", "achieved": adam_bytes / (kernel_ms["adam"] * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "work_per_launch": adam_bytes},
        }
        for k, r in roofs.items():
            r["kernel_ms"] = kernel_ms[k]
        roofs["sort"] = sort_roofline(args, N, P, W, H, kernel_ms, cpu["super_pairs"])
        # HBM bytes per launch from the committed counter summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated);
        # null when the kernel's sources changed since the counters were taken
        from differentiable_gaussian_splatting_amd import profiling
        traffic_md = os.path.join(ROOT, "profiles", f"hbm_counters_{args.workload}.md")
        for k, r in roofs.items():
            r["frac"] = r["achieved"] / r["peak"]
            if k == "sort":
                if r["scheme"] == "tile_depth":
                    kern = profiling.TILE_FIRST_SORT_KERNELS if r["tile_scan_ms"] > 0 else None
                else:
                    kern = profiling.sort_kernels(r["passes"])
                r["traffic"] = profiling.traffic_for(kern, traffic_md) if kern else None
                continue
            r["traffic"] = profiling.traffic_for(profiling.STAGE_KERNEL[k], traffic_md)
            if r["bound"] == "alu":
                # the share of the chip's VALU issue slots the kernel used: its VALU wave instructions per launch
                # (counter record) over this run's kernel time
                insts = profiling.valu_insts_for(profiling.STAGE_KERNEL[k], traffic_md)
                r["valu_insts_per_launch"] = insts
                r["valu_issue_frac"] = (None if insts is None else
                                        insts / (r["kernel_ms"] * 1e-3 * VALU_ISSUE_PER_S))
                # SIMD cycles in fp32 MFMA (the backward's reduction), which do not overlap VALU issue on a SIMD
                mcyc = profiling.mfma_busy_for(profiling.STAGE_KERNEL[k], traffic_md)
                r["mfma_busy_frac"] = (None if mcyc is None else
                                       mcyc / (r["kernel_ms"] * 1e-3 * 1024 * 2.4e9))
                # the hardware's own vector flop count over the same time: inactive lanes count (an upper bound on
                # the vector work) and matrix-core flops do not (the backward's moment sums run there)
                cf = profiling.counted_flops_for(profiling.STAGE_KERNEL[k], traffic_md)
                r["counted_tflops_upper"] = None if cf is None else cf / (r["kernel_ms"] * 1e-3) / 1e12
                r["counted_frac_upper"] = None if cf is None else r["counted_tflops_upper"] / ALU_PEAK_TFLOPS
        # the forward with the hardware exponential (GSR_OPT_FORWARD_EXP), the same operation count
        kf = fast_exp["kernel_ms"]
        roofs["forward_fast_exp"] = {"bound": "alu", "achieved": fwd_ops / (kf * 1e-3) / 1e12, "peak": ALU_PEAK_TFLOPS,
                                     "unit": "TFLOP/s", "work_per_launch": fwd_ops, "achieved_kind": eff,
                                     "kernel_ms": kf, "frac": fwd_ops / (kf * 1e-3) / 1e12 / ALU_PEAK_TFLOPS,
                                     "traffic": profiling.traffic_for(profiling.STAGE_KERNEL["forward_fast_exp"],
                                                                      traffic_md)}
        insts = profiling.valu_insts_for(profiling.STAGE_KERNEL["forward_fast_exp"], traffic_md)
        roofs["forward_fast_exp"]["valu_insts_per_launch"] = insts
        roofs["forward_fast_exp"]["valu_issue_frac"] = None if insts is None else insts / (kf * 1e-3 * VALU_ISSUE_PER_S)
        for k in ("forward", "backward", "forward_fast_exp"):
            roofs[k]["frac_of_nonpacked_78_6"] = roofs[k]["achieved"] / ALU_NONPACKED_TFLOPS
        dominant = max(("forward", "backward", "adam"), key=lambda k: kernel_ms[k])
        result["roofline"] = {"kernel": dominant, **roofs[dominant]}
        result["rooflines"] = roofs
        ct = cpu["times"]
        cpu_step = sum(ct.values())
        result["cpu_baseline"] = {"value": evals / cpu_step, "unit": UNIT, "cores": 1, "kind": "oracle",
                                  "sample": "one whole step of the same workload (bin + forward + backward + Adam "
                                            "over all 410k splats), single-threaded",
                                  "stage_s": ct, "host_cpus": os.cpu_count(), "host_cpu_model": cpu_model()}
        cm = cpu["times_mt"]
        result["cpu_baseline_all_cores"] = {"value": evals / sum(cm.values()), "unit": UNIT, "cores": cpu["threads"],
                                            "kind": "oracle",
                                            "sample": "the same step with the oracle's forward and backward run by "
                                                      f"{cpu['threads']} threads over bands of tile rows (binning "
                                                      "and Adam single-threaded)",
                                            "stage_s": cm}
    else:
        result["value"] = None
    # the pages' own figures, for context only (another GPU, their trained 409,660-splat checkpoint of the same image
    # size, not this synthetic workload): vs_baseline stays null
    result["context"] = {"pages_m4max_ms_per_iter_fwd_bwd_adam": 15.354, "pages_m4max_backward_ms_per_call": 4.65,
                         "pages_splats": 409660, "this_fwd_bwd_adam_ms": stage_ms["forward"] + stage_ms["backward"]
                         + stage_ms["adam"], "this_backward_ms": stage_ms["backward"]}
    stream = device_stream_gbs(torch)
    result["context"]["torch_stream_gbs"] = stream
    if result.get("rooflines"):
        result["context"]["adam_frac_of_torch_add"] = result["rooflines"]["adam"]["achieved"] / stream["add"]
    result["projection"] = bench_projection(args, ctx, gsr, scenes, sc, hp=hp, bc=bc)
    if not args.no_bin_stress:
        result["bin_stress"] = bench_bin_stress(args, ctx, gsr, scenes, torch, np)
    if not args.no_views:
        result["changing_views"] = bench_changing_views(args, ctx, gsr, scenes, torch, np)
    print(json.dumps(result), flush=True)
    ctx.close()


def bench_per_splat_backward(args, ctx, gsr, torch, np, splats, b, W, H, out_rgba, final_T, last_contrib, v_out,
                             grad):
    """The backward in the per-splat loop order (GSR_BACKWARD_PER_SPLAT) on the last step's bins and image: its
    kernel's time from the library's events over K launches, and the largest difference from the default order's
    gradients in units of the parity bar (both sum the same terms in other orders)."""
    ref = grad.clone()
    g = torch.empty_like(grad)
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_BACKWARD_SCHEME, gsr.GSR_BACKWARD_PER_SPLAT)
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_KERNEL_TIMING, args.steps)
    try:
        for _ in range(args.steps):
            gsr.gsr_render_backward(ctx, splats, b, W, H, out_rgba, final_T, last_contrib, v_out, g)
        kms = float(np.mean(gsr.gsr_kernel_times(ctx, gsr.GSR_STAGE_BACKWARD)))
    finally:
        gsr.gsr_set_option(ctx, gsr.GSR_OPT_KERNEL_TIMING, 0)
        gsr.gsr_set_option(ctx, gsr.GSR_OPT_BACKWARD_SCHEME, gsr.GSR_BACKWARD_PER_PIXEL)
    dev = ((g - ref).abs() / (1e-4 + 1e-4 * ref.abs())).max().item()
    return {"kernel_ms": kms, "max_diff_to_default_in_units_of_1e-4_abs_plus_rel": dev}


def scheme_opt(gsr, name):
    return {"tile_depth": gsr.GSR_BIN_TILE_DEPTH, "presort": gsr.GSR_BIN_PRESORT, "key64": gsr.GSR_BIN_KEY64}[name]


def sort_roofline(args, N, P, W, H, kernel_ms, Ps=None):
    """The binning's sorts against HBM: algorithmic bytes of the scheme per launch over their kernels' own time.
    Tile-first (the default): see the branch below. Presort: the two radix sorts. Depth sort: 4 passes of 8-bit
    digits over the n 32-bit depth keys with their indices, each pass reading the keys for the histogram (4 B) and
    reading and writing key and index (16 B). Tile sort: 2
    passes of 6-bit digits over the pairs; packed (tile and splat in one 32-bit word when they fit) a pass reads
    the words twice and writes them once (12 B), and the last one also writes the splat index (4 B), the 64-bit key
    (8 B) and gathers the depth (4 B); unpacked each pass moves tile id and index (20 B) and the last one adds the
    64-bit key and the depth gather (12 B). The pages' target is stated for their 64-bit key sort, P (8 + 24 d) B at
    d = 6 passes, at 70 % of the peak: its time is reported beside ours."""
    tiles = ((W + 15) // 16) * ((H + 15) // 16)
    bits = lambda v: int(v).bit_length()
    tile_bits = bits(tiles - 1)
    tile_passes = (tile_bits + 5) // 6
    packed = N > 0 and tile_bits > 0 and bits(N - 1) + tile_bits <= 32
    pages_bytes = P * (8 + 24 * 6)
    pages = {"pages_64bit_sort_bytes": pages_bytes,
             "pages_target_ms_at_70pct": pages_bytes / (0.7 * HBM_PEAK_GBS * 1e9) * 1e3}
    if args.bin_scheme == "tile_depth" and kernel_ms["tile_depth"] > 0:
        # tile-first. Under the box rule (the two-level counting sort, tile_scan > 0): the column scan reads the
        # [blocks of 1024 splats][tiles + super-tiles] count table twice and writes it once (12 B per entry), the
        # starts read the totals and write the starts (8 B per list) and the tiles' ranges (8 B per tile); the
        # scatter reads each splat's rectangle and depth (20 B), its block's row of the super-tile part of the table
        # and the super-tile starts (8 B per super-tile and block), and writes each (splat, super-tile) pair's 8 B
        # entry; the per-super-tile order reads those entries (8 B) and writes each (splat, tile) pair's value and
        # 64-bit key (12 B). Otherwise the tile ids' radix sort on packed words (12 B per pair and pass) and the
        # per-tile order (it reads each pair's splat and gathers its depth, 8 B, and writes 12 B).
        fused = kernel_ms["tile_scan"] > 0
        nblk = (N + 1023) // 1024
        sups = ((W + 31) // 32) * ((H + 31) // 32)
        if fused:
            by = (12 * P + 16 * Ps + 20 * N + 12 * nblk * (tiles + sups) + 8 * nblk * sups + 8 * (tiles + sups)
                  + 8 * tiles)
            ms = kernel_ms["tile_scan"] + kernel_ms["tile_sort"] + kernel_ms["tile_depth"]
            note = ("count table scan + list starts + scatter to super-tiles + per-super-tile order "
                    f"({Ps} super-tile pairs)")
        else:
            by = (12 * tile_passes + 20) * P
            ms = kernel_ms["tile_sort"] + kernel_ms["tile_depth"] + kernel_ms["tile_scan"]
            note = f"radix sort of the tile ids ({tile_passes} passes, packed words) + per-tile order"
        return {"bound": "hbm", "achieved": by / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "work_per_launch": by, "kernel_ms": ms, "scheme": "tile_depth", "bytes": note,
                "tile_scan_ms": kernel_ms["tile_scan"], "tile_sort_ms": kernel_ms["tile_sort"],
                "tile_depth_ms": kernel_ms["tile_depth"], **pages}
    per_pair = (12 * tile_passes + 16) if packed else (20 * tile_passes + 12)
    by = 4 * 20 * N + per_pair * P
    ms = kernel_ms["depth_sort"] + kernel_ms["tile_sort"]
    return {"bound": "hbm", "achieved": by / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "work_per_launch": by, "kernel_ms": ms, "scheme": "presort", "depth_sort_ms": kernel_ms["depth_sort"],
            "tile_sort_ms": kernel_ms["tile_sort"], "packed": packed, "passes": {"depth": 4, "tile": tile_passes},
            **pages}


def bench_bin_stress(args, ctx, gsr, scenes, torch, np):
    """The binning on its own on the 1M-splat stress scene (about 26M pairs under the box rule), under the tile-first
    default and the presort and 64-bit key schemes, timed with the library's events over K calls per repeat (median
    of the repeats' means). Sort rooflines on algorithmic bytes:
      tile_depth (the default): as sort_roofline's two-level form (the super-tile lists, about 15,000 entries each
        here, are ordered in chunks on chip);
      key64 (the pages' scheme): a stable LSD sort of the 64-bit (tile | depth) keys with their 32-bit values over
        d = ceil((tile bits + 32) / 8) passes, P (8 + 24 d) bytes: one read of the keys for the digit histograms and
        a read and a write of key and value per pass;
      presort: the depth sort of the n 32-bit depth keys with their indices (4 passes, 20 B per key
        per pass) and the tile sort of the pairs by their tile id (per pass 12 B per pair on packed 32-bit words;
        the last one adds the 4 B value, the 8 B 64-bit key and the 4 B depth gather)."""
    sc = scenes.make_scene("bin1m")
    W, H, N = sc.width, sc.height, sc.spec.n
    sp, dp = torch.from_numpy(sc.splats).cuda(), torch.from_numpy(sc.depths).cuda()
    tiles = ((W + 15) // 16) * ((H + 15) // 16)
    tile_bits = int(tiles - 1).bit_length()
    out = {"workload": f"bin1m: {W}x{H} image, {N} splats ({scene_label(sc.spec)}), box rule"}
    for scheme, opt in (("tile_depth", gsr.GSR_BIN_TILE_DEPTH), ("presort", gsr.GSR_BIN_PRESORT),
                        ("key64", gsr.GSR_BIN_KEY64)):
        gsr.gsr_set_option(ctx, gsr.GSR_OPT_BIN_SCHEME, opt)
        b = gsr.gsr_bin(ctx, sp, dp, W, H)
        P = b.num_pairs
        gsr.gsr_reserve(ctx, P, N)
        for _ in range(3):
            gsr.gsr_bin(ctx, sp, dp, W, H)
        reps = {"bin": [], "depth_sort": [], "tile_sort": [], "tile_scan": [], "tile_depth": []}
        for _ in range(args.repeats):
            gsr.gsr_set_option(ctx, gsr.GSR_OPT_KERNEL_TIMING, args.steps)
            for _ in range(args.steps):
                b = gsr.gsr_bin(ctx, sp, dp, W, H)
            torch.cuda.synchronize()
            for nm, stg in (("bin", gsr.GSR_STAGE_BIN), ("depth_sort", gsr.GSR_STAGE_DEPTH_SORT),
                            ("tile_sort", gsr.GSR_STAGE_TILE_SORT), ("tile_scan", gsr.GSR_STAGE_TILE_SCAN),
                            ("tile_depth", gsr.GSR_STAGE_TILE_DEPTH)):
                t = gsr.gsr_kernel_times(ctx, stg)
                reps[nm].append(float(np.mean(t)) if t else 0.0)
            gsr.gsr_set_option(ctx, gsr.GSR_OPT_KERNEL_TIMING, 0)
        ms = {nm: float(np.median(v)) for nm, v in reps.items()}
        if scheme == "tile_depth":
            keys, vals, _ = gsr.gsr_bins_copy(ctx, b)
            Ps = super_pairs(keys.cpu().numpy().view(np.uint64), vals.cpu().numpy().view(np.uint32), W)
            roof = sort_roofline(argparse.Namespace(bin_scheme="tile_depth"), N, P, W, H, ms, Ps)
            by, sort_ms, note = roof["work_per_launch"], roof["kernel_ms"], roof["bytes"]
        elif scheme == "key64":
            d = (tile_bits + 32 + 7) // 8
            by = P * (8 + 24 * d)
            sort_ms = ms["tile_sort"]
            note = f"64-bit key sort, {d} passes of 8-bit digits: P (8 + 24 d) B"
        else:
            packed = int(N - 1).bit_length() + tile_bits <= 32
            tp = (tile_bits + 5) // 6
            by = 4 * 20 * N + ((12 * tp + 16) if packed else (20 * tp + 12)) * P
            sort_ms = ms["depth_sort"] + ms["tile_sort"]
            note = (f"depth sort 4 x 20 B per splat + tile sort {tp} passes of 6-bit digits "
                    f"({'packed' if packed else 'unpacked'})")
        ach = by / (sort_ms * 1e-3) / 1e9
        # HBM bytes per bin from the committed counter record of this leg (copy-calibrated), or null
        from differentiable_gaussian_splatting_amd import profiling
        md = os.path.join(ROOT, "profiles", "hbm_counters_bin1m.md")
        if scheme == "tile_depth":
            kern = profiling.TILE_FIRST_SORT_KERNELS
        elif scheme == "key64":
            d = (tile_bits + 32 + 7) // 8
            kern = ("k_upsweep<uint64,16u,8u>", "k_scan_rows", "k_scatter<uint64,16u,8u,false,false>") * d
        else:
            kern = profiling.sort_kernels({"depth": 4, "tile": (tile_bits + 5) // 6})
        traffic = profiling.traffic_for(kern, md)
        out[scheme] = {"pairs": P, "bin_ms": ms["bin"], "depth_sort_ms": ms["depth_sort"],
                       "tile_sort_ms": ms["tile_sort"], "tile_scan_ms": ms["tile_scan"],
                       "tile_depth_ms": ms["tile_depth"], "sigma": {nm: float(np.std(v)) for nm, v in reps.items()},
                       "sort_roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                         "frac": ach / HBM_PEAK_GBS, "work_per_launch": by, "kernel_ms": sort_ms,
                                         "bytes": note, "traffic": traffic}}
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_BIN_SCHEME, scheme_opt(gsr, args.bin_scheme))
    k64 = out["key64"]["sort_roofline"]["work_per_launch"]
    out["pages_target_ms_at_70pct"] = k64 / (0.7 * HBM_PEAK_GBS * 1e9) * 1e3
    return out


def bench_changing_views(args, ctx, gsr, scenes, torch, np):
    """The raster kernels when every step sees a new view, as in training: gauss410k projected by a camera that
    turns 1 degree about its vertical axis per step (about 14 px, most of a tile, of image motion), then bin,
    forward and backward. The default launch order ranks the tiles by the walk counts of the previous forward -
    here a different view - so this leg times the forward and backward kernels (library events, min(K, 20) steps
    per repeat, so that the camera turns at most 20 degrees; median of the repeats) under each order: cost
    (default), list length, tile index."""
    nv = min(args.steps, 20)
    g3 = scenes.make_gaussians("gauss410k")
    W, H = g3.width, g3.height
    ps = [torch.from_numpy(a).cuda() for a in (g3.means, g3.log_scales, g3.quats, g3.raw_opacities, g3.sh)]
    v_out = torch.from_numpy(np.random.default_rng(31).normal(0.0, 0.01, (H, W, 4)).astype(np.float32)).cuda()
    cams = []
    for k in range(nv + 1):
        a = np.deg2rad(1.0 * k)
        Ry = np.array([[np.cos(a), 0.0, np.sin(a)], [0.0, 1.0, 0.0], [-np.sin(a), 0.0, np.cos(a)]])
        R = Ry @ np.asarray(g3.camera["R"], np.float64)
        cams.append(gsr.camera(R, g3.camera["tv"], g3.camera["fx"], g3.camera["fy"], g3.camera["cx"],
                               g3.camera["cy"], g3.camera["near"]))
    n = g3.spec.n
    sp = torch.empty((n, 9), dtype=torch.float32, device="cuda")
    dp = torch.empty(n, dtype=torch.float32, device="cuda")
    out = torch.empty((H, W, 4), dtype=torch.float32, device="cuda")
    ft = torch.empty((H, W), dtype=torch.float32, device="cuda")
    lc = torch.empty((H, W), dtype=torch.int32, device="cuda")
    grad = torch.empty((n, 9), dtype=torch.float32, device="cuda")
    res = {"workload": f"gauss410k: {n} 3D Gaussians, {W}x{H}, camera turning 1 degree per step",
           "pairs_first_last": None}
    pairs = []
    for name, order in (("cost", gsr.GSR_ORDER_COST), ("length", gsr.GSR_ORDER_LENGTH),
                        ("index", gsr.GSR_ORDER_NONE)):
        gsr.gsr_set_option(ctx, gsr.GSR_OPT_TILE_ORDER, order)
        reps = {"forward": [], "backward": []}
        for _ in range(args.repeats):
            # a forward on the first view, so that the first timed step ranks by a previous view's counts
            gsr.gsr_project_forward(ctx, cams[0], *ps, splats=sp, depths=dp)
            b = gsr.gsr_bin(ctx, sp, dp, W, H)
            gsr.gsr_render_forward(ctx, sp, b, W, H, out, ft, lc)
            torch.cuda.synchronize()
            gsr.gsr_set_option(ctx, gsr.GSR_OPT_KERNEL_TIMING, nv)
            for k in range(1, nv + 1):
                gsr.gsr_project_forward(ctx, cams[k], *ps, splats=sp, depths=dp)
                b = gsr.gsr_bin(ctx, sp, dp, W, H)
                gsr.gsr_render_forward(ctx, sp, b, W, H, out, ft, lc)
                gsr.gsr_render_backward(ctx, sp, b, W, H, out, ft, lc, v_out, grad)
                if name == "cost" and not pairs:
                    pairs.append(b.num_pairs)
            torch.cuda.synchronize()
            pairs.append(b.num_pairs)
            reps["forward"].append(float(np.mean(gsr.gsr_kernel_times(ctx, gsr.GSR_STAGE_FORWARD))))
            reps["backward"].append(float(np.mean(gsr.gsr_kernel_times(ctx, gsr.GSR_STAGE_BACKWARD))))
            gsr.gsr_set_option(ctx, gsr.GSR_OPT_KERNEL_TIMING, 0)
        res[name] = {k: float(np.median(v)) for k, v in reps.items()}
        res[name]["sigma"] = {k: float(np.std(v)) for k, v in reps.items()}
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_TILE_ORDER, gsr.GSR_ORDER_COST)
    res["pairs_first_last"] = [pairs[0], pairs[-1]]
    res["gain_of_cost_order_vs_length"] = {k: res["length"][k] / res["cost"][k] for k in ("forward", "backward")}
    return res


def bench_fast_exp_forward(args, ctx, gsr, torch, np, splats, b, W, H, out_rgba, final_T, last_contrib):
    """The forward with the hardware exponential (GSR_OPT_FORWARD_EXP = GSR_EXP_FAST) on the last step's bins:
    its kernel's time from the library's events over K launches per repeat (the median of the repeats' means), and
    how far its outputs are from the exact forward's: pixels whose last contributor differs, and the largest image
    difference elsewhere."""
    print("[bench] forward with the hardware exponential", file=sys.stderr, flush=True)
    o2, t2, l2 = torch.empty_like(out_rgba), torch.empty_like(final_T), torch.empty_like(last_contrib)
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_FORWARD_EXP, gsr.GSR_EXP_FAST)
    reps = []
    try:
        for _ in range(args.repeats):
            gsr.gsr_set_option(ctx, gsr.GSR_OPT_KERNEL_TIMING, args.steps)
            for _ in range(args.steps):
                gsr.gsr_render_forward(ctx, splats, b, W, H, o2, t2, l2)
            reps.append(float(np.mean(gsr.gsr_kernel_times(ctx, gsr.GSR_STAGE_FORWARD))))
            gsr.gsr_set_option(ctx, gsr.GSR_OPT_KERNEL_TIMING, 0)
    finally:
        gsr.gsr_set_option(ctx, gsr.GSR_OPT_KERNEL_TIMING, 0)
        gsr.gsr_set_option(ctx, gsr.GSR_OPT_FORWARD_EXP, gsr.GSR_EXP_EXACT)
    same = l2 == last_contrib
    d_img = float((o2 - out_rgba).abs().amax(dim=-1)[same].max().item()) if bool(same.any()) else 0.0
    return {"kernel_ms": float(np.median(reps)), "repeats": reps, "sigma": float(np.std(reps)),
            "pixels_stopping_apart_from_exact": int((~same).sum().item()),
            "max_image_diff_elsewhere": d_img}


def bench_sync_free(args, ctx, gsr, torch, np, step, bins_sync, walls_sync):
    """The same steps with GSR_OPT_BIN_SYNC_FREE: gsr_bin queues its launches without waiting for the pair count
    (buffers sized from the counts seen). Wall clock of K steps, `repeats` times, beside the waiting form's; checks
    that no call overflowed and that the bins equal the waiting form's."""
    print("[bench] sync-free binning", file=sys.stderr, flush=True)
    ref_keys, ref_vals, ref_ranges = gsr.gsr_bins_copy(ctx, bins_sync)
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_BIN_SYNC_FREE, 1)
    try:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        walls = []
        for _ in range(args.repeats):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                b = step()
            torch.cuda.synchronize()
            walls.append(time.perf_counter() - t0)
        pairs, over = gsr.gsr_bin_pair_count(ctx)
        keys, vals, ranges = gsr.gsr_bins_copy(ctx, b)
        P = bins_sync.num_pairs
        same = (not over and pairs == P and torch.equal(ranges, ref_ranges) and torch.equal(vals[:P], ref_vals)
                and (keys is None or torch.equal(keys[:P], ref_keys)))
    finally:
        gsr.gsr_set_option(ctx, gsr.GSR_OPT_BIN_SYNC_FREE, 0)
    ms = [w * 1e3 / args.steps for w in walls]
    ms_sync = [w * 1e3 / args.steps for w in walls_sync]
    return {"ms_per_step": float(np.median(ms)), "repeats": ms, "sigma": float(np.std(ms)),
            "ms_per_step_waiting": float(np.median(ms_sync)), "capacity": int(b.num_pairs), "pairs": pairs,
            "overflowed": over, "bins_equal_waiting_form": bool(same)}


def bench_deterministic_backward(args, ctx, gsr, torch, np, stream, splats, b, W, H, out_rgba, final_T, last_contrib,
                                 v_out, grad):
    """The backward with GSR_OPT_DETERMINISTIC on the last step's bins and image, timed like the step's stages
    (outside the step's timed region); a second run checks that the gradients repeat bit for bit, and the largest
    difference from the default mode's gradients is reported."""
    ref = grad.clone()
    g = [torch.empty_like(grad), torch.empty_like(grad)]
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_DETERMINISTIC, 1)
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_KERNEL_TIMING, args.steps)
    try:
        gsr.gsr_render_backward(ctx, splats, b, W, H, out_rgba, final_T, last_contrib, v_out, g[0])
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for k in range(args.steps):
            ev[k][0].record(stream)
            gsr.gsr_render_backward(ctx, splats, b, W, H, out_rgba, final_T, last_contrib, v_out, g[1])
            ev[k][1].record(stream)
        torch.cuda.synchronize()
        kms = float(np.mean(gsr.gsr_kernel_times(ctx, gsr.GSR_STAGE_BACKWARD)))
    finally:
        gsr.gsr_set_option(ctx, gsr.GSR_OPT_KERNEL_TIMING, 0)
        gsr.gsr_set_option(ctx, gsr.GSR_OPT_DETERMINISTIC, 0)
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    same = bool(torch.equal(g[0].view(torch.int32), g[1].view(torch.int32)))
    dev = ((g[0] - ref).abs() / (1e-4 + 1e-4 * ref.abs())).max().item()
    return {"ms": ms, "kernel_ms": kms, "repeats_bit_identical": same,
            "max_diff_to_default_in_units_of_1e-4_abs_plus_rel": dev}


def bench_projection(args, ctx, gsr, scenes, sc, hp, bc):
    """The steps on either side of the path, timed on their own (not part of `value`): the projection of 410k 3D
    Gaussians to splats and its backward pass, and a whole training iteration that chains them with the path
    (project, bin, forward, backward, project backward, Adam on the five parameter groups with those gradients)."""
    import numpy as np
    import torch
    from differentiable_gaussian_splatting_amd import profiling

    g3 = scenes.make_gaussians("gauss410k")
    n = g3.spec.n
    cam = gsr.camera(g3.camera["R"], g3.camera["tv"], g3.camera["fx"], g3.camera["fy"], g3.camera["cx"],
                     g3.camera["cy"], g3.camera["near"])
    ps = [torch.from_numpy(a).cuda() for a in (g3.means, g3.log_scales, g3.quats, g3.raw_opacities, g3.sh)]
    sg = torch.from_numpy(g3.splats_grad).cuda()
    sp, dp = gsr.gsr_project_forward(ctx, cam, *ps)
    grads = gsr.gsr_project_backward(ctx, cam, *ps, sg)
    stream = torch.cuda.current_stream()
    reps = max(5, args.steps)
    for _ in range(3):
        gsr.gsr_project_forward(ctx, cam, *ps, splats=sp, depths=dp)
        gsr.gsr_project_backward(ctx, cam, *ps, sg, grads=grads)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for k in range(reps):
        ev[k][0].record(stream)
        gsr.gsr_project_forward(ctx, cam, *ps, splats=sp, depths=dp)
        ev[k][1].record(stream)
        gsr.gsr_project_backward(ctx, cam, *ps, sg, grads=grads)
        ev[k][2].record(stream)
    torch.cuda.synchronize()
    f_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    b_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    # algorithmic bytes: forward reads 59 parameters and writes the 9-value record and the depth; the backward reads
    # the parameters and the record gradient and writes 59 gradients
    f_bytes, b_bytes = n * (59 + 10) * 4, n * (59 + 9 + 59) * 4
    traffic_md = os.path.join(ROOT, "profiles", f"hbm_counters_{args.workload}.md")
    roofs = {}
    for k, ms, by in (("project_forward", f_ms, f_bytes), ("project_backward", b_ms, b_bytes)):
        ach = by / (ms * 1e-3) / 1e9
        roofs[k] = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                    "work_per_launch": by, "traffic": profiling.traffic_for(profiling.STAGE_KERNEL[k], traffic_md)}

    # a whole training iteration on the projected splats, with the loss giving the backward its v_out
    W, H = sc.width, sc.height
    target = torch.from_numpy(scenes.make_target(W, H)).cuda()
    v_out = torch.empty((H, W, 4), dtype=torch.float32, device="cuda")
    loss_val = torch.empty(3, dtype=torch.float32, device="cuda")
    out = torch.empty((H, W, 4), dtype=torch.float32, device="cuda")
    ft = torch.empty((H, W), dtype=torch.float32, device="cuda")
    lc = torch.empty((H, W), dtype=torch.int32, device="cuda")
    rec_grad = torch.empty((n, 9), dtype=torch.float32, device="cuda")
    ms_ = [torch.zeros_like(p) for p in ps]
    vs_ = [torch.zeros_like(p) for p in ps]
    adam = [(p, g, m, v, hp["lr"]) for p, g, m, v in zip(ps, grads, ms_, vs_)]

    def iteration():
        gsr.gsr_project_forward(ctx, cam, *ps, splats=sp, depths=dp)
        b = gsr.gsr_bin(ctx, sp, dp, W, H)
        gsr.gsr_render_forward(ctx, sp, b, W, H, out, ft, lc)
        gsr.gsr_loss_l1_ssim(ctx, out, target, v_out, loss_val)
        gsr.gsr_render_backward(ctx, sp, b, W, H, out, ft, lc, v_out, rec_grad)
        gsr.gsr_project_backward(ctx, cam, *ps, rec_grad, grads=grads)
        gsr.gsr_adam_step(ctx, adam, hp["beta1"], hp["beta2"], hp["eps"], *bc)
        return b

    for _ in range(3):
        iteration()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        b = iteration()
    torch.cuda.synchronize()
    it_ms = (time.perf_counter() - t0) * 1e3 / reps
    loss_after = loss_val.tolist()
    # the loss alone, on the last rendered image
    lev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for k in range(reps):
        lev[k][0].record(stream)
        gsr.gsr_loss_l1_ssim(ctx, out, target, v_out, loss_val)
        lev[k][1].record(stream)
    torch.cuda.synchronize()
    l_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in lev]))
    loss_ops = 3 * W * H * LOSS_OPS
    roofs["loss_l1_ssim"] = {"bound": "alu", "achieved": loss_ops / (l_ms * 1e-3) / 1e12, "peak": ALU_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "work_per_launch": loss_ops,
                             "traffic": profiling.traffic_for(profiling.STAGE_KERNEL["loss_l1_ssim"], traffic_md)}
    roofs["loss_l1_ssim"]["frac"] = roofs["loss_l1_ssim"]["achieved"] / ALU_PEAK_TFLOPS

    # Visible-only Adam against the dense step, with the visibility of this view (b, the last iteration's bins) and
    # of the same camera panned by half the image width (its principal point moved by W / 2), which sees part of
    # the Gaussians; algorithmic bytes = 28 per element of a visible splat + 4 per splat for its pair count
    def time_adam(visible):
        ae = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for k in range(reps):
            ae[k][0].record(stream)
            if visible is None:
                gsr.gsr_adam_step(ctx, adam, hp["beta1"], hp["beta2"], hp["eps"], *bc)
            else:
                gsr.gsr_adam_step_visible(ctx, adam, hp["beta1"], hp["beta2"], hp["eps"], *bc, visible, n)
            ae[k][1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([e[0].elapsed_time(e[1]) for e in ae]))

    dense_ms = time_adam(None)
    sparse = {"dense_ms": dense_ms, "dense_bytes": 28 * 59 * n}
    pan = gsr.camera(g3.camera["R"], g3.camera["tv"], g3.camera["fx"], g3.camera["fy"], g3.camera["cx"] + W / 2,
                     g3.camera["cy"], g3.camera["near"])
    for view, c in (("this_view", None), ("panned_half_width", pan)):
        if c is None:
            vb = b
        else:
            sp2, dp2 = gsr.gsr_project_forward(ctx, c, *ps)
            vb = gsr.gsr_bin(ctx, sp2, dp2, W, H)
        nvis = int((gsr.gsr_bins_splat_pairs(ctx, vb) != 0).sum().item())
        ms = time_adam(vb)
        by = 28 * 59 * nvis + 4 * n
        ach = by / (ms * 1e-3) / 1e9
        sparse[view] = {"visible_fraction": nvis / n, "ms": ms, "speedup_vs_dense": dense_ms / ms,
                        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": ach / HBM_PEAK_GBS, "work_per_launch": by}}
    out_d = {"workload": f"gauss410k: {n} 3D Gaussians (means, log_scales, quats, raw_opacities, SH degree 3) seen "
                         f"by an {W}x{H} pinhole camera, projected sizes as the path's workload",
             "forward_ms": f_ms, "backward_ms": b_ms, "loss_ms": l_ms, "rooflines": roofs,
             "iteration_ms": it_ms, "iteration_pairs": b.num_pairs, "iteration_loss": loss_after,
             "adam_visible_only": sparse,
             "iteration": "project + bin + forward + L1/SSIM loss + backward + project backward + Adam on the 5 "
                          "groups"}
    if not args.no_cpu_baseline:
        from oracle import project as op
        ocam = op.Camera(R=g3.camera["R"], tv=g3.camera["tv"], fx=g3.camera["fx"], fy=g3.camera["fy"],
                         cx=g3.camera["cx"], cy=g3.camera["cy"], near=g3.camera["near"])
        par = (g3.means, g3.log_scales, g3.quats, g3.raw_opacities, g3.sh)
        t0 = time.perf_counter()
        op.project_forward(ocam, *par)
        t1 = time.perf_counter()
        op.project_backward(ocam, *par, g3.splats_grad)
        t2 = time.perf_counter()
        out_d["cpu_baseline"] = {"forward_s": t1 - t0, "backward_s": t2 - t1, "kind": "oracle",
                                 "cores": torch.get_num_threads(),
                                 "sample": "the oracle's fp64 projection and its automatic backward over all "
                                           f"{n} Gaussians"}
    return out_d


if __name__ == "__main__":
    main()
