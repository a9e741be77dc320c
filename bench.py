"""Benchmark: one training view (forward + backward + one Adam step) of the
tile rasterizer with load-budgeted leaves, on one MI355X.

Default workload: ~6M Gaussians (ground plane + clustered objects, SH degree
3), 16000 x 10560 view, 384 MiB leaf budget, L1 loss, leaf 2D gradients
summed, one projection backward, one Adam step per view.

Prints one JSON line: fwd+bwd Mpixel/s per view (value), with Gaussians/s,
peak working set (GiB), the roofline of the dominant kernel measured live with
HIP events, and the CPU oracle timed on a bounded sample of the same view.
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

MIB = 1 << 20
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E, GB/s
# 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz: f32 VALU instructions per second,
# counting one per lane (an fma counts once); packed f32 is not used.
PEAK_VALU_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# per (pixel, entry) pair of the raster backward: f32 VALU operations of the
# specified arithmetic (recompute power/exp/alpha 29, T recovery 6,
# dL/dalpha 12, the other partials 20, colour-behind update 9)
OPS_PER_PAIR_BWD = 76
OPS_PER_PAIR_FWD = 38


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="c5_plane16k")
    ap.add_argument("--n", type=int, default=None)
    ap.add_argument("--width", type=int, default=None)
    ap.add_argument("--height", type=int, default=None)
    ap.add_argument("--budget-mib", type=float, default=384.0)
    ap.add_argument("--no-adam", action="store_true")
    ap.add_argument("--cpu-baseline", type=int, default=1)
    ap.add_argument("--cpu-window", type=int, default=384, help="side (pixels) of the oracle's sampled window")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    from differentiable_gaussian_splatting_amd import binding as B
    from differentiable_gaussian_splatting_amd import scenes

    t0 = time.time()
    w = scenes.make_workload(args.workload, n=args.n, width=args.width, height=args.height)
    cam, sc = w.camera, w.scene
    budget = int(args.budget_mib * MIB)
    log(f"[bench] workload {w.name}: N={sc.n} {cam.width}x{cam.height} budget={args.budget_mib} MiB "
        f"(generated in {time.time() - t0:.1f}s)")

    B.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    ctx = B.Context()
    params = B.DeviceScene(sc, dev)
    m, v = B.like_scene(params), B.like_scene(params)
    target = torch.from_numpy(w.target).to(dev)
    torch.cuda.synchronize()
    P = cam.width * cam.height

    def step(k):
        adam = None if args.no_adam else dict(step=k, params=params, m=m, v=v, lr=1e-3)
        return B.gs_train_view(ctx, cam, params, target, budget_bytes=budget, loss="l1", adam=adam)

    k = 0
    for _ in range(args.warmup):
        k += 1
        r = step(k)
        log(f"[bench] warmup step {k}: loss {r['loss']:.6f} cand {r['n_cand']} isect {r['n_isect']} "
            f"leaves {r['n_leaves']}")
    torch.cuda.synchronize()
    base_alloc = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    B.gs_reset_timing(ctx)
    B.gs_set_timing(ctx, True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    results = []
    for _ in range(args.steps):
        k += 1
        results.append(step(k))
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    B.gs_set_timing(ctx, False)
    torch_peak = torch.cuda.max_memory_allocated(dev) - base_alloc
    ms_step = 1e3 * t_total / args.steps
    r = results[-1]
    log(f"[bench] {args.steps} steps in {t_total:.3f}s: {ms_step:.2f} ms/step, loss {r['loss']:.6f}, "
        f"leaves {r['n_leaves']}, isect {r['n_isect']}")

    kernels = ["project_flags", "project_write", "prefix2d", "scan", "rect_diff", "emit", "sort_tiles",
               "plan_split", "raster_fwd", "raster_bwd", "project_bwd", "adam"]
    ktimes = {}
    for name in kernels:
        ms, n = B.gs_kernel_time(ctx, name)
        if n:
            ktimes[name] = dict(total_ms=ms / args.steps, launches=n // args.steps, avg_ms=ms / n)
    log("[bench] per-step kernel time (ms): " +
        ", ".join(f"{k}={v['total_ms']:.2f}" for k, v in sorted(ktimes.items(), key=lambda kv: -kv[1]['total_ms'])))

    # work counters of the view (untimed): pairs the raster backward walks
    q_b = count_backward_pairs(B, ctx, cam, params, budget)
    dom = "raster_bwd"
    bwd = ktimes.get(dom, dict(total_ms=float("nan"), launches=0, avg_ms=float("nan")))
    achieved = OPS_PER_PAIR_BWD * q_b / (bwd["total_ms"] * 1e-3) / 1e12   # per-step totals
    roofline = dict(bound="alu", achieved=round(achieved, 3), peak=round(PEAK_VALU_TOPS, 2), unit="Top/s",
                    frac=round(achieved / PEAK_VALU_TOPS, 4), traffic=None, kernel=dom,
                    ops_per_unit=OPS_PER_PAIR_BWD, units_per_step=int(q_b),
                    avg_launch_ms=round(bwd["avg_ms"], 4), launches_per_step=bwd["launches"])

    cpu = None
    if args.cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_window)

    value = P / (ms_step * 1e-3) / 1e6
    out = {
        "metric": "fwd+bwd Mpixel/s per view and peak working set (GiB) on one MI355X",
        "value": round(value, 3),
        "unit": "Mpixel/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {sc.n} Gaussians SH{sc.sh_degree}, {cam.width}x{cam.height}, "
                               f"leaf budget {args.budget_mib:g} MiB, L1, leaf grads summed, "
                               + ("one Adam step per view" if not args.no_adam else "no update"),
                   "n_gaussians": sc.n, "width": cam.width, "height": cam.height,
                   "leaf_budget_mib": args.budget_mib, "parallelism": "single GPU"},
        "gaussians_per_s": round(sc.n / (ms_step * 1e-3), 1),
        "peak_working_set_gib": round(r["peak_bytes"] / 2 ** 30, 4),
        "peak_working_set_torch_gib": round(torch_peak / 2 ** 30, 4),
        "n_candidates": r["n_cand"],
        "n_intersections": r["n_isect"],
        "n_leaves": r["n_leaves"],
        "pairs_backward": int(q_b),
        "kernel_ms_per_step": {k: round(v["total_ms"], 3) for k, v in ktimes.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    ctx.close()


def count_backward_pairs(B, ctx, cam, params, budget):
    """Sum over pixels of the list position after the last included entry
    (the pairs the raster backward revisits), for the view as benchmarked."""
    import torch
    proj, _ = B.gs_project(ctx, cam, params)
    leaves = B.gs_plan_leaves(ctx, cam, proj, budget)
    total = 0
    for L in leaves:
        bins, _ = B.gs_bin_sort(ctx, cam, proj, L)
        ras = B.gs_render_fwd(ctx, cam, proj, bins)
        last = B.gs_export(ctx, ras, B.RASTER_LAST)
        total += int(last.to(torch.int64).sum().item())
        B.gs_release(ctx, ras)
        B.gs_release(ctx, bins)
    B.gs_release(ctx, proj)
    return total


def cpu_baseline(w, window):
    """The CPU oracle as it stands, single-threaded, on a bounded sample of the
    same view: every per-Gaussian stage (f32 and f64 projection, binning of all
    candidates, projection backward) over all N Gaussians, and per-pixel
    compositing forward + backward on a window x window pixel window at the
    image centre; the view time is the per-Gaussian time plus the window's
    pixel time scaled by P / P_window."""
    import oracle
    cam, sc = w.camera, w.scene
    TW, TH = cam.tiles_x, cam.tiles_y
    wt = max(1, window // 16)
    tx0, ty0 = max(0, TW // 2 - wt // 2), max(0, TH // 2 - wt // 2)
    leaf = oracle.rect(tx0, ty0, min(TW, tx0 + wt), min(TH, ty0 + wt))
    p_win = (min(leaf.tx1 * 16, cam.width) - leaf.tx0 * 16) * (min(leaf.ty1 * 16, cam.height) - leaf.ty0 * 16)
    t = time.perf_counter()
    p32 = oracle.project(cam, sc, "f32")
    p64 = oracle.project(cam, sc, "f64")
    ids = np.nonzero(p32["cand"])[0]
    slot_of = np.full(sc.n, -1, np.int64)
    slot_of[ids] = np.arange(ids.size)
    c32 = {k: p32[k][ids] for k in ("rect", "xy", "conic", "depth", "opacity", "rgb")}
    c64 = {k: p64[k][ids] for k in ("xy", "conic", "opacity", "rgb")}
    t_proj = time.perf_counter() - t
    t = time.perf_counter()
    bins = oracle.bin_leaf(TW, leaf, c32["rect"], c32["depth"], with_keys=False)
    t_bin = time.perf_counter() - t
    t = time.perf_counter()
    H, W = cam.height, cam.width
    image = np.zeros((3, H, W), np.float32)
    tf = np.ones((H, W), np.float32)
    last = np.zeros((H, W), np.int32)
    oracle.render_fwd(cam, leaf, bins, c32["xy"], c32["conic"], c32["opacity"], c32["rgb"], image, tf, last)
    dloss = np.zeros((3, H, W), np.float64)
    oracle.loss_l1(cam, leaf, image.astype(np.float64), w.target, dloss)
    grad2d = np.zeros((ids.size, 9), np.float64)
    oracle.render_bwd(cam, leaf, bins, (c32["xy"], c32["conic"], c32["opacity"]),
                      (c64["xy"], c64["conic"], c64["opacity"], c64["rgb"]), dloss, grad2d)
    t_pix = time.perf_counter() - t
    t = time.perf_counter()
    oracle.project_bwd(cam, sc, p32["cand"], p32["flags"], slot_of, grad2d)
    t_pbwd = time.perf_counter() - t
    P = W * H
    t_view = t_proj + t_bin + t_pbwd + t_pix * (P / p_win)
    log(f"[bench] cpu oracle: projection {t_proj:.1f}s, binning {t_bin:.1f}s, window raster {t_pix:.1f}s "
        f"({p_win} px), projection backward {t_pbwd:.1f}s -> view {t_view:.1f}s")
    return {"value": round(P / t_view / 1e6, 5), "unit": "Mpixel/s", "cores": 1, "kind": "oracle",
            "sample": f"all {sc.n} Gaussians through projection (f32 + f64), binning and projection backward; "
                      f"raster fwd+bwd on a {p_win}-pixel window at the image centre, scaled by P/P_window "
                      f"= {P / p_win:.1f}",
            "seconds_measured": round(t_proj + t_bin + t_pix + t_pbwd, 2), "seconds_view_estimate": round(t_view, 1)}


if __name__ == "__main__":
    main()
