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
# f32 VALU lane operations per second (an fma counts once): 256 CUs x 4 SIMD
# x 32 lanes x 2.4 GHz = 78.6 T, i.e. the published 157.3 TFLOP/s f32 vector
# rate.  gfx950 issues f32 add / mul / fma whose operands are VGPRs or inline
# constants at that rate without packed instructions (a wave64 instruction
# every 2 cycles per SIMD, measured); compares, min / max / med3, selects,
# conversions, shifts and instructions reading an SGPR take 4 cycles.
PEAK_VALU_TOPS = 256 * 4 * 32 * 2.4e9 / 1e12
# f32 VALU operations of the specified per-(pixel, entry) arithmetic:
#   every examined pair: offsets 2, power 5, range test 2, exp 14, alpha with
#     clamp and threshold 4                                            = 27
#   an included pair adds, forward: T' 2, stop test 1, weight 1,
#     colour 3 fma                                                     -> 34
#   backward: T recovery 3 (1 - alpha, reciprocal, product), weight 1,
#     colour dot dL/dout 3, dL/dalpha 2, colour behind 1, colour partials
#     3, clamp decision 1, opacity partial 1, -dL/dpower 1, the five
#     power moments q dx, q dy, q dx^2, q dx dy, q dy^2 accumulated 7
#     (the mean and conic partials follow from the moments once per
#     entry, not per pixel)                                            -> 50
OPS_EXAMINED = 27
OPS_INCLUDED_FWD = 34
OPS_INCLUDED_BWD = 50


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
    ap.add_argument("--cpu-window", type=int, default=384,
                    help="side (pixels) of each window the oracle rasterizes for the CPU baseline")
    ap.add_argument("--cpu-windows", type=int, default=16,
                    help="windows of the CPU baseline, one at a seeded position in each cell of a grid over the view")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="host threads of the CPU baseline (0: the cores the process may use, at most 16)")
    ap.add_argument("--attr-steps", type=int, default=2,
                    help="steps of the per-kernel attribution pass (events around every kernel)")
    ap.add_argument("--layout", default="auto",
                    help="auto: load-budgeted leaves; grid:N: a fixed N x N block layout rendered as given "
                         "(the fixed-block baselines)")
    ap.add_argument("--per-block-update", action="store_true",
                    help="with --layout grid:N: one Adam step after every block (each block a view of its own: "
                         "projection, binning, raster, backward and update), instead of one per view")
    ap.add_argument("--skip-gate", type=int, default=0, metavar="VIEWS",
                    help="a sequence over this many posed views with the SkipGS backward gate (warm-up: one pass "
                         "over the views); times --steps gated views after it and prints that line instead")
    ap.add_argument("--serial-leaves", action="store_true",
                    help="render one leaf at a time (no overlap of consecutive leaves' rasters: a smaller peak)")
    ap.add_argument("--cached-layout", action="store_true",
                    help="second-round views: every step after the first re-checks the first step's leaf layout "
                         "against the current model instead of planning afresh")
    ap.add_argument("--target-host", action="store_true",
                    help="keep the target image in pinned host memory; the library copies each leaf's pixels")
    ap.add_argument("--loss", default="auto", choices=["auto", "l1", "l1_ssim"],
                    help="override the workload's loss (l1_ssim: leaves rendered with an SSIM halo)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one device copy of this many MiB (a known-traffic kernel for counter scaling)")
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
    target = torch.from_numpy(w.target).pin_memory() if args.target_host else torch.from_numpy(w.target).to(dev)
    if args.loss != "auto":
        w.loss = args.loss
    torch.cuda.synchronize()
    P = cam.width * cam.height
    if args.calib_copy_mib:
        src = torch.ones(args.calib_copy_mib * MIB // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {args.calib_copy_mib} MiB read + {args.calib_copy_mib} MiB written")
        del src, dst

    if args.skip_gate:
        gated_sequence(args, B, scenes, torch, ctx, w, params, m, v, budget)
        return

    layout = []
    grid = None
    if args.layout.startswith("grid:"):
        nb = int(args.layout.split(":")[1])
        grid = B.gs_grid_leaves(B.load(), cam.tiles_x, cam.tiles_y, nb, nb)
    upd = [0]   # Adam steps taken

    def step(k, loss_out=None):
        if grid is not None:
            if not args.per_block_update:
                upd[0] += 1
                adam = None if args.no_adam else dict(step=upd[0], params=params, m=m, v=v, lr=1e-3)
                return B.gs_train_view(ctx, cam, params, target, budget_bytes=0, loss=w.loss, adam=adam,
                                       leaves_in=grid)
            tot = None
            for blk in grid:
                upd[0] += 1
                adam = None if args.no_adam else dict(step=upd[0], params=params, m=m, v=v, lr=1e-3)
                r = B.gs_train_view(ctx, cam, params, target, budget_bytes=0, loss=w.loss, adam=adam,
                                    leaves_in=[blk], partial=True)
                if tot is None:
                    tot = dict(r)
                else:
                    tot["loss"] += r["loss"]
                    tot["n_isect"] += r["n_isect"]
                    tot["n_leaves"] += r["n_leaves"]
                    tot["peak_bytes"] = max(tot["peak_bytes"], r["peak_bytes"])
            return tot
        adam = None if args.no_adam else dict(step=k, params=params, m=m, v=v, lr=1e-3)
        if not args.cached_layout:
            # loss_out: each view's loss stays on the device (a training loop
            # reads it when it needs it), so the host queues the next view
            # while this one's last kernels run
            return B.gs_train_view(ctx, cam, params, target, budget_bytes=budget, loss=w.loss, adam=adam,
                                   serial_leaves=args.serial_leaves, loss_out=loss_out)
        # the first step plans and returns its layout; later steps re-check it
        r = B.gs_train_view(ctx, cam, params, target, budget_bytes=budget, loss=w.loss, adam=adam,
                            max_leaves=0 if layout else 65536, leaves_in=layout or None)
        if not layout:
            layout.extend(r["leaves"])
        return r

    k = 0
    for _ in range(args.warmup):
        k += 1
        r = step(k)
        log(f"[bench] warmup step {k}: loss {r['loss']:.6f} cand {r['n_cand']} isect {r['n_isect']} "
            f"leaves {r['n_leaves']}")
    kernels = ["project_flags", "project_write", "prefix2d", "scan", "rect_diff", "bin_count", "emit", "radix",
               "seg_offsets", "fine", "plan_split", "leaf_groups", "raster_fwd", "raster_bwd", "raster_fused", "tile_order",
               "project_bwd", "adam", "bwd_adam"]

    def kernel_times(n_steps, names):
        out = {}
        for name in names:
            ms, n = B.gs_kernel_time(ctx, name)
            if n:
                out[name] = dict(total_ms=ms / n_steps, launches=n // n_steps, avg_ms=ms / n)
        return out

    # attribution pass (not timed as a whole): HIP events around every kernel
    # give the per-kernel split of a step and name the dominant kernel
    torch.cuda.synchronize()
    B.gs_reset_timing(ctx)
    B.gs_set_timing_only(ctx, None)
    B.gs_set_timing(ctx, True)
    for _ in range(args.attr_steps):
        k += 1
        step(k)
    torch.cuda.synchronize()
    B.gs_set_timing(ctx, False)
    ktimes = kernel_times(args.attr_steps, kernels)
    log("[bench] per-step kernel time (ms): " +
        ", ".join(f"{k}={v['total_ms']:.2f}" for k, v in sorted(ktimes.items(), key=lambda kv: -kv[1]['total_ms'])))
    # the dominant kernel among those with a work model (every kernel of a
    # view at full size; the small per-leaf scans only lead at tiny sizes)
    modeled = set(KERNEL_WORK_NAMES)
    dom = max((n for n in ktimes if n in modeled), key=lambda n: ktimes[n]["total_ms"])

    # timed region: HIP events only around the dominant kernel
    torch.cuda.synchronize()
    base_alloc = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    ctx.reset_peak()
    B.gs_reset_timing(ctx)
    B.gs_set_timing_only(ctx, dom)
    B.gs_set_timing(ctx, True)
    losses = torch.full((args.steps,), float("nan"), dtype=torch.float64, device=dev)
    async_loss = grid is None and not args.cached_layout
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    results = []
    for i in range(args.steps):
        k += 1
        results.append(step(k, losses[i:i + 1] if async_loss else None))
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    if async_loss:
        lv = losses.cpu().numpy()
        if not np.isfinite(lv).all():
            raise RuntimeError(f"non-finite loss in the timed steps: {lv}")
        for rr, lo in zip(results, lv):
            rr["loss"] = float(lo)
    B.gs_set_timing(ctx, False)
    B.gs_set_timing_only(ctx, None)
    dom_live = kernel_times(args.steps, [dom])[dom]
    torch_peak = torch.cuda.max_memory_allocated(dev) - base_alloc
    mem = ctx.mem_stats()
    ms_step = 1e3 * t_total / args.steps
    r = results[-1]
    log(f"[bench] {args.steps} steps in {t_total:.3f}s: {ms_step:.2f} ms/step, loss {r['loss']:.6f}, "
        f"leaves {r['n_leaves']}, isect {r['n_isect']}; {dom} {dom_live['avg_ms']:.4f} ms per launch (live)")

    # per leaf of one more (untimed) view: its estimate and the bytes the
    # library held for it
    leaf_rep = None
    if grid is None and not args.cached_layout and budget > 0:
        adam = None if args.no_adam else dict(step=k + 1, params=params, m=m, v=v, lr=1e-3)
        rl = B.gs_train_view(ctx, cam, params, target, budget_bytes=budget, loss=w.loss, adam=adam,
                             serial_leaves=args.serial_leaves, max_leaves=65536)
        k += 1
        est = [L["est_bytes"] for L in rl["leaves"]]
        held = [L["bytes"] for L in rl["leaves"]]
        leaf_rep = {"n_leaves": len(est), "max_est_mib": round(max(est) / MIB, 2),
                    "max_held_mib": round(max(held) / MIB, 2),
                    "max_held_over_est": round(max(h / e for h, e in zip(held, est)), 4),
                    "all_within_est": all(h <= e for h, e in zip(held, est)),
                    "held_mib_per_leaf": [round(h / MIB, 1) for h in held]}
        log(f"[bench] per-leaf bytes held / estimate: max {leaf_rep['max_held_mib']} MiB held, "
            f"max ratio {leaf_rep['max_held_over_est']}, all within: {leaf_rep['all_within_est']}")

    # work counters of the view (untimed pass): pairs examined / included /
    # revisited by the backward, intersections, candidates
    wc = count_work(B, ctx, cam, params, budget)
    work = kernel_work(wc, sc)
    rooflines = {}
    attain_s = 0.0      # sum over the timed kernels of max(bytes / BW, ops / VALU)
    step_bytes = 0      # algorithmic HBM bytes of the kernels that ran in the step
    counted = []
    for name, (bound, amount, unit_desc) in work.items():
        kt = dom_live if name == dom else ktimes.get(name)
        if not kt or kt["total_ms"] <= 0.0:
            continue
        sec = kt["total_ms"] * 1e-3
        if bound == "alu":
            ach = amount / sec / 1e12
            rooflines[name] = dict(bound="alu", achieved=round(ach, 3), peak=round(PEAK_VALU_TOPS, 2), unit="Top/s",
                                   frac=round(ach / PEAK_VALU_TOPS, 4), work=unit_desc)
            hbm = wc["raster_bytes"] if name == "raster_fused" else 0
            attain_s += max(amount / (PEAK_VALU_TOPS * 1e12), hbm / (PEAK_HBM_GBS * 1e9))
            step_bytes += hbm
        else:
            ach = amount / sec / 1e9
            rooflines[name] = dict(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                                   frac=round(ach / PEAK_HBM_GBS, 4), work=unit_desc)
            attain_s += amount / (PEAK_HBM_GBS * 1e9)
            step_bytes += amount
        counted.append(name)
    roofline = dict(rooflines[dom])
    roofline.update(traffic=measured_traffic(args.workload, dom, wc["n_leaves"]),
                    traffic_unit="HBM bytes per launch (counters)",
                    kernel=dom, avg_launch_ms=round(dom_live["avg_ms"], 4), launches_per_step=dom_live["launches"],
                    timing="HIP events around this kernel's launches inside the timed steps")
    # whole-step HBM fraction: the algorithmic bytes of the kernels that ran
    # in the step (and the fused raster's own bytes) over the step time;
    # attainable fraction: the step's time at the roof of each kernel's bound
    hbm_frac_step = step_bytes / (ms_step * 1e-3) / (PEAK_HBM_GBS * 1e9)
    attain_frac = attain_s / (ms_step * 1e-3)

    cpu = None
    if args.cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_window, args.cpu_windows, args.cpu_threads)

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
                               + (f"fixed {args.layout[5:]}x{args.layout[5:]} blocks, L1, "
                                  + ("one Adam step per block" if args.per_block_update
                                     else "block grads summed, one Adam step per view")
                                  if grid else
                                  f"leaf budget {args.budget_mib:g} MiB, "
                                  + ("L1" if w.loss == "l1" else "L1 + SSIM (one-tile halo per leaf)")
                                  + ", leaf grads summed, "
                                  + ("one Adam step per view" if not args.no_adam else "no update")
                                  + (", cached leaf layout re-checked per view" if args.cached_layout else "")
                                  + (", leaves rendered one at a time" if args.serial_leaves else "")
                                  + (", target in pinned host memory copied leaf by leaf" if args.target_host
                                     else "")),
                   "n_gaussians": sc.n, "width": cam.width, "height": cam.height,
                   "leaf_budget_mib": None if grid else args.budget_mib, "layout": args.layout,
                   "parallelism": "single GPU"},
        "gaussians_per_s": round(sc.n / (ms_step * 1e-3), 1),
        "peak_working_set_gib": round(r["peak_bytes"] / 2 ** 30, 4),
        "peak_working_set_torch_gib": round(torch_peak / 2 ** 30, 4),
        "peak_by_category_gib": {c: round(b / 2 ** 30, 4) for c, b in mem["peak_by_cat"].items()},
        "leaf_bytes": leaf_rep,
        "n_candidates": r["n_cand"],
        "n_intersections": r["n_isect"],
        "n_coarse_pairs": wc["cells"],
        "n_leaves": r["n_leaves"],
        "pairs": {"examined": wc["q_f"], "included": wc["q_inc"], "backward": wc["q_b"], "sum_last": wc["sum_last"]},
        "kernel_ms_per_step": {k: round(v["total_ms"], 3) for k, v in ktimes.items()},
        "kernel_ms_note": "HIP events around every kernel in a separate attribution pass of "
                          f"{args.attr_steps} steps before the timed steps, with the leaves binned in "
                          "series (the timed steps bin each next leaf on a second stream during the "
                          "current leaf's raster, so their step time is less than this sum)",
        "roofline": roofline,
        "rooflines_all": rooflines,
        "step_hbm": {"algorithmic_bytes": int(step_bytes), "frac_of_8TBps": round(hbm_frac_step, 4),
                     "kernels": counted, "raster_bytes": int(wc["raster_bytes"]),
                     "raster_bytes_note": "fused raster: 8 B slot + key per super-tile group entry, 36 B attributes per (leaf, "
                                          "candidate), 12 B target per pixel, 36 B 2D gradient per candidate"},
        "attainable_roofline_frac": round(attain_frac, 4),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    ctx.close()


def count_work(B, ctx, cam, params, budget):
    """Work counters of the view as benchmarked (untimed): pairs examined by
    the forward (q_f), pairs included (q_inc), pairs the backward revisits
    (q_b: those examined), intersections, candidates, leaves, tiles, pixels."""
    import torch
    proj, n_cand = B.gs_project(ctx, cam, params)
    # the leaves of the benchmarked L1 view (its own load model)
    leaves = (B.gs_plan_leaves(ctx, cam, proj, budget, cost=B.gs_train_cost_model()) if budget > 0 else
              [dict(tx0=0, ty0=0, tx1=cam.tiles_x, ty1=cam.tiles_y)])
    stats = torch.zeros(4, dtype=torch.int64, device=ctx.device)
    n_isect = 0
    tiles = 0
    radix_elems = 4 * n_cand           # the per-view depth sort: 4 passes over the candidates
    group_entries = 0
    cells = 0                          # coarse (super-tile of 8 x 8 tiles, candidate) pairs
    supers = 0
    rects = B.gs_export(ctx, proj, B.PROJ_RECT).cpu().numpy().astype(np.int64)
    for L in leaves:
        bins, ni = B.gs_bin_sort(ctx, cam, proj, L)
        n_isect += ni
        t_l = (L["tx1"] - L["tx0"]) * (L["ty1"] - L["ty0"])
        tiles += t_l
        meet = ((rects[:, 0] < L["tx1"]) & (rects[:, 2] > L["tx0"]) &
                (rects[:, 1] < L["ty1"]) & (rects[:, 3] > L["ty0"]))
        r = rects[meet]
        # image-aligned super-cells of 8 x 8 tiles met inside the leaf
        x0 = np.maximum(r[:, 0], L["tx0"])
        x1 = np.minimum(r[:, 2], L["tx1"])
        y0 = np.maximum(r[:, 1], L["ty0"])
        y1 = np.minimum(r[:, 3], L["ty1"])
        c_l = int((((x1 - 1) >> 3) - (x0 >> 3) + 1) @ (((y1 - 1) >> 3) - (y0 >> 3) + 1))
        s_l = (((L["tx1"] - 1) >> 3) - (L["tx0"] >> 3) + 1) * (((L["ty1"] - 1) >> 3) - (L["ty0"] >> 3) + 1)
        cells += c_l
        supers += s_l
        radix_elems += c_l * ((max(1, (s_l - 1).bit_length()) + 7) // 8) if s_l > 1 else 0
        group_entries += int(meet.sum())
        ras = B.gs_render_fwd(ctx, cam, proj, bins, stats=stats)
        B.gs_release(ctx, ras)
        B.gs_release(ctx, bins)
    B.gs_release(ctx, proj)
    q = stats.cpu().tolist()
    P = cam.width * cam.height
    # algorithmic bytes of the fused forward + L1 + backward (per-pixel state
    # stays in registers; tiles walk their super-tile groups): every group
    # entry once (slot + coarse key, 8 B), the attributes of each leaf's
    # candidates once (36 B), the target (12 B/px) and the 2D gradient rows
    # (36 B per candidate)
    raster_bytes = 8 * cells + 36 * group_entries + 12 * P + 36 * n_cand
    return dict(q_f=int(q[0]), q_inc=int(q[1]), q_b=int(q[3]), sum_last=int(q[2]), n_isect=int(n_isect),
                n_cand=int(n_cand),
                n_leaves=len(leaves), tiles=int(tiles), pixels=P, raster_bytes=int(raster_bytes),
                radix_elems=int(radix_elems), group_entries=int(group_entries), cells=int(cells),
                supers=int(supers))


KERNEL_WORK_NAMES = ("raster_fwd", "raster_bwd", "raster_fused", "radix", "emit", "bin_count", "seg_offsets", "fine", "rect_diff",
                     "project_flags", "project_write", "project_bwd", "adam", "bwd_adam")


def kernel_work(wc, sc):
    """Algorithmic work per step of each timed kernel: (bound, amount, description).
    alu: f32 VALU lane operations; hbm: bytes that must cross HBM."""
    K = (sc.sh_degree + 1) ** 2
    F = 11 + 3 * K
    N, Nc, I, T, L = sc.n, wc["n_cand"], wc["n_isect"], wc["tiles"], wc["n_leaves"]
    C = wc["cells"]
    qf, qi, qb = wc["q_f"], wc["q_inc"], wc["q_b"]
    return {
        "raster_fwd": ("alu", OPS_EXAMINED * (qf - qi) + OPS_INCLUDED_FWD * qi,
                       f"{OPS_EXAMINED} ops x examined-only pairs + {OPS_INCLUDED_FWD} x included pairs"),
        "raster_bwd": ("alu", OPS_EXAMINED * (qb - qi) + OPS_INCLUDED_BWD * qi,
                       f"{OPS_EXAMINED} ops x revisited-only pairs + {OPS_INCLUDED_BWD} x included pairs"),
        "raster_fused": ("alu", OPS_EXAMINED * (qf - qi) + OPS_INCLUDED_FWD * qi
                         + OPS_EXAMINED * (qb - qi) + OPS_INCLUDED_BWD * qi,
                         f"forward ({OPS_EXAMINED} ops x examined-only pairs + {OPS_INCLUDED_FWD} x included pairs) "
                         f"+ backward ({OPS_EXAMINED} x revisited-only + {OPS_INCLUDED_BWD} x included)"),
        "radix": ("hbm", 20 * wc["radix_elems"], "per pass and element: read the key twice, the value once, "
                                                   "write key and value (20 B)"),
        "emit": ("hbm", 8 * C + 20 * wc["group_entries"], "write 8 B (super-tile, slot) per coarse pair; read "
                                                           "depth position, slot, packed rectangle (8 B) and "
                                                           "offset per candidate visit"),
        "bin_count": ("hbm", 16 * wc["group_entries"] + 8 * T, "read depth position and packed rectangle, write "
                                                             "the count; gather the leaf's tile counts"),
        "seg_offsets": ("hbm", 4 * C + 8 * wc["supers"], "read sorted super-tile keys, write group offsets"),
        "fine": ("hbm", 4 * I + 20 * C + 8 * T, "read each coarse entry and its rectangle, the tile offsets; "
                                                "write one slot per intersection"),
        "rect_diff": ("hbm", 16 * Nc + 4 * T, "read rects, touch the count grid"),
        "project_flags": ("hbm", 40 * N, "read mean, log-scale, quaternion"),
        "project_write": ("hbm", N * (40 + 4 + 12 * K + 8) + Nc * 68, "read parameters, write compact state"),
        "project_bwd": ("hbm", Nc * (36 + 48 + 40 + 4 + 12 * K + 4 * F + 4), "read 2D grads, state, params; write 3D grads"),
        "adam": ("hbm", 24 * N * F + 4 * F * Nc + 4 * N, "read/write params, m, v; read compact grads"),
        "bwd_adam": ("hbm", 24 * N * F + 52 * Nc + 4 * N, "read/write params, m, v once; read the candidates' 2D "
                                                         "grads and flags, the slot map"),
    }


RASTER_SOURCES = ("differentiable_gaussian_splatting_amd/csrc/raster.hip",
                  "differentiable_gaussian_splatting_amd/csrc/gs_device.h")


def measured_traffic(workload, kernel, n_leaves):
    """HBM bytes per launch of a raster kernel from the committed counter
    summary (calibrated FETCH_SIZE + WRITE_SIZE), or None when there is none
    for this workload and leaf count, or the kernel sources have changed since
    it was taken."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", f"raster_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in RASTER_SOURCES:
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    fields = {}
    for line in open(path):
        parts = line.split()
        if not parts or parts[0].startswith("#"):
            continue
        fields[parts[0]] = parts[1:]
    if fields.get("source_sha256_16", [None])[0] != h.hexdigest()[:16] or kernel not in fields:
        return None
    if int(fields.get("n_leaves", ["-1"])[0]) != int(n_leaves):
        return None
    kv = fields[kernel]
    return int(dict(zip(kv[0::2], kv[1::2]))["traffic_bytes_per_launch"])


def gated_sequence(args, B, scenes, torch, ctx, w, params, m, v, budget):
    """A training sequence over posed views of one scene with the SkipGS
    gate: the warm-up is one pass over the views (every view runs its
    backward), then --steps views are timed one by one.  A view whose
    backward is skipped runs binning, forward and loss only; one that runs it
    renders its leaves twice (forward for the loss, then forward + backward),
    since the leaves' buffers are not kept between the passes."""
    import numpy as np
    nv = args.skip_gate
    rng = np.random.default_rng(5000)
    cams = [scenes.random_pose_camera(w.camera.width, w.camera.height, rng) for _ in range(nv)]
    targets = [torch.from_numpy(scenes.target_image(rng, w.camera.width, w.camera.height)).to(params.means.device)
               for _ in range(nv)]
    gate = B.Gate(nv, warmup=nv)
    k = [0]

    def view(i):
        k[0] += 1
        return B.gs_train_view(ctx, cams[i % nv], params, targets[i % nv], budget_bytes=budget, loss=w.loss,
                               adam=dict(step=k[0], params=params, m=m, v=v, lr=1e-3), gate=gate,
                               gate_view=i % nv)

    for i in range(nv):   # the warm-up pass
        view(i)
    torch.cuda.synchronize()
    times, runs, forced = [], [], 0
    t_all = time.perf_counter()
    for i in range(nv, nv + args.steps):
        t0 = time.perf_counter()
        r = view(i)
        times.append(time.perf_counter() - t0)
        runs.append(r["backward"])
        forced += 1 if r["forced"] else 0
    t_all = time.perf_counter() - t_all
    ms = 1e3 * t_all / args.steps
    ran = [t for t, b in zip(times, runs) if b]
    skipped = [t for t, b in zip(times, runs) if not b]
    st = gate.stats()
    P = w.camera.width * w.camera.height
    log(f"[bench] gated sequence: {args.steps} views in {t_all:.3f}s: {ms:.2f} ms/view, backward ratio "
        f"{sum(runs) / len(runs):.3f} (forced {forced}), floor {st['rho_min']}")
    out = {
        "metric": "fwd+bwd Mpixel/s per view and peak working set (GiB) on one MI355X",
        "value": round(P / (ms * 1e-3) / 1e6, 3),
        "unit": "Mpixel/s",
        "n_gpus": 1, "steps": args.steps, "warmup": nv, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.scene.n} Gaussians SH{w.scene.sh_degree}, "
                               f"{w.camera.width}x{w.camera.height}, leaf budget {args.budget_mib:g} MiB, L1, "
                               f"SkipGS gate over {nv} posed views, one Adam step per view that runs its backward",
                   "n_gaussians": w.scene.n, "width": w.camera.width, "height": w.camera.height,
                   "leaf_budget_mib": args.budget_mib, "parallelism": "single GPU"},
        "gate": {"views": nv, "warmup_steps": nv, "backward_ratio": round(sum(runs) / len(runs), 4),
                 "forced": forced, "rho_min": st["rho_min"],
                 "ms_view_with_backward": round(1e3 * sum(ran) / len(ran), 3) if ran else None,
                 "ms_view_skipped": round(1e3 * sum(skipped) / len(skipped), 3) if skipped else None},
        "peak_working_set_gib": None, "roofline": None, "cpu_baseline": None,
    }
    gate.close()
    print(json.dumps(out), flush=True)


def host_cpu():
    """(logical CPUs the process may use, CPU model name)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return n, model


def cpu_baseline(w, window, n_windows, threads):
    """The CPU oracle as it stands on a bounded sample of the same view, on
    several host threads (its C routines run outside the GIL, each thread on
    its own inputs and outputs; the arithmetic is the oracle's own):
      - projection (f32 and f64) and projection backward over all N
        Gaussians, split into equal bands of Gaussians over the threads;
      - per window: binning, forward, L1 and raster backward, for n_windows
        windows of window x window pixels, one at a seeded position in each
        cell of a grid over the view, the windows spread over the threads.
    The view time is the per-Gaussian time plus the windows' time scaled by
    P / (pixels of the windows)."""
    import concurrent.futures as cf

    import oracle
    from differentiable_gaussian_splatting_amd import scenes
    cam, sc = w.camera, w.scene
    W, H = cam.width, cam.height
    TW, TH = cam.tiles_x, cam.tiles_y
    avail, model = host_cpu()
    nt = threads if threads > 0 else max(1, min(16, avail))
    # the oracle's exp routines set up their constant tables on first use:
    # take that first use here, before any thread runs
    oracle.exp_cw(np.zeros(1, np.float32))
    oracle.exp_falloff(np.zeros(1, np.float32))
    pool = cf.ThreadPoolExecutor(max_workers=nt)

    def bands(n):
        e = np.linspace(0, n, nt + 1).astype(np.int64)
        return [(int(a), int(b)) for a, b in zip(e[:-1], e[1:]) if b > a]

    def sub(a, b):
        return scenes.Scene(*(x[a:b] for x in sc.arrays()), sh_degree=sc.sh_degree)

    # ---- projection over bands of Gaussians
    t = time.perf_counter()

    def proj_band(ab):
        s_ = sub(*ab)
        return oracle.project(cam, s_, "f32"), oracle.project(cam, s_, "f64")

    parts = list(pool.map(proj_band, bands(sc.n)))
    p32 = {k: np.concatenate([p[0][k] for p in parts]) for k in parts[0][0]}
    p64 = {k: np.concatenate([p[1][k] for p in parts]) for k in parts[0][1]}
    del parts
    t_proj = time.perf_counter() - t
    ids = np.nonzero(p32["cand"])[0]
    slot_of = np.full(sc.n, -1, np.int64)
    slot_of[ids] = np.arange(ids.size)
    c32 = {k: p32[k][ids] for k in ("rect", "xy", "conic", "depth", "opacity", "rgb")}
    c64 = {k: p64[k][ids] for k in ("xy", "conic", "opacity", "rgb")}

    # ---- windows: one per cell of a gx x gy grid, at a seeded position
    wt = max(1, window // 16)
    gx = max(1, min(TW, int(round(np.sqrt(n_windows * TW / TH)))))
    gy = max(1, min(TH, int(round(n_windows / gx))))
    rng = np.random.default_rng(12345)
    wins = []
    for j in range(gy):
        for i in range(gx):
            # inside its cell, so that no two windows share a pixel
            cx0, cx1 = i * TW // gx, (i + 1) * TW // gx
            cy0, cy1 = j * TH // gy, (j + 1) * TH // gy
            if cx1 <= cx0 or cy1 <= cy0:
                continue
            tx0 = int(rng.integers(cx0, max(cx0 + 1, cx1 - wt + 1)))
            ty0 = int(rng.integers(cy0, max(cy0 + 1, cy1 - wt + 1)))
            wins.append(oracle.rect(tx0, ty0, min(cx1, tx0 + wt), min(cy1, ty0 + wt)))
    image = np.zeros((3, H, W), np.float32)
    tf = np.ones((H, W), np.float32)
    last = np.zeros((H, W), np.int32)
    dloss = np.zeros((3, H, W), np.float64)

    def win_pixels(r):
        return (min(r.tx1 * 16, W) - r.tx0 * 16) * (min(r.ty1 * 16, H) - r.ty0 * 16)

    def run_window(r):
        bins = oracle.bin_leaf(TW, r, c32["rect"], c32["depth"], with_keys=False)
        oracle.render_fwd(cam, r, bins, c32["xy"], c32["conic"], c32["opacity"], c32["rgb"], image, tf, last)
        ys, xs = slice(r.ty0 * 16, min(r.ty1 * 16, H)), slice(r.tx0 * 16, min(r.tx1 * 16, W))
        # the L1 term of the window's pixels (the oracle's own loss routine
        # reads the window out of a full-size image)
        full64 = window_image64(ys, xs)
        oracle.loss_l1(cam, r, full64, w.target, dloss)
        g2 = np.zeros((ids.size, 9), np.float64)
        oracle.render_bwd(cam, r, bins, (c32["xy"], c32["conic"], c32["opacity"]),
                          (c64["xy"], c64["conic"], c64["opacity"], c64["rgb"]), dloss, g2)
        return g2

    img64_all = np.zeros((3, H, W), np.float64)

    def window_image64(ys, xs):
        img64_all[:, ys, xs] = image[:, ys, xs]
        return img64_all

    t = time.perf_counter()
    grads = list(pool.map(run_window, wins))
    t_pix = time.perf_counter() - t
    grad2d = grads[0]
    for g in grads[1:]:
        grad2d += g
    del grads
    p_win = sum(win_pixels(r) for r in wins)

    # ---- projection backward over bands of Gaussians
    t = time.perf_counter()
    list(pool.map(lambda ab: oracle.project_bwd(cam, sub(*ab), p32["cand"][ab[0]:ab[1]],
                                                p32["flags"][ab[0]:ab[1]], slot_of[ab[0]:ab[1]], grad2d),
                  bands(sc.n)))
    t_pbwd = time.perf_counter() - t
    pool.shutdown()
    P = W * H
    t_view = t_proj + t_pbwd + t_pix * (P / p_win)
    log(f"[bench] cpu oracle on {nt} threads ({avail} available, {model}): projection {t_proj:.1f}s, "
        f"{len(wins)} windows {t_pix:.1f}s ({p_win} px), projection backward {t_pbwd:.1f}s -> view {t_view:.1f}s")
    return {"value": round(P / t_view / 1e6, 5), "unit": "Mpixel/s", "cores": nt, "kind": "oracle",
            "host": {"cpus_available": avail, "cpu_model": model},
            "sample": f"all {sc.n} Gaussians through projection (f32 + f64) and projection backward, in "
                      f"{len(bands(sc.n))} bands over {nt} threads; binning + raster fwd + L1 + raster bwd on "
                      f"{len(wins)} windows of {wt}x{wt} tiles ({p_win} px), one at a seeded position in each "
                      f"cell of a {gx}x{gy} grid over the view, spread over {nt} threads; window time scaled by "
                      f"P/P_windows = {P / p_win:.1f}",
            "seconds_measured": round(t_proj + t_pix + t_pbwd, 2), "seconds_view_estimate": round(t_view, 1)}


if __name__ == "__main__":
    main()
