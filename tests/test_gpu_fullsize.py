"""GPU parity at the workloads' full sizes, leaf by leaf exactly as the
benchmark runs them (same calls, same leaves, same kernels and launch
shapes), checked where the oracle can follow:

  - projection of every Gaussian: bit-exact (ids, rectangles, depth, conic,
    mean2d, radius, opacity, rgb, flags);
  - the leaf plan: identical leaves and estimates;
  - per-tile counts of every tile of every leaf: bit-exact against the
    oracle's count grid; the total intersection count;
  - sampled tiles (the heaviest, random ones, the last row and column):
    sorted lists, image, T_final and last bit-exact against the oracle
    binning and rendering that tile alone;
  - the loss: the fused f64 L1 sum against the L1 of the GPU image
    recomputed on the host (a property at any size);
  - sampled candidates whose rectangle spans at most 6 x 6 tiles: their 2D
    gradient rows (summed over leaves on the GPU) and 3D gradient rows
    against the oracle's backward over exactly the tiles they touch, each
    group within 1e-3 relative L2.
"""
import sys

import numpy as np
import pytest

import oracle
from differentiable_gaussian_splatting_amd import binding as B
from differentiable_gaussian_splatting_amd import scenes
from tests.gpu_pipeline import GRAD2D_GROUPS, bits, grad3d_groups, rel_l2

pytestmark = pytest.mark.gpu

MIB = 1 << 20
GRAD_TOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ctx():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load()
    return B.Context()


def count_grid(rect_c, TW, TH):
    """Candidates per tile by a 2D difference array over the rectangles."""
    r = rect_c.astype(np.int64)
    S = (TH + 1) * (TW + 1)
    d = np.zeros(S, np.int64)
    for (yi, xi), sgn in (((1, 0), 1), ((1, 2), -1), ((3, 0), -1), ((3, 2), 1)):
        d += sgn * np.bincount(r[:, yi] * (TW + 1) + r[:, xi], minlength=S)
    return d.reshape(TH + 1, TW + 1).cumsum(0).cumsum(1)[:TH, :TW]


@pytest.mark.parametrize("name,budget_mib", [("c5_plane16k", 384), ("c4_plane5k", 384), ("c3_gmm4k", 128)])
def test_full_size_sampled_parity(ctx, name, budget_mib):
    import torch
    dev = ctx.device
    w = scenes.make_workload(name)
    cam, sc = w.camera, w.scene
    W, H = cam.width, cam.height
    TW, TH = cam.tiles_x, cam.tiles_y
    budget = budget_mib * MIB
    say(f"case {name}: N={sc.n} {W}x{H} budget {budget_mib} MiB")

    # ---------------- GPU, leaf by leaf
    ds = B.DeviceScene(sc, dev)
    target = torch.from_numpy(w.target).to(dev)
    proj, n_cand = B.gs_project(ctx, cam, ds)
    g = {k: B.gs_export(ctx, proj, f).cpu().numpy() for k, f in (
        ("ids", B.PROJ_IDS), ("rect", B.PROJ_RECT), ("xy", B.PROJ_XY), ("conic", B.PROJ_CONIC),
        ("depth", B.PROJ_DEPTH), ("radius", B.PROJ_RADIUS), ("opacity", B.PROJ_OPACITY), ("rgb", B.PROJ_RGB),
        ("flags", B.PROJ_FLAGS))}
    leaves = B.gs_plan_leaves(ctx, cam, proj, budget)
    say(f"  {n_cand} candidates, {len(leaves)} leaves")

    # ---------------- oracle projection (all Gaussians) and plan
    p32 = oracle.project(cam, sc, "f32")
    ids = np.nonzero(p32["cand"])[0]
    assert n_cand == ids.size
    assert np.array_equal(g["ids"].astype(np.int64), ids)
    assert np.array_equal(g["rect"], p32["rect"][ids])
    assert np.array_equal(bits(g["depth"]), bits(p32["depth"][ids]))
    assert np.array_equal(g["flags"].view(np.uint32), p32["flags"][ids])
    for k in ("xy", "conic", "radius", "opacity", "rgb"):
        assert np.array_equal(bits(g[k]), bits(p32[k][ids])), k
    say("  projection bit-exact")
    rect_c = p32["rect"][ids]
    o_leaves = oracle.plan_leaves(cam, rect_c, budget)
    got = [(L["tx0"], L["ty0"], L["tx1"], L["ty1"], L["est_bytes"], L["over_budget"]) for L in leaves]
    exp = [(L["tx0"], L["ty0"], L["tx1"], L["ty1"], L["est_bytes"], L["over_budget"]) for L in o_leaves]
    assert got == exp
    counts = count_grid(rect_c, TW, TH)

    # sampled tiles: the 6 heaviest, 10 random, the last row / column corners
    rng = np.random.default_rng(7)
    flat = counts.ravel()
    heavy = np.argsort(flat)[-6:]
    rand = rng.choice(flat.size, size=10, replace=False)
    corner = np.array([(TH - 1) * TW + TW - 1, (TH - 1) * TW, TW - 1])
    sample_tiles = sorted(set(int(t) for t in np.concatenate([heavy, rand, corner])))

    image = torch.zeros((3, H, W), dtype=torch.float32, device=dev)
    grad2d = torch.zeros((max(n_cand, 1), 9), dtype=torch.float32, device=dev)
    loss_acc = torch.zeros(1, dtype=torch.float64, device=dev)
    tile_lists, tile_tf, tile_last = {}, {}, {}
    total_isect = 0
    for L in leaves:
        bins, n_isect = B.gs_bin_sort(ctx, cam, proj, L)
        total_isect += n_isect
        TWL = L["tx1"] - L["tx0"]
        off = B.gs_export(ctx, bins, B.BINS_OFFSETS).cpu().numpy().view(np.uint64).astype(np.int64)
        sub = counts[L["ty0"]:L["ty1"], L["tx0"]:L["tx1"]].ravel()
        assert np.array_equal(np.diff(off), sub), "per-tile counts of a leaf"
        mine = [t for t in sample_tiles if L["tx0"] <= t % TW < L["tx1"] and L["ty0"] <= t // TW < L["ty1"]]
        vals = B.gs_export(ctx, bins, B.BINS_VALUES).cpu().numpy().view(np.uint32) if mine else None
        ras = B.gs_render_fwd(ctx, cam, proj, bins, target, loss_acc, image)
        B.gs_render_bwd(ctx, cam, proj, bins, ras, grad2d)
        if mine:
            tf = B.gs_export(ctx, ras, B.RASTER_TFINAL).cpu().numpy()
            la = B.gs_export(ctx, ras, B.RASTER_LAST).cpu().numpy()
            x0, y0 = L["tx0"] * 16, L["ty0"] * 16
            WL = min(L["tx1"] * 16, W) - x0
            HL = min(L["ty1"] * 16, H) - y0
            tf, la = tf.reshape(HL, WL), la.reshape(HL, WL)
            for t in mine:
                lt = (t // TW - L["ty0"]) * TWL + (t % TW - L["tx0"])
                tile_lists[t] = vals[off[lt]:off[lt + 1]].copy()
                px, py = (t % TW) * 16 - x0, (t // TW) * 16 - y0
                tile_tf[t] = tf[py:py + 16, px:px + 16].copy()
                tile_last[t] = la[py:py + 16, px:px + 16].copy()
        B.gs_release(ctx, ras)
        B.gs_release(ctx, bins)
    K = (sc.sh_degree + 1) ** 2
    F = 11 + 3 * K
    grad3d = torch.zeros((max(n_cand, 1), F), dtype=torch.float32, device=dev)
    B.gs_project_bwd(ctx, cam, ds, proj, grad2d, grad3d)
    torch.cuda.synchronize()
    B.gs_release(ctx, proj)
    area = ((rect_c[:, 2] - rect_c[:, 0]).astype(np.int64) * (rect_c[:, 3] - rect_c[:, 1])).sum()
    assert total_isect == int(area) == int(counts.sum())
    say(f"  {total_isect} intersections; every tile count bit-exact")

    # ---------------- loss: fused sum against the image it was formed from
    img = image.cpu().numpy()
    loss_gpu = float(loss_acc.cpu().numpy()[0]) / (3.0 * W * H)
    loss_host = sum(float(np.abs(img[c].astype(np.float64) - w.target[c].astype(np.float64)).sum())
                    for c in range(3)) / (3.0 * W * H)
    say(f"  loss {loss_gpu:.9f} (host sum of the GPU image {loss_host:.9f})")
    assert abs(loss_gpu - loss_host) <= 1e-9

    # ---------------- sampled tiles against the oracle
    depth_c = p32["depth"][ids]
    xy_c, conic_c, op_c, rgb_c = (p32[k][ids] for k in ("xy", "conic", "opacity", "rgb"))
    o_img = np.zeros((3, H, W), np.float32)
    o_tf = np.ones((H, W), np.float32)
    o_last = np.zeros((H, W), np.int32)
    for t in sample_tiles:
        tx, ty = t % TW, t // TW
        r = oracle.rect(tx, ty, tx + 1, ty + 1)
        ob = oracle.bin_leaf(TW, r, rect_c, depth_c, with_keys=False)
        assert np.array_equal(tile_lists[t], ob["values"]), f"tile {t} list"
        oracle.render_fwd(cam, r, ob, xy_c, conic_c, op_c, rgb_c, o_img, o_tf, o_last)
        ys, xs = slice(ty * 16, min(ty * 16 + 16, H)), slice(tx * 16, min(tx * 16 + 16, W))
        assert np.array_equal(bits(img[:, ys, xs]), bits(o_img[:, ys, xs])), f"tile {t} image"
        h, wd = ys.stop - ys.start, xs.stop - xs.start
        assert np.array_equal(bits(tile_tf[t][:h, :wd]), bits(o_tf[ys, xs])), f"tile {t} T_final"
        assert np.array_equal(tile_last[t][:h, :wd].astype(np.int64), o_last[ys, xs]), f"tile {t} last"
    say(f"  {len(sample_tiles)} sampled tiles bit-exact (lists, image, T_final, last); "
        f"longest list {max(len(v) for v in tile_lists.values())}")

    # ---------------- sampled gradients against the oracle over the tiles they touch
    g2 = grad2d.cpu().numpy()[:n_cand]
    g3 = grad3d.cpu().numpy()[:n_cand]
    p64 = oracle.project(cam, sc, "f64")
    c64 = {k: p64[k][ids] for k in ("xy", "conic", "opacity", "rgb")}
    span = (rect_c[:, 2] - rect_c[:, 0]) * (rect_c[:, 3] - rect_c[:, 1])
    small = ((rect_c[:, 2] - rect_c[:, 0]) <= 6) & ((rect_c[:, 3] - rect_c[:, 1]) <= 6)
    # most small rectangles at high resolution belong to distant, occluded
    # Gaussians whose gradient is exactly zero: take 40 with a contribution
    # (nonzero row on the GPU side) and 20 at random (zero rows must be zero
    # in the oracle too)
    live = np.nonzero(small & np.any(g2 != 0, axis=1))[0]
    anyc = np.nonzero(small)[0]
    pick = np.unique(np.concatenate([rng.choice(live, size=min(40, live.size), replace=False),
                                     rng.choice(anyc, size=min(20, anyc.size), replace=False)]))
    say(f"  gradient sample: {pick.size} candidates ({min(40, live.size)} of {live.size} with a contribution), "
        f"rectangles of {span[pick].min()}..{span[pick].max()} tiles")
    dl_img = np.zeros((3, H, W), np.float64)
    o_img64 = np.zeros((3, H, W), np.float64)
    o_g2 = np.zeros((n_cand, 9), np.float64)
    for s in pick:
        rc = rect_c[s]
        r = oracle.rect(rc[0], rc[1], rc[2], rc[3])
        ob = oracle.bin_leaf(TW, r, rect_c, depth_c, with_keys=False)
        oracle.render_fwd(cam, r, ob, xy_c, conic_c, op_c, rgb_c, o_img, o_tf, o_last)
        ys, xs = slice(rc[1] * 16, min(rc[3] * 16, H)), slice(rc[0] * 16, min(rc[2] * 16, W))
        o_img64[:, ys, xs] = o_img[:, ys, xs]
        oracle.loss_l1(cam, r, o_img64, w.target, dl_img)
        part = np.zeros((n_cand, 9), np.float64)
        oracle.render_bwd(cam, r, ob, (xy_c, conic_c, op_c), (c64["xy"], c64["conic"], c64["opacity"],
                                                             c64["rgb"]), dl_img, part)
        o_g2[s] = part[s]
    assert np.array_equal(np.any(g2[pick] != 0, axis=1), np.any(o_g2[pick] != 0, axis=1))
    for gname, sl in GRAD2D_GROUPS.items():
        assert np.linalg.norm(o_g2[pick][:, sl]) > 0, gname
        e = rel_l2(g2[pick][:, sl], o_g2[pick][:, sl])
        say(f"  grad2d {gname:8s} rel L2 {e:.2e}")
        assert e <= GRAD_TOL, gname
    slot_of = np.full(sc.n, -1, np.int64)
    slot_of[ids] = np.arange(ids.size)
    o_g3 = oracle.project_bwd(cam, sc, p32["cand"], p32["flags"], slot_of, o_g2)[ids[pick]]
    gg, og = grad3d_groups(g3[pick], sc.sh_degree), grad3d_groups(o_g3, sc.sh_degree)
    for gname in gg:
        assert np.linalg.norm(og[gname]) > 0, gname
        e = rel_l2(gg[gname], og[gname])
        say(f"  grad3d {gname:10s} rel L2 {e:.2e}")
        assert e <= GRAD_TOL, gname
