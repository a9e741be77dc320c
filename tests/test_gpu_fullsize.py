"""GPU parity at the workloads' full sizes, checked where the oracle can follow.

Two paths per workload:
  view: gs_train_view exactly as the benchmark times it (planned leaves, each
        next leaf binned on the second stream, the fused forward + L1 +
        backward raster on two overlapped render streams in the plan's tile
        order, the projection backward fused with the Adam step over all N);
        its image and the Adam moments it writes are compared;
  abi:  the six calls leaf by leaf (gs_project, gs_plan_leaves, gs_bin_sort,
        gs_render_fwd, gs_render_bwd, gs_project_bwd): the separate kernels.
Checked:
  - the leaf plan: identical leaves and estimates; per leaf, the bytes the
    library held for it within its estimate (view);
  - projection of every Gaussian bit-exact; per-tile counts of every tile of
    every leaf bit-exact; sampled tile lists, T_final and walk ends bit-exact
    (abi);
  - the loss: the fused f64 L1 sum against the L1 of the GPU image
    recomputed on the host (a property at any size);
  - the image bit-exact on sampled tiles (the heaviest, random ones, the
    last row and column) and on whole regions of 24..40 x 24..40 tiles
    centred on leaf junctions;
  - the gradients of every candidate whose rectangle lies inside such a
    region (rectangles of up to the region's size, many crossing two to four
    leaves, so summed over leaves, render streams and atomics), against the
    oracle's backward of the region: 2D rows (abi) and 3D rows, each group
    within 1e-3 relative L2.  In the view path the 3D gradient is read from
    the first Adam moment the fused update wrote (m = (1 - beta1) g from
    m = 0), and every update is checked against Adam of that gradient;
  - non-candidates: zero moment and unchanged parameters (view).
The workloads: C5 (6M and 12M Gaussians, 16000 x 10560, 384 and 128 MiB
leaves), C4 (6M, 5000 x 3300, 384 MiB), C3 (1M, 3840 x 2160, full image and
128 MiB leaves); C2 (100k, 1920 x 1080, L1 + SSIM) against the oracle's whole
view, the whole image as one leaf and split into leaves.
"""
import sys
import time

import numpy as np
import pytest

import oracle
from differentiable_gaussian_splatting_amd import binding as B
from tests import fullsize as F
from tests.gpu_pipeline import GRAD2D_GROUPS, bits, grad3d_groups, rel_l2

pytestmark = pytest.mark.gpu

MIB = 1 << 20
GRAD_TOL = 1e-3
BETA1 = 0.9


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ctx():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load()
    c = B.Context()
    yield c
    F._CACHE.clear()
    c.close()


def leaf_tuples(leaves):
    return [(L["tx0"], L["ty0"], L["tx1"], L["ty1"], L["est_bytes"], L["over_budget"]) for L in leaves]


def regions_for(ov, leaves, name):
    TW, TH = ov.TW, ov.TH
    if name == "c3_gmm4k":
        heavy = int(np.argmax(ov.counts))
        aims, R = [(heavy % TW, heavy // TW), (TW // 4, TH // 4)], 24
    else:
        # near the camera at the bottom (the largest rectangles), the centre
        # (the dense clusters) and two off-axis quarters
        aims = [(TW // 2, TH - 1), (TW // 2, TH // 2), (TW // 4, 3 * TH // 4), (3 * TW // 4, TH // 4)]
        R = 32 if ov.sc.n > 8_000_000 else 40
    return F.leaf_regions(leaves, TW, TH, R, aims)


def check_grads(name, got, exp, groups):
    """Per-group relative L2 of gradient rows (and the same rows nonzero)."""
    assert np.array_equal(np.any(got != 0, axis=1), np.any(exp != 0, axis=1)), f"{name}: nonzero rows differ"
    for gname, sl in groups.items():
        e = rel_l2(got[:, sl], exp[:, sl])
        say(f"  {name} {gname:10s} rel L2 {e:.2e}")
        assert np.linalg.norm(exp[:, sl]) > 0, gname
        assert e <= GRAD_TOL, (name, gname)


CASES = [
    ("c5_plane16k", 384, "view"),
    ("c5_plane16k", 128, "view"),
    ("c5_plane16k", 384, "abi"),
    ("c5_plane16k_12m", 384, "view"),
    ("c5_plane16k_12m", 128, "view"),
    ("c4_plane5k", 384, "view"),
    ("c4_plane5k", 384, "abi"),
    ("c3_gmm4k", 0, "view"),
    ("c3_gmm4k", 128, "abi"),
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,budget_mib,path", CASES)
def test_full_size_parity(ctx, name, budget_mib, path):
    import torch
    dev = ctx.device
    t0 = time.time()
    say(f"case {name} budget {budget_mib} MiB path {path}")
    ov = F.oracle_view(name)
    w, cam, sc = ov.w, ov.cam, ov.sc
    W, H, TW, TH = ov.W, ov.H, ov.TW, ov.TH
    ids, rect_c = ov.ids, ov.rect_c
    budget = budget_mib * MIB
    say(f"  N={sc.n} {W}x{H}: {ids.size} candidates (oracle ready in {time.time() - t0:.0f}s)")
    # the view plans with the load model of the raster it takes, the six calls with the default one
    view_cost = oracle.TRAIN_COST if oracle.walks_groups(rect_c) else None
    o_leaves = oracle.plan_leaves(cam, rect_c, budget, view_cost if path == "view" else None) if budget else \
        [dict(tx0=0, ty0=0, tx1=TW, ty1=TH, est_bytes=0, over_budget=False)]
    area = int(((rect_c[:, 2] - rect_c[:, 0]).astype(np.int64) * (rect_c[:, 3] - rect_c[:, 1])).sum())
    assert area == int(ov.counts.sum())
    K = (sc.sh_degree + 1) ** 2
    F_ = 11 + 3 * K
    target = torch.from_numpy(w.target).to(dev)
    ds = B.DeviceScene(sc, dev)
    image = torch.zeros((3, H, W), dtype=torch.float32, device=dev)
    rng = np.random.default_rng(7)
    tiles = F.sample_tiles(ov.counts, rng)
    regions = regions_for(ov, o_leaves, name)
    lid = F.leaf_ids(o_leaves, TW, TH)

    if path == "view":
        p0 = [t.clone() for t in ds.tensors()]
        m, v = B.like_scene(ds), B.like_scene(ds)
        r = B.gs_train_view(ctx, cam, ds, target, budget_bytes=budget, image_out=image,
                            adam=dict(step=1, params=ds, m=m, v=v), max_leaves=1 << 14)
        torch.cuda.synchronize()
        say(f"  GPU view: {r['n_leaves']} leaves, {r['n_isect']} intersections, loss {r['loss']:.9f}, "
            f"groups walked {r['groups_walked']}")
        assert r["groups_walked"] == (bool(budget) and oracle.walks_groups(rect_c))
        assert r["n_cand"] == ids.size and r["n_isect"] == area
        if budget:
            assert leaf_tuples(r["leaves"]) == leaf_tuples(o_leaves)
        else:
            assert r["n_leaves"] == 1
        held = [L["bytes"] for L in r["leaves"]]
        say(f"  bytes held per leaf: max {max(held) / MIB:.1f} MiB (largest estimate "
            f"{max(L['est_bytes'] for L in r['leaves']) / MIB:.1f} MiB)")
        if budget:
            assert all(L["bytes"] <= L["est_bytes"] for L in r["leaves"]), "a leaf held more than its estimate"
        loss_gpu = r["loss"]
        # non-candidates: zero gradient, so zero first moment and unchanged parameters
        noncand = torch.from_numpy(ov.slot_of < 0).to(dev)
        for t, t0_, mm in zip(ds.tensors(), p0, m.tensors()):
            assert bool((mm[noncand] == 0).all()) and bool(torch.equal(t[noncand], t0_[noncand]))
        del noncand
    else:
        proj, n_cand = B.gs_project(ctx, cam, ds)
        assert n_cand == ids.size
        g = {k: B.gs_export(ctx, proj, f).cpu().numpy() for k, f in (
            ("ids", B.PROJ_IDS), ("rect", B.PROJ_RECT), ("xy", B.PROJ_XY), ("conic", B.PROJ_CONIC),
            ("depth", B.PROJ_DEPTH), ("radius", B.PROJ_RADIUS), ("opacity", B.PROJ_OPACITY), ("rgb", B.PROJ_RGB),
            ("flags", B.PROJ_FLAGS))}
        p32 = ov.p32
        assert np.array_equal(g["ids"].astype(np.int64), ids)
        assert np.array_equal(g["rect"], rect_c)
        assert np.array_equal(g["flags"].view(np.uint32), p32["flags"][ids])
        for k in ("xy", "conic", "depth", "radius", "opacity", "rgb"):
            assert np.array_equal(bits(g[k]), bits(p32[k][ids])), k
        del g
        say("  projection bit-exact")
        leaves = B.gs_plan_leaves(ctx, cam, proj, budget) if budget else o_leaves
        assert leaf_tuples(leaves) == leaf_tuples(o_leaves)
        grad2d = torch.zeros((max(n_cand, 1), 9), dtype=torch.float32, device=dev)
        loss_acc = torch.zeros(1, dtype=torch.float64, device=dev)
        tile_lists, tile_tf, tile_last = {}, {}, {}
        total = 0
        for L in leaves:
            bins, n_isect = B.gs_bin_sort(ctx, cam, proj, L)
            total += n_isect
            TWL = L["tx1"] - L["tx0"]
            off = B.gs_export(ctx, bins, B.BINS_OFFSETS).cpu().numpy().view(np.uint64).astype(np.int64)
            assert np.array_equal(np.diff(off), ov.counts[L["ty0"]:L["ty1"], L["tx0"]:L["tx1"]].ravel())
            mine = [t for t in tiles if L["tx0"] <= t % TW < L["tx1"] and L["ty0"] <= t // TW < L["ty1"]]
            vals = B.gs_export(ctx, bins, B.BINS_VALUES).cpu().numpy().view(np.uint32) if mine else None
            ras = B.gs_render_fwd(ctx, cam, proj, bins, target, loss_acc, image)
            B.gs_render_bwd(ctx, cam, proj, bins, ras, grad2d)
            if mine:
                tf = B.gs_export(ctx, ras, B.RASTER_TFINAL).cpu().numpy()
                la = B.gs_export(ctx, ras, B.RASTER_LAST).cpu().numpy()
                x0, y0 = L["tx0"] * 16, L["ty0"] * 16
                WL, HL = min(L["tx1"] * 16, W) - x0, min(L["ty1"] * 16, H) - y0
                tf, la = tf.reshape(HL, WL), la.reshape(HL, WL)
                for t in mine:
                    lt = (t // TW - L["ty0"]) * TWL + (t % TW - L["tx0"])
                    tile_lists[t] = vals[off[lt]:off[lt + 1]].astype(np.int64)
                    px, py = (t % TW) * 16 - x0, (t // TW) * 16 - y0
                    tile_tf[t] = tf[py:py + 16, px:px + 16].copy()
                    tile_last[t] = la[py:py + 16, px:px + 16].copy()
            B.gs_release(ctx, ras)
            B.gs_release(ctx, bins)
        assert total == area
        grad3d = torch.zeros((max(n_cand, 1), F_), dtype=torch.float32, device=dev)
        B.gs_project_bwd(ctx, cam, ds, proj, grad2d, grad3d)
        torch.cuda.synchronize()
        B.gs_release(ctx, proj)
        loss_gpu = float(loss_acc.cpu().numpy()[0]) / (3.0 * W * H)
        say(f"  every tile count bit-exact ({total} intersections)")

    # ---- the loss against the L1 of the GPU image
    img = image.cpu().numpy()
    del image
    loss_host = sum(float(np.abs(img[c].astype(np.float64) - w.target[c].astype(np.float64)).sum())
                    for c in range(3)) / (3.0 * W * H)
    say(f"  loss {loss_gpu:.9f} (host L1 of the GPU image {loss_host:.9f})")
    assert abs(loss_gpu - loss_host) <= 1e-9

    # ---- sampled tiles against the oracle rendering each alone
    lists = ov.render_tiles(tiles)
    b = ov.buffers()
    for t in tiles:
        ys, xs = ov.pix(oracle.rect(t % TW, t // TW, t % TW + 1, t // TW + 1))
        assert np.array_equal(bits(img[:, ys, xs]), bits(b["img"][:, ys, xs])), f"tile {t} image"
        if path == "abi":
            h, wd = ys.stop - ys.start, xs.stop - xs.start
            assert np.array_equal(tile_lists[t], lists[t]), f"tile {t} list"
            assert np.array_equal(bits(tile_tf[t][:h, :wd]), bits(b["tf"][ys, xs])), f"tile {t} T_final"
            assert np.array_equal(tile_last[t][:h, :wd].astype(np.int64), b["last"][ys, xs]), f"tile {t} last"
    say(f"  {len(tiles)} sampled tiles bit-exact; longest list {max(len(x) for x in lists.values())}")

    # ---- regions: image and the gradients of the candidates inside them
    slots, g2o = [], []
    for reg in regions:
        tr = time.time()
        ins, g2 = ov.render_region(reg)
        ys, xs = ov.pix(reg)
        assert np.array_equal(bits(img[:, ys, xs]), bits(b["img"][:, ys, xs])), "region image"
        span = np.maximum(rect_c[ins, 2] - rect_c[ins, 0], rect_c[ins, 3] - rect_c[ins, 1])
        live = np.any(g2 != 0, axis=1)
        nleaf = np.array([F.leaves_spanned(rect_c[s], lid) for s in ins[live]])
        say(f"  region tiles ({reg.tx0},{reg.ty0})-({reg.tx1},{reg.ty1}) image bit-exact; {ins.size} candidates "
            f"inside, {int(live.sum())} with a gradient, largest rectangle {span[live].max() if live.any() else 0} "
            f"tiles, {int((nleaf > 1).sum())} across 2+ leaves ({time.time() - tr:.0f}s)")
        slots.append(ins)
        g2o.append(g2)
    slots = np.concatenate(slots)
    g2o = np.concatenate(g2o)
    g3o = ov.project_bwd_rows(slots, g2o)
    del img
    if path == "abi":
        check_grads("grad2d", grad2d.cpu().numpy()[slots].astype(np.float64), g2o, GRAD2D_GROUPS)
        got3 = grad3d[torch.from_numpy(slots).to(dev)].cpu().numpy().astype(np.float64)
    else:
        gid = torch.from_numpy(ids[slots]).to(dev)
        mrows = [t.reshape(sc.n, -1)[gid].cpu().numpy() for t in m.tensors()]
        vrows = [t.reshape(sc.n, -1)[gid].cpu().numpy() for t in v.tensors()]
        prow = [t.reshape(sc.n, -1)[gid].cpu().numpy() for t in ds.tensors()]
        p0row = [t.reshape(sc.n, -1)[gid].cpu().numpy() for t in p0]
        c1 = np.float32(1.0) - np.float32(BETA1)
        got3 = np.concatenate(mrows, axis=1).astype(np.float64) / np.float64(c1)
        # the update of these rows is one Adam step (from zero moments) of
        # the gradient held in m, and it moves each parameter against the
        # oracle gradient's sign wherever that gradient is not negligible
        mm, vv = np.concatenate(mrows, axis=1), np.concatenate(vrows, axis=1)
        pp, q0 = np.concatenate(prow, axis=1), np.concatenate(p0row, axis=1)
        pe, _, _ = oracle.adam(got3, q0, np.zeros_like(mm), np.zeros_like(vv), step=1)
        ulp = np.spacing(np.abs(pe).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(pp - pe) <= 2 * ulp + 1e-6 * np.abs(pe - q0)), "update of the sampled rows"
        big = np.abs(g3o) >= 1e-2 * np.sqrt(np.mean(g3o ** 2, axis=0, keepdims=True))
        assert np.all(np.sign(pp - q0)[big] == -np.sign(g3o)[big]), "update direction"
        say(f"  Adam rows consistent with the moment's gradient; {int(big.sum())} significant values move "
            f"against the oracle gradient's sign")
    g3groups = {k: sl for k, sl in zip(["means", "log_scales", "quats", "logits", "sh"],
                                       [slice(0, 3), slice(3, 6), slice(6, 10), slice(10, 11), slice(11, F_)])}
    check_grads("grad3d", got3, g3o, g3groups)
    ov.release_buffers()
    say(f"  case done in {time.time() - t0:.0f}s")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("budget_mib", [0, 48])
def test_full_size_ssim_view(ctx, budget_mib):
    """C2 at its full size: 100k Gaussians, SH3, 1920 x 1080, loss
    0.8 L1 + 0.2 (1 - SSIM) (SkipGS notes, "loss function"), through
    gs_train_view as one leaf and split into leaves with the SSIM halo,
    against the oracle's whole view: loss and image within 1e-4, every
    Gaussian's 3D gradient, each group within 1e-3 relative L2."""
    import torch
    from differentiable_gaussian_splatting_amd import scenes
    if "c2" not in F._CACHE:
        F._CACHE.clear()
        w = scenes.make_workload("c2_hd")
        F._CACHE["c2"] = (w, oracle.train_view(w.camera, w.scene, w.target, loss="l1_ssim"))
    w, o = F._CACHE["c2"]
    cam, sc = w.camera, w.scene
    dev = ctx.device
    ds = B.DeviceScene(sc, dev)
    target = torch.from_numpy(w.target).to(dev)
    K = (sc.sh_degree + 1) ** 2
    g3 = torch.zeros((sc.n, 11 + 3 * K), dtype=torch.float32, device=dev)
    img = torch.zeros((3, cam.height, cam.width), dtype=torch.float32, device=dev)
    r = B.gs_train_view(ctx, cam, ds, target, budget_bytes=budget_mib * MIB, loss="l1_ssim", image_out=img,
                        grad3d_out=g3, max_leaves=4096)
    say(f"C2 full size, budget {budget_mib} MiB: {r['n_leaves']} leaves; loss gpu {r['loss']:.9f} "
        f"oracle {o['loss']:.9f}")
    if budget_mib:
        assert r["n_leaves"] > 2
        assert all(L["bytes"] <= L["est_bytes"] for L in r["leaves"])
    assert r["n_cand"] == o["n_cand"]
    assert abs(r["loss"] - o["loss"]) <= 1e-4
    err = float(np.abs(img.cpu().numpy().astype(np.float64) - o["image"]).max())
    say(f"  image max abs err {err:.2e}")
    assert err <= 1e-4
    gg, og = grad3d_groups(g3.cpu().numpy(), 3), grad3d_groups(o["grad3d"], 3)
    for gname in gg:
        e = rel_l2(gg[gname], og[gname])
        say(f"  grad3d {gname:10s} rel L2 {e:.2e}")
        assert e <= GRAD_TOL, gname
