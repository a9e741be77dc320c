"""GPU (HIP, through the C ABI) versus the CPU oracle on the same seeded
inputs.  Bars: bit-exact for candidates, rectangles, depth keys, counts,
offsets, sorted keys and values, leaves; images and loss within 1e-4 max abs;
every gradient group within 1e-3 relative L2 (non-candidates exactly zero)."""
import sys

import numpy as np
import pytest

import oracle
from differentiable_gaussian_splatting_amd import binding as B
from differentiable_gaussian_splatting_amd import scenes
from tests.gpu_pipeline import GRAD2D_GROUPS, bits, grad3d_groups, rel_l2, run_gpu_view

pytestmark = pytest.mark.gpu

IMG_TOL = 1e-4
LOSS_TOL = 1e-4
GRAD_TOL = 1e-3


@pytest.fixture(scope="module")
def ctx():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load()
    return B.Context()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def compare_view(w, g, o, check_bins=True):
    deg = w.scene.sh_degree
    # ---- projection: bit-exact
    ids = o["ids"]
    assert g["n_cand"] == ids.size
    assert np.array_equal(g["ids"].astype(np.int64), ids)
    p = o["proj32"]
    assert np.array_equal(g["rect"], p["rect"][ids])
    assert np.array_equal(bits(g["depth"]), bits(p["depth"][ids]))
    assert np.array_equal(g["flags"].view(np.uint32), p["flags"][ids])
    for k in ("xy", "conic", "radius", "opacity", "rgb"):
        assert np.array_equal(bits(g[k]), bits(p[k][ids])), (k, np.abs(g[k] - p[k][ids]).max())
    slot_of = np.full(w.scene.n, -1, np.int64)
    slot_of[ids] = np.arange(ids.size)
    assert np.array_equal(g["slot_of"].astype(np.int64), slot_of)
    # ---- binning: bit-exact per leaf
    if check_bins:
        for gb, ob in zip(g["bins"], o["bins"]):
            assert gb["n_isect"] == ob["n_isect"]
            assert np.array_equal(gb["offsets"].view(np.uint64), ob["offsets"])
            assert np.array_equal(gb["values"].view(np.uint32), ob["values"])
            assert np.array_equal(gb["keys"].view(np.uint64), ob["keys"])
    # ---- forward
    err = np.abs(g["image"].astype(np.float64) - o["image"].astype(np.float64)).max()
    say(f"  image max abs err {err:.3e} (bitwise: {np.array_equal(bits(g['image']), bits(o['image']))})")
    assert err <= IMG_TOL
    assert np.array_equal(g["last"], o["last"])
    assert np.abs(g["t_final"] - o["t_final"]).max() <= 1e-6
    say(f"  loss gpu {g['loss']:.9f} oracle {o['loss']:.9f}")
    assert abs(g["loss"] - o["loss"]) <= LOSS_TOL
    # ---- gradients
    for name, sl in GRAD2D_GROUPS.items():
        e = rel_l2(g["grad2d"][:, sl], o["grad2d"][:, sl])
        say(f"  grad2d {name:8s} rel L2 {e:.2e}")
        assert e <= GRAD_TOL, name
    gg, og = grad3d_groups(g["grad3d"], deg), grad3d_groups(o["grad3d"], deg)
    for name in gg:
        e = rel_l2(gg[name], og[name])
        say(f"  grad3d {name:10s} rel L2 {e:.2e}")
        assert e <= GRAD_TOL, name
    non = np.ones(w.scene.n, bool)
    non[ids] = False
    assert not g["grad3d"][non].any()


def test_exp_bitwise(ctx):
    import torch
    x = np.concatenate([np.linspace(-87.0, 88.0, 1_000_001, dtype=np.float32),
                        np.array([0.0, -0.0, -87.5, -1e30, 89.0, np.inf, -np.inf], np.float32)])
    xg = torch.from_numpy(x).to(ctx.device)
    y = B.gs_util_exp(ctx, xg).cpu().numpy()
    assert np.array_equal(bits(y), bits(oracle.exp_cw(x)))


def test_exp_falloff_bitwise(ctx):
    import torch
    x = np.concatenate([np.linspace(-7.0, 0.5, 1_000_001, dtype=np.float32),
                        np.arange(0x80000000, 0x80000000 + 100_000, dtype=np.uint32).view(np.float32),
                        np.array([0.0, -0.0, -6.0, -87.5, -1e30, 89.0, np.inf, -np.inf], np.float32)])
    xg = torch.from_numpy(x).to(ctx.device)
    y = B.gs_util_exp_falloff(ctx, xg).cpu().numpy()
    assert np.array_equal(bits(y), bits(oracle.exp_falloff(x)))


@pytest.mark.parametrize("name,kw,budget", [
    ("c1_small", dict(), None),
    ("c1_small", dict(posed=True, seed=101), None),
    ("c2_hd", dict(n=20000, width=400, height=300, posed=True, seed=102), None),
    ("c3_gmm4k", dict(n=40000, width=497, height=283, seed=103), None),
    ("c3_gmm4k", dict(n=40000, width=497, height=283, seed=103), 2_500_000),
    ("c4_plane5k", dict(n=50000, width=520, height=343, seed=104), 3_000_000),
])
def test_view_parity(ctx, name, kw, budget):
    w = scenes.make_workload(name, **kw)
    cost = dict(b_isect=20, b_pixel=20, b_tile=64, b_const=1 << 20)
    say(f"case {name} {kw} budget={budget}")
    g = run_gpu_view(ctx, w, budget=budget, cost=cost)
    o = oracle.train_view(w.camera, w.scene, w.target, loss=w.loss, budget=budget, cost=cost, keep_bins=True)
    if budget is not None:
        got = [(L["tx0"], L["ty0"], L["tx1"], L["ty1"], L["est_bytes"], L["over_budget"]) for L in g["leaves"]]
        exp = [(L["tx0"], L["ty0"], L["tx1"], L["ty1"], L["est_bytes"], L["over_budget"]) for L in o["leaves"]]
        assert got == exp
        assert len(got) > 2
        say(f"  {len(got)} leaves")
    compare_view(w, g, o)


def test_leaf_mode_equals_full_mode_on_gpu(ctx):
    w = scenes.make_workload("c3_gmm4k", n=30000, width=384, height=256, seed=105)
    cost = dict(b_isect=20, b_pixel=20, b_tile=64, b_const=1 << 20)
    full = run_gpu_view(ctx, w, keep_bins=False)
    leaf = run_gpu_view(ctx, w, budget=1_800_000, cost=cost, keep_bins=False)
    assert len(leaf["leaves"]) > 3
    assert np.array_equal(bits(full["image"]), bits(leaf["image"]))
    assert abs(full["loss"] - leaf["loss"]) <= 1e-9
    for name, sl in GRAD2D_GROUPS.items():
        assert rel_l2(leaf["grad2d"][:, sl], full["grad2d"][:, sl]) <= 1e-5


def test_train_view_entry_point(ctx):
    import torch
    w = scenes.make_workload("c2_hd", n=8000, width=250, height=170, posed=True, seed=106)
    ds = B.DeviceScene(w.scene, ctx.device)
    target = torch.from_numpy(w.target).to(ctx.device)
    K = (w.scene.sh_degree + 1) ** 2
    g3 = torch.zeros((w.scene.n, 11 + 3 * K), dtype=torch.float32, device=ctx.device)
    img = torch.zeros((3, 170, 250), dtype=torch.float32, device=ctx.device)
    r = B.gs_train_view(ctx, w.camera, ds, target, loss="l1_ssim", image_out=img, grad3d_out=g3)
    o = oracle.train_view(w.camera, w.scene, w.target, loss="l1_ssim")
    assert abs(r["loss"] - o["loss"]) <= LOSS_TOL
    assert np.abs(img.cpu().numpy() - o["image"]).max() <= IMG_TOL
    gg, og = grad3d_groups(g3.cpu().numpy(), 3), grad3d_groups(o["grad3d"], 3)
    for name in gg:
        assert rel_l2(gg[name], og[name]) <= GRAD_TOL, name
    assert r["n_cand"] == o["n_cand"] and r["n_isect"] == o["n_isect"]


@pytest.mark.parametrize("seed,budget,corner,serial", [(109, 2_500_000, False, False), (110, 1_400_000, False, False),
                                                      (111, 1_400_000, True, False), (110, 1_400_000, False, True)])
def test_train_view_leaves_pipelined(ctx, seed, budget, corner, serial):
    """gs_train_view over several planned leaves bins each next leaf on a
    second stream while the current one is rendered: loss, image, leaves,
    intersections and every 3D gradient group against the oracle's leaf mode,
    and the fused update against the oracle's Adam step.  In the corner case
    every centre projects into the top-left ninth of the image, so the leaves
    planned over the rest of it hold few or no intersections."""
    import torch
    w = scenes.make_workload("c3_gmm4k", n=40000, width=497, height=283, seed=seed)
    if corner:
        c, sc = w.camera, w.scene
        pc = sc.means.astype(np.float64) @ c.R.T.astype(np.float64) + c.t
        u = c.fx * pc[:, 0] / pc[:, 2] + c.cx
        v = c.fy * pc[:, 1] / pc[:, 2] + c.cy
        keep = (pc[:, 2] > 1.0) & (u < c.width / 3) & (v < c.height / 3)
        assert keep.sum() > 500
        w.scene = scenes.Scene(*(a[keep] for a in sc.arrays()), sh_degree=sc.sh_degree)
    cost = dict(b_isect=20, b_pixel=20, b_tile=64, b_const=1 << 20)
    ds = B.DeviceScene(w.scene, ctx.device)
    target = torch.from_numpy(w.target).to(ctx.device)
    K = (w.scene.sh_degree + 1) ** 2
    g3 = torch.zeros((w.scene.n, 11 + 3 * K), dtype=torch.float32, device=ctx.device)
    img = torch.zeros((3, w.camera.height, w.camera.width), dtype=torch.float32, device=ctx.device)
    r = B.gs_train_view(ctx, w.camera, ds, target, budget_bytes=budget, cost=cost, image_out=img, grad3d_out=g3,
                        max_leaves=64, serial_leaves=serial)
    o = oracle.train_view(w.camera, w.scene, w.target, budget=budget, cost=cost, keep_bins=corner)
    say(f"case seed {seed} budget {budget} corner {corner}: {r['n_leaves']} leaves")
    assert r["n_leaves"] == len(o["leaves"]) and r["n_leaves"] > 2
    if corner:
        per_leaf = [b["n_isect"] for b in o["bins"]]
        say(f"  intersections per leaf {per_leaf}")
        assert min(per_leaf) == 0 and max(per_leaf) > 0
    got = [(L["tx0"], L["ty0"], L["tx1"], L["ty1"]) for L in r["leaves"]]
    assert got == [(L["tx0"], L["ty0"], L["tx1"], L["ty1"]) for L in o["leaves"]]
    assert r["n_isect"] == o["n_isect"]
    assert abs(r["loss"] - o["loss"]) <= LOSS_TOL
    assert np.abs(img.cpu().numpy() - o["image"]).max() <= IMG_TOL
    gg, og = grad3d_groups(g3.cpu().numpy(), 3), grad3d_groups(o["grad3d"], 3)
    for name in gg:
        e = rel_l2(gg[name], og[name])
        say(f"  grad3d {name:10s} rel L2 {e:.2e}")
        assert e <= GRAD_TOL, name
    # the same view with the fused update
    rng = np.random.default_rng(seed)
    m0 = [rng.normal(0, 1e-3, size=t.shape) for t in w.scene.arrays()]
    v0 = [rng.uniform(0, 1e-6, size=t.shape) for t in w.scene.arrays()]
    ds2 = B.DeviceScene(w.scene, ctx.device)
    m, v = B.like_scene(ds2), B.like_scene(ds2)
    for dst, src in zip(m.tensors(), m0):
        dst.copy_(torch.from_numpy(src.astype(np.float32)))
    for dst, src in zip(v.tensors(), v0):
        dst.copy_(torch.from_numpy(src.astype(np.float32)))
    r2 = B.gs_train_view(ctx, w.camera, ds2, target, budget_bytes=budget, cost=cost,
                         adam=dict(step=2, params=ds2, m=m, v=v))
    assert abs(r2["loss"] - o["loss"]) <= LOSS_TOL
    groups = grad3d_groups(o["grad3d"], 3)
    for k, (t, name) in enumerate(zip(ds2.tensors(), ["means", "log_scales", "quats", "logits", "sh"])):
        p0 = w.scene.arrays()[k].astype(np.float64)
        p, mm, vv = oracle.adam(groups[name].reshape(p0.shape), p0, m0[k].astype(np.float32),
                                v0[k].astype(np.float32), step=2)
        got = t.cpu().numpy().astype(np.float64)
        ulp = np.spacing(np.abs(p).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(got - p) <= 1e-3 * np.abs(p - p0) + 2 * ulp), name


def test_adam_step_matches_oracle(ctx):
    import torch
    w = scenes.make_workload("c2_hd", n=5000, width=200, height=150, posed=True, seed=107)
    o = oracle.train_view(w.camera, w.scene, w.target)
    ds = B.DeviceScene(w.scene, ctx.device)
    proj, n_cand = B.gs_project(ctx, w.camera, ds)
    assert n_cand == o["n_cand"]
    rng = np.random.default_rng(0)
    # moments from an earlier step (oracle-side numbers), oracle gradients as input
    m0 = [rng.normal(0, 1e-3, size=t.shape) for t in w.scene.arrays()]
    v0 = [rng.uniform(0, 1e-6, size=t.shape) for t in w.scene.arrays()]
    m = B.like_scene(ds)
    v = B.like_scene(ds)
    for dst, src in zip(m.tensors(), m0):
        dst.copy_(torch.from_numpy(src.astype(np.float32)))
    for dst, src in zip(v.tensors(), v0):
        dst.copy_(torch.from_numpy(src.astype(np.float32)))
    g3c = torch.from_numpy(o["grad3d"][o["ids"]].astype(np.float32)).to(ctx.device)
    B.gs_adam_step(ctx, proj, ds, m, v, g3c, step=3, lr=1e-3)
    B.gs_release(ctx, proj)
    groups = grad3d_groups(o["grad3d"], 3)
    for k, (t, name) in enumerate(zip(ds.tensors(), ["means", "log_scales", "quats", "logits", "sh"])):
        p0 = w.scene.arrays()[k].astype(np.float64)
        gr = groups[name].reshape(p0.shape)
        p, mm, vv = oracle.adam(gr, p0, m0[k].astype(np.float32), v0[k].astype(np.float32), step=3)
        got = t.cpu().numpy().astype(np.float64)
        assert np.abs(got - p).max() <= 1e-6 * max(1.0, np.abs(p0).max()), name
        assert rel_l2(got - p0, p - p0) <= 1e-3, name


def _walk_workload():
    """C1's generator at 1024 x 768 with splats e^0.7 times larger: its
    Gaussians cover 0.48 of their super-tiles' tiles, so an L1 view walks the
    super-tile groups (the small scenes above cover 0.03-0.06 and take the
    per-tile lists)."""
    w = scenes.make_workload("c1_small", n=2000, width=1024, height=768, seed=121)
    w.scene.log_scales = (w.scene.log_scales + np.float32(0.7)).astype(np.float32)
    return w


@pytest.mark.parametrize("budget,serial", [(1_110_000, False), (1_150_000, False), (1_110_000, True), (None, False)])
def test_train_view_group_walk(ctx, budget, serial):
    """gs_train_view of a view whose coverage calls for the group-walking
    raster, with the default load model (L1 group walk), over several leaves
    pipelined and one at a time (and the whole image as one planned leaf):
    the raster choice, the leaves, loss, image and every 3D gradient group
    against the oracle's train_view with its own default."""
    import torch
    w = _walk_workload()
    p32 = oracle.project(w.camera, w.scene, "f32")
    assert oracle.walks_groups(p32["rect"][p32["cand"]])
    ds = B.DeviceScene(w.scene, ctx.device)
    target = torch.from_numpy(w.target).to(ctx.device)
    K = (w.scene.sh_degree + 1) ** 2
    g3 = torch.zeros((w.scene.n, 11 + 3 * K), dtype=torch.float32, device=ctx.device)
    img = torch.zeros((3, w.camera.height, w.camera.width), dtype=torch.float32, device=ctx.device)
    b = budget if budget is not None else 1 << 40
    r = B.gs_train_view(ctx, w.camera, ds, target, budget_bytes=b, image_out=img, grad3d_out=g3,
                        max_leaves=64, serial_leaves=serial)
    o = oracle.train_view(w.camera, w.scene, w.target, budget=b)
    say(f"group walk budget {budget} serial {serial}: {r['n_leaves']} leaves, walked {r['groups_walked']}")
    assert r["groups_walked"]
    assert r["n_leaves"] == len(o["leaves"]) and (budget is None or r["n_leaves"] > 2)
    got = [(L["tx0"], L["ty0"], L["tx1"], L["ty1"], L["est_bytes"]) for L in r["leaves"]]
    assert got == [(L["tx0"], L["ty0"], L["tx1"], L["ty1"], L["est_bytes"]) for L in o["leaves"]]
    assert all(L["bytes"] <= L["est_bytes"] for L in r["leaves"])
    assert r["n_isect"] == o["n_isect"]
    assert abs(r["loss"] - o["loss"]) <= LOSS_TOL
    assert np.array_equal(bits(img.cpu().numpy()), bits(o["image"].astype(np.float32)))
    gg, og = grad3d_groups(g3.cpu().numpy(), 3 if K == 16 else 0), grad3d_groups(o["grad3d"], 3 if K == 16 else 0)
    for name in gg:
        e = rel_l2(gg[name], og[name])
        say(f"  grad3d {name:10s} rel L2 {e:.2e}")
        assert e <= GRAD_TOL, name


def test_low_coverage_view_takes_the_lists(ctx):
    """A view whose Gaussians cover few of their super-tiles' tiles renders
    from per-tile lists, planned with the default model, as the oracle's
    train_view plans it."""
    import torch
    w = scenes.make_workload("c3_gmm4k", n=40000, width=497, height=283, seed=109)
    p32 = oracle.project(w.camera, w.scene, "f32")
    assert not oracle.walks_groups(p32["rect"][p32["cand"]])
    ds = B.DeviceScene(w.scene, ctx.device)
    target = torch.from_numpy(w.target).to(ctx.device)
    img = torch.zeros((3, w.camera.height, w.camera.width), dtype=torch.float32, device=ctx.device)
    r = B.gs_train_view(ctx, w.camera, ds, target, budget_bytes=3_000_000, image_out=img, max_leaves=64)
    o = oracle.train_view(w.camera, w.scene, w.target, budget=3_000_000)
    assert not r["groups_walked"]
    assert [(L["tx0"], L["ty0"], L["tx1"], L["ty1"]) for L in r["leaves"]] == \
        [(L["tx0"], L["ty0"], L["tx1"], L["ty1"]) for L in o["leaves"]]
    assert r["n_leaves"] > 1
    assert abs(r["loss"] - o["loss"]) <= LOSS_TOL
    assert np.array_equal(bits(img.cpu().numpy()), bits(o["image"].astype(np.float32)))


@pytest.mark.parametrize("chunk,deg", [(700, 3), (0, 3), (0, 1), (0, 0)])
def test_train_view_chunked_update_matches_oracle(ctx, chunk, deg):
    """gs_train_view with Adam and no dense gradient output: chunk 0 (the
    default) fuses the projection backward with the update over all
    Gaussians; chunk 700 runs them chunk by chunk of candidate slots (several
    chunks and a ragged last one).  N = 5000 leaves a ragged last wavefront."""
    import torch
    w = scenes.make_workload("c2_hd", n=5000, width=200, height=150, posed=True, seed=108, sh_degree=deg)
    o = oracle.train_view(w.camera, w.scene, w.target)
    assert o["n_cand"] > 2 * 700
    rng = np.random.default_rng(1)
    m0 = [rng.normal(0, 1e-3, size=t.shape) for t in w.scene.arrays()]
    v0 = [rng.uniform(0, 1e-6, size=t.shape) for t in w.scene.arrays()]
    ds = B.DeviceScene(w.scene, ctx.device)
    m, v = B.like_scene(ds), B.like_scene(ds)
    for dst, src in zip(m.tensors(), m0):
        dst.copy_(torch.from_numpy(src.astype(np.float32)))
    for dst, src in zip(v.tensors(), v0):
        dst.copy_(torch.from_numpy(src.astype(np.float32)))
    target = torch.from_numpy(w.target).to(ctx.device)
    r = B.gs_train_view(ctx, w.camera, ds, target, adam=dict(step=3, params=ds, m=m, v=v, chunk=chunk))
    assert abs(r["loss"] - o["loss"]) <= LOSS_TOL
    groups = grad3d_groups(o["grad3d"], deg)
    for k, (t, name) in enumerate(zip(ds.tensors(), ["means", "log_scales", "quats", "logits", "sh"])):
        p0 = w.scene.arrays()[k].astype(np.float64)
        p, mm, vv = oracle.adam(groups[name].reshape(p0.shape), p0, m0[k].astype(np.float32),
                                v0[k].astype(np.float32), step=3)
        got = t.cpu().numpy().astype(np.float64)
        say(f"  {name:10s} update rel L2 {rel_l2(got - p0, p - p0):.2e}")
        # each update within 1e-3 of the oracle's, beside the rounding of the
        # stored f32 parameter (its ulp is ~2e-6 at the means' depth of ~20)
        ulp = np.spacing(np.abs(p).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(got - p) <= 1e-3 * np.abs(p - p0) + 2 * ulp), name


@pytest.mark.parametrize("chunk", [0, 1, 700])
def test_train_view_update_without_candidates(ctx, chunk):
    """A view in which every Gaussian is culled still takes its one Adam step
    (zero gradients: the moments decay and the parameters move by the decayed
    first moment), in the fused form (chunk 0) and chunk by chunk of
    candidate slots (no slot exists, so no projection backward runs)."""
    import torch
    w = scenes.make_workload("c2_hd", n=3000, width=120, height=90, seed=112)
    w.scene.means[:, 2] = -5.0
    o = oracle.train_view(w.camera, w.scene, w.target)
    assert o["n_cand"] == 0
    rng = np.random.default_rng(2)
    m0 = [rng.normal(0, 1e-3, size=t.shape) for t in w.scene.arrays()]
    v0 = [rng.uniform(1e-8, 1e-6, size=t.shape) for t in w.scene.arrays()]
    ds = B.DeviceScene(w.scene, ctx.device)
    m, v = B.like_scene(ds), B.like_scene(ds)
    for dst, src in zip(m.tensors(), m0):
        dst.copy_(torch.from_numpy(src.astype(np.float32)))
    for dst, src in zip(v.tensors(), v0):
        dst.copy_(torch.from_numpy(src.astype(np.float32)))
    target = torch.from_numpy(w.target).to(ctx.device)
    r = B.gs_train_view(ctx, w.camera, ds, target, adam=dict(step=4, params=ds, m=m, v=v, chunk=chunk))
    assert r["n_cand"] == 0 and r["n_isect"] == 0
    assert abs(r["loss"] - o["loss"]) <= LOSS_TOL
    for k, t in enumerate(ds.tensors()):
        p0 = w.scene.arrays()[k].astype(np.float64)
        p, mm, vv = oracle.adam(np.zeros_like(p0), p0, m0[k].astype(np.float32), v0[k].astype(np.float32), step=4)
        got = t.cpu().numpy().astype(np.float64)
        ulp = np.spacing(np.abs(p).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(got - p) <= 1e-3 * np.abs(p - p0) + 2 * ulp), k
        assert rel_l2(m.tensors()[k].cpu().numpy(), mm) <= 1e-6, k
        assert rel_l2(v.tensors()[k].cpu().numpy(), vv) <= 1e-6, k


@pytest.mark.parametrize("case", ["empty", "all_culled", "one_pixel", "ragged", "huge", "dense_tile"])
def test_edge_cases(ctx, case):
    rng = np.random.default_rng(200)
    say(f"edge case {case}")
    if case == "empty":
        w = scenes.make_workload("c1_small", n=0, width=40, height=24)
    elif case == "all_culled":
        w = scenes.make_workload("c1_small", n=300, width=40, height=24)
        w.scene.means[:, 2] = -5.0
    elif case == "one_pixel":
        w = scenes.make_workload("c1_small", n=500, width=1, height=1)
    elif case == "ragged":
        w = scenes.make_workload("c2_hd", n=3000, width=17, height=33, posed=True, seed=201)
    elif case == "huge":
        w = scenes.make_workload("c1_small", n=400, width=300, height=200, seed=202)
        w.scene.log_scales[:5] = 1.5          # rectangles covering the whole grid (wave-wide emission)
        w.scene.logits[:5] = -3.0
    else:
        # one tile receives far more than 8192 entries (a long list split into many fine segments)
        n = 12000
        w = scenes.make_workload("c1_small", n=n, width=96, height=64, seed=203)
        w.scene.means[:, 0] = rng.uniform(-0.05, 0.05, n)
        w.scene.means[:, 1] = rng.uniform(-0.05, 0.05, n)
        # anisotropic: an exactly isotropic Gaussian has an identically zero
        # rotation gradient, which f32 and f64 would only show as rounding noise
        w.scene.log_scales[:] = (-6.0 + rng.normal(0, 0.3, size=(n, 3))).astype(np.float32)
        w.scene.logits[:] = -4.0
    g = run_gpu_view(ctx, w)
    o = oracle.train_view(w.camera, w.scene, w.target, loss=w.loss, keep_bins=True)
    if case == "dense_tile":
        assert max(np.diff(b["offsets"].view(np.uint64)).max() for b in g["bins"]) > 8192
    if case == "huge":
        assert (o["proj32"]["rect"][:5, 2] - o["proj32"]["rect"][:5, 0] > 10).all()
    compare_view(w, g, o)


def test_cull_threshold_at_box_edges_and_corners(ctx):
    """Gaussians whose alpha is exactly at 1/255 (one f32 logit step either
    side) at the corner or edge pixel of an 8 x 8 box they lie outside
    (tests/cull_cases.py): the sub-tile cull keeps every entry some pixel
    includes, so lists, images, T_final and walk ends are bit-exact against
    the oracle (which culls nothing), through the separate kernels and the
    fused raster, and the gradients meet the bar."""
    import torch
    from tests import cull_cases as cc
    cam, sc, cases = cc.threshold_scene()
    rng = np.random.default_rng(301)
    w = scenes.Workload(name="threshold", scene=sc, camera=cam,
                        target=scenes.target_image(rng, cam.width, cam.height), loss="l1", budgets=())
    o = oracle.train_view(cam, sc, w.target, keep_bins=True)
    inc = [bool(o["image"][:, py, px].any()) for (_, _, _, side, px, py) in cases]
    say(f"  {len(cases)} threshold Gaussians, {sum(inc)} of their pixels lit in the oracle image")
    g = run_gpu_view(ctx, w)
    compare_view(w, g, o)
    assert np.array_equal(bits(g["t_final"]), bits(o["t_final"]))
    assert np.array_equal(g["last"], o["last"].astype(np.int64))
    ds = B.DeviceScene(sc, ctx.device)
    img = torch.zeros((3, cam.height, cam.width), dtype=torch.float32, device=ctx.device)
    g3 = torch.zeros((sc.n, 14), dtype=torch.float32, device=ctx.device)
    r = B.gs_train_view(ctx, cam, ds, torch.from_numpy(w.target).to(ctx.device), image_out=img, grad3d_out=g3)
    assert np.array_equal(bits(img.cpu().numpy()), bits(o["image"]))
    assert abs(r["loss"] - o["loss"]) <= LOSS_TOL
    gg, og = grad3d_groups(g3.cpu().numpy(), 0), grad3d_groups(o["grad3d"], 0)
    for name in gg:
        assert rel_l2(gg[name], og[name]) <= GRAD_TOL, name


def test_isotropic_rotation_gradient_is_negligible(ctx):
    # rotating an isotropic Gaussian changes nothing: its quaternion gradient
    # is rounding noise, tiny next to the scale gradient of the same Gaussian
    w = scenes.make_workload("c1_small", n=800, width=96, height=64, seed=204)
    w.scene.log_scales[:] = -3.0
    g = run_gpu_view(ctx, w, keep_bins=False)
    gg = grad3d_groups(g["grad3d"], 0)
    assert np.linalg.norm(gg["quats"]) <= 1e-4 * np.linalg.norm(gg["log_scales"])


def _rects(leaves):
    return [(L["tx0"], L["ty0"], L["tx1"], L["ty1"], L["est_bytes"], L["over_budget"]) for L in leaves]


@pytest.mark.parametrize("budget_b", [1_400_000, 700_000, 4_000_000])
def test_replan_cached_layout_matches_oracle(ctx, budget_b):
    """A layout planned on one view, re-checked on another (moved camera,
    other budget) through gs_replan_leaves: the same leaves and estimates as
    the oracle's re-check, bit for bit."""
    cost = dict(b_isect=20, b_pixel=20, b_tile=64, b_const=1 << 20)
    wa = scenes.make_workload("c3_gmm4k", n=40000, width=497, height=283, posed=True, seed=121)
    wb = scenes.make_workload("c3_gmm4k", n=40000, width=497, height=283, posed=True, seed=122)
    da = B.DeviceScene(wa.scene, ctx.device)
    pa, _ = B.gs_project(ctx, wa.camera, da)
    cached = B.gs_plan_leaves(ctx, wa.camera, pa, 1_400_000, cost=cost)
    B.gs_release(ctx, pa)
    db = B.DeviceScene(wb.scene, ctx.device)
    pb, _ = B.gs_project(ctx, wb.camera, db)
    got = B.gs_replan_leaves(ctx, wb.camera, pb, budget_b, cached, cost=cost)
    B.gs_release(ctx, pb)
    o32 = oracle.project(wb.camera, wb.scene, "f32")
    rect_c = o32["rect"][o32["cand"]]
    expect = oracle.plan_leaves(wb.camera, rect_c, budget_b, cost, roots=cached)
    say(f"cached {len(cached)} leaves -> {len(got)} at budget {budget_b}")
    assert len(cached) > 2
    assert _rects(got) == _rects(expect)


def test_train_view_with_cached_layout(ctx):
    """The first view of a sequence returns its layout; the next view
    re-checks that layout instead of planning afresh: loss, image,
    leaves and every gradient group against the oracle's view over the
    oracle's re-check of the same layout."""
    import torch
    cost = dict(b_isect=20, b_pixel=20, b_tile=64, b_const=1 << 20)
    budget = 1_400_000
    wa = scenes.make_workload("c3_gmm4k", n=40000, width=497, height=283, posed=True, seed=123)
    wb = scenes.make_workload("c3_gmm4k", n=40000, width=497, height=283, posed=True, seed=124)
    da = B.DeviceScene(wa.scene, ctx.device)
    ra = B.gs_train_view(ctx, wa.camera, da, torch.from_numpy(wa.target).to(ctx.device), budget_bytes=budget,
                         cost=cost, max_leaves=256)
    cached = ra["leaves"]
    db = B.DeviceScene(wb.scene, ctx.device)
    K = (wb.scene.sh_degree + 1) ** 2
    g3 = torch.zeros((wb.scene.n, 11 + 3 * K), dtype=torch.float32, device=ctx.device)
    img = torch.zeros((3, wb.camera.height, wb.camera.width), dtype=torch.float32, device=ctx.device)
    rb = B.gs_train_view(ctx, wb.camera, db, torch.from_numpy(wb.target).to(ctx.device), budget_bytes=budget,
                         cost=cost, max_leaves=256, leaves_in=cached, image_out=img, grad3d_out=g3)
    o32 = oracle.project(wb.camera, wb.scene, "f32")
    leaves = oracle.plan_leaves(wb.camera, o32["rect"][o32["cand"]], budget, cost, roots=cached)
    o = oracle.train_view(wb.camera, wb.scene, wb.target, leaves=leaves, cost=cost)
    say(f"next view: {len(cached)} cached leaves -> {rb['n_leaves']}")
    assert _rects(rb["leaves"]) == _rects(leaves)
    assert abs(rb["loss"] - o["loss"]) <= LOSS_TOL
    assert np.abs(img.cpu().numpy() - o["image"]).max() <= IMG_TOL
    gg, og = grad3d_groups(g3.cpu().numpy(), 3), grad3d_groups(o["grad3d"], 3)
    for name in gg:
        assert rel_l2(gg[name], og[name]) <= GRAD_TOL, name


def test_replan_rejects_a_layout_that_does_not_tile_the_grid(ctx):
    w = scenes.make_workload("c1_small", n=300, width=96, height=64, seed=125)
    d = B.DeviceScene(w.scene, ctx.device)
    p, _ = B.gs_project(ctx, w.camera, d)
    TW, TH = w.camera.tiles_x, w.camera.tiles_y
    bad = [[dict(tx0=0, ty0=0, tx1=TW, ty1=TH), dict(tx0=0, ty0=0, tx1=1, ty1=1)],   # overlap
           [dict(tx0=0, ty0=0, tx1=TW - 1, ty1=TH)],                                  # a column uncovered
           [dict(tx0=0, ty0=0, tx1=TW + 1, ty1=TH)]]                                  # outside the grid
    for layout in bad:
        with pytest.raises(B.GsError) as ei:
            B.gs_replan_leaves(ctx, w.camera, p, 1 << 30, layout)
        assert B.STATUS_NAMES[ei.value.status] == "GS_ERR_INVALID_ARG"
    ok = B.gs_replan_leaves(ctx, w.camera, p, 1 << 30, [dict(tx0=0, ty0=0, tx1=TW, ty1=TH)])
    assert [(L["tx0"], L["ty0"], L["tx1"], L["ty1"]) for L in ok] == [(0, 0, TW, TH)]
    B.gs_release(ctx, p)


@pytest.mark.parametrize("nx,ny,blocks", [(3, 2, None), (3, 2, [1, 4]), (9, 8, None)])
def test_fixed_grid_views_match_oracle(ctx, nx, ny, blocks):
    """The fixed-block baselines: a 3 x 2 grid rendered as given (budget 0),
    all blocks (one update per view) or some of them (the view of one
    per-block update step: only those pixels are rendered and differentiated).
    Loss, image (pixels outside the blocks untouched), leaves and every
    gradient group against the oracle's view over the same blocks.  The 9 x 8
    grid has more leaves than the candidate-to-leaf grouping tests one by one
    (it looks the rectangle corners up in a tile -> leaf map)."""
    import torch
    w = scenes.make_workload("c3_gmm4k", n=30000, width=400, height=250, posed=True, seed=131)
    lib = B.load()
    grid = B.gs_grid_leaves(lib, w.camera.tiles_x, w.camera.tiles_y, nx, ny)
    assert [(L["tx0"], L["ty0"], L["tx1"], L["ty1"]) for L in grid] == \
        [(L["tx0"], L["ty0"], L["tx1"], L["ty1"]) for L in oracle.grid_leaves(w.camera.tiles_x, w.camera.tiles_y, nx, ny)]
    assert len(grid) == nx * ny
    layout = grid if blocks is None else [grid[k] for k in blocks]
    ds = B.DeviceScene(w.scene, ctx.device)
    K = (w.scene.sh_degree + 1) ** 2
    g3 = torch.zeros((w.scene.n, 11 + 3 * K), dtype=torch.float32, device=ctx.device)
    img = torch.full((3, w.camera.height, w.camera.width), -1.0, dtype=torch.float32, device=ctx.device)
    r = B.gs_train_view(ctx, w.camera, ds, torch.from_numpy(w.target).to(ctx.device), budget_bytes=0,
                        leaves_in=layout, partial=blocks is not None, image_out=img, grad3d_out=g3, max_leaves=128)
    o = oracle.train_view(w.camera, w.scene, w.target, leaves=[dict(L, est_bytes=0, over_budget=False)
                                                               for L in layout])
    assert [(L["tx0"], L["ty0"], L["tx1"], L["ty1"]) for L in r["leaves"]] == \
        [(L["tx0"], L["ty0"], L["tx1"], L["ty1"]) for L in layout]
    assert abs(r["loss"] - o["loss"]) <= LOSS_TOL
    got = img.cpu().numpy()
    inside = np.zeros((w.camera.height, w.camera.width), bool)
    for L in layout:
        inside[L["ty0"] * 16:L["ty1"] * 16, L["tx0"] * 16:L["tx1"] * 16] = True
    assert np.abs(got[:, inside] - o["image"][:, inside]).max() <= IMG_TOL
    assert (got[:, ~inside] == -1.0).all()
    gg, og = grad3d_groups(g3.cpu().numpy(), 3), grad3d_groups(o["grad3d"], 3)
    for name in gg:
        assert rel_l2(gg[name], og[name]) <= GRAD_TOL, name
    if blocks is not None:
        with pytest.raises(B.GsError):   # a partial layout with overlapping blocks
            B.gs_train_view(ctx, w.camera, ds, torch.from_numpy(w.target).to(ctx.device), budget_bytes=0,
                            leaves_in=[grid[0], grid[0]], partial=True)


@pytest.mark.parametrize("loss", ["l1", "l1_ssim"])
def test_train_view_loss_left_on_device(ctx, loss):
    """loss_out: the view's loss is written to the device (no read-back), with
    the bits of the read-back value; the returned loss is None, the element
    before it is untouched, and a gated view refuses the option."""
    import torch
    w = scenes.make_workload("c3_gmm4k", n=20000, width=400, height=250, posed=True, seed=151)
    ds = B.DeviceScene(w.scene, ctx.device)
    target = torch.from_numpy(w.target).to(ctx.device)
    kw = dict(budget_bytes=1_400_000, cost=dict(b_isect=20, b_pixel=20, b_tile=64, b_const=1 << 20), loss=loss)
    say(f"case loss_out {loss}")
    r = B.gs_train_view(ctx, w.camera, ds, target, **kw)
    out = torch.full((2,), float("nan"), dtype=torch.float64, device=ctx.device)
    r2 = B.gs_train_view(ctx, w.camera, ds, target, loss_out=out[1:], **kw)
    assert r2["loss"] is None and r2["n_leaves"] == r["n_leaves"] and r["n_leaves"] > 1
    got = out.cpu().numpy()
    assert np.isnan(got[0]) and got[1] == r["loss"]
    with pytest.raises(B.GsError):
        B.gs_train_view(ctx, w.camera, ds, target, loss_out=out[1:], gate=B.Gate(2, warmup=2), gate_view=0, **kw)


@pytest.mark.parametrize("budget,factors,falling", [
    (0, [1.0, 1.0, 0.8, 1.25, 0.9, 1.1, 1.05, 0.7, 1.3, 0.85], False),
    (1_400_000, [1.0, 1.0, 0.8, 1.25, 0.9, 1.1, 1.05, 0.7, 1.3, 0.85], False),
    # falling losses: the skips bring the backward ratio under the floor,
    # which then forces backwards
    (1_400_000, [1.0, 1.0, 0.9, 0.9, 0.8, 0.8, 0.7, 0.7, 0.6, 0.6], True)])
def test_gated_view_sequence_matches_oracle(ctx, budget, factors, falling):
    """A sequence of views through gs_train_view with the SkipGS gate: every
    step's loss and decision against the oracle's gate fed with the oracle's
    loss; a step that runs its backward gives the oracle's gradients, one
    that skips it leaves the gradient buffer untouched.  The targets change
    from step to step so that no score sits near 1."""
    import torch
    cost = dict(b_isect=20, b_pixel=20, b_tile=64, b_const=1 << 20)
    views = [scenes.make_workload("c3_gmm4k", n=20000, width=400, height=250, posed=True, seed=s)
             for s in (141, 142)]
    scene = views[0].scene
    ds = B.DeviceScene(scene, ctx.device)
    K = (scene.sh_degree + 1) ** 2
    gate = B.Gate(2, warmup=2)
    og = oracle.SkipGate(2, warmup=2)
    ran = skipped = forced = 0
    for t, f in enumerate(factors):
        v = t % 2
        w = views[v]
        tgt = (w.target * np.float32(f)).astype(np.float32)
        g3 = torch.full((scene.n, 11 + 3 * K), float("nan"), dtype=torch.float32, device=ctx.device)
        r = B.gs_train_view(ctx, w.camera, ds, torch.from_numpy(tgt).to(ctx.device), budget_bytes=budget,
                            cost=cost, grad3d_out=g3, gate=gate, gate_view=v)
        o = oracle.train_view(w.camera, scene, tgt, budget=budget if budget else None, cost=cost)
        od = og.step(v, o["loss"])
        say(f"step {t + 1} view {v}: loss {r['loss']:.6f} / {o['loss']:.6f}, score {r['score']:.4f}, "
            f"backward {r['backward']} forced {r['forced']}")
        assert abs(r["loss"] - o["loss"]) <= LOSS_TOL
        assert (r["backward"], r["forced"]) == (od["backward"], od["forced"])
        assert np.isinf(od["score"]) or abs(od["score"] - 1.0) > 1e-3
        got = g3.cpu().numpy()
        forced += 1 if r["forced"] else 0
        if r["backward"]:
            ran += 1
            gg, ogr = grad3d_groups(got, 3), grad3d_groups(o["grad3d"], 3)
            for name in gg:
                assert rel_l2(gg[name], ogr[name]) <= GRAD_TOL, name
        else:
            skipped += 1
            assert np.isnan(got).all()
    st = gate.stats()
    assert st["backwards"] == og.b and st["rho_min"] == og.rho_min
    assert ran > 2 and skipped > 0
    if falling:
        assert forced > 0
    gate.close()


@pytest.mark.parametrize("opaque", ["none", "some", "all"])
def test_alpha_clamp_batches_bit_exact(ctx, opaque):
    """Opacities above the alpha clamp (0.99) in none, some or all of the
    Gaussians, so that the clamp binds on some pixels: the image is bit-exact
    against the oracle, and the gradients (zero through a clamped alpha) and
    the loss meet the bar, in every mix."""
    import torch
    w = scenes.make_workload("c1_small", n=2500, width=96, height=64, seed=205)
    if opaque == "some":
        w.scene.logits[::7] = 6.0          # opacity 0.9975
    elif opaque == "all":
        w.scene.logits[:] = 6.0
    sc, cam = w.scene, w.camera
    o = oracle.train_view(cam, sc, w.target)
    ds = B.DeviceScene(sc, ctx.device)
    img = torch.zeros((3, cam.height, cam.width), dtype=torch.float32, device=ctx.device)
    g3 = torch.zeros((sc.n, 11 + 3 * (sc.sh_degree + 1) ** 2), dtype=torch.float32, device=ctx.device)
    r = B.gs_train_view(ctx, cam, ds, torch.from_numpy(w.target).to(ctx.device), image_out=img, grad3d_out=g3)
    assert np.array_equal(bits(img.cpu().numpy()), bits(o["image"]))
    assert abs(r["loss"] - o["loss"]) <= LOSS_TOL
    gg, og = grad3d_groups(g3.cpu().numpy(), sc.sh_degree), grad3d_groups(o["grad3d"], sc.sh_degree)
    for name in gg:
        assert rel_l2(gg[name], og[name]) <= GRAD_TOL, name


def test_train_view_more_leaves_than_a_block(ctx):
    """A budget below every single tile's estimate: the plan is one leaf per
    tile, 1200 of them, more than the 1024 threads that sum the leaves' tile
    bases (so each thread takes a run of leaves).  Leaves, intersections,
    loss, image and the 3D gradient groups against the oracle's leaf mode."""
    import torch
    w = scenes.make_workload("c3_gmm4k", n=6000, width=640, height=480, seed=206)
    cost = dict(b_isect=20, b_pixel=20, b_tile=64, b_const=1 << 20)
    ds = B.DeviceScene(w.scene, ctx.device)
    K = (w.scene.sh_degree + 1) ** 2
    g3 = torch.zeros((w.scene.n, 11 + 3 * K), dtype=torch.float32, device=ctx.device)
    img = torch.zeros((3, w.camera.height, w.camera.width), dtype=torch.float32, device=ctx.device)
    r = B.gs_train_view(ctx, w.camera, ds, torch.from_numpy(w.target).to(ctx.device), budget_bytes=1, cost=cost,
                        image_out=img, grad3d_out=g3, max_leaves=2048)
    o = oracle.train_view(w.camera, w.scene, w.target, budget=1, cost=cost)
    say(f"{r['n_leaves']} leaves")
    assert r["n_leaves"] == 40 * 30 == len(o["leaves"])
    got = [(L["tx0"], L["ty0"], L["tx1"], L["ty1"]) for L in r["leaves"]]
    assert got == [(L["tx0"], L["ty0"], L["tx1"], L["ty1"]) for L in o["leaves"]]
    assert r["n_isect"] == o["n_isect"]
    assert abs(r["loss"] - o["loss"]) <= LOSS_TOL
    assert np.abs(img.cpu().numpy() - o["image"]).max() <= IMG_TOL
    gg, og = grad3d_groups(g3.cpu().numpy(), w.scene.sh_degree), grad3d_groups(o["grad3d"], w.scene.sh_degree)
    for name in gg:
        assert rel_l2(gg[name], og[name]) <= GRAD_TOL, name
