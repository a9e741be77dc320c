"""Pins of the oracle's analytic backward (raster backward + projection
backward) by f64 central finite differences of the f64 forward, for every
parameter of tiny posed scenes, and the leaf == full-image invariant."""
import hashlib

import numpy as np
import pytest

from differentiable_gaussian_splatting_amd import scenes

GROUPS = ("means", "log_scales", "quats", "logits", "sh")


def tiny_scene(rng, n, deg):
    means = np.stack([rng.uniform(-0.8, 0.8, n), rng.uniform(-0.6, 0.6, n), rng.uniform(3.0, 5.0, n)], 1)
    q = rng.normal(size=(n, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    K = (deg + 1) ** 2
    sh = rng.normal(0, 0.4, size=(n, K, 3))
    sh[:, 0, :] = rng.uniform(-1.5, 1.5, size=(n, 3))
    return scenes.Scene(means=means, log_scales=rng.normal(-1.6, 0.3, size=(n, 3)), quats=q,
                        logits=rng.normal(0.5, 1.0, size=n), sh=sh, sh_degree=deg)


def decisions(r, target):
    h = hashlib.sha256()
    p = r["proj64"]
    for a in (p["cand"], p["rect"], p["flags"], np.sign(r["image"] - target.astype(np.float64))):
        h.update(np.ascontiguousarray(a).tobytes())
    h.update(str(r["signature"]).encode())
    return h.hexdigest()


def fd_check(oracle_lib, cam, sc, target, loss, rng, probes_per_group=None, rel_tol=2e-5):
    base = oracle_lib.train_view(cam, sc, target, loss=loss, mode="reference")
    sig0 = decisions(base, target)
    an = oracle_lib.split_grad3d(base["grad3d"], sc.sh_degree)
    arrays = dict(means=sc.means, log_scales=sc.log_scales, quats=sc.quats, logits=sc.logits, sh=sc.sh)
    checked = 0
    for g in GROUPS:
        arr = arrays[g]
        idx = list(np.ndindex(arr.shape))
        if probes_per_group is not None and len(idx) > probes_per_group:
            idx = [idx[k] for k in rng.choice(len(idx), probes_per_group, replace=False)]
        fd_vals, an_vals = [], []
        for ix in idx:
            x0 = arr[ix]
            h = 1e-6 * max(1.0, abs(x0))
            arr[ix] = x0 + h
            rp = oracle_lib.train_view(cam, sc, target, loss=loss, mode="reference")
            arr[ix] = x0 - h
            rm = oracle_lib.train_view(cam, sc, target, loss=loss, mode="reference")
            arr[ix] = x0
            if decisions(rp, target) != sig0 or decisions(rm, target) != sig0:
                continue   # a decision flips inside [x-h, x+h]: the loss is not smooth there
            fd_vals.append((rp["loss"] - rm["loss"]) / (2 * h))
            an_vals.append(an[g][ix if g != "logits" else ix[0]])
        fd_vals, an_vals = np.array(fd_vals), np.array(an_vals)
        if fd_vals.size == 0:
            continue
        scale = max(np.abs(an_vals).max(), 1e-12)
        err = np.abs(fd_vals - an_vals)
        assert np.all(err <= rel_tol * scale + 1e-6 * np.abs(an_vals)), \
            (g, np.max(err / scale), fd_vals[:6], an_vals[:6])
        checked += fd_vals.size
    return checked, base


@pytest.mark.parametrize("seed,n,deg,size", [(1, 1, 0, (32, 32)), (2, 4, 1, (40, 32)),
                                             (3, 8, 3, (48, 40)), (4, 16, 2, (48, 48))])
def test_fd_all_parameters_l1(oracle_lib, seed, n, deg, size):
    rng = np.random.default_rng(seed)
    cam = scenes.random_pose_camera(size[0], size[1], rng, max_angle_deg=10, max_shift=0.2)
    sc = tiny_scene(rng, n, deg)
    target = rng.random((3, size[1], size[0])).astype(np.float32)
    checked, base = fd_check(oracle_lib, cam, sc, target, "l1", rng)
    assert base["n_cand"] == n
    assert checked >= 0.8 * n * (11 + 3 * (deg + 1) ** 2)


def test_fd_l1_ssim(oracle_lib):
    rng = np.random.default_rng(12)
    cam = scenes.random_pose_camera(36, 30, rng, max_angle_deg=10, max_shift=0.2)
    sc = tiny_scene(rng, 6, 3)
    target = rng.random((3, 30, 36)).astype(np.float32)
    checked, _ = fd_check(oracle_lib, cam, sc, target, "l1_ssim", rng, probes_per_group=20)
    assert checked >= 60


def test_fd_with_alpha_and_colour_clamps(oracle_lib):
    # high opacities (alpha clamps at 0.99) and dark colours (rgb clamps at 0)
    rng = np.random.default_rng(21)
    cam = scenes.random_pose_camera(40, 40, rng, max_angle_deg=5, max_shift=0.1)
    sc = tiny_scene(rng, 10, 1)
    sc.logits[:] = 6.0
    sc.sh[:5, 0, :] = -2.5
    target = rng.random((3, 40, 40)).astype(np.float32)
    base = oracle_lib.train_view(cam, sc, target, mode="reference")
    assert (base["proj64"]["flags"] & 7).any()
    checked, _ = fd_check(oracle_lib, cam, sc, target, "l1", rng)
    assert checked >= 0.8 * 10 * 23


def test_parity_gradients_track_reference(oracle_lib):
    w = scenes.make_workload("c2_hd", n=3000, width=160, height=120, posed=True)
    rp = oracle_lib.train_view(w.camera, w.scene, w.target, mode="parity")
    rr = oracle_lib.train_view(w.camera, w.scene, w.target, mode="reference")
    assert abs(rp["loss"] - rr["loss"]) < 1e-5
    gp = oracle_lib.split_grad3d(rp["grad3d"], 3)
    gr = oracle_lib.split_grad3d(rr["grad3d"], 3)
    for g in GROUPS:
        assert np.linalg.norm(gp[g] - gr[g]) <= 1e-3 * np.linalg.norm(gr[g]), g


@pytest.mark.parametrize("budget", [200_000, 60_000])
def test_leaves_equal_full_image(oracle_lib, budget):
    w = scenes.make_workload("c3_gmm4k", n=6000, width=200, height=136, posed=True)
    full = oracle_lib.train_view(w.camera, w.scene, w.target, mode="parity")
    cost = dict(b_isect=20, b_pixel=20, b_tile=64, b_const=4096)
    lv = oracle_lib.train_view(w.camera, w.scene, w.target, mode="parity", budget=budget, cost=cost)
    assert len(lv["leaves"]) > 2
    assert np.array_equal(full["image"], lv["image"])          # bitwise
    assert np.array_equal(full["last"], lv["last"])
    assert abs(lv["loss"] - full["loss"]) <= 1e-12 * full["loss"]
    np.testing.assert_allclose(lv["grad2d"], full["grad2d"], rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose(lv["grad3d"], full["grad3d"], rtol=1e-9, atol=1e-15)
    assert lv["n_isect"] == full["n_isect"]
    assert lv["q_f"] == full["q_f"] and lv["q_b"] == full["q_b"]
