"""Scenes whose Gaussians put alpha exactly at the 1/255 threshold on the
edges and corners of the 8 x 8 pixel boxes the rasterizer culls against.

For each case a Gaussian (random anisotropic scale and rotation) is centred
outside one 8 x 8 box of a tile, beyond one of the box's corners or edges,
so that the box's pixel centre nearest to it is that corner or edge pixel.
Its opacity logit is then bisected over the ordered f32 values with the
oracle (projecting and rendering the Gaussian alone), down to the two
adjacent logits at which that pixel's alpha moves from below 1/255 (the
entry is skipped) to at least 1/255 (the entry is included).  Both are kept,
each as a Gaussian of its own placed in a box of its own: one that reaches
exactly one pixel of the box by the smallest margin f32 allows, and one that
reaches none of it by the same margin.  A cull that drops an entry some
pixel of the box includes changes the image, which the parity tests compare
bit for bit with the oracle (which culls nothing).
"""
from __future__ import annotations

import math

import numpy as np

import oracle
from differentiable_gaussian_splatting_amd import scenes

W = H = 256


def _f32_order(x):
    """Monotone map f32 -> int64 (ordered like the floats)."""
    b = np.array([x], np.float32).view(np.int32)[0].astype(np.int64)
    return b if b >= 0 else -(b & 0x7FFFFFFF)


def _f32_from_order(k):
    b = k if k >= 0 else (-k) | 0x80000000
    return float(np.array([b & 0xFFFFFFFF], np.uint32).view(np.float32)[0])


def included(cam, g, logit, px, py):
    """Whether pixel (px, py) includes Gaussian g (alone) at this logit."""
    sc = scenes.Scene(g["means"], g["log_scales"], g["quats"], np.array([logit], np.float32), g["sh"],
                      sh_degree=0)
    p = oracle.project(cam, sc, "f32")
    if not p["cand"][0]:
        return False
    tx, ty = px // 16, py // 16
    r = oracle.rect(tx, ty, tx + 1, ty + 1)
    bins = oracle.bin_leaf(cam.tiles_x, r, p["rect"], p["depth"], with_keys=False)
    img, _, _, _ = oracle.render_fwd(cam, r, bins, p["xy"], p["conic"], p["opacity"], p["rgb"])
    return bool(img[:, py, px].any())


def threshold_scene(n_cases=96, seed=300):
    """(camera, scene, cases): cases[i] = (box x0, box y0, feature, side,
    pixel x, pixel y) for Gaussian i, with side 'in' (the pixel includes it,
    not at the next smaller f32 logit) or 'out' (the pixel skips it, not at
    the next larger f32 logit)."""
    rng = np.random.default_rng(seed)
    cam = scenes.pinhole_camera(W, H)
    boxes = [(bx, by) for by in range(0, H, 8) for bx in range(0, W, 8)]
    order = rng.permutation(len(boxes))
    used = 0
    feats = ["corner00", "corner10", "corner01", "corner11", "edge_l", "edge_r", "edge_t", "edge_b"]
    means, scales, quats, logits, cases = [], [], [], [], []
    Z = 4.0
    while len(cases) < 2 * n_cases and used + 2 <= len(boxes):
        feat = feats[len(cases) // 2 % len(feats)]
        ls = rng.normal(-3.0, 0.6, size=3).astype(np.float32)
        q = rng.normal(size=4)
        q = (q / np.linalg.norm(q)).astype(np.float32)
        sh = np.zeros((1, 1, 3), np.float32) + np.float32(1.0)
        # outward offset from the feature pixel's centre, in pixels
        d = float(rng.uniform(0.6, 3.5))
        pair = []
        for _ in range(2):
            bx, by = boxes[order[used]]
            used += 1
            if feat.startswith("corner"):
                sx, sy = int(feat[6]), int(feat[7])
                ppx, ppy = bx + 7 * sx, by + 7 * sy
                ox, oy = (1 if sx else -1) * d / math.sqrt(2), (1 if sy else -1) * d / math.sqrt(2)
            else:
                side = feat[5]
                ppx = bx + (0 if side == "l" else 7 if side == "r" else int(rng.integers(1, 7)))
                ppy = by + (0 if side == "t" else 7 if side == "b" else int(rng.integers(1, 7)))
                ox = -d if side == "l" else d if side == "r" else 0.0
                oy = -d if side == "t" else d if side == "b" else 0.0
            cx, cy = ppx + 0.5 + ox, ppy + 0.5 + oy
            X = (cx - cam.cx) * Z / cam.fx
            Y = (cy - cam.cy) * Z / cam.fy
            pair.append((bx, by, ppx, ppy, np.array([[X, Y, Z]], np.float32)))
        # bisect on the first placement's pixel; the second gets the same
        # shape at its own box (its boundary found the same way)
        found = []
        for bx, by, ppx, ppy, mu in pair:
            g = dict(means=mu, log_scales=ls[None], quats=q[None], sh=sh)
            lo, hi = _f32_order(np.float32(-12.0)), _f32_order(np.float32(12.0))
            if included(cam, g, _f32_from_order(lo), ppx, ppy) or not included(cam, g, _f32_from_order(hi),
                                                                                 ppx, ppy):
                found = None
                break
            while hi - lo > 1:
                mid = (lo + hi) // 2
                if included(cam, g, _f32_from_order(mid), ppx, ppy):
                    hi = mid
                else:
                    lo = mid
            found.append((bx, by, ppx, ppy, mu, _f32_from_order(lo), _f32_from_order(hi)))
        if not found:
            continue
        (bx0, by0, px0, py0, mu0, lo0, hi0), (bx1, by1, px1, py1, mu1, lo1, hi1) = found
        for bx, by, ppx, ppy, mu, lg, side in ((bx0, by0, px0, py0, mu0, hi0, "in"),
                                               (bx1, by1, px1, py1, mu1, lo1, "out")):
            means.append(mu[0])
            scales.append(ls)
            quats.append(q)
            logits.append(lg)
            cases.append((bx, by, feat, side, ppx, ppy))
    n = len(means)
    sc = scenes.Scene(np.array(means, np.float32), np.array(scales, np.float32), np.array(quats, np.float32),
                      np.array(logits, np.float32), np.ones((n, 1, 3), np.float32), sh_degree=0)
    return cam, sc, cases
