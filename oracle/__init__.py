"""CPU oracle for one training view of the BoundedGS-style tile rasterizer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check
(``__graft_entry__.smoke``) and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the GPU library; the only common piece
is the seeded input generator module (which holds none of the method's
arithmetic).

The arithmetic lives in plain C (``gso.c``, ``gso_real.inc``); this module
marshals numpy arrays and chains the stages the way the pages describe one
view (BoundedGS page, "01" and "02 / method", Fig. 3):

    projection -> [leaf planning] -> for each leaf: binning, forward,
    loss, raster backward (2D gradients summed over leaves) ->
    one projection backward -> [one Adam step]

Decisions (candidates, rectangles, keys, included pairs, stops, L1 signs) are
taken in f32 (``mode="parity"``), losses and gradients are computed in f64.
``mode="reference"`` runs every step in f64 (for finite differences).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build
from .skipgate import SkipGate, decide as gate_decide, rho_min_of  # noqa: F401

_lib = None


class Camera_c(C.Structure):
    _fields_ = [("R", C.c_float * 9), ("t", C.c_float * 3), ("fx", C.c_float), ("fy", C.c_float),
                ("cx", C.c_float), ("cy", C.c_float), ("near_z", C.c_float), ("bg", C.c_float * 3),
                ("width", C.c_int32), ("height", C.c_int32)]


class Rect_c(C.Structure):
    _fields_ = [("tx0", C.c_int32), ("ty0", C.c_int32), ("tx1", C.c_int32), ("ty1", C.c_int32)]


class Leaf_c(C.Structure):
    _fields_ = [("tx0", C.c_int32), ("ty0", C.c_int32), ("tx1", C.c_int32), ("ty1", C.c_int32),
                ("est_bytes", C.c_uint64), ("over_budget", C.c_int32), ("pad", C.c_int32)]


class Cost_c(C.Structure):
    _fields_ = [("b_isect", C.c_uint64), ("b_pixel", C.c_uint64), ("b_tile", C.c_uint64),
                ("b_const", C.c_uint64), ("b_cell", C.c_uint64)]


FLAG_CLAMP_R, FLAG_CLAMP_G, FLAG_CLAMP_B, FLAG_CLAMP_UX, FLAG_CLAMP_UY = 1, 2, 4, 8, 16


def lib():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        _lib = C.CDLL(path)
        _declare(_lib)
    return _lib


def _p(a):
    return a.ctypes.data_as(C.c_void_p) if a is not None else None


def _declare(L):
    vp, i64, i32, u64, dbl = C.c_void_p, C.c_int64, C.c_int32, C.c_uint64, C.c_double
    L.gso_exp_cw.restype = C.c_float
    L.gso_exp_cw.argtypes = [C.c_float]
    L.gso_exp_cw_array.argtypes = [vp, vp, i64]
    L.gso_exp_falloff_array.argtypes = [vp, vp, i64]
    L.gso_sh_basis_f32.argtypes = [C.c_int, vp, vp, i64]
    L.gso_sh_basis_f64.argtypes = [C.c_int, vp, vp, i64]
    proj = [C.POINTER(Camera_c), i64, C.c_int] + [vp] * 5 + [vp] * 9
    L.gso_project_f32.argtypes = proj
    L.gso_project_f64.argtypes = proj
    L.gso_bin.restype = i64
    L.gso_bin.argtypes = [i32, Rect_c, i64, vp, vp, vp, vp, vp, vp, vp, i64]
    fwd = [C.POINTER(Camera_c), Rect_c, vp, vp, vp, vp, vp, vp, vp, vp, vp, C.POINTER(i64)]
    L.gso_render_fwd_f32.argtypes = fwd
    L.gso_render_fwd_f64.argtypes = fwd
    L.gso_loss_l1.restype = dbl
    L.gso_loss_l1.argtypes = [i32, i32, Rect_c, vp, vp, vp]
    L.gso_loss_ssim.restype = dbl
    L.gso_loss_ssim.argtypes = [i32, i32, vp, vp, dbl, vp, C.POINTER(dbl)]
    L.gso_render_bwd_f32dec.argtypes = [C.POINTER(Camera_c), Rect_c, vp, vp, vp, vp, vp, vp, vp, vp,
                                        vp, vp, vp, C.POINTER(i64), C.POINTER(u64)]
    L.gso_render_bwd_f64dec.argtypes = [C.POINTER(Camera_c), Rect_c, vp, vp, vp, vp, vp, vp, vp, vp,
                                        C.POINTER(i64), C.POINTER(u64)]
    L.gso_project_bwd.argtypes = [C.POINTER(Camera_c), i64, C.c_int] + [vp] * 5 + [vp] * 5
    L.gso_plan_leaves.restype = i32
    L.gso_plan_leaves.argtypes = [i32, i32, i64, vp, u64, C.POINTER(Cost_c), vp, i32, vp]
    L.gso_replan_leaves.restype = i32
    L.gso_replan_leaves.argtypes = [i32, i32, i64, vp, u64, C.POINTER(Cost_c), vp, i32, vp, i32, vp]
    L.gso_leaf_estimate.restype = u64
    L.gso_leaf_estimate.argtypes = [i32, i32, Rect_c, u64, u64, C.POINTER(Cost_c)]
    L.gso_adam.argtypes = [i64, vp, vp, vp, vp, i32, dbl, dbl, dbl, dbl]


# --------------------------------------------------------------------------- helpers

def camera_struct(cam) -> Camera_c:
    c = Camera_c()
    R = np.asarray(cam.R, dtype=np.float32).reshape(9)
    for k in range(9):
        c.R[k] = float(R[k])
    for k in range(3):
        c.t[k] = float(np.float32(cam.t[k]))
        c.bg[k] = float(cam.bg[k])
    c.fx, c.fy, c.cx, c.cy = cam.fx, cam.fy, cam.cx, cam.cy
    c.near_z = cam.near_z
    c.width, c.height = cam.width, cam.height
    return c


def rect(tx0, ty0, tx1, ty1) -> Rect_c:
    return Rect_c(int(tx0), int(ty0), int(tx1), int(ty1))


def full_rect(cam) -> Rect_c:
    return rect(0, 0, (cam.width + 15) // 16, (cam.height + 15) // 16)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def exp_cw(x):
    x = _c(x, np.float32)
    y = np.empty_like(x)
    lib().gso_exp_cw_array(_p(x), _p(y), x.size)
    return y


def exp_falloff(x):
    """exp of the Gaussian falloff as the f32 compositing pass takes it."""
    x = _c(x, np.float32)
    y = np.empty_like(x)
    lib().gso_exp_falloff_array(_p(x), _p(y), x.size)
    return y


def sh_basis(deg, dirs, dtype=np.float64):
    dirs = _c(dirs, dtype)
    n = dirs.shape[0]
    Y = np.empty((n, (deg + 1) ** 2), dtype=dtype)
    fn = lib().gso_sh_basis_f32 if dtype == np.float32 else lib().gso_sh_basis_f64
    fn(deg, _p(dirs), _p(Y), n)
    return Y


def project(cam, scene, precision="f32"):
    """Dense per-Gaussian projection outputs (index = Gaussian id)."""
    dt = np.float32 if precision == "f32" else np.float64
    n = scene.n
    arrs = [_c(a, dt) for a in scene.arrays()]
    out = dict(cand=np.zeros(n, np.uint8), rect=np.zeros((n, 4), np.int32),
               xy=np.zeros((n, 2), dt), conic=np.zeros((n, 3), dt), depth=np.zeros(n, dt),
               radius=np.zeros(n, dt), opacity=np.zeros(n, dt), rgb=np.zeros((n, 3), dt),
               flags=np.zeros(n, np.uint32))
    fn = lib().gso_project_f32 if dt == np.float32 else lib().gso_project_f64
    cs = camera_struct(cam)
    fn(C.byref(cs), n, scene.sh_degree, *[_p(a) for a in arrs],
       _p(out["cand"]), _p(out["rect"]), _p(out["xy"]), _p(out["conic"]), _p(out["depth"]),
       _p(out["radius"]), _p(out["opacity"]), _p(out["rgb"]), _p(out["flags"]))
    out["cand"] = out["cand"].astype(bool)
    return out


def bin_leaf(tiles_x, leaf: Rect_c, rect_c, depth_c, with_keys=True):
    """Binning over one tile rectangle; rect_c/depth_c are compact by slot."""
    rect_c = _c(rect_c, np.int32)
    depth64 = _c(depth_c, np.float64)
    bits = depth_c.astype(np.float32).view(np.uint32) if (with_keys and depth_c.dtype == np.float32) else None
    bits = _c(bits, np.uint32) if bits is not None else None
    TL = (leaf.tx1 - leaf.tx0) * (leaf.ty1 - leaf.ty0)
    counts = np.zeros(TL, np.uint32)
    offsets = np.zeros(TL + 1, np.uint64)
    n_c = rect_c.shape[0]
    total = lib().gso_bin(tiles_x, leaf, n_c, _p(rect_c), _p(depth64), _p(bits), _p(counts),
                          _p(offsets), None, None, 0)
    values = np.zeros(max(total, 1), np.uint32)
    keys = np.zeros(max(total, 1), np.uint64) if bits is not None else None
    lib().gso_bin(tiles_x, leaf, n_c, _p(rect_c), _p(depth64), _p(bits), _p(counts), _p(offsets),
                  _p(values), _p(keys), total)
    return dict(n_isect=int(total), counts=counts, offsets=offsets, values=values[:total],
                keys=keys[:total] if keys is not None else None, leaf=leaf)


def render_fwd(cam, leaf, bins, xy, conic, opacity, rgb, image=None, t_final=None, last=None):
    dt = xy.dtype
    W, H = cam.width, cam.height
    if image is None:
        image = np.zeros((3, H, W), dt)
        t_final = np.ones((H, W), dt)
        last = np.zeros((H, W), np.int32)
    q = C.c_int64(0)
    fn = lib().gso_render_fwd_f32 if dt == np.float32 else lib().gso_render_fwd_f64
    xy, conic, opacity, rgb = (_c(a, dt) for a in (xy, conic, opacity, rgb))
    vals = bins["values"] if bins["n_isect"] else np.zeros(1, np.uint32)
    fn(C.byref(camera_struct(cam)), leaf, _p(bins["offsets"]), _p(vals), _p(xy), _p(conic),
       _p(opacity), _p(rgb), _p(image), _p(t_final), _p(last), C.byref(q))
    return image, t_final, last, int(q.value)


def loss_l1(cam, leaf, image64, target, dloss):
    return float(lib().gso_loss_l1(cam.width, cam.height, leaf, _p(_c(image64, np.float64)),
                                   _p(_c(target, np.float32)), _p(dloss)))


def loss_ssim(cam, image64, target, lam=0.2):
    dloss = np.zeros((3, cam.height, cam.width), np.float64)
    ssim = C.c_double(0)
    L = lib().gso_loss_ssim(cam.width, cam.height, _p(_c(image64, np.float64)),
                            _p(_c(target, np.float32)), lam, _p(dloss), C.byref(ssim))
    return float(L), dloss, float(ssim.value)


def render_bwd(cam, leaf, bins, dec_state, val_state, dloss, grad2d, signature=None):
    """dec_state: (xy, conic, opacity) in f32 (parity) or None (decisions in f64
    from val_state).  val_state: (xy, conic, opacity, rgb) f64, compact."""
    qb = C.c_uint64(0) if False else C.c_int64(0)
    sig = C.c_uint64(signature if signature is not None else 1469598103934665603)
    vals = bins["values"] if bins["n_isect"] else np.zeros(1, np.uint32)
    xy, conic, op, rgb = (_c(a, np.float64) for a in val_state)
    cs = camera_struct(cam)
    if dec_state is not None:
        x32, c32, o32 = (_c(a, np.float32) for a in dec_state)
        lib().gso_render_bwd_f32dec(C.byref(cs), leaf, _p(bins["offsets"]), _p(vals), _p(x32), _p(c32),
                                    _p(o32), _p(xy), _p(conic), _p(op), _p(rgb), _p(dloss), _p(grad2d),
                                    C.byref(qb), C.byref(sig))
    else:
        lib().gso_render_bwd_f64dec(C.byref(cs), leaf, _p(bins["offsets"]), _p(vals), _p(xy), _p(conic),
                                    _p(op), _p(rgb), _p(dloss), _p(grad2d), C.byref(qb), C.byref(sig))
    return int(qb.value), int(sig.value)


def project_bwd(cam, scene, cand, flags, slot_of, grad2d):
    n = scene.n
    K = (scene.sh_degree + 1) ** 2
    F = 11 + 3 * K
    arrs = [_c(a, np.float64) for a in scene.arrays()]
    grad3d = np.zeros((n, F), np.float64)
    lib().gso_project_bwd(C.byref(camera_struct(cam)), n, scene.sh_degree, *[_p(a) for a in arrs],
                          _p(_c(cand, np.uint8)), _p(_c(flags, np.uint32)), _p(_c(slot_of, np.int64)),
                          _p(_c(grad2d, np.float64)), _p(grad3d))
    return grad3d


DEFAULT_COST = dict(b_isect=4, b_cell=19, b_pixel=9, b_tile=320, b_const=1 << 20)
# the load model of a leaf whose L1 raster walks its super-tile groups (no
# per-tile lists, no per-pixel state): coarse sort per pair, group offsets
# per tile
TRAIN_COST = dict(b_isect=0, b_cell=19, b_pixel=0, b_tile=8, b_const=1 << 20)


def walks_groups(rect_c):
    """Whether an L1 view's rasters walk the super-tile groups: when the
    candidates' intersections I are at least 0.18 of 64 times their
    (candidate, super-cell) pairs Cb (the super-cells of 8 x 8 tiles, aligned
    to the image, that each rectangle meets)."""
    r = np.asarray(rect_c, np.int64).reshape(-1, 4)
    I = int(((r[:, 2] - r[:, 0]) * (r[:, 3] - r[:, 1])).sum())
    Cb = int(((((r[:, 2] - 1) >> 3) - (r[:, 0] >> 3) + 1) * (((r[:, 3] - 1) >> 3) - (r[:, 1] >> 3) + 1)).sum())
    return 100 * I >= 1152 * Cb


def cost_struct(cost=None) -> Cost_c:
    """A cost given without b_cell has no super-cell term."""
    c = dict(DEFAULT_COST) if cost is None else dict(dict(b_cell=0), **cost)
    return Cost_c(c["b_isect"], c["b_pixel"], c["b_tile"], c["b_const"], c["b_cell"])


def plan_leaves(cam, rect_c, budget, cost=None, with_sat=False, roots=None):
    """Leaf plan of the candidates' tile rectangles; with roots (cached leaves,
    dicts with tx0..ty1) the re-check of that layout instead of a fresh plan."""
    W, H = cam.width, cam.height
    TW, TH = (W + 15) // 16, (H + 15) // 16
    rect_c = _c(rect_c, np.int32)
    cs = cost_struct(cost)
    sat = np.zeros((TH + 1, TW + 1), np.uint64) if with_sat else None
    if roots is None:
        rr, nr = None, 0
    else:
        rr = (Rect_c * max(len(roots), 1))(*[Rect_c(r["tx0"], r["ty0"], r["tx1"], r["ty1"]) for r in roots])
        rr, nr = C.cast(rr, C.c_void_p), len(roots)
    n = lib().gso_replan_leaves(W, H, rect_c.shape[0], _p(rect_c), int(budget), C.byref(cs), rr, nr, None, 0, None)
    out = (Leaf_c * max(n, 1))()
    lib().gso_replan_leaves(W, H, rect_c.shape[0], _p(rect_c), int(budget), C.byref(cs), rr, nr,
                            C.cast(out, C.c_void_p), n, _p(sat))
    leaves = [dict(tx0=o.tx0, ty0=o.ty0, tx1=o.tx1, ty1=o.ty1, est_bytes=int(o.est_bytes),
                   over_budget=bool(o.over_budget)) for o in out[:n]]
    return (leaves, sat) if with_sat else leaves


def grid_leaves(TW, TH, nx, ny):
    """The fixed-block layout: nx x ny blocks of the tile grid, row by row;
    block (i, j) covers tiles [i TW // nx, (i + 1) TW // nx) x [j TH // ny,
    (j + 1) TH // ny) (BoundedGS "03 / results", Fig. 5 and 6)."""
    return [dict(tx0=i * TW // nx, ty0=j * TH // ny, tx1=(i + 1) * TW // nx, ty1=(j + 1) * TH // ny)
            for j in range(ny) for i in range(nx)]


def leaf_estimate(cam, r: Rect_c, n_isect, cost=None, n_cells=0):
    cs = cost_struct(cost)
    return int(lib().gso_leaf_estimate(cam.width, cam.height, r, int(n_isect), int(n_cells), C.byref(cs)))


def adam(grad, param, m, v, step, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-15):
    grad, param, m, v = (_c(a, np.float64).copy() for a in (grad, param, m, v))
    lib().gso_adam(grad.size, _p(grad), _p(param), _p(m), _p(v), int(step), lr, beta1, beta2, eps)
    return param, m, v


# --------------------------------------------------------------------------- a whole view

def _compact(d, ids):
    return {k: (v[ids] if isinstance(v, np.ndarray) and v.shape[:1] == d["cand"].shape else v)
            for k, v in d.items()}


def train_view(cam, scene, target, loss="l1", budget=None, leaves=None, mode="parity",
               cost=None, keep_bins=False, lam=0.2):
    """One view: projection, (planned or given) leaves, per-leaf binning /
    forward / loss / raster backward with 2D gradients summed over leaves,
    then one projection backward.

    Returns a dict with loss (f64), image, grad2d (compact, f64), grad3d
    (dense [N,F], f64), candidate ids, per-leaf bins and statistics.
    """
    W, H = cam.width, cam.height
    TW = (W + 15) // 16
    p32 = project(cam, scene, "f32")
    p64 = project(cam, scene, "f64")
    dec = p32 if mode == "parity" else p64
    ids = np.nonzero(dec["cand"])[0]
    slot_of = np.full(scene.n, -1, np.int64)
    slot_of[ids] = np.arange(ids.size)
    c32 = _compact(p32, ids)
    c64 = _compact(p64, ids)
    cdec = c32 if mode == "parity" else c64
    if leaves is None:
        if budget is not None:
            if cost is None and loss == "l1":
                cost = TRAIN_COST if walks_groups(cdec["rect"]) else DEFAULT_COST
            leaves = plan_leaves(cam, cdec["rect"], budget, cost)
        else:
            leaves = [dict(tx0=0, ty0=0, tx1=TW, ty1=(H + 15) // 16, est_bytes=0, over_budget=False)]
    if loss == "l1_ssim" and len(leaves) != 1:
        raise ValueError("the SSIM loss is defined on the full image (one leaf)")

    dt = np.float32 if mode == "parity" else np.float64
    image = np.zeros((3, H, W), dt)
    t_final = np.ones((H, W), dt)
    last = np.zeros((H, W), np.int32)
    grad2d = np.zeros((ids.size, 9), np.float64)
    dloss = np.zeros((3, H, W), np.float64)
    total_loss = 0.0
    q_f = q_b = n_isect = 0
    sig = 1469598103934665603
    all_bins = []
    ssim = None
    for lf in leaves:
        r = rect(lf["tx0"], lf["ty0"], lf["tx1"], lf["ty1"])
        bins = bin_leaf(TW, r, cdec["rect"], cdec["depth"], with_keys=(mode == "parity"))
        n_isect += bins["n_isect"]
        _, _, _, q = render_fwd(cam, r, bins, cdec["xy"], cdec["conic"], cdec["opacity"], cdec["rgb"],
                                image, t_final, last)
        q_f += q
        if loss == "l1":
            total_loss += loss_l1(cam, r, image.astype(np.float64), target, dloss)
        else:
            total_loss, dloss, ssim = loss_ssim(cam, image.astype(np.float64), target, lam)
        dec_state = (c32["xy"], c32["conic"], c32["opacity"]) if mode == "parity" else None
        qb, sig = render_bwd(cam, r, bins, dec_state,
                             (c64["xy"], c64["conic"], c64["opacity"], c64["rgb"]), dloss, grad2d, sig)
        q_b += qb
        if keep_bins:
            all_bins.append(bins)
    grad3d = project_bwd(cam, scene, dec["cand"], dec["flags"], slot_of, grad2d)
    return dict(loss=total_loss, image=image, t_final=t_final, last=last, grad2d=grad2d,
                grad3d=grad3d, ids=ids, slot_of=slot_of, leaves=leaves, bins=all_bins,
                n_cand=int(ids.size), n_isect=int(n_isect), q_f=int(q_f), q_b=int(q_b),
                signature=int(sig), proj32=p32, proj64=p64, ssim=ssim, dloss=dloss)


def split_grad3d(grad3d, sh_degree):
    """Split a [N,F] gradient into the parameter groups."""
    K = (sh_degree + 1) ** 2
    return dict(means=grad3d[:, 0:3], log_scales=grad3d[:, 3:6], quats=grad3d[:, 6:10],
                logits=grad3d[:, 10], sh=grad3d[:, 11:].reshape(-1, K, 3))
