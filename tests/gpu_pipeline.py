"""Test-side driver of the GPU library, stage by stage through the C ABI, and
the comparison helpers against the oracle."""
from __future__ import annotations

import numpy as np

from differentiable_gaussian_splatting_amd import binding as B


def to_np(t):
    return t.detach().cpu().numpy()


def run_gpu_view(ctx, w, budget=None, cost=None, loss=None, lam=0.2, keep_bins=True):
    """projection -> (plan) -> per leaf: bin_sort, render_fwd (+ L1 fused or
    SSIM), render_bwd -> project_bwd.  Returns numpy copies of everything."""
    import torch
    cam, dev = w.camera, ctx.device
    loss = loss or w.loss
    ds = B.DeviceScene(w.scene, dev)
    target = torch.from_numpy(w.target).to(dev)
    proj, n_cand = B.gs_project(ctx, cam, ds)
    out = dict(n_cand=n_cand)
    for name, f in (("ids", B.PROJ_IDS), ("rect", B.PROJ_RECT), ("xy", B.PROJ_XY), ("conic", B.PROJ_CONIC),
                    ("depth", B.PROJ_DEPTH), ("radius", B.PROJ_RADIUS), ("opacity", B.PROJ_OPACITY),
                    ("rgb", B.PROJ_RGB), ("flags", B.PROJ_FLAGS), ("slot_of", B.PROJ_SLOT_OF)):
        out[name] = to_np(B.gs_export(ctx, proj, f))
    TW, TH = cam.tiles_x, cam.tiles_y
    if budget is not None:
        leaves = B.gs_plan_leaves(ctx, cam, proj, budget, cost)
    else:
        leaves = [dict(tx0=0, ty0=0, tx1=TW, ty1=TH)]
    out["leaves"] = leaves
    H, W = cam.height, cam.width
    image = torch.zeros((3, H, W), dtype=torch.float32, device=dev)
    grad2d = torch.zeros((max(n_cand, 1), 9), dtype=torch.float32, device=dev)
    loss_acc = torch.zeros(1, dtype=torch.float64, device=dev)
    t_final = np.ones((H, W), np.float32)
    last = np.zeros((H, W), np.int64)
    bins_out = []
    ssim_loss = None
    for L in leaves:
        bins, n_isect = B.gs_bin_sort(ctx, cam, proj, L)
        if keep_bins:
            bins_out.append(dict(n_isect=n_isect, offsets=to_np(B.gs_export(ctx, bins, B.BINS_OFFSETS)),
                                 values=to_np(B.gs_export(ctx, bins, B.BINS_VALUES)),
                                 keys=to_np(B.gs_export(ctx, bins, B.BINS_KEYS))))
        if loss == "l1":
            ras = B.gs_render_fwd(ctx, cam, proj, bins, target, loss_acc, image)
            B.gs_render_bwd(ctx, cam, proj, bins, ras, grad2d)
        else:
            ras = B.gs_render_fwd(ctx, cam, proj, bins, None, None, image)
            dl = torch.empty_like(image)
            ssim_loss, _ = B.gs_loss_ssim(ctx, image, target, dl, lam)
            B.gs_render_bwd(ctx, cam, proj, bins, ras, grad2d, dl_dimage=dl)
        x0, y0 = L["tx0"] * 16, L["ty0"] * 16
        x1, y1 = min(L["tx1"] * 16, W), min(L["ty1"] * 16, H)
        t_final[y0:y1, x0:x1] = to_np(B.gs_export(ctx, ras, B.RASTER_TFINAL)).reshape(y1 - y0, x1 - x0)
        last[y0:y1, x0:x1] = to_np(B.gs_export(ctx, ras, B.RASTER_LAST)).reshape(y1 - y0, x1 - x0)
        B.gs_release(ctx, ras)
        B.gs_release(ctx, bins)
    K = (w.scene.sh_degree + 1) ** 2
    F = 11 + 3 * K
    grad3d = torch.zeros((max(n_cand, 1), F), dtype=torch.float32, device=dev)
    B.gs_project_bwd(ctx, cam, ds, proj, grad2d, grad3d)
    B.gs_release(ctx, proj)
    out.update(image=to_np(image), t_final=t_final, last=last, bins=bins_out,
               grad2d=to_np(grad2d)[:n_cand], grad3d_c=to_np(grad3d)[:n_cand],
               loss=(float(to_np(loss_acc)[0]) / (3.0 * W * H)) if loss == "l1" else ssim_loss)
    dense = np.zeros((w.scene.n, F), np.float32)
    dense[out["ids"].astype(np.int64)] = out["grad3d_c"]
    out["grad3d"] = dense
    return out


def rel_l2(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-12))


GRAD2D_GROUPS = dict(mean2d=slice(0, 2), conic=slice(2, 5), opacity=slice(5, 6), rgb=slice(6, 9))


def grad3d_groups(g, deg):
    K = (deg + 1) ** 2
    return dict(means=g[:, 0:3], log_scales=g[:, 3:6], quats=g[:, 6:10], logits=g[:, 10:11], sh=g[:, 11:11 + 3 * K])


def bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)
