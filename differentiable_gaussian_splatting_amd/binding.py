"""Thin ctypes binding of libgsmi (the C ABI declared in include/gs.h).

Argument marshalling only: every numeric step runs in the library's HIP
kernels.  PyTorch provides device memory (its caching allocator is handed to
the library as the allocator callback, so torch's memory statistics see the
library's working set) and the stream.  The functions keep the C names.

The library is loaded from the package directory (built in-tree by
``differentiable_gaussian_splatting_amd._build``); there is no fallback: if
it is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes as C
import os
import re
import traceback

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgsmi.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "gs.h")

GS_OK, GS_ERR_INVALID_ARG, GS_ERR_OOM, GS_ERR_DEVICE, GS_ERR_OVERFLOW, GS_ERR_BUDGET, GS_ERR_STATE = range(7)
STATUS_NAMES = ["GS_OK", "GS_ERR_INVALID_ARG", "GS_ERR_OOM", "GS_ERR_DEVICE", "GS_ERR_OVERFLOW", "GS_ERR_BUDGET",
                "GS_ERR_STATE"]
MEM_CATS = ["proj", "raster", "grad", "loss", "scratch"]

# export fields
PROJ_IDS, PROJ_RECT, PROJ_XY, PROJ_CONIC, PROJ_DEPTH, PROJ_RADIUS, PROJ_OPACITY, PROJ_RGB, PROJ_FLAGS, PROJ_SLOT_OF = \
    range(10)
BINS_OFFSETS, BINS_VALUES, BINS_KEYS = 20, 21, 22
RASTER_TFINAL, RASTER_LAST = 30, 31


class GsError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES[status] if 0 <= status < 7 else status}: {msg}")
        self.status = status


class gs_camera(C.Structure):
    _fields_ = [("R", C.c_float * 9), ("t", C.c_float * 3), ("fx", C.c_float), ("fy", C.c_float),
                ("cx", C.c_float), ("cy", C.c_float), ("near_z", C.c_float), ("bg", C.c_float * 3),
                ("width", C.c_int32), ("height", C.c_int32)]


class gs_params(C.Structure):
    _fields_ = [("n", C.c_int64), ("sh_degree", C.c_int32), ("pad", C.c_int32), ("means", C.c_void_p),
                ("log_scales", C.c_void_p), ("quats", C.c_void_p), ("opacity_logits", C.c_void_p),
                ("sh", C.c_void_p)]


class gs_param_ptrs(C.Structure):
    _fields_ = [("means", C.c_void_p), ("log_scales", C.c_void_p), ("quats", C.c_void_p),
                ("opacity_logits", C.c_void_p), ("sh", C.c_void_p)]


class gs_tile_rect(C.Structure):
    _fields_ = [("tx0", C.c_int32), ("ty0", C.c_int32), ("tx1", C.c_int32), ("ty1", C.c_int32)]


class gs_leaf(C.Structure):
    _fields_ = [("tx0", C.c_int32), ("ty0", C.c_int32), ("tx1", C.c_int32), ("ty1", C.c_int32),
                ("est_bytes", C.c_uint64), ("over_budget", C.c_int32), ("pad", C.c_int32)]


class gs_cost_model(C.Structure):
    _fields_ = [("b_isect", C.c_uint64), ("b_pixel", C.c_uint64), ("b_tile", C.c_uint64), ("b_const", C.c_uint64),
                ("b_cell", C.c_uint64)]


def cost_struct(cost):
    """gs_cost_model from a dict; a cost given without b_cell has no super-cell term."""
    return gs_cost_model(cost["b_isect"], cost["b_pixel"], cost["b_tile"], cost["b_const"], cost.get("b_cell", 0))


class gs_mem_stats(C.Structure):
    _fields_ = [("live_bytes", C.c_uint64), ("peak_bytes", C.c_uint64), ("live_by_cat", C.c_uint64 * 5),
                ("peak_by_cat", C.c_uint64 * 5), ("n_alloc", C.c_uint64), ("n_free", C.c_uint64)]


class gs_view_opts(C.Structure):
    _fields_ = [("budget_bytes", C.c_uint64), ("loss_kind", C.c_int32), ("ssim_lambda", C.c_float),
                ("adam_step", C.c_int32), ("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float),
                ("eps", C.c_float), ("strict_budget", C.c_int32), ("max_leaves", C.c_int32),
                ("leaves_out", C.c_void_p), ("cost", C.c_void_p), ("image_out", C.c_void_p),
                ("grad3d_out", C.c_void_p), ("params_rw", C.c_void_p), ("adam_m", C.c_void_p),
                ("adam_v", C.c_void_p), ("adam_chunk", C.c_int64), ("leaves_in", C.c_void_p),
                ("n_leaves_in", C.c_int32), ("leaves_in_partial", C.c_int32), ("gate", C.c_void_p),
                ("gate_view", C.c_int32), ("serial_leaves", C.c_int32), ("target_host", C.c_int32),
                ("leaf_bytes_out", C.c_void_p), ("loss_out", C.c_void_p)]


class gs_gate_decision(C.Structure):
    _fields_ = [("backward", C.c_int32), ("forced", C.c_int32), ("score", C.c_double), ("rho_cum", C.c_double)]


class gs_gate_stats(C.Structure):
    _fields_ = [("steps", C.c_int64), ("backwards", C.c_int64), ("warmup_counted", C.c_int64),
                ("warmup_proposed", C.c_int64), ("calibrated", C.c_int32), ("pad", C.c_int32),
                ("rho_min", C.c_double)]


class gs_view_result(C.Structure):
    _fields_ = [("loss", C.c_double), ("n_cand", C.c_int64), ("n_isect", C.c_int64), ("n_leaves", C.c_int32),
                ("groups_walked", C.c_int32), ("peak_bytes", C.c_uint64), ("gate_backward", C.c_int32),
                ("gate_forced", C.c_int32), ("gate_score", C.c_double)]


ALLOC_FN = C.CFUNCTYPE(C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p)
FREE_FN = C.CFUNCTYPE(None, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p)

_lib = None


def header_functions():
    """Names of the functions declared in include/gs.h."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gs_[a-z0-9_]+)\s*\(", src)) - {"gs_alloc_fn", "gs_free_fn"})


def load(path: str = LIB_PATH):
    """Load libgsmi.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with differentiable_gaussian_splatting_amd._build.build()")
    L = C.CDLL(path)
    vp, i32, i64, u64, st = C.c_void_p, C.c_int32, C.c_int64, C.c_uint64, C.c_int
    P = C.POINTER
    sig = {
        "gs_ctx_create": (st, [P(vp), vp, ALLOC_FN, FREE_FN, vp]),
        "gs_ctx_destroy": (None, [vp]),
        "gs_last_error": (C.c_char_p, [vp]),
        "gs_mem_stats_get": (st, [vp, P(gs_mem_stats)]),
        "gs_mem_reset_peak": (st, [vp]),
        "gs_set_timing": (st, [vp, i32]),
        "gs_kernel_time": (st, [vp, C.c_char_p, P(C.c_double), P(i64)]),
        "gs_reset_timing": (st, [vp]),
        "gs_set_timing_only": (st, [vp, C.c_char_p]),
        "gs_default_cost_model": (gs_cost_model, []),
        "gs_train_cost_model": (gs_cost_model, []),
        "gs_project": (st, [vp, P(gs_camera), P(gs_params), P(vp), P(i64)]),
        "gs_plan_leaves": (st, [vp, P(gs_camera), vp, u64, vp, i32, vp, i32, P(i32)]),
        "gs_replan_leaves": (st, [vp, P(gs_camera), vp, u64, vp, i32, vp, i32, vp, i32, P(i32)]),
        "gs_grid_leaves": (st, [i32, i32, i32, i32, vp]),
        "gs_gate_create": (st, [i32, i32, C.c_double, C.c_double, C.c_double, P(vp)]),
        "gs_gate_destroy": (None, [vp]),
        "gs_gate_step": (st, [vp, i32, C.c_double, P(gs_gate_decision)]),
        "gs_gate_get_stats": (st, [vp, P(gs_gate_stats)]),
        "gs_bin_sort": (st, [vp, P(gs_camera), vp, gs_tile_rect, P(vp), P(i64)]),
        "gs_render_fwd": (st, [vp, P(gs_camera), vp, vp, vp, vp, vp, vp, P(vp)]),
        "gs_render_bwd": (st, [vp, P(gs_camera), vp, vp, vp, vp, vp]),
        "gs_project_bwd": (st, [vp, P(gs_camera), P(gs_params), vp, vp, vp]),
        "gs_loss_ssim": (st, [vp, i32, i32, vp, vp, C.c_float, vp, P(C.c_double), P(C.c_double)]),
        "gs_loss_ssim_static": (st, [vp, i32, i32, vp, vp, C.c_float, vp, P(C.c_double), P(C.c_double)]),
        "gs_adam_step": (st, [vp, vp, i64, i32, P(gs_param_ptrs), P(gs_param_ptrs), P(gs_param_ptrs), vp, i32,
                              C.c_float, C.c_float, C.c_float, C.c_float]),
        "gs_release": (None, [vp, vp]),
        "gs_export": (st, [vp, vp, i32, vp, C.c_size_t]),
        "gs_export_size": (st, [vp, vp, i32, P(C.c_size_t)]),
        "gs_util_exp": (st, [vp, vp, vp, i64]),
        "gs_util_exp_falloff": (st, [vp, vp, vp, i64]),
        "gs_train_view": (st, [vp, P(gs_camera), P(gs_params), vp, P(gs_view_opts), P(gs_view_result)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


# ---------------------------------------------------------------------------- context

TORCH_ALLOC_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgsmi_torchalloc.so")
_talloc = None


def _torch_alloc_lib():
    """The C allocator callbacks over torch's HIP caching allocator
    (libgsmi_torchalloc.so, built with libgsmi.so), or None if not built."""
    global _talloc
    if _talloc is None and os.path.exists(TORCH_ALLOC_LIB):
        import torch  # noqa: F401  (loads libc10_hip, which the callbacks call)
        _talloc = C.CDLL(TORCH_ALLOC_LIB)
    return _talloc


class Context:
    """A library context on the current torch device and stream, allocating
    through torch's caching allocator: by C callbacks into it when
    libgsmi_torchalloc.so is built, else (or with torch_allocator="python")
    by Python callbacks; torch_allocator=False: the library's own
    hipMallocAsync."""

    def __init__(self, device=None, stream=None, torch_allocator=True):
        import torch
        self.torch = torch
        self.lib = load()
        self.device = torch.device("cuda", torch.cuda.current_device() if device is None else device)
        self.stream = torch.cuda.current_stream(self.device) if stream is None else stream
        self._sizes = {}
        dev_index = self.device.index
        raw_stream = self.stream.cuda_stream

        def _alloc(user, nbytes, strm):
            try:
                # stream-ordered on the stream the library allocates for
                return torch.cuda.caching_allocator_alloc(int(nbytes), dev_index, strm if strm else raw_stream)
            except Exception:   # the library turns NULL into GS_ERR_OOM
                traceback.print_exc()
                return None

        def _free(user, ptr, nbytes, strm):
            try:
                torch.cuda.caching_allocator_delete(ptr)
            except Exception:
                traceback.print_exc()

        shim = _torch_alloc_lib() if torch_allocator is True else None
        if shim is not None:
            self._alloc_cb = ALLOC_FN(("gs_torch_alloc", shim))
            self._free_cb = FREE_FN(("gs_torch_free", shim))
        elif torch_allocator:
            self._alloc_cb, self._free_cb = ALLOC_FN(_alloc), FREE_FN(_free)
        else:
            self._alloc_cb, self._free_cb = C.cast(None, ALLOC_FN), C.cast(None, FREE_FN)
        h = C.c_void_p()
        self.check(self.lib.gs_ctx_create(C.byref(h), C.c_void_p(raw_stream), self._alloc_cb, self._free_cb, None),
                   ctx=None)
        self.handle = h

    def check(self, status, ctx="self"):
        if status != GS_OK:
            msg = self.lib.gs_last_error(self.handle).decode() if ctx == "self" else ""
            raise GsError(status, msg)

    def close(self):
        if getattr(self, "handle", None):
            self.lib.gs_ctx_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reset_peak(self):
        """Restart the high-water marks (all and per category) at the live bytes."""
        self.check(self.lib.gs_mem_reset_peak(self.handle))

    def mem_stats(self):
        s = gs_mem_stats()
        self.check(self.lib.gs_mem_stats_get(self.handle, C.byref(s)))
        return dict(live=s.live_bytes, peak=s.peak_bytes, n_alloc=s.n_alloc, n_free=s.n_free,
                    live_by_cat={k: s.live_by_cat[i] for i, k in enumerate(MEM_CATS)},
                    peak_by_cat={k: s.peak_by_cat[i] for i, k in enumerate(MEM_CATS)})


def camera_struct(cam) -> gs_camera:
    c = gs_camera()
    R = np.asarray(cam.R, dtype=np.float32).reshape(9)
    for k in range(9):
        c.R[k] = float(R[k])
    for k in range(3):
        c.t[k] = float(np.float32(cam.t[k]))
        c.bg[k] = float(cam.bg[k])
    c.fx, c.fy, c.cx, c.cy, c.near_z = cam.fx, cam.fy, cam.cx, cam.cy, cam.near_z
    c.width, c.height = cam.width, cam.height
    return c


class DeviceScene:
    """Gaussian parameters as contiguous float32 device tensors."""

    def __init__(self, scene, device="cuda"):
        import torch
        f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
        self.means, self.log_scales, self.quats = f(scene.means), f(scene.log_scales), f(scene.quats)
        self.logits, self.sh = f(scene.logits), f(scene.sh)
        self.sh_degree = int(scene.sh_degree)
        self.n = int(scene.n)

    def tensors(self):
        return [self.means, self.log_scales, self.quats, self.logits, self.sh]

    def struct(self) -> gs_params:
        return gs_params(self.n, self.sh_degree, 0, self.means.data_ptr(), self.log_scales.data_ptr(),
                         self.quats.data_ptr(), self.logits.data_ptr(), self.sh.data_ptr())

    def ptrs(self) -> gs_param_ptrs:
        return gs_param_ptrs(*[t.data_ptr() for t in self.tensors()])


def like_scene(ds: DeviceScene) -> DeviceScene:
    """A zero-filled DeviceScene of the same shapes (Adam moments)."""
    import torch
    z = DeviceScene.__new__(DeviceScene)
    z.means, z.log_scales, z.quats, z.logits, z.sh = (torch.zeros_like(t) for t in ds.tensors())
    z.sh_degree, z.n = ds.sh_degree, ds.n
    return z


# ---------------------------------------------------------------------------- the calls

def gs_project(ctx: Context, cam, params: DeviceScene):
    h = C.c_void_p()
    n = C.c_int64()
    ctx.check(ctx.lib.gs_project(ctx.handle, C.byref(camera_struct(cam)), C.byref(params.struct()), C.byref(h),
                                 C.byref(n)))
    return h, int(n.value)


def gs_plan_leaves(ctx: Context, cam, proj, budget_bytes: int, cost=None, strict=False, max_leaves=4096):
    cs = None
    if cost is not None:
        cs = cost_struct(cost)
    n = C.c_int32()
    while True:
        arr = (gs_leaf * max_leaves)()
        ctx.check(ctx.lib.gs_plan_leaves(ctx.handle, C.byref(camera_struct(cam)), proj, int(budget_bytes),
                                         C.byref(cs) if cs is not None else None, int(strict),
                                         C.cast(arr, C.c_void_p), max_leaves, C.byref(n)))
        if n.value <= max_leaves:
            break
        max_leaves = n.value
    return [dict(tx0=a.tx0, ty0=a.ty0, tx1=a.tx1, ty1=a.ty1, est_bytes=int(a.est_bytes),
                 over_budget=bool(a.over_budget)) for a in arr[:n.value]]


def _leaf_array(leaves):
    arr = (gs_leaf * max(len(leaves), 1))()
    for k, L in enumerate(leaves):
        arr[k].tx0, arr[k].ty0, arr[k].tx1, arr[k].ty1 = L["tx0"], L["ty0"], L["tx1"], L["ty1"]
    return arr


def gs_replan_leaves(ctx: Context, cam, proj, budget_bytes: int, cached, cost=None, strict=False, max_leaves=4096):
    cs = cost_struct(cost) if cost is not None else None
    src = _leaf_array(cached)
    n = C.c_int32()
    while True:
        arr = (gs_leaf * max_leaves)()
        ctx.check(ctx.lib.gs_replan_leaves(ctx.handle, C.byref(camera_struct(cam)), proj, int(budget_bytes),
                                           C.byref(cs) if cs is not None else None, int(strict),
                                           C.cast(src, C.c_void_p), len(cached), C.cast(arr, C.c_void_p),
                                           max_leaves, C.byref(n)))
        if n.value <= max_leaves:
            break
        max_leaves = n.value
    return [dict(tx0=a.tx0, ty0=a.ty0, tx1=a.tx1, ty1=a.ty1, est_bytes=int(a.est_bytes),
                 over_budget=bool(a.over_budget)) for a in arr[:n.value]]


def gs_grid_leaves(lib, tiles_x: int, tiles_y: int, nx: int, ny: int):
    """Fixed nx x ny block layout of the tile grid (host only; lib = the loaded library)."""
    arr = (gs_leaf * max(nx * ny, 1))()
    stv = lib.gs_grid_leaves(int(tiles_x), int(tiles_y), int(nx), int(ny), C.cast(arr, C.c_void_p))
    if stv != GS_OK:
        raise GsError(stv, "gs_grid_leaves")
    return [dict(tx0=a.tx0, ty0=a.ty0, tx1=a.tx1, ty1=a.ty1, est_bytes=0, over_budget=False)
            for a in arr[:nx * ny]]


class Gate:
    """The library's SkipGS backward gate (host only; see gs_gate_* in include/gs.h)."""

    def __init__(self, n_views, warmup=500, beta=0.95, rho_lo=0.5, eps=1e-8, lib=None):
        self.lib = lib or load()
        self.handle = C.c_void_p()
        stv = self.lib.gs_gate_create(int(n_views), int(warmup), float(beta), float(rho_lo), float(eps),
                                      C.byref(self.handle))
        if stv != GS_OK:
            raise GsError(stv, "gs_gate_create")

    def step(self, view, loss):
        d = gs_gate_decision()
        stv = self.lib.gs_gate_step(self.handle, int(view), float(loss), C.byref(d))
        if stv != GS_OK:
            raise GsError(stv, "gs_gate_step")
        return dict(backward=bool(d.backward), forced=bool(d.forced), score=d.score, rho_cum=d.rho_cum)

    def stats(self):
        s = gs_gate_stats()
        stv = self.lib.gs_gate_get_stats(self.handle, C.byref(s))
        if stv != GS_OK:
            raise GsError(stv, "gs_gate_get_stats")
        return dict(steps=s.steps, backwards=s.backwards, warmup_counted=s.warmup_counted,
                    warmup_proposed=s.warmup_proposed, calibrated=bool(s.calibrated),
                    rho_min=s.rho_min if s.calibrated else None)

    def close(self):
        if self.handle:
            self.lib.gs_gate_destroy(self.handle)
            self.handle = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gs_bin_sort(ctx: Context, cam, proj, leaf):
    h = C.c_void_p()
    n = C.c_int64()
    r = gs_tile_rect(leaf["tx0"], leaf["ty0"], leaf["tx1"], leaf["ty1"]) if isinstance(leaf, dict) else \
        gs_tile_rect(*leaf)
    ctx.check(ctx.lib.gs_bin_sort(ctx.handle, C.byref(camera_struct(cam)), proj, r, C.byref(h), C.byref(n)))
    return h, int(n.value)


def gs_render_fwd(ctx: Context, cam, proj, bins, target=None, loss_accum=None, image_out=None, stats=None):
    """stats: optional int64 device tensor [4] accumulating (pairs examined,
    pairs included, sum of last, pairs the backward revisits)."""
    h = C.c_void_p()
    ctx.check(ctx.lib.gs_render_fwd(ctx.handle, C.byref(camera_struct(cam)), proj, bins, _ptr(target),
                                    _ptr(loss_accum), _ptr(image_out), _ptr(stats), C.byref(h)))
    return h


def gs_render_bwd(ctx: Context, cam, proj, bins, raster, grad2d, dl_dimage=None):
    ctx.check(ctx.lib.gs_render_bwd(ctx.handle, C.byref(camera_struct(cam)), proj, bins, raster, _ptr(dl_dimage),
                                    _ptr(grad2d)))


def gs_project_bwd(ctx: Context, cam, params: DeviceScene, proj, grad2d, grad3d):
    ctx.check(ctx.lib.gs_project_bwd(ctx.handle, C.byref(camera_struct(cam)), C.byref(params.struct()), proj,
                                     _ptr(grad2d), _ptr(grad3d)))


def gs_loss_ssim(ctx: Context, image, target, dl_dimage, lam=0.2):
    loss, ssim = C.c_double(), C.c_double()
    H, W = int(image.shape[1]), int(image.shape[2])
    ctx.check(ctx.lib.gs_loss_ssim(ctx.handle, W, H, _ptr(image), _ptr(target), float(lam), _ptr(dl_dimage),
                                   C.byref(loss), C.byref(ssim)))
    return float(loss.value), float(ssim.value)


def gs_loss_ssim_static(ctx: Context, image, target, dl_dimage, lam=0.2, sums=True):
    """gs_loss_ssim with the library's static work buffers (allocates
    nothing); sums=False: the gradient only, asynchronous."""
    loss, ssim = C.c_double(), C.c_double()
    H, W = int(image.shape[1]), int(image.shape[2])
    ctx.check(ctx.lib.gs_loss_ssim_static(ctx.handle, W, H, _ptr(image), _ptr(target), float(lam), _ptr(dl_dimage),
                                          C.byref(loss) if sums else None, C.byref(ssim) if sums else None))
    return (float(loss.value), float(ssim.value)) if sums else None


def gs_adam_step(ctx: Context, proj, params: DeviceScene, m: DeviceScene, v: DeviceScene, grad3d, step,
                 lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-15):
    ctx.check(ctx.lib.gs_adam_step(ctx.handle, proj, params.n, params.sh_degree, C.byref(params.ptrs()),
                                   C.byref(m.ptrs()), C.byref(v.ptrs()), _ptr(grad3d), int(step), float(lr),
                                   float(beta1), float(beta2), float(eps)))


def gs_release(ctx: Context, handle):
    if handle is not None and handle.value:
        ctx.lib.gs_release(ctx.handle, handle)


_EXPORT_DTYPES = {PROJ_IDS: ("int32", 1), PROJ_RECT: ("int32", 4), PROJ_XY: ("float32", 2),
                  PROJ_CONIC: ("float32", 3), PROJ_DEPTH: ("float32", 1), PROJ_RADIUS: ("float32", 1),
                  PROJ_OPACITY: ("float32", 1), PROJ_RGB: ("float32", 3), PROJ_FLAGS: ("int32", 1),
                  PROJ_SLOT_OF: ("int32", 1), BINS_OFFSETS: ("int64", 1), BINS_VALUES: ("int32", 1),
                  BINS_KEYS: ("int64", 1), RASTER_TFINAL: ("float32", 1), RASTER_LAST: ("int32", 1)}


def gs_export(ctx: Context, handle, field: int):
    """Copy a handle's field into a new device tensor (unsigned fields are
    returned in the signed torch dtype of the same width; reinterpret on the
    host)."""
    import torch
    nbytes = C.c_size_t()
    ctx.check(ctx.lib.gs_export_size(ctx.handle, handle, field, C.byref(nbytes)))
    dt, width = _EXPORT_DTYPES[field]
    tdt = getattr(torch, dt)
    esz = torch.tensor([], dtype=tdt).element_size()
    n = nbytes.value // (esz * width)
    out = torch.empty((n, width) if width > 1 else (n,), dtype=tdt, device=ctx.device)
    if n:
        ctx.check(ctx.lib.gs_export(ctx.handle, handle, field, _ptr(out), nbytes.value))
    return out


def gs_util_exp(ctx: Context, x):
    y = x.new_empty(x.shape)
    ctx.check(ctx.lib.gs_util_exp(ctx.handle, _ptr(x), _ptr(y), x.numel()))
    return y


def gs_util_exp_falloff(ctx: Context, x):
    y = x.new_empty(x.shape)
    ctx.check(ctx.lib.gs_util_exp_falloff(ctx.handle, _ptr(x), _ptr(y), x.numel()))
    return y


def gs_set_timing(ctx: Context, on: bool):
    ctx.check(ctx.lib.gs_set_timing(ctx.handle, int(on)))


def gs_set_timing_only(ctx: Context, name):
    ctx.check(ctx.lib.gs_set_timing_only(ctx.handle, None if name is None else name.encode()))


def gs_reset_timing(ctx: Context):
    ctx.check(ctx.lib.gs_reset_timing(ctx.handle))


def gs_kernel_time(ctx: Context, name: str):
    ms, n = C.c_double(), C.c_int64()
    ctx.check(ctx.lib.gs_kernel_time(ctx.handle, name.encode(), C.byref(ms), C.byref(n)))
    return float(ms.value), int(n.value)


def gs_default_cost_model():
    c = load().gs_default_cost_model()
    return dict(b_isect=c.b_isect, b_pixel=c.b_pixel, b_tile=c.b_tile, b_const=c.b_const, b_cell=c.b_cell)


def gs_train_cost_model():
    c = load().gs_train_cost_model()
    return dict(b_isect=c.b_isect, b_pixel=c.b_pixel, b_tile=c.b_tile, b_const=c.b_const, b_cell=c.b_cell)


def gs_train_view(ctx: Context, cam, params: DeviceScene, target, budget_bytes=0, loss="l1", lam=0.2,
                  adam=None, image_out=None, grad3d_out=None, strict=False, cost=None, max_leaves=0,
                  leaves_in=None, partial=False, gate=None, gate_view=0, serial_leaves=False, loss_out=None):
    """One whole view in the library (see gs_train_view in include/gs.h).
    adam: None or dict(step, params=DeviceScene (updated), m, v, lr, beta1, beta2, eps, chunk).
    leaves_in: a cached layout (list of leaf dicts) to re-check instead of planning afresh.
    max_leaves > 0: the view's leaves are returned, each with its est_bytes and the high-water
    mark of the bytes the library held for it ("bytes").
    target: a device tensor, or a CPU tensor (pinned for the copies to overlap), which the
    library copies leaf by leaf.
    loss_out: a device float64 tensor (one element used): the loss is written there and not read
    back (the call does not wait for the view's end); the returned "loss" is then None."""
    o = gs_view_opts()
    o.serial_leaves = int(bool(serial_leaves))
    o.target_host = int(not target.is_cuda)
    if not target.is_cuda and not target.is_contiguous():
        raise ValueError("a host target must be contiguous [3][H][W] float32")
    src = _leaf_array(leaves_in) if leaves_in else None
    if leaves_in:
        o.leaves_in = C.cast(src, C.c_void_p)
        o.n_leaves_in = len(leaves_in)
        o.leaves_in_partial = int(bool(partial))
    if gate is not None:
        o.gate = gate.handle
        o.gate_view = int(gate_view)
    o.budget_bytes = int(budget_bytes)
    o.loss_kind = 0 if loss == "l1" else 1
    o.ssim_lambda = float(lam)
    leaves_arr = (gs_leaf * max(max_leaves, 1))()
    leaf_bytes = (C.c_uint64 * max(max_leaves, 1))()
    o.max_leaves = int(max_leaves)
    o.leaves_out = C.cast(leaves_arr, C.c_void_p) if max_leaves else None
    o.leaf_bytes_out = C.cast(leaf_bytes, C.c_void_p) if max_leaves else None
    cs = cost_struct(cost) if cost else None
    o.cost = C.cast(C.pointer(cs), C.c_void_p) if cs is not None else None
    o.image_out = image_out.data_ptr() if image_out is not None else None
    o.grad3d_out = grad3d_out.data_ptr() if grad3d_out is not None else None
    if loss_out is not None:
        import torch
        if not loss_out.is_cuda or loss_out.dtype != torch.float64 or loss_out.numel() < 1:
            raise ValueError("loss_out must be a device float64 tensor")
        o.loss_out = loss_out.data_ptr()
    o.strict_budget = int(strict)
    keep = []
    if adam is not None:
        o.adam_step = int(adam["step"])
        o.lr, o.beta1, o.beta2, o.eps = (float(adam.get(k, d)) for k, d in
                                         (("lr", 1e-3), ("beta1", 0.9), ("beta2", 0.999), ("eps", 1e-15)))
        o.adam_chunk = int(adam.get("chunk", 0))
        pr, pm, pv = adam["params"].ptrs(), adam["m"].ptrs(), adam["v"].ptrs()
        keep += [pr, pm, pv]
        o.params_rw, o.adam_m, o.adam_v = (C.cast(C.pointer(x), C.c_void_p) for x in (pr, pm, pv))
    res = gs_view_result()
    ctx.check(ctx.lib.gs_train_view(ctx.handle, C.byref(camera_struct(cam)), C.byref(params.struct()),
                                    _ptr(target), C.byref(o), C.byref(res)))
    out = dict(loss=None if loss_out is not None else res.loss, n_cand=res.n_cand, n_isect=res.n_isect,
               n_leaves=res.n_leaves,
               peak_bytes=res.peak_bytes, groups_walked=bool(res.groups_walked))
    if gate is not None:
        out.update(backward=bool(res.gate_backward), forced=bool(res.gate_forced), score=res.gate_score)
    if max_leaves:
        nl = min(res.n_leaves, max_leaves)
        out["leaves"] = [dict(tx0=a.tx0, ty0=a.ty0, tx1=a.tx1, ty1=a.ty1, est_bytes=int(a.est_bytes),
                              over_budget=bool(a.over_budget), bytes=int(leaf_bytes[i]))
                         for i, a in enumerate(leaves_arr[:nl])]
    del keep
    return out
