"""MI355X (gfx950) implementation of one training view of differentiable
tile-based 3D Gaussian splatting with load-budgeted leaf regions (BoundedGS).

The numeric work runs in hand-written HIP kernels behind the C ABI of
``libgsmi.so`` (declared in ``include/gs.h``); ``binding`` is a thin ctypes
layer over it that uses PyTorch only for device memory and streams, and
``scenes`` draws the seeded synthetic inputs.
"""
from . import scenes
from .binding import (Context, DeviceScene, GsError, like_scene, load, gs_project, gs_plan_leaves, gs_bin_sort,
                      gs_render_fwd, gs_render_bwd, gs_project_bwd, gs_loss_ssim, gs_adam_step, gs_release,
                      gs_export, gs_util_exp, gs_train_view, gs_set_timing, gs_set_timing_only, gs_reset_timing,
                      gs_kernel_time, gs_default_cost_model, gs_train_cost_model)

__all__ = ["scenes", "Context", "DeviceScene", "GsError", "like_scene", "load", "gs_project", "gs_plan_leaves",
           "gs_bin_sort", "gs_render_fwd", "gs_render_bwd", "gs_project_bwd", "gs_loss_ssim", "gs_adam_step",
           "gs_release", "gs_export", "gs_util_exp", "gs_train_view", "gs_set_timing", "gs_set_timing_only",
           "gs_reset_timing", "gs_kernel_time", "gs_default_cost_model", "gs_train_cost_model"]
