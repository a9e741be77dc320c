"""The C-ABI library loads and exports every function include/gs.h declares,
and the binding carries the same names.  No compute calls (no GPU needed)."""
import ctypes

import differentiable_gaussian_splatting_amd as dgs
from differentiable_gaussian_splatting_amd import binding


def test_library_exports_every_declared_symbol():
    names = binding.header_functions()
    assert "gs_render_bwd" in names and "gs_plan_leaves" in names
    lib = ctypes.CDLL(binding.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_the_six_calls_and_binding_names():
    six = ["gs_project", "gs_bin_sort", "gs_render_fwd", "gs_render_bwd", "gs_project_bwd", "gs_plan_leaves"]
    names = binding.header_functions()
    for n in six:
        assert n in names
        assert hasattr(dgs, n)
    binding.load()   # argtypes for every declared function are set without error


def test_default_cost_model_is_an_upper_bound_of_allocations():
    c = dgs.gs_default_cost_model()   # a pure host function: no device needed
    # per coarse pair: keys u32 x 2 and slots u32 x 2 (radix ping-pong) + 256
    # u32 histogram bins and their scan per 2048 pairs
    assert c["b_cell"] >= 16 + 2 * 256 * 4 / 2048
    # per intersection: the sorted slot u32
    assert c["b_isect"] >= 4
    # per pixel: T_final f32 + last u32 + packed L1 signs u8
    assert c["b_pixel"] >= 4 + 4 + 1
    # per tile: 4 f64 L1 partials; fine work items (at most one per tile
    # beyond one per 512 pairs) with 64 u32 positions, super-tile id and offsets
    assert c["b_tile"] >= 32 + 64 * 4 + 4 + 12
