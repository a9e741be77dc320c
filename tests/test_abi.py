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
    # per coarse pair: keys u32 x 2 and slots u32 x 2 (radix ping-pong), the
    # 1024 u32 digit counts of a 10-bit pass per 2048 pairs, and the fine
    # level's 64 u32 positions per work item of up to 512 pairs
    assert c["b_cell"] >= 16 + 1024 * 4 / 2048 + 64 * 4 / 512
    # per intersection: the sorted slot u32
    assert c["b_isect"] >= 4
    # per pixel: T_final f32 + last u32 + packed L1 signs u8
    assert c["b_pixel"] >= 4 + 4 + 1
    # per tile: 4 f64 L1 partials; fine work items (at most one per tile
    # beyond one per 512 pairs) with 64 u32 positions, super-tile id and offsets
    assert c["b_tile"] >= 32 + 64 * 4 + 4 + 12


def test_train_cost_model_is_an_upper_bound_of_the_group_walking_view():
    import oracle
    c = dgs.gs_train_cost_model()
    # an L1 view's leaf holds its coarse sort only (keys and slots ping-pong
    # plus the 10-bit digit counts per 2048 pairs) and its group offsets (a
    # u64 per super-tile, at most one per tile); no per-tile list, no
    # per-pixel state
    assert c["b_cell"] >= 16 + 1024 * 4 / 2048
    assert c["b_tile"] >= 8
    assert c["b_isect"] == 0 and c["b_pixel"] == 0
    assert c == oracle.TRAIN_COST


def test_grid_layout_matches_the_oracle_and_tiles_the_grid():
    """gs_grid_leaves is host-only: its blocks are the oracle's fixed-block
    layout, they tile the grid exactly, and invalid shapes are refused."""
    import numpy as np
    import oracle
    lib = binding.load()
    rng = np.random.default_rng(7)
    for _ in range(200):
        TW, TH = int(rng.integers(1, 400)), int(rng.integers(1, 300))
        nx, ny = int(rng.integers(1, min(TW, 12) + 1)), int(rng.integers(1, min(TH, 12) + 1))
        got = binding.gs_grid_leaves(lib, TW, TH, nx, ny)
        assert [(L["tx0"], L["ty0"], L["tx1"], L["ty1"]) for L in got] == \
            [(L["tx0"], L["ty0"], L["tx1"], L["ty1"]) for L in oracle.grid_leaves(TW, TH, nx, ny)]
        cover = np.zeros((TH, TW), np.int32)
        for L in got:
            assert L["tx0"] < L["tx1"] and L["ty0"] < L["ty1"]
            cover[L["ty0"]:L["ty1"], L["tx0"]:L["tx1"]] += 1
        assert (cover == 1).all()
    for bad in [(10, 10, 0, 1), (10, 10, 11, 1), (10, 10, 1, 11), (0, 10, 1, 1)]:
        try:
            binding.gs_grid_leaves(lib, *bad)
        except binding.GsError as e:
            assert binding.STATUS_NAMES[e.status] == "GS_ERR_INVALID_ARG"
        else:
            raise AssertionError(bad)


def test_gate_decisions_equal_the_oracle_gate():
    """The library's SkipGS gate (host only) against the oracle's gate on
    random view / loss sequences: every decision, forced flag, score, ratio
    and the calibrated floor identical (both compute in double, same order)."""
    import numpy as np
    import oracle
    lib = binding.load()
    rng = np.random.default_rng(11)
    for trial in range(30):
        nv = int(rng.integers(1, 9))
        warm = int(rng.integers(0, 60))
        beta = float(rng.choice([0.95, 0.9, 0.5]))
        g = binding.Gate(nv, warmup=warm, beta=beta, lib=lib)
        o = oracle.SkipGate(nv, warmup=warm, beta=beta)
        loss = 1.0
        for t in range(int(rng.integers(50, 400))):
            v = int(rng.integers(0, nv))
            loss = max(1e-6, loss * float(rng.choice([0.97, 0.99, 1.0, 1.02])) + float(rng.normal(0, 1e-3)))
            a, b = g.step(v, loss), o.step(v, loss)
            assert (a["backward"], a["forced"]) == (b["backward"], b["forced"]), (trial, t)
            assert a["score"] == b["score"] and a["rho_cum"] == b["rho_cum"]
        s = g.stats()
        assert s["backwards"] == o.b and s["steps"] == o.t
        assert (s["rho_min"] is None) == (o.rho_min is None)
        if o.rho_min is not None:
            assert s["rho_min"] == o.rho_min
        g.close()


def test_gate_rejects_bad_arguments():
    lib = binding.load()
    for args in [(0, 10, 0.95, 0.5, 1e-8), (2, -1, 0.95, 0.5, 1e-8), (2, 10, 1.0, 0.5, 1e-8),
                 (2, 10, 0.95, 1.5, 1e-8), (2, 10, 0.95, 0.5, 0.0)]:
        try:
            binding.Gate(*args[:1], warmup=args[1], beta=args[2], rho_lo=args[3], eps=args[4], lib=lib)
        except binding.GsError as e:
            assert binding.STATUS_NAMES[e.status] == "GS_ERR_INVALID_ARG"
        else:
            raise AssertionError(args)
    g = binding.Gate(2, lib=lib)
    for view, loss in [(2, 1.0), (-1, 1.0), (0, float("nan")), (0, float("inf"))]:
        try:
            g.step(view, loss)
        except binding.GsError:
            pass
        else:
            raise AssertionError((view, loss))
    assert g.stats()["steps"] == 0


def test_binding_structs_match_the_header_layout(tmp_path):
    """Every struct the binding passes across the ABI has the header's size
    and field offsets (a C program built with gcc from include/gs.h prints
    them)."""
    import os
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        import pytest
        pytest.skip("gcc not available")
    structs = [binding.gs_camera, binding.gs_params, binding.gs_param_ptrs, binding.gs_tile_rect, binding.gs_leaf,
               binding.gs_cost_model, binding.gs_mem_stats, binding.gs_view_opts, binding.gs_gate_decision,
               binding.gs_gate_stats, binding.gs_view_result]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "gs.h"', "int main(void) {"]
    for st in structs:
        n = st.__name__
        lines.append(f'    printf("{n} %zu\\n", sizeof({n}));')
        for f in st._fields_:
            lines.append(f'    printf("{n}.{f[0]} %zu\\n", offsetof({n}, {f[0]}));')
    lines += ["    return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run(["gcc", "-std=c11", "-I", inc, str(src), "-o", str(exe)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], check=True, capture_output=True,
                                                        text=True).stdout.splitlines())
    for st in structs:
        n = st.__name__
        assert int(got[n]) == ctypes.sizeof(st), n
        for f in st._fields_:
            assert int(got[f"{n}.{f[0]}"]) == getattr(st, f[0]).offset, (n, f[0])
