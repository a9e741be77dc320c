"""The boundary's error contract, through the C ABI (include/gs.h,
"Conventions"): every call returns a status; on error every temporary of the
call is released, outputs are left untouched (gs_train_view: parameters and
Adam moments untouched) and the context stays usable.

* The allocator callback fails on its k-th call, for every k a call makes:
  GS_ERR_OOM, the library's live bytes back to their value before the call,
  no handle returned, and the next call without failures gives the same
  result as on a fresh context.
* Strict planning with a budget below one tile's load: GS_ERR_BUDGET, the
  leaves still written with the over-budget tile flagged (BoundedGS "02 /
  method": regions over the budget are subdivided, down to single tiles).
* Counts beyond the index widths: GS_ERR_OVERFLOW before any device work.
* Invalid arguments and handles: GS_ERR_INVALID_ARG, GS_ERR_STATE.
* Per leaf, the bytes the library held for it stay within the leaf's
  estimate under the default cost model (pipelined, overlapped, serial, host
  target and SSIM views).
"""
import ctypes as C
import sys

import pytest

from differentiable_gaussian_splatting_amd import binding as B
from differentiable_gaussian_splatting_amd import scenes
from tests.gpu_pipeline import rel_l2

pytestmark = pytest.mark.gpu

MIB = 1 << 20


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class FailingContext(B.Context):
    """A context whose allocator (torch's caching allocator) returns NULL on
    its fail_at-th call (0: never) and counts its calls."""

    def __init__(self):
        import torch
        self.torch = torch
        self.lib = B.load()
        self.device = torch.device("cuda", torch.cuda.current_device())
        self.stream = torch.cuda.current_stream(self.device)
        self.calls = 0
        self.fail_at = 0
        dev_index, raw = self.device.index, self.stream.cuda_stream

        def _alloc(user, nbytes, strm):
            self.calls += 1
            if self.calls == self.fail_at:
                return None
            return torch.cuda.caching_allocator_alloc(int(nbytes), dev_index, strm if strm else raw)

        def _free(user, ptr, nbytes, strm):
            torch.cuda.caching_allocator_delete(ptr)

        self._alloc_cb, self._free_cb = B.ALLOC_FN(_alloc), B.FREE_FN(_free)
        h = C.c_void_p()
        self.check(self.lib.gs_ctx_create(C.byref(h), C.c_void_p(raw), self._alloc_cb, self._free_cb, None), ctx=None)
        self.handle = h

    def arm(self, k):
        self.calls = 0
        self.fail_at = k


@pytest.fixture(scope="module")
def fctx():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    c = FailingContext()
    yield c
    c.close()


def expect(status, fn, *a, **kw):
    try:
        fn(*a, **kw)
    except B.GsError as e:
        assert e.status == status, (B.STATUS_NAMES[e.status], str(e))
        return str(e)
    raise AssertionError(f"expected {B.STATUS_NAMES[status]}")


def _workload(name="c3_gmm4k", **kw):
    return scenes.make_workload(name, **kw)


@pytest.mark.parametrize("mode", ["pipelined", "serial", "one_leaf", "ssim", "host_target", "chunked", "wide"])
def test_train_view_allocation_failure_at_every_call(fctx, mode):
    """gs_train_view with the allocator failing at each of its calls in turn:
    GS_ERR_OOM, live bytes back, parameters and moments untouched; then a
    view without failures equals the one before.  "wide": 640 x 480, enough
    tiles (over 1024) that the view's L1 sum runs in chunks, whose buffer
    must be allocated before the update starts."""
    import torch
    wide = mode == "wide"
    w = _workload(n=20000, width=640 if wide else 300, height=480 if wide else 200, seed=151)
    dev = fctx.device
    ds = B.DeviceScene(w.scene, dev)
    m, v = B.like_scene(ds), B.like_scene(ds)
    target = torch.from_numpy(w.target)
    target = target.pin_memory() if mode == "host_target" else target.to(dev)
    kw = dict(budget_bytes=0 if mode == "one_leaf" else 900_000,
              cost=dict(b_isect=20, b_pixel=20, b_tile=64, b_const=1 << 18),
              serial_leaves=mode == "serial", loss="l1_ssim" if mode == "ssim" else "l1")
    adam = dict(step=1, params=ds, m=m, v=v, chunk=500 if mode == "chunked" else 0)
    snap = [t.clone() for t in ds.tensors() + m.tensors() + v.tensors()]

    def run():
        return B.gs_train_view(fctx, w.camera, ds, target, adam=adam, **kw)

    # the calls a view makes (reference run on copies of the state)
    fctx.arm(0)
    live0 = fctx.mem_stats()["live"]
    ref = run()
    n_calls = fctx.calls
    assert fctx.mem_stats()["live"] == live0
    ref_state = [t.clone() for t in ds.tensors() + m.tensors() + v.tensors()]
    for t, s in zip(ds.tensors() + m.tensors() + v.tensors(), snap):
        t.copy_(s)
    say(f"mode {mode}: {ref['n_leaves']} leaves, {n_calls} allocations per view")
    assert ref["n_leaves"] >= (1 if mode == "one_leaf" else 3) and n_calls > 5
    for k in range(1, n_calls + 1):
        fctx.arm(k)
        msg = expect(B.GS_ERR_OOM, run)
        assert fctx.calls >= k, (k, fctx.calls)
        assert fctx.mem_stats()["live"] == live0, (k, msg)
        torch.cuda.synchronize()
        for t, s in zip(ds.tensors() + m.tensors() + v.tensors(), snap):
            assert torch.equal(t, s), (k, msg)
    fctx.arm(0)
    again = run()
    assert again["loss"] == ref["loss"] and again["n_isect"] == ref["n_isect"]
    for t, s in zip(ds.tensors() + m.tensors() + v.tensors(), ref_state):
        assert rel_l2(t.cpu().numpy(), s.cpu().numpy()) <= 1e-6


def test_stage_calls_allocation_failure_at_every_call(fctx):
    """gs_project, gs_plan_leaves, gs_bin_sort (planned leaf and a leaf
    outside the plan), gs_render_fwd and gs_loss_ssim with the allocator
    failing at each of their calls: GS_ERR_OOM, no handle, live bytes back."""
    import torch
    w = _workload(n=15000, width=280, height=190, seed=152)
    cam, dev = w.camera, fctx.device
    ds = B.DeviceScene(w.scene, dev)
    target = torch.from_numpy(w.target).to(dev)
    cost = dict(b_isect=20, b_pixel=20, b_tile=64, b_const=1 << 18)

    def sweep(name, fn, cleanup):
        # reference calls count the allocations (the first also makes what
        # a projection caches on first use); then each failing call must
        # leave the live bytes as they were before it
        fctx.arm(0)
        cleanup(fn())
        fctx.arm(0)
        cleanup(fn())       # the steady state: nothing left to cache
        n = fctx.calls
        for k in range(1, n + 1):
            live0 = fctx.mem_stats()["live"]
            fctx.arm(k)
            expect(B.GS_ERR_OOM, fn)
            assert fctx.mem_stats()["live"] == live0, (name, k)
        fctx.arm(0)
        say(f"  {name}: {n} allocations, each failure clean")

    sweep("gs_project", lambda: B.gs_project(fctx, cam, ds), lambda o: B.gs_release(fctx, o[0]))
    fctx.arm(0)
    proj, n_cand = B.gs_project(fctx, cam, ds)
    # a successful plan stays attached to the projection; a failed one
    # leaves the projection's bytes as they were
    sweep("gs_plan_leaves", lambda: B.gs_plan_leaves(fctx, cam, proj, 900_000, cost), lambda o: None)
    fctx.arm(0)
    leaves = B.gs_plan_leaves(fctx, cam, proj, 900_000, cost)
    assert len(leaves) > 2
    outside = dict(tx0=1, ty0=1, tx1=cam.tiles_x - 1, ty1=cam.tiles_y - 2)
    for L in (leaves[1], outside):
        sweep(f"gs_bin_sort {L['tx0'], L['ty0'], L['tx1'], L['ty1']}", lambda: B.gs_bin_sort(fctx, cam, proj, L),
              lambda o: B.gs_release(fctx, o[0]))
    fctx.arm(0)
    bins, _ = B.gs_bin_sort(fctx, cam, proj, leaves[1])
    acc = torch.zeros(1, dtype=torch.float64, device=dev)
    sweep("gs_render_fwd", lambda: B.gs_render_fwd(fctx, cam, proj, bins, target, acc),
          lambda o: B.gs_release(fctx, o))
    B.gs_release(fctx, bins)
    B.gs_release(fctx, proj)
    img = torch.rand((3, 60, 70), device=dev)
    dl = torch.empty_like(img)
    sweep("gs_loss_ssim", lambda: B.gs_loss_ssim(fctx, img, target[:, :60, :70].contiguous(), dl),
          lambda o: None)


def test_strict_budget(fctx):
    """A budget below one tile's estimate: the planner still writes every
    leaf (single tiles over the budget flagged) and returns GS_ERR_BUDGET in
    strict mode; gs_train_view in strict mode stops with GS_ERR_BUDGET and
    leaves the parameters untouched."""
    import torch
    w = _workload(n=20000, width=160, height=96, seed=153)
    cam, dev = w.camera, fctx.device
    ds = B.DeviceScene(w.scene, dev)
    fctx.arm(0)
    proj, _ = B.gs_project(fctx, cam, ds)
    cost = dict(b_isect=20, b_pixel=20, b_tile=64, b_const=1 << 18)
    budget = 100_000   # below b_const alone: every tile is over it
    leaves = B.gs_plan_leaves(fctx, cam, proj, budget, cost)   # not strict: OK, tiles flagged
    assert len(leaves) == cam.tiles_x * cam.tiles_y and all(L["over_budget"] for L in leaves)
    arr = (B.gs_leaf * 4096)()
    n = C.c_int32()
    cs = B.cost_struct(cost)
    st = fctx.lib.gs_plan_leaves(fctx.handle, C.byref(B.camera_struct(cam)), proj, budget, C.byref(cs), 1,
                                 C.cast(arr, C.c_void_p), 4096, C.byref(n))
    assert st == B.GS_ERR_BUDGET and n.value == len(leaves)
    assert [(a.tx0, a.ty0, a.tx1, a.ty1, a.over_budget) for a in arr[:n.value]] == \
        [(L["tx0"], L["ty0"], L["tx1"], L["ty1"], 1) for L in leaves]
    assert "budget" in fctx.lib.gs_last_error(fctx.handle).decode()
    # a budget that fits every tile but not the whole view: no flag, strict OK
    ok = B.gs_plan_leaves(fctx, cam, proj, 700_000, cost, strict=True)
    assert len(ok) > 1 and not any(L["over_budget"] for L in ok)
    B.gs_release(fctx, proj)
    m, v = B.like_scene(ds), B.like_scene(ds)
    snap = [t.clone() for t in ds.tensors()]
    live0 = fctx.mem_stats()["live"]
    expect(B.GS_ERR_BUDGET, B.gs_train_view, fctx, cam, ds, torch.from_numpy(w.target).to(dev),
           budget_bytes=budget, cost=cost, strict=True, adam=dict(step=1, params=ds, m=m, v=v))
    assert fctx.mem_stats()["live"] == live0
    for t, s in zip(ds.tensors(), snap):
        assert torch.equal(t, s)


def test_overflow_and_invalid_arguments(fctx):
    """GS_ERR_OVERFLOW for N >= 2^31 Gaussians and for a tile grid of 2^31
    tiles or more (checked before any device work: the parameter pointers
    are never read); GS_ERR_INVALID_ARG and GS_ERR_STATE for bad arguments
    and handles."""
    import torch
    lib, dev = fctx.lib, fctx.device
    w = _workload("c1_small", n=100, width=64, height=48)
    ds = B.DeviceScene(w.scene, dev)
    live0 = fctx.mem_stats()["live"]
    big = ds.struct()
    big.n = 1 << 31
    h, n = C.c_void_p(), C.c_int64()
    cam = B.camera_struct(w.camera)
    assert lib.gs_project(fctx.handle, C.byref(cam), C.byref(big), C.byref(h), C.byref(n)) == B.GS_ERR_OVERFLOW
    assert not h.value
    o, res = B.gs_view_opts(), B.gs_view_result()
    tgt = torch.zeros((3, 48, 64), device=dev)
    assert lib.gs_train_view(fctx.handle, C.byref(cam), C.byref(big), C.c_void_p(tgt.data_ptr()), C.byref(o),
                             C.byref(res)) == B.GS_ERR_OVERFLOW
    huge = B.camera_struct(w.camera)
    huge.width, huge.height = 1 << 20, 1 << 20   # (2^16)^2 = 2^32 tiles
    assert lib.gs_project(fctx.handle, C.byref(huge), C.byref(ds.struct()), C.byref(h), C.byref(n)) == \
        B.GS_ERR_OVERFLOW
    bad = ds.struct()
    bad.sh_degree = 4
    assert lib.gs_project(fctx.handle, C.byref(cam), C.byref(bad), C.byref(h), C.byref(n)) == B.GS_ERR_INVALID_ARG
    neg = ds.struct()
    neg.n = -1
    assert lib.gs_project(fctx.handle, C.byref(cam), C.byref(neg), C.byref(h), C.byref(n)) == B.GS_ERR_INVALID_ARG
    zero = B.camera_struct(w.camera)
    zero.width = 0
    assert lib.gs_project(fctx.handle, C.byref(zero), C.byref(ds.struct()), C.byref(h), C.byref(n)) == \
        B.GS_ERR_INVALID_ARG
    assert fctx.mem_stats()["live"] == live0
    fctx.arm(0)
    proj, _ = B.gs_project(fctx, w.camera, ds)
    expect(B.GS_ERR_INVALID_ARG, B.gs_bin_sort, fctx, w.camera, proj, dict(tx0=0, ty0=0, tx1=99, ty1=1))
    expect(B.GS_ERR_INVALID_ARG, B.gs_bin_sort, fctx, w.camera, proj, dict(tx0=2, ty0=0, tx1=2, ty1=1))
    expect(B.GS_ERR_INVALID_ARG, B.gs_plan_leaves, fctx, w.camera, proj, 0)
    other = B.Context()
    expect(B.GS_ERR_STATE, B.gs_bin_sort, other, w.camera, proj, dict(tx0=0, ty0=0, tx1=1, ty1=1))
    other.close()
    moved = scenes.pinhole_camera(80, 48)
    expect(B.GS_ERR_STATE, B.gs_plan_leaves, fctx, moved, proj, 1 << 20)
    B.gs_release(fctx, proj)
    assert fctx.mem_stats()["live"] == live0


@pytest.mark.parametrize("mode", ["overlapped", "serial", "host_target", "ssim"])
def test_leaf_bytes_within_estimate(fctx, mode):
    """Under the library's default cost model, the bytes the library holds
    for each planned leaf (its binning buffers, slot array, target slice,
    SSIM buffers) stay within the leaf's estimate."""
    import torch
    w = _workload(n=150000, width=1400, height=900, seed=154)
    dev = fctx.device
    ds = B.DeviceScene(w.scene, dev)
    target = torch.from_numpy(w.target)
    target = target.pin_memory() if mode == "host_target" else target.to(dev)
    fctx.arm(0)
    # a budget that splits this view into several leaves under each mode's
    # default model (L1: the group-walking one, SSIM: the per-tile one)
    budget = 5 * MIB if mode == "ssim" else 3 * MIB
    r = B.gs_train_view(fctx, w.camera, ds, target, budget_bytes=budget, max_leaves=4096,
                        serial_leaves=mode == "serial", loss="l1_ssim" if mode == "ssim" else "l1")
    held = [L["bytes"] for L in r["leaves"]]
    est = [L["est_bytes"] for L in r["leaves"]]
    say(f"mode {mode}: {len(held)} leaves, largest held {max(held) / MIB:.2f} MiB, largest estimate "
        f"{max(est) / MIB:.2f} MiB, max held/estimate {max(h / e for h, e in zip(held, est)):.3f}")
    assert len(held) > 3 and min(held) > 0
    assert all(h <= e for h, e in zip(held, est))
