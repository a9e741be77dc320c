"""Oracle-side helpers for the full-size GPU parity tests: the workload and
its oracle projection (one workload cached at a time), sampled tiles, and
regions of the view rendered forward and backward by the oracle.

At the full sizes (up to 16000 x 10560 pixels and 12M Gaussians) the oracle
cannot render whole views in a test's time, so it follows the GPU where it
can, on the host's threads (the oracle's C routines run outside the GIL; each
thread works on its own outputs):
  - every Gaussian's projection (bands of Gaussians over the threads);
  - sampled tiles, each binned and rendered alone;
  - square regions of tiles, split into blocks rendered forward, L1 and
    backward over the threads.  The 2D gradient of a candidate whose tile
    rectangle lies inside a region is complete once the region's blocks are
    summed (every pixel that includes it is inside), so its gradient rows
    (2D, and 3D by the oracle's projection backward) can be compared with
    the GPU's, whatever the size of its rectangle and however many leaves it
    crosses.
Binning a tile or block visits only the candidates whose rectangle meets it;
their relative order (ascending slot) is kept, so the sorted lists are the
oracle's lists over all candidates, mapped back to global slots.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

import oracle
from differentiable_gaussian_splatting_amd import scenes

_CACHE: dict = {}


def threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _warm_oracle():
    # the oracle's exp routines set up their constant tables on first use:
    # take that first use on this thread, before any worker thread runs
    oracle.exp_cw(np.zeros(1, np.float32))
    oracle.exp_falloff(np.zeros(1, np.float32))


def project_bands(cam, sc, precision):
    """oracle.project over bands of Gaussians on the host's threads."""
    _warm_oracle()
    nt = threads()
    e = np.linspace(0, sc.n, nt + 1).astype(np.int64)
    bands = [(int(a), int(b)) for a, b in zip(e[:-1], e[1:]) if b > a]
    if not bands:
        return oracle.project(cam, sc, precision)

    def run(ab):
        return oracle.project(cam, scenes.Scene(*(x[ab[0]:ab[1]] for x in sc.arrays()), sh_degree=sc.sh_degree),
                              precision)

    with cf.ThreadPoolExecutor(nt) as ex:
        parts = list(ex.map(run, bands))
    return {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}


def count_grid(rect_c, TW, TH):
    """Candidates per tile by a 2D difference array over the rectangles."""
    r = rect_c.astype(np.int64)
    S = (TH + 1) * (TW + 1)
    d = np.zeros(S, np.int64)
    for (yi, xi), sgn in (((1, 0), 1), ((1, 2), -1), ((3, 0), -1), ((3, 2), 1)):
        d += sgn * np.bincount(r[:, yi] * (TW + 1) + r[:, xi], minlength=S)
    return d.reshape(TH + 1, TW + 1).cumsum(0).cumsum(1)[:TH, :TW]


class OracleView:
    """A workload, its oracle projection in f32 (decisions) and f64 (values),
    compact by candidate slot, and the per-tile candidate counts."""

    def __init__(self, name):
        self.name = name
        self.w = w = scenes.make_workload(name)
        cam, sc = w.camera, w.scene
        self.cam, self.sc = cam, sc
        self.W, self.H, self.TW, self.TH = cam.width, cam.height, cam.tiles_x, cam.tiles_y
        self.p32 = project_bands(cam, sc, "f32")
        p64 = project_bands(cam, sc, "f64")
        self.ids = np.nonzero(self.p32["cand"])[0]
        self.slot_of = np.full(sc.n, -1, np.int64)
        self.slot_of[self.ids] = np.arange(self.ids.size)
        self.rect_c = self.p32["rect"][self.ids]
        self.depth_c = self.p32["depth"][self.ids]
        self.c32 = {k: self.p32[k][self.ids] for k in ("xy", "conic", "opacity", "rgb")}
        self.c64 = {k: p64[k][self.ids] for k in ("xy", "conic", "opacity", "rgb")}
        del p64
        self.counts = count_grid(self.rect_c, self.TW, self.TH)
        self._bufs = None

    def buffers(self):
        """Full-size oracle image / T_final / last / f64 image / dL/dout,
        written only where tiles or regions are rendered."""
        if self._bufs is None:
            H, W = self.H, self.W
            self._bufs = dict(img=np.zeros((3, H, W), np.float32), tf=np.ones((H, W), np.float32),
                              last=np.zeros((H, W), np.int32), img64=np.zeros((3, H, W), np.float64),
                              dl=np.zeros((3, H, W), np.float64))
        return self._bufs

    def release_buffers(self):
        self._bufs = None

    def meeting(self, r):
        rc = self.rect_c
        return np.nonzero((rc[:, 0] < r.tx1) & (rc[:, 2] > r.tx0) & (rc[:, 1] < r.ty1) & (rc[:, 3] > r.ty0))[0]

    def pix(self, r):
        return (slice(r.ty0 * 16, min(r.ty1 * 16, self.H)), slice(r.tx0 * 16, min(r.tx1 * 16, self.W)))

    def render_block(self, r, sub, backward):
        """Bin, forward (and L1 + raster backward) of tile rectangle r over the
        candidates sub (ascending slots, a superset of those meeting r).
        Returns (the sorted list of each tile in global slots, concatenated,
        its offsets, the block's 2D gradient rows in sub's order or None)."""
        b = self.buffers()
        ob = oracle.bin_leaf(self.TW, r, self.rect_c[sub], self.depth_c[sub], with_keys=False)
        c = {k: v[sub] for k, v in self.c32.items()}
        oracle.render_fwd(self.cam, r, ob, c["xy"], c["conic"], c["opacity"], c["rgb"], b["img"], b["tf"],
                          b["last"])
        part = None
        if backward:
            ys, xs = self.pix(r)
            b["img64"][:, ys, xs] = b["img"][:, ys, xs]
            oracle.loss_l1(self.cam, r, b["img64"], self.w.target, b["dl"])
            part = np.zeros((sub.size, 9), np.float64)
            c64 = {k: v[sub] for k, v in self.c64.items()}
            oracle.render_bwd(self.cam, r, ob, (c["xy"], c["conic"], c["opacity"]),
                              (c64["xy"], c64["conic"], c64["opacity"], c64["rgb"]), b["dl"], part)
        return sub[ob["values"]], ob["offsets"].astype(np.int64), part

    def render_tiles(self, tiles):
        """Each sampled tile binned and rendered alone: its list (global
        slots), image, T_final and walk ends, keyed by tile id."""
        _warm_oracle()
        self.buffers()

        def one(t):
            tx, ty = t % self.TW, t // self.TW
            r = oracle.rect(tx, ty, tx + 1, ty + 1)
            vals, _, _ = self.render_block(r, self.meeting(r), False)
            return t, vals

        with cf.ThreadPoolExecutor(threads()) as ex:
            return dict(ex.map(one, tiles))

    def render_region(self, region, block=8):
        """Forward, L1 and backward of a tile rectangle, in blocks of block x
        block tiles over the threads.  Returns (inside: the slots of the
        candidates whose rectangle lies inside the region, g2: their summed 2D
        gradient rows [inside.size][9] f64)."""
        _warm_oracle()
        self.buffers()
        sub = self.meeting(region)
        blocks = [oracle.rect(x, y, min(x + block, region.tx1), min(y + block, region.ty1))
                  for y in range(region.ty0, region.ty1, block) for x in range(region.tx0, region.tx1, block)]

        def one(r):
            s = sub[np.nonzero((self.rect_c[sub, 0] < r.tx1) & (self.rect_c[sub, 2] > r.tx0) &
                               (self.rect_c[sub, 1] < r.ty1) & (self.rect_c[sub, 3] > r.ty0))[0]]
            _, _, part = self.render_block(r, s, True)
            return s, part

        acc = np.zeros((sub.size, 9), np.float64)
        pos = np.full(self.ids.size, -1, np.int64)
        pos[sub] = np.arange(sub.size)
        with cf.ThreadPoolExecutor(threads()) as ex:
            for s, part in ex.map(one, blocks):
                acc[pos[s]] += part      # s holds distinct slots
        rc = self.rect_c[sub]
        ins = (rc[:, 0] >= region.tx0) & (rc[:, 2] <= region.tx1) & (rc[:, 1] >= region.ty0) & (rc[:, 3] <= region.ty1)
        return sub[ins], acc[ins]

    def project_bwd_rows(self, slots, g2):
        """The oracle's 3D gradient rows [slots.size][F] (f64) of candidates
        `slots` from their complete 2D gradient rows g2."""
        gid = self.ids[slots]
        sc = self.sc
        part = scenes.Scene(*(a[gid] for a in sc.arrays()), sh_degree=sc.sh_degree)
        return oracle.project_bwd(self.cam, part, np.ones(gid.size, np.uint8), self.p32["flags"][gid],
                                  np.arange(gid.size, dtype=np.int64), g2)


def oracle_view(name) -> OracleView:
    """The cached OracleView of a workload (the previous one is dropped)."""
    if name not in _CACHE:
        _CACHE.clear()
        _CACHE[name] = OracleView(name)
    return _CACHE[name]


def sample_tiles(counts, rng, n_heavy=6, n_random=10):
    """The heaviest tiles, random ones and the last row / column corners."""
    TH, TW = counts.shape
    flat = counts.ravel()
    heavy = np.argsort(flat, kind="stable")[-n_heavy:]
    rand = rng.choice(flat.size, size=min(n_random, flat.size), replace=False)
    corner = np.array([(TH - 1) * TW + TW - 1, (TH - 1) * TW, TW - 1])
    return sorted(set(int(t) for t in np.concatenate([heavy, rand, corner])))


def leaf_regions(leaves, TW, TH, R, aims):
    """Square regions of R x R tiles (clipped to the grid), each centred on
    the leaf junction (a point where three or four leaves meet) nearest to an
    aim point (tile coordinates); with no junction, centred on the aim."""
    from collections import Counter
    cnt = Counter()
    for L in leaves:
        for c in ((L["tx0"], L["ty0"]), (L["tx1"], L["ty0"]), (L["tx0"], L["ty1"]), (L["tx1"], L["ty1"])):
            cnt[c] += 1
    junctions = [c for c, k in cnt.items() if k >= 3 and 0 < c[0] < TW and 0 < c[1] < TH]
    out = []
    for ax, ay in aims:
        cx, cy = min(junctions, key=lambda c: (c[0] - ax) ** 2 + (c[1] - ay) ** 2) if junctions else (ax, ay)
        Rx, Ry = min(R, TW), min(R, TH)
        x0 = int(max(0, min(TW - Rx, cx - Rx // 2)))
        y0 = int(max(0, min(TH - Ry, cy - Ry // 2)))
        r = oracle.rect(x0, y0, x0 + Rx, y0 + Ry)
        if all(r.tx1 <= q.tx0 or q.tx1 <= r.tx0 or r.ty1 <= q.ty0 or q.ty1 <= r.ty0 for q in out):
            out.append(r)
    return out


def leaf_ids(leaves, TW, TH):
    lid = np.full((TH, TW), -1, np.int32)
    for i, L in enumerate(leaves):
        lid[L["ty0"]:L["ty1"], L["tx0"]:L["tx1"]] = i
    return lid


def leaves_spanned(rect, lid):
    return len(np.unique(lid[rect[1]:rect[3], rect[0]:rect[2]]))
