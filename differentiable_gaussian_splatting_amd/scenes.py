"""Seeded synthetic inputs for one training view (scenes, cameras, targets).

This module only draws random numbers and assembles arrays: it holds none of
the method's arithmetic, and it is the one piece shared by the GPU path's
tests/benchmark and by the CPU oracle.

The pages measure on dataset scenes (the "Bicycle" model with about 5.99M
and 11.98M Gaussians, Mip-NeRF 360, Tanks and Temples; BoundedGS page, "03"
and Fig. 5/6).  Those are not available; the generators below stand in for
their shapes: a clustered ground-plane-plus-object layout, a heavy-tailed
Gaussian mixture, and uniform boxes.  Nothing here reproduces a dataset item.

Parameter layout (all float32, host numpy):
    means [N,3], log_scales [N,3], quats [N,4] (w,x,y,z), logits [N],
    sh [N,K,3] with K = (deg+1)^2, target [3,H,W] (CHW).
Camera: world->camera p = R mu + t, pinhole with horizontal field of view
60 degrees, fx = fy = (W/2)/tan(30 deg), principal point at the image centre,
near plane 0.2, black background.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

SQRT_PI = math.sqrt(math.pi)


@dataclasses.dataclass
class Camera:
    R: np.ndarray          # [3,3] float32 row-major, world->camera
    t: np.ndarray          # [3] float32
    fx: float
    fy: float
    cx: float
    cy: float
    width: int
    height: int
    near_z: float = 0.2
    bg: tuple = (0.0, 0.0, 0.0)

    @property
    def tiles_x(self) -> int:
        return (self.width + 15) // 16

    @property
    def tiles_y(self) -> int:
        return (self.height + 15) // 16


@dataclasses.dataclass
class Scene:
    means: np.ndarray
    log_scales: np.ndarray
    quats: np.ndarray
    logits: np.ndarray
    sh: np.ndarray
    sh_degree: int

    @property
    def n(self) -> int:
        return int(self.means.shape[0])

    def arrays(self):
        return (self.means, self.log_scales, self.quats, self.logits, self.sh)


def pinhole_camera(width: int, height: int, fov_x_deg: float = 60.0, R=None, t=None) -> Camera:
    f = np.float32((width / 2.0) / math.tan(math.radians(fov_x_deg) / 2.0))
    R = np.eye(3, dtype=np.float32) if R is None else np.asarray(R, dtype=np.float32)
    t = np.zeros(3, dtype=np.float32) if t is None else np.asarray(t, dtype=np.float32)
    return Camera(R=R, t=t, fx=float(f), fy=float(f), cx=float(np.float32(width / 2.0)),
                  cy=float(np.float32(height / 2.0)), width=int(width), height=int(height))


def random_pose_camera(width: int, height: int, rng: np.random.Generator,
                       max_angle_deg: float = 15.0, max_shift: float = 0.5) -> Camera:
    """Pinhole camera with a random small rotation (axis uniform, angle up to
    max_angle_deg) and translation (each component up to max_shift)."""
    axis = rng.normal(size=3)
    axis /= np.linalg.norm(axis)
    ang = math.radians(rng.uniform(0.0, max_angle_deg))
    K = np.array([[0, -axis[2], axis[1]], [axis[2], 0, -axis[0]], [-axis[1], axis[0], 0]])
    R = np.eye(3) + math.sin(ang) * K + (1 - math.cos(ang)) * (K @ K)
    t = rng.uniform(-max_shift, max_shift, size=3)
    return pinhole_camera(width, height, R=R.astype(np.float32), t=t.astype(np.float32))


def _quats(rng, n):
    q = rng.normal(size=(n, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    return q.astype(np.float32)


def _finish(rng, means, log_mu, log_sd, deg, sh_sd=0.2, sh0_uniform=False) -> Scene:
    n = means.shape[0]
    log_scales = rng.normal(log_mu, log_sd, size=(n, 3)).astype(np.float32)
    quats = _quats(rng, n)
    logits = rng.normal(0.0, 1.0, size=n).astype(np.float32)
    K = (deg + 1) ** 2
    if sh0_uniform:
        # degree-0 colour uniform in [0,1] per channel: the DC coefficient is
        # drawn uniform in [-sqrt(pi), sqrt(pi)] (the DC basis value is
        # 1/(2 sqrt(pi)) and colour = 0.5 + basis * coefficient)
        sh = rng.uniform(-SQRT_PI, SQRT_PI, size=(n, K, 3)).astype(np.float32)
    else:
        sh = rng.normal(0.0, sh_sd, size=(n, K, 3)).astype(np.float32)
    return Scene(means=means.astype(np.float32), log_scales=log_scales, quats=quats,
                 logits=logits, sh=sh, sh_degree=deg)


def target_image(rng: np.random.Generator, width: int, height: int) -> np.ndarray:
    """Supervision image, i.i.d. U[0,1] f32 CHW."""
    return rng.random(size=(3, height, width), dtype=np.float32)


# -- the five workloads --------------------------------------------------------

def uniform_box_scene(rng, n, half=1.0, depth=4.0, log_mu=-3.0, log_sd=0.5, deg=0,
                      sh0_uniform=True) -> Scene:
    """Means uniform in [-half,half]^3 shifted to z + depth."""
    means = rng.uniform(-half, half, size=(n, 3))
    means[:, 2] += depth
    return _finish(rng, means, log_mu, log_sd, deg, sh0_uniform=sh0_uniform)


def gmm_scene(rng, n, components=64, deg=3, log_mu=-4.0, log_sd=0.7, zipf=1.5,
              centre_half=5.0, depth=20.0, sigma_lo=0.1, sigma_hi=1.0) -> Scene:
    """Isotropic Gaussian mixture, Zipf-weighted components (heavy-tailed
    cluster sizes), centres uniform in a box in front of the camera, component
    spreads log-uniform in [sigma_lo, sigma_hi]."""
    w = np.arange(1, components + 1, dtype=np.float64) ** (-zipf)
    w /= w.sum()
    counts = np.floor(w * n).astype(np.int64)
    counts[0] += n - counts.sum()
    centres = rng.uniform(-centre_half, centre_half, size=(components, 3))
    centres[:, 2] += depth
    sig = np.exp(rng.uniform(math.log(sigma_lo), math.log(sigma_hi), size=components))
    comp = np.repeat(np.arange(components), counts)
    rng.shuffle(comp)
    means = centres[comp] + rng.normal(size=(n, 3)) * sig[comp, None]
    return _finish(rng, means, log_mu, log_sd, deg)


def ground_object_scene(rng, n, deg=3, log_mu=-4.0, log_sd=0.7, plane_frac=0.7,
                        clusters=8) -> Scene:
    """Ground plane plus objects: plane_frac of the Gaussians lie within 2
    units of the plane y = 2 (x in [-30,30], z in [2,60]); the rest fall in
    equal dense isotropic clusters in front of the camera."""
    n_plane = int(round(plane_frac * n))
    n_obj = n - n_plane
    plane = np.empty((n_plane, 3))
    plane[:, 0] = rng.uniform(-30.0, 30.0, size=n_plane)
    plane[:, 1] = 2.0 + rng.uniform(-2.0, 2.0, size=n_plane)
    plane[:, 2] = rng.uniform(2.0, 60.0, size=n_plane)
    centres = np.stack([rng.uniform(-4, 4, clusters), rng.uniform(-1, 1.5, clusters),
                        rng.uniform(8, 16, clusters)], axis=1)
    sig = rng.uniform(0.3, 1.0, size=clusters)
    comp = np.arange(n_obj) % clusters
    rng.shuffle(comp)
    obj = centres[comp] + rng.normal(size=(n_obj, 3)) * sig[comp, None]
    means = np.concatenate([plane, obj], axis=0)
    perm = rng.permutation(n)
    return _finish(rng, means[perm], log_mu, log_sd, deg)


@dataclasses.dataclass
class Workload:
    name: str
    scene: Scene
    camera: Camera
    target: np.ndarray
    loss: str               # "l1" or "l1_ssim"
    budgets: tuple          # leaf budgets in bytes; () = full image only


MIB = 1 << 20


def make_workload(name: str, seed: int | None = None, n: int | None = None,
                  width: int | None = None, height: int | None = None,
                  posed: bool = False, sh_degree: int | None = None) -> Workload:
    """Workloads by name, with optional size overrides (parity tests shrink
    them while keeping the generator and its structure):

      c1_small     2,000 Gaussians, box at z+4, SH0 rgb U[0,1], 128x128, L1
      c2_hd        100k, 10-unit box at z+20, SH3, 1920x1080, L1 + 0.2 (1-SSIM)
      c3_gmm4k     1M, 64-component Zipf mixture, SH3, 3840x2160, L1
      c4_plane5k   6M ground plane + 8 clusters, SH3, 5000x3300, 384 MiB leaves
      c5_plane16k  6M same generator, 16000x10560, 384 MiB leaves, one Adam step
      c5_plane16k_12m  12M, same

    sh_degree overrides the SH degree of the box scenes (c1_small, c2_hd).
    """
    table = {
        "c1_small": dict(seed=1, n=2000, w=128, h=128, loss="l1", budgets=()),
        "c2_hd": dict(seed=2, n=100_000, w=1920, h=1080, loss="l1_ssim", budgets=()),
        "c3_gmm4k": dict(seed=3, n=1_000_000, w=3840, h=2160, loss="l1",
                         budgets=(384 * MIB, 128 * MIB)),
        "c4_plane5k": dict(seed=4, n=6_000_000, w=5000, h=3300, loss="l1", budgets=(384 * MIB,)),
        "c5_plane16k": dict(seed=5, n=6_000_000, w=16000, h=10560, loss="l1",
                            budgets=(384 * MIB, 128 * MIB)),
        "c5_plane16k_12m": dict(seed=6, n=12_000_000, w=16000, h=10560, loss="l1",
                                budgets=(384 * MIB, 128 * MIB)),
    }
    if name not in table:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(table)}")
    spec = table[name]
    seed = spec["seed"] if seed is None else seed
    n = spec["n"] if n is None else n
    w = spec["w"] if width is None else width
    h = spec["h"] if height is None else height
    rng = np.random.default_rng(seed)
    if sh_degree is not None and name not in ("c1_small", "c2_hd"):
        raise ValueError(f"sh_degree override applies to c1_small and c2_hd only, not {name!r}")
    if name == "c1_small":
        scene = uniform_box_scene(rng, n, half=1.0, depth=4.0, log_mu=-3.0, log_sd=0.5,
                                  deg=0 if sh_degree is None else sh_degree)
    elif name == "c2_hd":
        scene = uniform_box_scene(rng, n, half=5.0, depth=20.0, log_mu=-4.0, log_sd=0.7,
                                  deg=3 if sh_degree is None else sh_degree, sh0_uniform=False)
    elif name == "c3_gmm4k":
        scene = gmm_scene(rng, n)
    else:
        scene = ground_object_scene(rng, n)
    cam = random_pose_camera(w, h, rng) if posed else pinhole_camera(w, h)
    target = target_image(rng, w, h)
    return Workload(name=name, scene=scene, camera=cam, target=target, loss=spec["loss"],
                    budgets=spec["budgets"])
