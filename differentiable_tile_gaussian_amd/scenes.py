"""Seeded synthetic scenes and cameras for the five rasteriser workloads.

This module only draws random numbers and builds camera poses.  It holds none
of the rasteriser's arithmetic, so both the HIP path and the CPU oracle can
take their inputs from it.

Parameter layout (structure of arrays, float32, plane-major ``[P][N]``):

* planes 0-2   mean x, y, z (world units)
* planes 3-5   log-scales
* planes 6-9   quaternion w, x, y, z
* plane 10     opacity logit
* planes 11-13 colour DC r, g, b (colour units)
* plane 14 + 3*(k-1) + ch, k = 1..(deg+1)^2-1: higher spherical-harmonic bands

so P = 11 + 3*(deg+1)^2: 14 at degree 0, 59 at degree 3.

Camera convention: OpenCV axes (x right, y down, z forward), ``p_c = R p_w + t``
with R row-major, pixel (i, j) centred at (i + 0.5, j + 0.5).

Seeds: ``default_rng(1000*cfg + role)``, role 0 = scene, 1 = target scene or
perturbation, 2 = cameras.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

PLANE_MEAN = 0
PLANE_LOGSCALE = 3
PLANE_QUAT = 6
PLANE_LOGIT = 10
PLANE_DC = 11
PLANE_SH = 14


def num_planes(sh_degree: int) -> int:
    return 11 + 3 * (sh_degree + 1) ** 2


@dataclasses.dataclass
class Camera:
    R: np.ndarray            # (3, 3) float32, world -> camera rotation
    t: np.ndarray            # (3,) float32
    campos: np.ndarray       # (3,) float32, camera centre in world coordinates
    fx: float
    fy: float
    cx: float
    cy: float
    width: int
    height: int
    znear: float = 0.2
    bg: tuple = (0.0, 0.0, 0.0)

    @property
    def tiles_x(self) -> int:
        return (self.width + 15) // 16

    @property
    def tiles_y(self) -> int:
        return (self.height + 15) // 16


@dataclasses.dataclass
class Scene:
    params: np.ndarray       # (P, N) float32
    sh_degree: int

    @property
    def n(self) -> int:
        return int(self.params.shape[1])


@dataclasses.dataclass
class Workload:
    name: str
    scene: Scene
    cameras: list            # list[Camera]
    target_scene: Scene | None   # target image = render of this scene from the same camera
    description: str


def look_at_origin(C, width, height, f, cx=None, cy=None) -> Camera:
    """Camera at world point C looking at the origin, world +y as 'down'.

    Rows of R: x_c = normalize((0,1,0) x z_c), y_c = z_c x x_c, z_c = normalize(-C);
    t = -R C.  C = (0, 0, -r) gives R = I, t = (0, 0, r).
    """
    C = np.asarray(C, dtype=np.float64)
    zc = -C / np.linalg.norm(C)
    xc = np.cross(np.array([0.0, 1.0, 0.0]), zc)
    xc /= np.linalg.norm(xc)
    yc = np.cross(zc, xc)
    R = np.stack([xc, yc, zc]).astype(np.float32)
    t = (-(R.astype(np.float64) @ C)).astype(np.float32)
    return Camera(R=R, t=t, campos=C.astype(np.float32), fx=float(f), fy=float(f),
                  cx=float(width / 2 if cx is None else cx),
                  cy=float(height / 2 if cy is None else cy),
                  width=int(width), height=int(height))


def identity_camera(width, height, f, cx=None, cy=None, position=(0.0, 0.0, 0.0)) -> Camera:
    """Camera with R = I placed at ``position`` (t = -position)."""
    pos = np.asarray(position, dtype=np.float32)
    return Camera(R=np.eye(3, dtype=np.float32), t=(-pos).astype(np.float32), campos=pos.copy(),
                  fx=float(f), fy=float(f),
                  cx=float(width / 2 if cx is None else cx),
                  cy=float(height / 2 if cy is None else cy),
                  width=int(width), height=int(height))


def _normal(rng, shape, mean, std):
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std) + np.float32(mean))


def _unit_quaternions(rng, n):
    q = rng.standard_normal((4, n), dtype=np.float32)
    q /= np.linalg.norm(q, axis=0, keepdims=True)
    return q


def _fill_common(rng, params, n, sh_degree, logscale_mean, logscale_std, logit_mean, logit_std):
    params[PLANE_LOGSCALE:PLANE_LOGSCALE + 3] = _normal(rng, (3, n), logscale_mean, logscale_std)
    params[PLANE_QUAT:PLANE_QUAT + 4] = _unit_quaternions(rng, n)
    params[PLANE_LOGIT] = _normal(rng, (n,), logit_mean, logit_std)
    params[PLANE_DC:PLANE_DC + 3] = rng.random((3, n), dtype=np.float32)
    rest = 3 * ((sh_degree + 1) ** 2 - 1)
    if rest:
        params[PLANE_SH:PLANE_SH + rest] = _normal(rng, (rest, n), 0.0, 0.05)


def _perturbed(scene: Scene, rng, std=0.01) -> Scene:
    p = scene.params.copy()
    p[0:3] += _normal(rng, (3, scene.n), 0.0, std)
    return Scene(p, scene.sh_degree)


def _clusters(rng, n, n_clusters, lo_xy, hi_xy, lo_z, hi_z):
    centres = np.empty((n_clusters, 3), dtype=np.float32)
    centres[:, 0:2] = rng.uniform(lo_xy, hi_xy, (n_clusters, 2)).astype(np.float32)
    centres[:, 2] = rng.uniform(lo_z, hi_z, n_clusters).astype(np.float32)
    stds = rng.uniform(0.05, 0.8, (n_clusters, 3)).astype(np.float32)
    assign = rng.integers(0, n_clusters, n)
    means = centres[assign].T + stds[assign].T * rng.standard_normal((3, n), dtype=np.float32)
    return means


def config1(seed_base=1000) -> Workload:
    """1,024 Gaussians, SH degree 0, 128x128, camera at (0,0,-4) looking +z."""
    n, deg = 1024, 0

    def make(role):
        rng = np.random.default_rng(seed_base + role)
        p = np.zeros((num_planes(deg), n), dtype=np.float32)
        p[0:3] = rng.uniform(-1.0, 1.0, (3, n)).astype(np.float32)
        _fill_common(rng, p, n, deg, math.log(0.03), 0.3, 0.0, 1.0)
        return Scene(p, deg)

    cam = look_at_origin((0.0, 0.0, -4.0), 128, 128, 128.0, 64.0, 64.0)
    return Workload("cfg1_tiny_1k_sh0_128px", make(0), [cam], make(1),
                    "1,024 Gaussians, SH0, 128x128; target rendered from a second seeded scene")


def config2(seed_base=2000) -> Workload:
    """100,000 Gaussians near the unit sphere, SH degree 3, 800x800 orbit camera."""
    n, deg = 100_000, 3
    rng = np.random.default_rng(seed_base + 0)
    p = np.zeros((num_planes(deg), n), dtype=np.float32)
    d = rng.standard_normal((3, n), dtype=np.float32)
    d /= np.linalg.norm(d, axis=0, keepdims=True)
    p[0:3] = d * (1.0 + _normal(rng, (n,), 0.0, 0.02))
    _fill_common(rng, p, n, deg, math.log(0.01), 0.5, 0.0, 1.5)
    scene = Scene(p, deg)
    target = _perturbed(scene, np.random.default_rng(seed_base + 1))
    theta = float(np.random.default_rng(seed_base + 2).uniform(0.0, 2.0 * math.pi))
    cam = look_at_origin((4.0 * math.sin(theta), 0.0, -4.0 * math.cos(theta)), 800, 800, 1100.0)
    return Workload("cfg2_mid_100k_sh3_800px", scene, [cam], target,
                    "100k Gaussians on a unit sphere shell, SH3, 800x800 orbit r=4")


def config3(seed_base=3000) -> Workload:
    """1,000,000 Gaussians in 64 anisotropic clusters at depth 2-20, 1920x1080."""
    n, deg = 1_000_000, 3
    rng = np.random.default_rng(seed_base + 0)
    p = np.zeros((num_planes(deg), n), dtype=np.float32)
    p[0:3] = _clusters(rng, n, 64, -5.0, 5.0, 2.0, 20.0)
    _fill_common(rng, p, n, deg, math.log(0.02), 0.6, 0.0, 2.0)
    scene = Scene(p, deg)
    target = _perturbed(scene, np.random.default_rng(seed_base + 1))
    cam = identity_camera(1920, 1080, 1500.0, 960.0, 540.0)
    return Workload("cfg3_large_1m_sh3_1080p", scene, [cam], target,
                    "1M Gaussians, 64 clusters (x,y in [-5,5], z in [2,20]), SH3, 1920x1080")


def config4(seed_base=4000) -> Workload:
    """3,000,000 Gaussians packed in a 2x2x10 slab in front of a 1280x720 camera."""
    n, deg = 3_000_000, 3
    rng = np.random.default_rng(seed_base + 0)
    p = np.zeros((num_planes(deg), n), dtype=np.float32)
    p[0:2] = rng.uniform(-1.0, 1.0, (2, n)).astype(np.float32)
    p[2] = rng.uniform(2.0, 12.0, n).astype(np.float32)
    _fill_common(rng, p, n, deg, math.log(0.05), 0.3, -2.0, 1.0)
    scene = Scene(p, deg)
    target = _perturbed(scene, np.random.default_rng(seed_base + 1))
    cam = identity_camera(1280, 720, 900.0, 640.0, 360.0)
    return Workload("cfg4_stress_3m_sh3_720p", scene, [cam], target,
                    "3M Gaussians in a 2x2x10 slab at depth 2-12, SH3, 1280x720, logits ~N(-2,1)")


def config5(seed_base=5000, n_cameras=100, n=6_000_000) -> Workload:
    """6,000,000 Gaussians, 64 clusters over [-20,20]^3, 100 orbit cameras r=25, 1920x1080."""
    deg = 3
    rng = np.random.default_rng(seed_base + 0)
    p = np.zeros((num_planes(deg), n), dtype=np.float32)
    p[0:3] = _clusters(rng, n, 64, -20.0, 20.0, -20.0, 20.0)
    _fill_common(rng, p, n, deg, math.log(0.02), 0.6, 0.0, 2.0)
    scene = Scene(p, deg)
    target = _perturbed(scene, np.random.default_rng(seed_base + 1))
    thetas = np.random.default_rng(seed_base + 2).uniform(0.0, 2.0 * math.pi, n_cameras)
    cams = [look_at_origin((25.0 * math.sin(th), 0.0, -25.0 * math.cos(th)), 1920, 1080, 1500.0,
                           960.0, 540.0) for th in thetas]
    return Workload("cfg5_train_6m_sh3_1080p", scene, cams, target,
                    "6M Gaussians, 64 clusters over [-20,20]^3, SH3, 100 orbit cameras r=25, 1920x1080")


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def random_scene(seed, n, sh_degree, spread=1.0, depth=(3.0, 6.0), logscale_mean=math.log(0.05),
                 logscale_std=0.3, logit_mean=0.0, logit_std=1.0) -> Scene:
    """Small generic scene in front of an identity camera (for parity and edge cases)."""
    rng = np.random.default_rng(seed)
    p = np.zeros((num_planes(sh_degree), n), dtype=np.float32)
    p[0:2] = rng.uniform(-spread, spread, (2, n)).astype(np.float32)
    p[2] = rng.uniform(depth[0], depth[1], n).astype(np.float32)
    _fill_common(rng, p, n, sh_degree, logscale_mean, logscale_std, logit_mean, logit_std)
    return Scene(p, sh_degree)


def random_image(seed, height, width):
    """Smooth-ish seeded image in [0, 1], shape (3, H, W) float32."""
    rng = np.random.default_rng(seed)
    img = rng.random((3, height, width), dtype=np.float32)
    return img
