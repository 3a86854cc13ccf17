"""The oracle's camera-pose gradient, pinned to central differences of the smooth render
(thresholds off, fp64) with respect to the camera: translation t (the centre moving as
-R^T t) and a rotation applied on the left, R <- expm([w]x) R.  The scene has anisotropic
Gaussians and SH degree 1, so the covariance path (T = J W) and the view direction's path
through the camera centre are both exercised ([GSG] "Forgiving the camera and the light")."""
import numpy as np
from scipy.linalg import expm

from differentiable_tile_gaussian_amd import scenes


def _skew(w):
    return np.array([[0, -w[2], w[1]], [w[2], 0, -w[0]], [-w[1], w[0], 0]], np.float64)


def _moved(cam, R, t):
    c = scenes.Camera(**{f.name: getattr(cam, f.name) for f in __import__("dataclasses").fields(cam)})
    c.R = R.astype(np.float32)
    c.t = t.astype(np.float32)
    c.campos = (-(R.T @ t)).astype(np.float32)
    return c


def test_camera_grad_matches_central_differences(oracle):
    s = scenes.random_scene(5, 40, 1, spread=1.0, logscale_std=0.5)
    s.params[14:] = np.random.default_rng(8).normal(0, 0.4, s.params[14:].shape).astype(np.float32)
    cam = scenes.look_at_origin((1.0, 0.8, -4.0), 40, 30, 40.0)
    dLdI = np.random.default_rng(9).standard_normal((3, 30, 40))
    _, gscreen, _ = oracle.smooth_grad(s.params, 1, cam, dLdI)
    cg = oracle.camera_grad(s.params, 1, cam, gscreen, smooth=True, dtype=np.float64)
    R0, t0 = cam.R.astype(np.float64), cam.t.astype(np.float64)

    def L(c):
        return float((dLdI * oracle.smooth_render(s.params, 1, c)[0]).sum())
    h = 5e-4   # central differences converge as h^2 here (the error is 1e-4 of the largest component at 5e-4)
    for k in range(3):
        e = np.zeros(3)
        e[k] = h
        fd_t = (L(_moved(cam, R0, t0 + e)) - L(_moved(cam, R0, t0 - e))) / (2 * h)
        fd_w = (L(_moved(cam, expm(_skew(e)) @ R0, t0)) - L(_moved(cam, expm(_skew(-e)) @ R0, t0))) / (2 * h)
        scale_t, scale_w = np.abs(cg[3:]).max(), np.abs(cg[:3]).max()
        assert abs(cg[3 + k] - fd_t) <= 1e-3 * scale_t, (k, cg[3 + k], fd_t)
        assert abs(cg[k] - fd_w) <= 1e-3 * scale_w, (k, cg[k], fd_w)
    assert np.abs(cg).min() > 0
