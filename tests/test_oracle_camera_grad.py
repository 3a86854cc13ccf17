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


def test_position_only_is_the_pages_torque(oracle):
    """The trainer's terms ([GSG] "Forgiving the camera and the light": the torque
    (p - t) x dp and dp, from each Gaussian's camera-space position gradient).  With SH
    degree 0 the position gradient is dp_i = W dL/dm_i, so the sums are W sum_i m_i x dL/dm_i
    and W sum_i dL/dm_i, with dL/dm from the oracle's own parameter gradients."""
    s = scenes.random_scene(6, 40, 0, spread=1.0, logscale_std=0.5)
    cam = scenes.look_at_origin((1.0, 0.8, -4.0), 40, 30, 40.0)
    dLdI = np.random.default_rng(10).standard_normal((3, 30, 40))
    g, gscreen, _ = oracle.smooth_grad(s.params, 0, cam, dLdI)
    pos = oracle.camera_grad(s.params, 0, cam, gscreen, smooth=True, dtype=np.float64, position_only=True)
    full = oracle.camera_grad(s.params, 0, cam, gscreen, smooth=True, dtype=np.float64)
    W = cam.R.astype(np.float64)
    m = s.params[0:3].astype(np.float64)
    gm = g[0:3]
    want_w = W @ np.cross(m.T, gm.T).sum(axis=0)
    want_t = W @ gm.sum(axis=1)
    # (W a) x (W b) = W (a x b) and W W^T = I hold to the rounding of the fp32 rotation (1e-7)
    np.testing.assert_allclose(pos[:3], want_w, rtol=1e-6, atol=1e-7 * np.abs(want_w).max())
    np.testing.assert_allclose(pos[3:], want_t, rtol=1e-6, atol=1e-7 * np.abs(want_t).max())
    # the covariance path is not negligible for these anisotropic Gaussians
    assert np.abs(full[:3] - pos[:3]).max() > 1e-3 * np.abs(full[:3]).max()
    np.testing.assert_allclose(full[3:], pos[3:], rtol=1e-12)    # degree 0: no view-direction term
