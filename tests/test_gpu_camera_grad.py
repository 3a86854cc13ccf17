"""The camera-pose gradient on the GPU (gs_camera_grad), through the C ABI.

Against the oracle's camera_grad on the screen partials the GPU's backward left (so that
both sides differentiate the same gscreen): the GPU's per-Gaussian chain is fp32 like the
oracle's fp32 run, in another order of operations, so its distance from the fp64 oracle is
allowed four times the fp32 oracle's own distance from it (the largest of the group of three,
rotation or translation), plus 1e-6 of the group's largest component.

At the full training size (6M Gaussians, 1080p) also an identity that holds whatever the
scene: moving every mean and the camera centre by the same vector changes nothing, so
dL/dt = W sum_i dL/dm_i, with the mean gradients from the chain of gs_render_bwd.
"""
import numpy as np
import pytest

from differentiable_tile_gaussian_amd import scenes
from tests import parity_util as pu

pytestmark = pytest.mark.gpu


@pytest.fixture
def gs_cam():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from differentiable_tile_gaussian_amd import gs
    return gs


def _backward(torch, gs, params, deg, cam, seed, scale=1e-2, cfg=None):
    pl, c = pu.gpu_forward(params, deg, cam, cfg)
    h, w = cam.height, cam.width
    pl.dLdI.copy_(torch.from_numpy((np.random.default_rng(seed).standard_normal((3, h, w)) * scale)
                                   .astype(np.float32)))
    gs.gs_render_bwd(pl.params, deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI, pl.gscreen,
                     pl.grads, pl.ws_render, cfg=pl.cfg)
    torch.cuda.synchronize()
    return pl, c


def _camera_grad(torch, gs, pl, deg, c, position_only=False):
    """The pose gradient with the pipeline's own settings (those its backward used)."""
    out = torch.full((6,), float("nan"), dtype=torch.float64, device="cuda")
    ws = gs.workspace(gs.GS_WS_CAMERA_GRAD, n=pl.n)
    gs.gs_camera_grad(pl.params, deg, pl.proj, c, pl.gscreen, out, ws, position_only=position_only, cfg=pl.cfg)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check_against_oracle(oracle, got, params, deg, cam, gscreen_9n, position_only=False):
    o32 = oracle.camera_grad(params, deg, cam, gscreen_9n, dtype=np.float32, position_only=position_only)
    o64 = oracle.camera_grad(params, deg, cam, gscreen_9n, dtype=np.float64, position_only=position_only)
    for grp in (slice(0, 3), slice(3, 6)):
        e32 = np.abs(o32[grp] - o64[grp]).max()
        tol = 4.0 * e32 + 1e-6 * np.abs(o64[grp]).max()
        err = np.abs(got[grp] - o64[grp])
        print(f"  group {grp}: gpu err {err.max():.3e}  fp32 oracle err {e32:.3e}  tol {tol:.3e}", flush=True)
        assert (err <= tol).all(), (got, o64, o32)
    assert np.abs(o64).min() > 0


def _scene(seed, n, deg):
    s = scenes.random_scene(seed, n, deg, spread=1.3, logscale_std=0.5)
    s.params[0:3] *= 0.8
    if deg > 0:
        s.params[14:] = np.random.default_rng(seed + 1).normal(0, 0.3, s.params[14:].shape).astype(np.float32)
    return s


@pytest.mark.parametrize("deg,active", [(0, -1), (1, -1), (3, -1), (3, 1)])
def test_camera_grad_matches_oracle(gs_cam, oracle, deg, active):
    import torch
    gs = gs_cam
    print(f"camera grad: deg={deg} active={active}", flush=True)
    s = _scene(40 + deg, 3000, deg)
    cam = scenes.look_at_origin((0.7, 0.4, -4.5), 160, 120, 150.0)
    oracle.set_active_sh_degree(active)
    try:
        pl, c = _backward(torch, gs, s.params, deg, cam, seed=deg, cfg=gs.GsConfig(active_sh_degree=active))
        got = _camera_grad(torch, gs, pl, deg, c)
        _check_against_oracle(oracle, got, s.params, deg, cam, pl.gscreen[:s.n].T.cpu().numpy())
    finally:
        oracle.set_active_sh_degree(-1)
    # the same call again: the same words (fixed summation order)
    again = _camera_grad(torch, gs, pl, deg, c)
    np.testing.assert_array_equal(got.view(np.uint64), again.view(np.uint64))


@pytest.mark.parametrize("deg", [0, 3])
def test_camera_grad_position_only(gs_cam, oracle, deg):
    """The trainer's own terms (position path only: torque (p - t) x dp, and dp)."""
    import torch
    gs = gs_cam
    s = _scene(60 + deg, 3000, deg)
    cam = scenes.look_at_origin((-0.4, 0.5, -4.4), 160, 120, 150.0)
    pl, c = _backward(torch, gs, s.params, deg, cam, seed=7 + deg)
    got = _camera_grad(torch, gs, pl, deg, c, position_only=True)
    _check_against_oracle(oracle, got, s.params, deg, cam, pl.gscreen[:s.n].T.cpu().numpy(), position_only=True)
    full = _camera_grad(torch, gs, pl, deg, c)
    assert np.abs(full[:3] - got[:3]).max() > 1e-3 * np.abs(full[:3]).max()


def test_camera_grad_ragged_and_empty(gs_cam, oracle):
    """A population that is not a multiple of 64 (the last group's padding carries no
    Gaussian), and the empty one (zeros)."""
    import torch
    gs = gs_cam
    s = _scene(50, 1001, 2)
    cam = scenes.look_at_origin((-0.6, 0.2, -4.2), 96, 72, 90.0)
    pl, c = _backward(torch, gs, s.params, 2, cam, seed=3)
    got = _camera_grad(torch, gs, pl, 2, c)
    _check_against_oracle(oracle, got, s.params, 2, cam, pl.gscreen[:s.n].T.cpu().numpy())
    out = torch.full((6,), float("nan"), dtype=torch.float64, device="cuda")
    gs.gs_camera_grad(torch.zeros(1, device="cuda"), 0, gs.Proj(0), c, torch.zeros((1, 9), device="cuda"), out,
                      gs.workspace(gs.GS_WS_CAMERA_GRAD, n=0))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), np.zeros(6))


def test_camera_grad_full_size(gs_cam, oracle):
    """6M Gaussians at 1920x1080 (the training workload's population and view): against the
    oracle, and the translation identity against the chain's mean gradients."""
    import torch
    gs = gs_cam
    wl = scenes.CONFIGS[5]()
    cam = wl.cameras[0]
    deg = wl.scene.sh_degree
    print("camera grad at 6M: forward + backward", flush=True)
    pl, c = _backward(torch, gs, wl.scene.params, deg, cam, seed=11, scale=1e-3)
    got = _camera_grad(torch, gs, pl, deg, c)
    gm = pl.planar(pl.grads)[0:3].double().sum(dim=1).cpu().numpy()
    W = cam.R.astype(np.float64)
    want_t = W @ gm
    print(f"  dL/dt {got[3:]}  W sum dL/dm {want_t}", flush=True)
    np.testing.assert_allclose(got[3:], want_t, rtol=0, atol=1e-4 * np.abs(want_t).max())
    print("  oracle at 6M", flush=True)
    _check_against_oracle(oracle, got, wl.scene.params, deg, cam, pl.gscreen[:pl.n].T.cpu().numpy())
