"""Mip-Splatting opacity compensation on the GPU (gs_config.mip_compensation), against the
oracle with the same switch, to the bar of the plain path: records, depths, rectangles,
tile counts, pairs and ranges bit for bit (the factor is formed with the same
contraction-free fp32 operations on both sides), the image within its flip risk, the screen
partials and parameter gradients as in the backward parity tests; the fused update's
projection for the next camera equals gs_preprocess; and the camera-pose gradient, which
the factor reaches through the screen covariance.
"""
import math

import numpy as np
import pytest

from tests import parity_util as pu
from tests.test_gpu_camera_grad import _camera_grad, _check_against_oracle
from tests.test_gpu_parity import _oracle_all, _proj_arrays, _scene_and_camera, _small_cases

pytestmark = pytest.mark.gpu


@pytest.fixture
def mip_on(oracle):
    """The binding and a gs_config with the compensation on (the oracle's switch on too)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from differentiable_tile_gaussian_amd import gs
    oracle.set_mip_compensation(True)
    try:
        yield gs, gs.GsConfig(mip_compensation=True)
    finally:
        oracle.set_mip_compensation(False)


@pytest.mark.parametrize("case", [_small_cases()[k] for k in (0, 2, 3, 4)])
def test_mip_forward_and_backward(mip_on, oracle, case):
    import torch
    gs, cfg = mip_on
    seed, n, deg, w, h = case
    print(f"mip: seed={seed} n={n} deg={deg} {w}x{h}", flush=True)
    s, cam = _scene_and_camera(*case)
    dLdI = (np.random.default_rng(seed).standard_normal((3, h, w)) * 1e-3).astype(np.float32)
    o = _oracle_all(oracle, s.params, deg, cam, dLdI)
    vis = o["pre"]["tiles"] > 0
    plain = 1.0 / (1.0 + np.exp(-s.params[10].astype(np.float64)))
    assert (o["pre"]["opac"][vis] / plain[vis]).min() < 0.8          # the factor matters here
    pl, c = pu.gpu_forward(s.params, deg, cam, cfg)
    o["risk"] = pu.observed_risk(oracle, o, cam, pu.render_to_numpy(pl), dLdI)
    pu.check_preprocess(pu.proj_to_numpy(pl), o["pre"])
    keys, vals, ranges = pu.sorted_to_numpy(pl)
    np.testing.assert_array_equal(keys, pu.tile_of_key(o["keys"]))
    np.testing.assert_array_equal(vals, o["vals"])
    np.testing.assert_array_equal(ranges, o["ranges"])
    pu.check_render(pu.render_to_numpy(pl), o["fwd"], o["risk"])
    pl.dLdI.copy_(torch.from_numpy(dLdI))
    gs.gs_render_bwd(pl.params, deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI, pl.gscreen,
                     pl.grads, pl.ws_render, cfg=cfg)
    torch.cuda.synchronize()
    pu.check_screen_grads(pl.gscreen[:n].T.cpu().numpy(), o["gscreen"], o["risk"]["g"], o["slack"])
    keep = pu.calm(o["risk"]["g"], o["gscreen"])
    pu.check_param_grads(pl.planar(pl.grads).cpu().numpy(), o, oracle, s.params, deg, cam, keep)


def test_mip_fused_update_projects_the_next_camera(mip_on):
    import torch
    gs, cfg = mip_on
    args = _small_cases()[3]
    s, cam = _scene_and_camera(*args)
    cam2 = _scene_and_camera(args[0] + 3, *args[1:])[1]
    deg, n = s.sh_degree, s.n
    dLdI = (np.random.default_rng(5).standard_normal((3, cam.height, cam.width)) * 1e-3).astype(np.float32)
    c2 = gs.make_camera(cam2)
    pl, c = pu.gpu_forward(s.params, deg, cam, cfg)
    pl.dLdI.copy_(torch.from_numpy(dLdI))
    pairs = gs.gs_render_bwd_adam_project(pl.params, deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc,
                                          pl.dLdI, pl.gscreen, pl.m, pl.v, pl.lr, 0.9, 0.999, 1e-8, 1,
                                          pl.ws_render, c2, pl.proj, pl.ws_pre, cfg=cfg)
    torch.cuda.synchronize()
    fused = _proj_arrays(pl.proj, n)
    ref_proj = gs.Proj(n)
    assert pairs == gs.gs_preprocess(pl.params, deg, c2, ref_proj, gs.workspace(gs.GS_WS_PREPROCESS, n=n), cfg=cfg)
    torch.cuda.synchronize()
    ref = _proj_arrays(ref_proj, n)
    for k in ref:
        np.testing.assert_array_equal(fused[k], ref[k], err_msg=k)
    # the records carry the compensated opacity
    logit = pl.planar(pl.params)[10].cpu().numpy().astype(np.float64)
    vis = ref["tiles"] > 0
    opac = ref["splat"].view(np.float32)[:, 5].astype(np.float64)
    assert (opac[vis] < 1.0 / (1.0 + np.exp(-logit[vis]))).all()


def test_mip_camera_grad(mip_on, oracle):
    import torch
    gs, cfg = mip_on
    args = _small_cases()[2]
    s, cam = _scene_and_camera(*args)
    deg = s.sh_degree
    pl, c = pu.gpu_forward(s.params, deg, cam, cfg)
    pl.dLdI.copy_(torch.from_numpy((np.random.default_rng(9).standard_normal((3, cam.height, cam.width)) * 1e-2)
                                   .astype(np.float32)))
    gs.gs_render_bwd(pl.params, deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI, pl.gscreen,
                     pl.grads, pl.ws_render, cfg=cfg)
    torch.cuda.synchronize()
    got = _camera_grad(torch, gs, pl, deg, c)
    _check_against_oracle(oracle, got, s.params, deg, cam, pl.gscreen[:s.n].T.cpu().numpy())
    assert math.isfinite(got.sum())
