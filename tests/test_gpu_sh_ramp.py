"""The SH degree ramp on the GPU (gs_config.active_sh_degree).

A degree-3 scene with active degree d against the degree-d scene made of its first planes
(the degree-d layout is a prefix of the degree-3 one): records, depths, rectangles, tile
counts and the rendered image bit for bit, and, with fixed-point gradient sums (so that
two backward runs add in the same way), the parameter gradients of the first planes bit
for bit and zero on the others.  The fused update with projection leaves the inactive
bands unchanged, and the oracle with the same active degree renders the same image.
"""
import numpy as np
import pytest

from differentiable_tile_gaussian_amd import scenes
from tests import parity_util as pu

pytestmark = pytest.mark.gpu


@pytest.fixture
def gs_ramp():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from differentiable_tile_gaussian_amd import gs
    return gs


def _scene():
    s = scenes.random_scene(21, 3000, 3, spread=1.3)
    s.params[0:3] *= 0.8
    s.params[14:] = np.random.default_rng(5).normal(0, 0.3, s.params[14:].shape).astype(np.float32)
    cam = scenes.look_at_origin((0.7, 0.4, -4.5), 160, 120, 150.0)
    return s, cam


def _forward_backward(torch, gs, params, deg, cam, dLdI, cfg):
    pl, c = pu.gpu_forward(params, deg, cam, cfg)
    pl.dLdI.copy_(dLdI)
    gs.gs_render_bwd(pl.params, deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI, pl.gscreen,
                     pl.grads, pl.ws_render, cfg=cfg)
    torch.cuda.synchronize()
    return pl


@pytest.mark.parametrize("d", [0, 1, 2])
def test_active_degree_equals_the_prefix_scene(gs_ramp, d):
    import torch
    gs = gs_ramp
    s, cam = _scene()
    dLdI = torch.from_numpy((np.random.default_rng(6).standard_normal((3, 120, 160)) * 1e-2).astype(np.float32)).cuda()
    Pd = scenes.num_planes(d)
    ref = _forward_backward(torch, gs, np.ascontiguousarray(s.params[:Pd]), d, cam, dLdI,
                            gs.GsConfig(grad_sums=gs.GS_GRAD_SUMS_FIXED))
    got = _forward_backward(torch, gs, s.params, 3, cam, dLdI,
                            gs.GsConfig(grad_sums=gs.GS_GRAD_SUMS_FIXED, active_sh_degree=d))
    n = s.n
    for name in ("splat", "depth", "rect", "tiles"):
        a = getattr(got.proj, name)[:n].cpu().numpy().view(np.uint32)
        b = getattr(ref.proj, name)[:n].cpu().numpy().view(np.uint32)
        np.testing.assert_array_equal(a, b, err_msg=name)
    np.testing.assert_array_equal(got.rgb.cpu().numpy(), ref.rgb.cpu().numpy())
    g3 = got.planar(got.grads).cpu().numpy()
    gd = ref.planar(ref.grads).cpu().numpy()
    np.testing.assert_array_equal(g3[:Pd], gd)
    assert not g3[Pd:].any()
    assert np.abs(gd[11:]).max() > 0


def test_ramp_against_the_oracle_and_in_the_fused_update(gs_ramp, oracle):
    import torch
    gs = gs_ramp
    s, cam = _scene()
    cfg = gs.GsConfig(active_sh_degree=1)
    oracle.set_active_sh_degree(1)
    try:
        o = oracle.forward(s.params, 3, cam)
    finally:
        oracle.set_active_sh_degree(-1)
    pl, c = pu.gpu_forward(s.params, 3, cam, cfg)
    risk = oracle.flip_risk(o[0], o[2], o[3], cam, np.zeros((3, 120, 160), np.float32))
    pu.check_render(pu.render_to_numpy(pl), o[4], risk)
    # one fused update with the next projection: the inactive bands keep their values
    before = pl.planar(pl.params).cpu().numpy()
    pl.dLdI.copy_(torch.from_numpy((np.random.default_rng(7).standard_normal((3, 120, 160)) * 1e-2)
                                   .astype(np.float32)))
    cam2 = gs.make_camera(scenes.look_at_origin((-0.5, 0.3, -4.4), 160, 120, 150.0))
    pairs = gs.gs_render_bwd_adam_project(pl.params, 3, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc,
                                          pl.dLdI, pl.gscreen, pl.m, pl.v, pl.lr, 0.9, 0.999, 1e-8, 1, pl.ws_render,
                                          cam2, pl.proj, pl.ws_pre, cfg=cfg)
    torch.cuda.synchronize()
    after = pl.planar(pl.params).cpu().numpy()
    P1 = scenes.num_planes(1)
    np.testing.assert_array_equal(after[P1:], before[P1:])
    assert np.abs(after[:P1] - before[:P1]).max() > 0
    ref = gs.Proj(s.n)
    assert pairs == gs.gs_preprocess(pl.params, 3, cam2, ref, gs.workspace(gs.GS_WS_PREPROCESS, n=s.n), cfg=cfg)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pl.proj.splat[:s.n].cpu().numpy().view(np.uint32),
                                  ref.splat[:s.n].cpu().numpy().view(np.uint32))
