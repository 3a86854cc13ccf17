"""Several views per step (gs_render_bwd_weighted and Pipeline.step_views), on the GPU.

With fixed-point gradient sums every backward is reproducible bit for bit, so the weighted
and accumulated gradients are checked exactly: weight 1 without accumulation is
gs_render_bwd's gradient; two views with weight 1/2, the second accumulated, give
fl(fl(g_a / 2) + fl(g_b / 2)) in fp32 element by element; and Pipeline.step_views over
those two views ends with the parameters and moments of one gs_adam_step on that gradient.
The single-view gradients themselves are checked against the oracle elsewhere.
"""
import numpy as np
import pytest

from differentiable_tile_gaussian_amd import scenes
from tests import parity_util as pu

pytestmark = pytest.mark.gpu


@pytest.fixture
def fixed_sums():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from differentiable_tile_gaussian_amd import gs
    gs.gs_set_grad_sums(gs.GS_GRAD_SUMS_FIXED)
    try:
        yield gs
    finally:
        gs.gs_set_grad_sums(gs.GS_GRAD_SUMS_FLOAT)


def _views():
    s = scenes.random_scene(61, 4000, 2, spread=1.3, logscale_std=0.5)
    s.params[0:3] *= 0.8
    cams = [scenes.look_at_origin((0.6, 0.4, -4.5), 160, 120, 150.0),
            scenes.look_at_origin((-2.5, 0.2, -3.8), 160, 120, 150.0)]
    rng = np.random.default_rng(7)
    targets = [rng.random((3, 120, 160), dtype=np.float32) for _ in cams]
    return s, cams, targets


def _view_grad(torch, gs, pl, cam, target, weight=None, accumulate=False):
    c = gs.make_camera(cam)
    pl.forward(c)
    gs.gs_loss_l1_dssim(pl.rgb, target, pl.lam, pl.loss, pl.dLdI, pl.ws_loss)
    if weight is None:
        gs.gs_render_bwd(pl.params, pl.deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI,
                         pl.gscreen, pl.grads, pl.ws_render)
    else:
        gs.gs_render_bwd_weighted(pl.params, pl.deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI,
                                  pl.gscreen, pl.grads, pl.ws_render, weight, accumulate)
    torch.cuda.synchronize()
    return pl.planar(pl.grads).cpu().numpy()


def test_weighted_and_accumulated_gradients(fixed_sums):
    import torch
    gs = fixed_sums
    from differentiable_tile_gaussian_amd.pipeline import Pipeline
    s, cams, targets = _views()
    tg = [torch.from_numpy(t).cuda() for t in targets]
    pl = Pipeline(torch.from_numpy(s.params).cuda(), 2, 160, 120)
    g_a = _view_grad(torch, gs, pl, cams[0], tg[0])
    g_b = _view_grad(torch, gs, pl, cams[1], tg[1])
    assert np.count_nonzero(g_a) > 1000 and np.count_nonzero(g_b) > 1000
    one = _view_grad(torch, gs, pl, cams[0], tg[0], weight=1.0, accumulate=False)
    np.testing.assert_array_equal(one.view(np.uint32), g_a.view(np.uint32))
    _view_grad(torch, gs, pl, cams[0], tg[0], weight=0.5, accumulate=False)
    both = _view_grad(torch, gs, pl, cams[1], tg[1], weight=0.5, accumulate=True)
    half = np.float32(0.5)
    want = (half * g_a).astype(np.float32) + (half * g_b).astype(np.float32)
    np.testing.assert_array_equal(both.view(np.uint32), want.astype(np.float32).view(np.uint32))


def test_step_views_is_one_adam_update_of_the_mean(fixed_sums):
    import torch
    gs = fixed_sums
    from differentiable_tile_gaussian_amd.pipeline import Pipeline
    s, cams, targets = _views()
    tg = [torch.from_numpy(t).cuda() for t in targets]
    gcams = [gs.make_camera(c) for c in cams]
    p1 = Pipeline(torch.from_numpy(s.params).cuda(), 2, 160, 120)
    losses = p1.step_views(gcams, tg)
    torch.cuda.synchronize()
    # the same by hand: the mean gradient, then gs_adam_step
    p2 = Pipeline(torch.from_numpy(s.params).cuda(), 2, 160, 120)
    g_a = _view_grad(torch, gs, p2, cams[0], tg[0])
    l_a = p2.loss.cpu().numpy().copy()
    g_b = _view_grad(torch, gs, p2, cams[1], tg[1])
    half = np.float32(0.5)
    mean = ((half * g_a).astype(np.float32) + (half * g_b).astype(np.float32)).astype(np.float32)
    p2.set_planar(p2.grads, torch.from_numpy(mean).cuda())
    p2.adam()
    torch.cuda.synchronize()
    for a, b in ((p1.params, p2.params), (p1.m, p2.m), (p1.v, p2.v)):
        np.testing.assert_array_equal(p1.planar(a).cpu().numpy().view(np.uint32),
                                      p2.planar(b).cpu().numpy().view(np.uint32))
    np.testing.assert_array_equal(losses[0].cpu().numpy(), l_a)
    assert np.isfinite(losses.cpu().numpy()).all()
