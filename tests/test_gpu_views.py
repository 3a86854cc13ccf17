"""Several views per step (gs_render_bwd_weighted and Pipeline.step_views), on the GPU.

Against the oracle (float sums, the training path's default): the GPU's gradient of two
views, weights 0.7 and 0.3, the second accumulated, equals the oracle's per-view
gradients combined with those weights in fp64, each view's tolerance (the usual 1e-3
relative bar plus its flip risk and rounding slack carried through the chain) weighted
likewise.  Each view's backward is fed the oracle's image gradient of that view.

With fixed-point gradient sums every backward is reproducible bit for bit, so the weighted
and accumulated gradients are also checked exactly: weight 1 without accumulation is
gs_render_bwd's gradient; two views with weight 1/2, the second accumulated, give
fl(fl(g_a / 2) + fl(g_b / 2)) in fp32 element by element; and Pipeline.step_views over
those two views ends with the parameters and moments of one gs_adam_step on that gradient.
"""
import numpy as np
import pytest

from differentiable_tile_gaussian_amd import scenes
from tests import parity_util as pu

pytestmark = pytest.mark.gpu


@pytest.fixture
def fixed_sums():
    """The binding and a gs_config with fixed-point sums."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from differentiable_tile_gaussian_amd import gs
    return gs, gs.GsConfig(grad_sums=gs.GS_GRAD_SUMS_FIXED)


def _views():
    s = scenes.random_scene(61, 4000, 2, spread=1.3, logscale_std=0.5)
    s.params[0:3] *= 0.8
    cams = [scenes.look_at_origin((0.6, 0.4, -4.5), 160, 120, 150.0),
            scenes.look_at_origin((-2.5, 0.2, -3.8), 160, 120, 150.0)]
    rng = np.random.default_rng(7)
    targets = [rng.random((3, 120, 160), dtype=np.float32) for _ in cams]
    return s, cams, targets


def _view_grad(torch, gs, pl, cam, target, weight=None, accumulate=False, dLdI=None):
    """The parameter gradient of one view (dLdI: the image gradient to feed the backward,
    else the GPU loss's)."""
    c = gs.make_camera(cam)
    pl.forward(c)
    gs.gs_loss_l1_dssim(pl.rgb, target, pl.lam, pl.loss, pl.dLdI, pl.ws_loss)
    if dLdI is not None:
        pl.dLdI.copy_(torch.from_numpy(np.ascontiguousarray(dLdI, np.float32)))
    if weight is None:
        gs.gs_render_bwd(pl.params, pl.deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI,
                         pl.gscreen, pl.grads, pl.ws_render, cfg=pl.cfg)
    else:
        gs.gs_render_bwd_weighted(pl.params, pl.deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI,
                                  pl.gscreen, pl.grads, pl.ws_render, weight, accumulate, cfg=pl.cfg)
    torch.cuda.synchronize()
    return pl.planar(pl.grads).cpu().numpy()


def _view_tolerance(oracle, ref, params, deg, cam, rtol=pu.GRAD_RTOL):
    """[P][n] tolerance of one view's parameter gradient: rtol of the element plus rtol of its
    group's rms, plus the view's flip risk and rounding slack on the screen partials carried
    through the chain (linear in them) plane by plane."""
    g = ref["gparams"].astype(np.float64)
    tol = rtol * np.abs(g)
    for sl in pu.grad_groups(deg).values():
        tol[sl] += rtol * np.sqrt((g[sl] ** 2).mean())
    bound = ref["risk"]["g"].astype(np.float64) + ref["slack"]
    for k in range(9):
        gk = np.zeros((9, g.shape[1]), np.float32)
        gk[k] = bound[k]
        tol += np.abs(oracle.preprocess_bwd(params, deg, cam, gk).astype(np.float64))
    return tol


def test_weighted_views_against_the_oracle(oracle):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from differentiable_tile_gaussian_amd import gs
    from differentiable_tile_gaussian_amd.pipeline import Pipeline
    s, cams, targets = _views()
    deg = 2
    weights = (0.7, 0.3)
    refs = [oracle.train_step_grads(s.params, deg, cam, t) for cam, t in zip(cams, targets)]
    pl = Pipeline(torch.from_numpy(s.params).cuda(), deg, 160, 120)
    for k, (cam, t, ref, w) in enumerate(zip(cams, targets, refs, weights)):
        got = _view_grad(torch, gs, pl, cam, torch.from_numpy(t).cuda(), weight=w, accumulate=k > 0,
                         dLdI=ref["dLdI"])
        ref["risk"] = pu.observed_risk(oracle, ref, cam, pu.render_to_numpy(pl), ref["dLdI"])
    want = sum(w * ref["gparams"].astype(np.float64) for w, ref in zip(weights, refs))
    tol = sum(w * _view_tolerance(oracle, ref, s.params, deg, cam) for w, ref, cam in zip(weights, refs, cams))
    keep = np.ones(s.n, bool)
    for ref in refs:
        keep &= pu.calm(ref["risk"]["g"], ref["gscreen"])
    print(f"  views: flips {[r['risk']['flips'] for r in refs]}, Gaussians not calm {int((~keep).sum())} "
          f"of {s.n}", flush=True)
    assert keep.mean() > 0.9
    d = np.abs(got.astype(np.float64) - want)[:, keep]
    assert (d <= tol[:, keep]).all(), f"{int((d > tol[:, keep]).sum())} elements off, max excess " \
                                      f"{(d - tol[:, keep]).max()}"
    for name, sl in pu.grad_groups(deg).items():
        nb = np.linalg.norm(want[sl][:, keep])
        assert np.linalg.norm(d[sl]) <= 1e-3 * nb + np.linalg.norm(tol[sl][:, keep] - 1e-3 * np.abs(want[sl][:, keep])), name


def test_weighted_and_accumulated_gradients(fixed_sums):
    import torch
    gs, cfg = fixed_sums
    from differentiable_tile_gaussian_amd.pipeline import Pipeline
    s, cams, targets = _views()
    tg = [torch.from_numpy(t).cuda() for t in targets]
    pl = Pipeline(torch.from_numpy(s.params).cuda(), 2, 160, 120, cfg=cfg)
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
    gs, cfg = fixed_sums
    from differentiable_tile_gaussian_amd.pipeline import Pipeline
    s, cams, targets = _views()
    tg = [torch.from_numpy(t).cuda() for t in targets]
    gcams = [gs.make_camera(c) for c in cams]
    p1 = Pipeline(torch.from_numpy(s.params).cuda(), 2, 160, 120, cfg=cfg)
    losses = p1.step_views(gcams, tg)
    torch.cuda.synchronize()
    # the same by hand: the mean gradient, then gs_adam_step
    p2 = Pipeline(torch.from_numpy(s.params).cuda(), 2, 160, 120, cfg=cfg)
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


def test_position_learning_rate_schedule(fixed_sums):
    """Pipeline(lr_schedule=...): each fused update uses the rates the schedule gives for
    its step.  Two fused steps with a decaying means rate end bit for bit where two fused
    steps end whose constant rates are set by hand to the schedule's before each step,
    and differ from the constant-rate run in the means only."""
    import torch
    gs, cfg = fixed_sums
    from differentiable_tile_gaussian_amd.pipeline import Pipeline, position_lr_decay, DEFAULT_LR
    s, cams, targets = _views()
    tg = [torch.from_numpy(t).cuda() for t in targets]
    gcams = [gs.make_camera(c) for c in cams]
    sched = position_lr_decay(1.6e-6, 2)
    assert sched(1)[0] == pytest.approx(1.6e-4) and sched(2)[0] == pytest.approx(1.6e-6)
    assert sched(2)[1:] == DEFAULT_LR[1:]
    runs = {}
    for name in ("schedule", "by_hand", "constant"):
        p = Pipeline(torch.from_numpy(s.params).cuda(), 2, 160, 120, cfg=cfg,
                     lr_schedule=sched if name == "schedule" else None)
        for k in range(2):
            if name == "by_hand":
                p.lr = sched(k + 1)
            p.step(gcams[k], tg[k])
        torch.cuda.synchronize()
        runs[name] = p.planar(p.params).cpu().numpy()
    np.testing.assert_array_equal(runs["schedule"].view(np.uint32), runs["by_hand"].view(np.uint32))
    assert not np.array_equal(runs["schedule"][0:3], runs["constant"][0:3])
    np.testing.assert_array_equal(runs["schedule"][3:].view(np.uint32), runs["constant"][3:].view(np.uint32))
