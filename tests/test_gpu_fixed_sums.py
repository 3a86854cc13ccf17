"""Fixed-point gradient sums (gs_config.grad_sums = GS_GRAD_SUMS_FIXED), [GSG] "Making the
parallel sums exact": the backward's results are reproducible bit for bit, and equal the
oracle's within the usual tolerance plus the rounding of the fixed-point unit.

Each wave-summed moment is rounded once to an integer of the unit 1 / (16384 * 3 W H)
(the second moments after division by the footprint's size factor 1 + trace of its
screen covariance), so a Gaussian's moment sum is off by at most half a unit per
contributing wave, and there are at most as many contributing waves as contributing
pixels (the oracle counts them; a few more are allowed for threshold flips).  The
decode applies the conic and 1 / opacity to those bounds.
"""
import numpy as np
import pytest

from differentiable_tile_gaussian_amd import scenes
from tests import parity_util as pu
from tests.test_gpu_parity import _oracle_all, _scene_and_camera, _small_cases

pytestmark = pytest.mark.gpu


@pytest.fixture
def fixed_mode():
    """The binding and a gs_config with fixed-point sums."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from differentiable_tile_gaussian_amd import gs
    return gs, gs.GsConfig(grad_sums=gs.GS_GRAD_SUMS_FIXED)


def quantisation_slack(pre, count, w, h):
    """[9][n] bound on what the fixed-point rounding adds to each screen partial."""
    unit = 16384.0 * 3.0 * w * h
    A, B, C = (pre["conic"][k].astype(np.float64) for k in range(3))
    o = pre["opac"].astype(np.float64)
    with np.errstate(all="ignore"):
        det = A * C - B * B
        f = np.where(det > 0, 1.0 + (A + C) / det, 1.0) * (1 + 1e-6)
        e = 0.5 * (count.astype(np.float64) + 8.0) / unit
        s = np.zeros((9, A.size))
        s[0] = (np.abs(A) + np.abs(B)) * e
        s[1] = (np.abs(B) + np.abs(C)) * e
        s[2] = 0.5 * e * f
        s[3] = e * f
        s[4] = 0.5 * e * f
        s[5] = np.where(o > 0, e / o, 0.0)
        s[6:9] = e
    return np.nan_to_num(s, posinf=0.0)


@pytest.mark.parametrize("case", [_small_cases()[k] for k in (0, 2, 3)])
def test_fixed_sums_match_oracle(fixed_mode, oracle, case):
    import torch
    gs, cfg = fixed_mode
    seed, n, deg, w, h = case
    print(f"fixed sums: seed={seed} n={n} deg={deg} {w}x{h}", flush=True)
    s, cam = _scene_and_camera(*case)
    dLdI = (np.random.default_rng(seed).standard_normal((3, h, w)) * 1e-3).astype(np.float32)
    o = _oracle_all(oracle, s.params, deg, cam, dLdI)
    _, mass, count = oracle.render_bwd(o["pre"], o["vals"], o["ranges"], cam, o["fwd"], dLdI, with_mass=True)
    o["slack"] = o["slack"] + quantisation_slack(o["pre"], count, w, h)
    pl, c = pu.gpu_forward(s.params, deg, cam, cfg)
    o["risk"] = pu.observed_risk(oracle, o, cam, pu.render_to_numpy(pl), dLdI)
    pl.dLdI.copy_(torch.from_numpy(dLdI))
    gs.gs_render_bwd(pl.params, deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI, pl.gscreen,
                     pl.grads, pl.ws_render, cfg=cfg)
    torch.cuda.synchronize()
    pu.check_screen_grads(pl.gscreen[:n].T.cpu().numpy(), o["gscreen"], o["risk"]["g"], o["slack"])
    keep = pu.calm(o["risk"]["g"], o["gscreen"])
    pu.check_param_grads(pl.planar(pl.grads).cpu().numpy(), o, oracle, s.params, deg, cam, keep)


def test_fixed_sums_reproducible(fixed_mode):
    """The same backward twice, and the same two fused training steps twice from the same
    start: every word identical (100k Gaussians at 800x800, SH degree 3)."""
    import torch
    gs, cfg = fixed_mode
    wl = scenes.CONFIGS[2]()
    cam0 = wl.cameras[0]
    cam1 = scenes.look_at_origin((3.0, 0.5, -2.5), cam0.width, cam0.height, cam0.fx)
    rng = np.random.default_rng(4)
    dLdI = torch.from_numpy((rng.standard_normal((3, cam0.height, cam0.width)) * 1e-3).astype(np.float32)).cuda()
    pl, c = pu.gpu_forward(wl.scene.params, 3, cam0, cfg)
    pl.dLdI.copy_(dLdI)
    runs = []
    for _ in range(2):
        gs.gs_render_bwd(pl.params, 3, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI,
                         pl.gscreen, pl.grads, pl.ws_render, cfg=cfg)
        torch.cuda.synchronize()
        runs.append((pl.gscreen.cpu().numpy().view(np.uint32).copy(), pl.grads.cpu().numpy().view(np.uint32).copy()))
    np.testing.assert_array_equal(runs[0][0], runs[1][0])
    np.testing.assert_array_equal(runs[0][1], runs[1][1])
    assert np.count_nonzero(runs[0][0]) > 10000
    # two fused steps (backward, chain, Adam, next projection), twice
    from differentiable_tile_gaussian_amd.pipeline import Pipeline
    cams = [gs.make_camera(cam0), gs.make_camera(cam1)]
    targets = [torch.from_numpy(rng.random((3, cam0.height, cam0.width), dtype=np.float32)).cuda() for _ in cams]
    finals = []
    for _ in range(2):
        p = Pipeline(torch.from_numpy(wl.scene.params).cuda(), 3, cam0.width, cam0.height, cfg=cfg)
        for k in range(2):
            p.step(cams[k], targets[k], next_cam=cams[1 - k])
        torch.cuda.synchronize()
        finals.append([t.cpu().numpy().view(np.uint32).copy() for t in (p.params, p.m, p.v)])
    for a, b in zip(*finals):
        np.testing.assert_array_equal(a, b)


def test_fixed_sums_of_a_screen_filling_gaussian(fixed_mode, oracle):
    """One Gaussian covering a whole 1920 x 1080 image behind a smaller one, and an image
    gradient of one sign everywhere (the L1 term's 0.8 / 3HW): its colour and opacity
    partials sum about 1.3e10 units, far past what an i32 holds.  The fixed-point sums,
    the float sums and the fp64 oracle agree."""
    import torch
    gs, cfg = fixed_mode
    from differentiable_tile_gaussian_amd.pipeline import Pipeline
    W, H = 1920, 1080
    cam = scenes.identity_camera(W, H, 1500.0)
    P = scenes.num_planes(0)
    p = np.zeros((P, 2), np.float32)
    p[0:3, 0] = (0.0, 0.0, 6.0)
    p[3:6, 0] = np.log([40.0, 30.0, 1.0])
    p[0:3, 1] = (0.3, -0.2, 3.0)
    p[3:6, 1] = np.log([0.2, 0.3, 0.2])
    p[6, :] = 1.0
    p[10] = (0.0, 1.0)
    p[11:14, 0] = (0.9, 0.2, 0.4)
    p[11:14, 1] = (0.1, 0.7, 0.3)
    dLdI = np.full((3, H, W), 0.8 / (3 * W * H), np.float32)
    pre, keys, vals, ranges, fwd = oracle.forward(p, 0, cam)
    assert pre["tiles"][0] == cam.tiles_x * cam.tiles_y
    ref = oracle.render_bwd_f64(pre, vals, ranges, cam, fwd, dLdI)
    unit = 16384.0 * 3 * W * H
    assert abs(ref[6, 0]) * unit > 2.0 ** 31          # an i32 sum would wrap
    got = {}
    for mode in (gs.GS_GRAD_SUMS_FIXED, gs.GS_GRAD_SUMS_FLOAT):
        c = gs.GsConfig(grad_sums=mode)
        pl = Pipeline(torch.from_numpy(p).cuda(), 0, W, H, cfg=c)
        cc = gs.make_camera(cam)
        pl.forward(cc)
        pl.dLdI.copy_(torch.from_numpy(dLdI))
        gs.gs_render_bwd(pl.params, 0, pl.proj, pl.vals, pl.ranges, pl.pairs, cc, pl.T, pl.nc, pl.dLdI, pl.gscreen,
                         pl.grads, pl.ws_render, cfg=c)
        torch.cuda.synchronize()
        got[mode] = pl.gscreen[:2].T.cpu().numpy().astype(np.float64)
    for k in range(9):
        for g in range(2):
            scale = max(abs(ref[k, g]), 1e-12)
            assert abs(got[gs.GS_GRAD_SUMS_FIXED][k, g] - ref[k, g]) <= 1e-4 * scale + 1e-9, (k, g)
            assert abs(got[gs.GS_GRAD_SUMS_FLOAT][k, g] - ref[k, g]) <= 1e-3 * scale + 1e-9, (k, g)
