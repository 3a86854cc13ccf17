"""Density control on the GPU, through the C ABI, against the oracle.

gs_densify: the new count, the counts kept / cloned / split and every output word
(parameters, moments, statistics) equal the oracle's bit for bit (decisions on the stored
logit and log-scales against the same rounded thresholds; split children from the same
normals with the same fp32 roundings).  gs_densify_accumulate and the statistics of the
projecting update: as the oracle's accumulation of the same screen gradients.
"""
import numpy as np
import pytest

from differentiable_tile_gaussian_amd import scenes
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

THR = dict(grad_threshold=2e-4, prune_opacity=0.005, prune_scale=1.0, split_scale=0.05)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _population(n, deg, seed):
    """A scene with a spread of opacities and sizes, statistics, moments and normals."""
    p = scenes.random_scene(seed, n, deg).params.copy()
    rng = np.random.default_rng(seed + 1)
    p[10] = rng.normal(0.0, 3.0, n)
    p[3:6] += rng.normal(0.0, 1.0, (3, n)).astype(np.float32)
    p[6:10, ::97] = 0.0                       # some zero quaternions
    cnt = rng.integers(0, 6, n).astype(np.float32)
    stats = np.stack([rng.random(n) * 1e-3 * cnt, cnt], 1).astype(np.float32)
    m = rng.standard_normal(p.shape).astype(np.float32)
    v = rng.random(p.shape).astype(np.float32)
    rand = rng.standard_normal((n, 2, 3)).astype(np.float32)
    return p, m, v, stats, rand


def _bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def _run(torch, gs, p, m, v, stats, rand, deg, reset, capacity=None):
    n = p.shape[1]
    dev = torch.device("cuda")
    pb, mb, vb = (gs.to_blocked(torch.from_numpy(np.ascontiguousarray(a)).to(dev), deg) for a in (p, m, v))
    st, rd = torch.from_numpy(stats).to(dev), torch.from_numpy(rand).to(dev)
    ws = gs.workspace(gs.GS_WS_DENSIFY, n=n)
    n_new, counts = gs.gs_densify(pb, mb, vb, st, rd, n, deg, ws=ws, reset_opacity=reset, **THR)
    cap = n_new if capacity is None else capacity
    outs = [gs.empty_blocked(max(cap, 1), deg, dev).fill_(float("nan")) for _ in range(3)]
    so = torch.full((max(cap, 1), 2), float("nan"), device=dev)
    n_chk, _ = gs.gs_densify(pb, mb, vb, st, rd, n, deg, ws=ws, reset_opacity=reset, params_out=outs[0],
                             m_out=outs[1], v_out=outs[2], stats_out=so, capacity=cap, **THR)
    torch.cuda.synchronize()
    assert n_chk == n_new
    return n_new, counts, outs, so


@pytest.mark.parametrize("n,deg,reset", [(1, 0, False), (1000, 0, False), (4097, 3, True), (20000, 1, False),
                                         (20000, 3, True)])
def test_densify_matches_oracle(torch_cuda, oracle, n, deg, reset):
    torch = torch_cuda
    from differentiable_tile_gaussian_amd import gs
    p, m, v, stats, rand = _population(n, deg, seed=n + deg)
    print(f"densify n={n} deg={deg} reset={reset}", flush=True)
    ref = oracle.densify(p, m, v, stats, rand, deg, reset_opacity=reset, **THR)
    n_new, counts, outs, so = _run(torch, gs, p, m, v, stats, rand, deg, reset)
    assert n_new == ref["params"].shape[1]
    assert counts == tuple(int(c) for c in ref["counts"])
    for name, blocked in zip(("params", "m", "v"), outs):
        got = gs.from_blocked(blocked, n_new, deg).cpu().numpy()
        np.testing.assert_array_equal(_bits(got), _bits(ref[name]), err_msg=name)
        # padding of the last group untouched (still the NaN fill)
        flat = blocked.cpu().numpy()
        groups, P, _ = flat.shape
        if n_new % 64:
            assert np.isnan(flat[n_new // 64, :, n_new % 64:]).all(), name
    np.testing.assert_array_equal(so[:n_new].cpu().numpy(), np.zeros((n_new, 2), np.float32))


def test_densify_capacity_and_counting(torch_cuda, oracle):
    torch = torch_cuda
    from differentiable_tile_gaussian_amd import gs
    p, m, v, stats, rand = _population(3000, 2, seed=11)
    ref = oracle.densify(p, m, v, stats, rand, 2, **THR)
    n_ref = ref["params"].shape[1]
    with pytest.raises(gs.GsError) as err:
        _run(torch, gs, p, m, v, stats, rand, 2, False, capacity=n_ref - 1)
    assert err.value.status == gs.GS_ERR_CAPACITY


def test_densify_full_size(torch_cuda, oracle):
    """The 6M-Gaussian population of the training workload, with synthetic statistics."""
    torch = torch_cuda
    from differentiable_tile_gaussian_amd import gs
    wl = scenes.CONFIGS[5]()
    p = wl.scene.params
    n, deg = wl.scene.n, wl.scene.sh_degree
    rng = np.random.default_rng(21)
    cnt = rng.integers(0, 4, n).astype(np.float32)
    stats = np.stack([rng.random(n, dtype=np.float32) * 6e-4 * cnt, cnt], 1).astype(np.float32)
    z = np.zeros_like(p)
    rand = rng.standard_normal((n, 2, 3), dtype=np.float32)
    print("oracle densify at 6M", flush=True)
    ref = oracle.densify(p, z, z, stats, rand, deg, **THR)
    print(f"  counts {ref['counts']}", flush=True)
    n_new, counts, outs, so = _run(torch, gs, p, z, z, stats, rand, deg, False)
    assert counts == tuple(int(c) for c in ref["counts"])
    got = gs.from_blocked(outs[0], n_new, deg).cpu().numpy()
    np.testing.assert_array_equal(_bits(got), _bits(ref["params"]))


def test_accumulate_matches_oracle(torch_cuda, oracle):
    """gs_densify_accumulate twice on one backward's screen gradients."""
    torch = torch_cuda
    from differentiable_tile_gaussian_amd import gs
    s = scenes.random_scene(31, 3000, 1, spread=1.3)
    s.params[0:3] *= 0.8
    cam = scenes.look_at_origin((0.0, 0.4, -4.5), 160, 120, 150.0)
    pl, c = pu.gpu_forward(s.params, 1, cam)
    pl.dLdI.copy_(torch.from_numpy(np.random.default_rng(2).standard_normal((3, 120, 160)).astype(np.float32)))
    gs.gs_render_bwd(pl.params, 1, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI, pl.gscreen,
                     pl.grads, pl.ws_render)
    pl.enable_density_stats()
    for _ in range(2):
        gs.gs_densify_accumulate(pl.proj, pl.gscreen, pl.dstats)
    torch.cuda.synchronize()
    tiles = pl.proj.tiles[:s.n].cpu().numpy().view(np.uint32)
    g = pl.gscreen[:s.n].T.cpu().numpy()
    want = oracle.densify_accumulate(tiles, g, np.zeros((s.n, 2), np.float32))
    want = oracle.densify_accumulate(tiles, g, want)
    np.testing.assert_array_equal(pl.dstats[:s.n].cpu().numpy(), want)
    assert (want[:, 1] > 0).sum() > 100


def test_projecting_update_accumulates_this_steps_observations(torch_cuda):
    """The statistics added by gs_render_bwd_adam_project (fused into its chain kernel)
    against gs_densify_accumulate after gs_render_bwd_adam on the same step: counts equal,
    lengths equal up to the order of the gradient atomics."""
    torch = torch_cuda
    from differentiable_tile_gaussian_amd import gs
    wl = scenes.CONFIGS[2]()
    cam2 = gs.make_camera(scenes.look_at_origin((3.0, 0.5, -2.5), 800, 800, 1100.0))
    rng = np.random.default_rng(3)
    dLdI = torch.from_numpy((rng.standard_normal((3, 800, 800)) * 1e-3).astype(np.float32)).cuda()
    res = []
    for fused in (True, False):
        pl, c = pu.gpu_forward(wl.scene.params, 3, wl.cameras[0])
        pl.enable_density_stats()
        pl.dLdI.copy_(dLdI)
        pl.t = 1
        if fused:
            gs.gs_render_bwd_adam_project(pl.params, 3, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc,
                                          pl.dLdI, pl.gscreen, pl.m, pl.v, pl.lr, 0.9, 0.999, 1e-8, 1, pl.ws_render,
                                          cam2, pl.proj, pl.ws_pre, pl.dstats)
        else:
            gs.gs_render_bwd_adam(pl.params, 3, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI,
                                  pl.gscreen, pl.m, pl.v, pl.lr, 0.9, 0.999, 1e-8, 1, pl.ws_render)
            gs.gs_densify_accumulate(pl.proj, pl.gscreen, pl.dstats)
        torch.cuda.synchronize()
        res.append(pl.dstats[:pl.n].cpu().numpy())
    np.testing.assert_array_equal(res[0][:, 1], res[1][:, 1])
    np.testing.assert_allclose(res[0][:, 0], res[1][:, 0], rtol=1e-4, atol=1e-12)
    assert (res[0][:, 1] > 0).sum() > 1000


def test_training_loop_with_density_control(torch_cuda):
    """Pipeline: fused steps that accumulate statistics, a densification, and fused steps
    on the new population; after it, the projection the last update made for the next
    camera equals gs_preprocess of the parameters it wrote."""
    torch = torch_cuda
    from differentiable_tile_gaussian_amd import gs
    from differentiable_tile_gaussian_amd.pipeline import Pipeline
    wl = scenes.CONFIGS[2]()
    cams = [gs.make_camera(c) for c in (wl.cameras[0],
                                        scenes.look_at_origin((3.0, 0.5, -2.5), 800, 800, 1100.0),
                                        scenes.look_at_origin((-3.5, -0.4, -2.0), 800, 800, 1100.0))]
    rng = np.random.default_rng(6)
    targets = [torch.from_numpy(rng.random((3, 800, 800), dtype=np.float32)).cuda() for _ in cams]
    pl = Pipeline(torch.from_numpy(wl.scene.params).cuda(), 3, 800, 800)
    pl.enable_density_stats()
    for k in range(6):
        pl.step(cams[k % 3], targets[k % 3], next_cam=cams[(k + 1) % 3])
    torch.cuda.synchronize()
    st = pl.dstats[:pl.n].cpu().numpy()
    assert st[:, 1].max() <= 6 and (st[:, 1] > 0).sum() > 1000
    thr = float(np.quantile(st[st[:, 1] > 0, 0] / st[st[:, 1] > 0, 1], 0.9))
    n0 = pl.n
    counts = pl.densify(thr, 0.005, 1.0, 0.01, generator=torch.Generator(device="cuda").manual_seed(1))
    kept, cloned, split = counts
    assert pl.n == kept + cloned + 2 * split and cloned + split > 0 and kept <= n0
    for k in range(3):
        loss = pl.step(cams[k], targets[k], next_cam=cams[(k + 1) % 3])
    torch.cuda.synchronize()
    assert np.isfinite(loss.cpu().numpy()).all()
    ref = gs.Proj(pl.n)
    pairs = gs.gs_preprocess(pl.params, 3, cams[0], ref, gs.workspace(gs.GS_WS_PREPROCESS, n=pl.n))
    torch.cuda.synchronize()
    assert pairs == pl.pairs
    for name in ("splat", "depth", "rect", "tiles"):
        a = getattr(pl.proj, name)[:pl.n].cpu().numpy()
        b = getattr(ref, name)[:pl.n].cpu().numpy()
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32), err_msg=name)


def test_scheduled_density_control_and_sh_ramp(torch_cuda):
    """Pipeline.after_step with a compressed TrainingSchedule (densify after steps 2 and 4,
    the opacity reset with the one after step 4, one more SH band every two steps): the
    population changes only after those steps, by the counts gs_densify reports, every
    opacity is at most the cap right after the reset, and each step passes the active SH
    degree the ramp gives."""
    import math
    torch = torch_cuda
    from differentiable_tile_gaussian_amd import gs
    from differentiable_tile_gaussian_amd.pipeline import Pipeline, TrainingSchedule
    s = scenes.random_scene(71, 4000, 3, spread=1.3, logscale_std=0.5)
    s.params[0:3] *= 0.8
    cams = [gs.make_camera(scenes.look_at_origin((0.6, 0.4, -4.5), 160, 120, 150.0)),
            gs.make_camera(scenes.look_at_origin((-2.5, 0.2, -3.8), 160, 120, 150.0))]
    rng = np.random.default_rng(8)
    targets = [torch.from_numpy(rng.random((3, 120, 160), dtype=np.float32)).cuda() for _ in cams]
    sched = TrainingSchedule(start=1, every=2, stop=6, reset_every=4, sh_every=2)
    pl = Pipeline(torch.from_numpy(s.params).cuda(), 3, 160, 120, cfg=gs.GsConfig(active_sh_degree=sched.sh_degree(1, 3)))
    pl.enable_density_stats()
    gen = torch.Generator(device="cuda").manual_seed(3)
    cap = float(np.float32(math.log(0.01 / 0.99)))
    for t in range(1, 7):
        assert pl.cfg.active_sh_degree == sched.sh_degree(t, 3)
        loss = pl.step(cams[t % 2], targets[t % 2], next_cam=cams[(t + 1) % 2])
        assert pl.t == t
        n0 = pl.n
        counts = pl.after_step(sched, 0.0, 0.005, 1.0, 0.05, generator=gen)
        torch.cuda.synchronize()
        assert np.isfinite(loss.cpu().numpy()).all()
        if t in (2, 4):
            kept, cloned, split = counts
            assert pl.n == kept + cloned + 2 * split and cloned + split > 0
        else:
            assert counts is None and pl.n == n0
        if t == 4:
            assert (pl.planar(pl.params)[10].cpu().numpy() <= cap).all()
