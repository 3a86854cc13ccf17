"""GPU (HIP, through the C ABI) against the CPU oracle, stage by stage.

Keys, values, tile ranges, counts, rectangles and depths bit-exact; pixels within
1e-5 absolute; gradients within 1e-3 relative (per element against |g| plus the
group's rms, and in norm).  Pixels whose skip/stop decisions sit within 1e-5 of a
threshold are excluded from the tight pixel check and counted; Gaussians seen by
such pixels are excluded from the tight gradient check.
"""
import math

import numpy as np
import pytest

from differentiable_tile_gaussian_amd import scenes
from tests import parity_util as pu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _small_cases():
    cases = []
    for seed, (n, deg, w, h) in enumerate([(300, 0, 100, 70), (500, 1, 64, 64), (800, 2, 130, 97),
                                          (1200, 3, 161, 33), (64, 3, 17, 300)]):
        cases.append((seed, n, deg, w, h))
    return cases


def _scene_and_camera(seed, n, deg, w, h):
    s = scenes.random_scene(100 + seed, n, deg, spread=1.3, logscale_std=0.6, logit_std=1.5)
    th = 0.3 * seed
    cam = scenes.look_at_origin((4.5 * math.sin(th), 0.4, -4.5 * math.cos(th)), w, h, 0.9 * max(w, h))
    s.params[0:3] -= np.array([[0.0], [0.0], [4.5]], np.float32)   # centre the cloud on the origin
    s.params[0:3] *= 0.8
    return s, cam


def _oracle_all(oracle, params, deg, cam, dLdI=None):
    pre, keys, vals, ranges, fwd = oracle.forward(params, deg, cam)
    out = dict(pre=pre, keys=keys, vals=vals, ranges=ranges, fwd=fwd)
    if dLdI is not None:
        gscreen, mass, count = oracle.render_bwd(pre, vals, ranges, cam, fwd, dLdI, with_mass=True)
        out["gscreen"] = gscreen
        out["slack"] = oracle.rounding_slack(mass, count)
        out["gparams"] = oracle.preprocess_bwd(params, deg, cam, gscreen)
    else:
        dLdI = np.zeros((3, cam.height, cam.width), np.float32)
    out["risk"] = oracle.flip_risk(pre, vals, ranges, cam, dLdI)
    return out


@pytest.mark.parametrize("case", _small_cases())
def test_forward_stages_small(torch_cuda, oracle, case):
    seed, n, deg, w, h = case
    print(f"case seed={seed} n={n} deg={deg} {w}x{h}", flush=True)
    s, cam = _scene_and_camera(*case)
    o = _oracle_all(oracle, s.params, deg, cam)
    pl, c = pu.gpu_forward(s.params, deg, cam)
    pu.check_preprocess(pu.proj_to_numpy(pl), o["pre"])
    assert pl.pairs == len(o["keys"]) > 0
    keys, vals, ranges = pu.sorted_to_numpy(pl)
    np.testing.assert_array_equal(keys, pu.tile_of_key(o["keys"]))
    np.testing.assert_array_equal(vals, o["vals"])
    np.testing.assert_array_equal(ranges, o["ranges"])
    pu.check_render(pu.render_to_numpy(pl), o["fwd"], o["risk"])


@pytest.mark.parametrize("case", _small_cases())
def test_backward_small(torch_cuda, oracle, case):
    torch = torch_cuda
    seed, n, deg, w, h = case
    print(f"case seed={seed} n={n} deg={deg} {w}x{h}", flush=True)
    s, cam = _scene_and_camera(*case)
    dLdI = (np.random.default_rng(seed).standard_normal((3, h, w)) * 1e-3).astype(np.float32)
    o = _oracle_all(oracle, s.params, deg, cam, dLdI)
    pl, c = pu.gpu_forward(s.params, deg, cam)
    o["risk"] = pu.observed_risk(oracle, o, cam, pu.render_to_numpy(pl), dLdI)
    pl.dLdI.copy_(torch.from_numpy(dLdI))
    from differentiable_tile_gaussian_amd import gs
    gs.gs_render_bwd(pl.params, deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI, pl.gscreen,
                     pl.grads, pl.ws_render)
    torch.cuda.synchronize()
    gscreen = pl.gscreen[:n].T.cpu().numpy()
    gparams = pl.planar(pl.grads).cpu().numpy()
    pu.check_screen_grads(gscreen, o["gscreen"], o["risk"]["g"], o["slack"])
    keep = pu.calm(o["risk"]["g"], o["gscreen"])
    print(f"  flips {o['risk']['flips']}, gaussians not calm: {int((~keep).sum())} of {n}", flush=True)
    pu.check_param_grads(gparams, o, oracle, s.params, deg, cam, keep)
    # culled Gaussians get exactly zero
    culled = o["pre"]["tiles"] == 0
    assert np.all(gparams[:, culled] == 0.0)


def test_backward_into_unaligned_screen_gradients(torch_cuda):
    """The screen partials written through a pointer that is not 16-byte aligned (the
    clear then takes its 4-byte path over the whole array): equal to the aligned result
    after the same forward, with stale values in the buffer beforehand.  Float sums whose
    atomics may land in another order, so within rounding."""
    torch = torch_cuda
    from differentiable_tile_gaussian_amd import gs
    case = _small_cases()[2]
    seed, n, deg, w, h = case
    s, cam = _scene_and_camera(*case)
    pl, c = pu.gpu_forward(s.params, deg, cam)
    dLdI = (np.random.default_rng(seed).standard_normal((3, h, w)) * 1e-3).astype(np.float32)
    pl.dLdI.copy_(torch.from_numpy(dLdI))
    gs.gs_render_bwd(pl.params, deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI, pl.gscreen,
                     pl.grads, pl.ws_render)
    torch.cuda.synchronize()
    ref = pl.gscreen[:n].cpu().numpy().astype(np.float64)
    big = torch.full((9 * n + 8,), 7.0, dtype=torch.float32, device="cuda")   # stale values
    un = big[1:1 + 9 * n].view(n, 9)
    assert un.data_ptr() % 16 != 0
    gs.gs_render_bwd(pl.params, deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI, un,
                     pl.grads, pl.ws_render)
    torch.cuda.synchronize()
    got = un.cpu().numpy().astype(np.float64)
    scale = np.abs(ref).max(axis=0) + 1e-30
    assert np.all(np.abs(got - ref) <= 1e-5 * scale), float((np.abs(got - ref) / scale).max())
    # the words around the array are untouched
    assert float(big[0]) == 7.0 and float(big[9 * n + 1]) == 7.0


def _full_step_checks(torch, gs, oracle, pl, c, ref, target, params, deg, cam):
    """Every stage of one step against the oracle: projection, pairs and ranges
    bit-exact; pixels, loss and image gradient; then the backward fed the oracle's
    image gradient (so that only the blend's own decisions can differ): all screen
    partials with their flip risk, parameter gradients of the calm Gaussians.
    Returns the GPU's parameter gradients [P][n]."""
    n = ref["pre"]["n"]
    pu.check_preprocess(pu.proj_to_numpy(pl), ref["pre"])
    keys, vals, ranges = pu.sorted_to_numpy(pl)
    np.testing.assert_array_equal(keys, pu.tile_of_key(ref["keys"]))
    np.testing.assert_array_equal(vals, ref["vals"])
    np.testing.assert_array_equal(ranges, ref["ranges"])
    render = pu.render_to_numpy(pl)
    ref["risk"] = pu.observed_risk(oracle, ref, cam, render, ref["dLdI"])
    px = pu.check_render(render, ref["fwd"], ref["risk"])
    tgt = torch.from_numpy(target).cuda()
    gs.gs_loss_l1_dssim(pl.rgb, tgt, pl.lam, pl.loss, pl.dLdI, pl.ws_loss)
    torch.cuda.synchronize()
    n_img = pu.check_loss(pl.loss.cpu().numpy(), pl.dLdI.cpu().numpy(), ref, target)
    # the loss on the oracle's own image: every element of dL/dimage against the oracle
    (terms, g_ref, mag) = oracle.loss(ref["fwd"]["rgb"], target, pl.lam, with_mag=True)
    img = torch.from_numpy(np.ascontiguousarray(ref["fwd"]["rgb"], np.float32)).cuda()
    out = torch.zeros(3, device="cuda")
    g = torch.empty_like(img)
    gs.gs_loss_l1_dssim(img, tgt, pl.lam, out, g, pl.ws_loss)
    torch.cuda.synchronize()
    pu.check_loss_everywhere(out.cpu().numpy(), g.cpu().numpy(), terms, g_ref, mag)
    pl.dLdI.copy_(torch.from_numpy(np.ascontiguousarray(ref["dLdI"], np.float32)))
    gs.gs_render_bwd(pl.params, deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI, pl.gscreen,
                     pl.grads, pl.ws_render)
    torch.cuda.synchronize()
    pu.check_screen_grads(pl.gscreen[:n].T.cpu().numpy(), ref["gscreen"], ref["risk"]["g"], ref["slack"])
    keep = pu.calm(ref["risk"]["g"], ref["gscreen"])
    g = pl.planar(pl.grads).cpu().numpy()
    pu.check_param_grads(g, ref, oracle, params, deg, cam, keep)
    print(f"  flips {ref['risk']['flips']} over {px['near']} px; image-gradient elements checked on the GPU's "
          f"image {n_img}; Gaussians not calm {int((~keep).sum())} of {n}", flush=True)
    return g


def test_config1_full_step(torch_cuda, oracle):
    """The tiny workload end to end, including the loss and one Adam step."""
    torch = torch_cuda
    from differentiable_tile_gaussian_amd import gs
    wl = scenes.config1()
    cam = wl.cameras[0]
    deg = wl.scene.sh_degree
    target = oracle.forward(wl.target_scene.params, deg, cam)[4]["rgb"]
    ref = oracle.train_step_grads(wl.scene.params, deg, cam, target)
    pl, c = pu.gpu_forward(wl.scene.params, deg, cam)
    gparams = _full_step_checks(torch, gs, oracle, pl, c, ref, target, wl.scene.params, deg, cam)
    # one Adam step from zero moments, against the oracle's fp64 Adam on the GPU's gradient
    p0 = wl.scene.params.astype(np.float64)
    pl.adam()
    torch.cuda.synchronize()
    lr = np.array([1.6e-4, 5e-3, 1e-3, 5e-2, 2.5e-3])
    p_ref, m_ref, v_ref = oracle.adam(p0, gparams.astype(np.float64), np.zeros_like(p0), np.zeros_like(p0), deg,
                                      lr, step=1)
    np.testing.assert_allclose(pl.planar(pl.params).cpu().numpy(), p_ref, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(pl.planar(pl.m).cpu().numpy(), m_ref, rtol=1e-6, atol=1e-12)
    np.testing.assert_allclose(pl.planar(pl.v).cpu().numpy(), v_ref, rtol=1e-6, atol=1e-14)
    del gs


def test_loss_parity(torch_cuda, oracle):
    torch = torch_cuda
    from differentiable_tile_gaussian_amd import gs
    for (h, w) in [(37, 53), (128, 128), (200, 77), (1080, 1920)]:
        img = scenes.random_image(h * w, h, w)
        tgt = np.clip(img + 0.1 * np.random.default_rng(w).standard_normal(img.shape).astype(np.float32), 0, 1)
        terms, g_ref, mag = oracle.loss(img, tgt, 0.2, with_mag=True)
        ti, tt = torch.from_numpy(img).cuda(), torch.from_numpy(tgt).cuda()
        out = torch.zeros(3, device="cuda")
        g = torch.empty_like(ti)
        ws = gs.workspace(gs.GS_WS_LOSS, W=w, H=h)
        gs.gs_loss_l1_dssim(ti, tt, 0.2, out, g, ws)
        torch.cuda.synchronize()
        pu.check_loss_everywhere(out.cpu().numpy(), g.cpu().numpy(), terms, g_ref, mag)


def _blocked_np(planar):
    """The blocked layout written out from its definition (numpy), padding NaN."""
    P, n = planar.shape
    groups = (n + 63) // 64
    out = np.full((groups, P, 64), np.nan, np.float32)
    for i in range(n):
        out[i // 64, :, i % 64] = planar[:, i]
    return out


@pytest.mark.parametrize("n,deg", [(1, 0), (64, 3), (129, 1), (1003, 2)])
def test_layout_round_trip(torch_cuda, n, deg):
    torch = torch_cuda
    from differentiable_tile_gaussian_amd import gs
    P = scenes.num_planes(deg)
    a = np.random.default_rng(n).standard_normal((P, n)).astype(np.float32)
    b = gs.to_blocked(torch.from_numpy(a).cuda(), deg)
    torch.cuda.synchronize()
    assert b.numel() == gs.gs_param_floats(n, deg) == ((n + 63) // 64) * 64 * P
    want = _blocked_np(a)
    got = b.cpu().numpy()
    pad = np.isnan(want)
    np.testing.assert_array_equal(got[~pad], want[~pad])
    assert np.all(got[pad] == 0.0)
    back = gs.from_blocked(b, n, deg).cpu().numpy()
    np.testing.assert_array_equal(back, a)


@pytest.mark.parametrize("aligned", [True, False])
def test_adam_parity(torch_cuda, oracle, aligned):
    """gs_adam_step on blocked arrays (the vector kernel when 16-byte aligned, the
    scalar one otherwise) against the oracle's fp64 Adam; padding is left untouched."""
    torch = torch_cuda
    from differentiable_tile_gaussian_amd import gs
    rng = np.random.default_rng(3)
    for n, deg in [(1003, 3), (4096, 0), (1, 1), (130, 2)]:
        P = scenes.num_planes(deg)
        th = rng.standard_normal((P, n)).astype(np.float32)
        g = rng.standard_normal((P, n)).astype(np.float32)
        m = (0.1 * rng.standard_normal((P, n))).astype(np.float32)
        v = (0.01 * rng.random((P, n))).astype(np.float32)
        lr = np.array([1.6e-4, 5e-3, 1e-3, 5e-2, 2.5e-3])
        ref = oracle.adam(th, g, m, v, deg, lr, step=7)
        nf = gs.gs_param_floats(n, deg)
        T = []
        for a in (th, g, m, v):
            buf = torch.full((nf + 1,), 7.0, dtype=torch.float32, device="cuda")
            t = buf[:nf] if aligned else buf[1:]
            gs.to_blocked(torch.from_numpy(a).cuda(), deg, out=t)
            padding = np.isnan(_blocked_np(a).reshape(-1))
            t[torch.from_numpy(padding).cuda()] = 7.0     # sentinel in the padding slots
            T.append(t)
        gs.gs_adam_step(T[0], T[1], T[2], T[3], n, deg, lr, 0.9, 0.999, 1e-8, 7)
        torch.cuda.synchronize()
        out = [gs.from_blocked(t, n, deg).cpu().numpy() for t in T]
        padmask = np.isnan(_blocked_np(th).reshape(-1))
        for t in (T[0], T[2], T[3]):
            assert np.all(t.cpu().numpy()[padmask] == 7.0)
        # fp32 rounding is relative to the operands of each update, which can cancel
        m_scale = 0.9 * np.abs(m) + 0.1 * np.abs(g)
        v_scale = 0.999 * np.abs(v) + 0.001 * g * g
        assert np.all(np.abs(out[2] - ref[1]) <= 1e-6 * m_scale + 1e-30)
        assert np.all(np.abs(out[3] - ref[2]) <= 1e-6 * v_scale + 1e-30)
        # one fp32 rounding of theta itself plus a small relative error on the step
        bound = 1.2e-7 * np.abs(ref[0]) + 1e-5 * np.abs(th - ref[0]) + 1e-12
        assert np.all(np.abs(out[0] - ref[0]) <= bound)


# ---------------------------------------------------------------- edge cases
def test_empty_scene(torch_cuda, oracle):
    import torch
    cam = scenes.identity_camera(40, 30, 40.0)
    cam.bg = (0.2, 0.3, 0.4)
    params = np.zeros((14, 0), np.float32)
    from differentiable_tile_gaussian_amd import gs
    from differentiable_tile_gaussian_amd.pipeline import Pipeline
    pl = Pipeline(torch.zeros((14, 0), device="cuda"), 0, 40, 30)
    c = gs.make_camera(cam)
    pl.forward(c)
    torch.cuda.synchronize()
    assert pl.pairs == 0
    rgb = pl.rgb.cpu().numpy()
    np.testing.assert_allclose(rgb, np.broadcast_to(np.array(cam.bg, np.float32)[:, None, None], rgb.shape))
    assert np.all(pl.nc.cpu().numpy() == 0) and np.all(pl.T.cpu().numpy() == 1.0)
    pl.backward(c, torch.zeros((3, 30, 40), device="cuda"))
    torch.cuda.synchronize()
    del params, oracle


def test_single_gaussian_and_all_culled(torch_cuda, oracle):
    cam = scenes.identity_camera(48, 48, 60.0)
    s = scenes.random_scene(5, 1, 0)
    s.params[0:3, 0] = (0.0, 0.0, 3.0)
    o = _oracle_all(oracle, s.params, 0, cam)
    pl, c = pu.gpu_forward(s.params, 0, cam)
    pu.check_preprocess(pu.proj_to_numpy(pl), o["pre"])
    pu.check_render(pu.render_to_numpy(pl), o["fwd"], o["risk"])
    # everything behind the camera or with a zero quaternion
    s2 = scenes.random_scene(6, 200, 0)
    s2.params[2, :100] = -s2.params[2, :100]
    s2.params[6:10, 100:] = 0.0
    pl2, _ = pu.gpu_forward(s2.params, 0, cam)
    assert pl2.pairs == 0
    assert np.all(pl2.proj.tiles.cpu().numpy() == 0)


def test_all_in_one_tile_and_non_finite(torch_cuda, oracle):
    cam = scenes.identity_camera(64, 64, 200.0, 8.0, 8.0)
    s = scenes.random_scene(8, 700, 3, spread=0.01, logscale_mean=math.log(0.002), logscale_std=0.2)
    s.params[3, 0] = np.nan          # non-finite scale: culled, not binned
    s.params[0, 1] = np.inf
    o = _oracle_all(oracle, s.params, 3, cam)
    assert o["pre"]["tiles"][0] == 0 and o["pre"]["tiles"][1] == 0
    pl, c = pu.gpu_forward(s.params, 3, cam)
    pu.check_preprocess(pu.proj_to_numpy(pl), o["pre"])
    keys, vals, ranges = pu.sorted_to_numpy(pl)
    np.testing.assert_array_equal(keys, pu.tile_of_key(o["keys"]))
    np.testing.assert_array_equal(vals, o["vals"])
    np.testing.assert_array_equal(ranges, o["ranges"])
    pu.check_render(pu.render_to_numpy(pl), o["fwd"], o["risk"])


@pytest.mark.parametrize("far", [900.0, 5.0e4])
def test_depth_order_over_a_wide_depth_range(torch_cuda, oracle, far):
    """Depths from just above znear to far, log-uniform, with runs of exactly equal
    depths (ties broken by id).  At far = 5e4 the depth key (the depth's bits less
    znear's) needs more than 27 bits, so the depth sort makes its fourth pass; at 900 it
    makes three.  Pairs and ranges bit-exact against the oracle."""
    n, w, h, f = 3000, 96, 80, 60.0
    rng = np.random.default_rng(int(far))
    s = scenes.random_scene(40, n, 0)
    cam = scenes.identity_camera(w, h, f)
    z = np.exp(rng.uniform(math.log(cam.znear * 1.0001), math.log(far), n)).astype(np.float32)
    z[:40] = np.float32(cam.znear) * np.float32(1.0000001)   # just above the near plane
    z[40:400] = z[400]                                         # one long run of equal depths
    z[1000:1100:3] = np.float32(far)                           # equal depths at the far end
    s.params[2] = z
    s.params[0] = rng.uniform(-0.7, 0.7, n).astype(np.float32) * z * (w / (2 * f))
    s.params[1] = rng.uniform(-0.7, 0.7, n).astype(np.float32) * z * (h / (2 * f))
    s.params[3:6] = np.log(0.04 * z)[None, :].astype(np.float32) + rng.normal(0, 0.2, (3, n)).astype(np.float32)
    d_bits = z.view(np.uint32).astype(np.int64) - np.array([cam.znear], np.float32).view(np.uint32)[0]
    assert (d_bits.max() >= 1 << 27) == (far > 2.0e4)
    pre, okeys, ovals, oranges, _ = oracle.forward(s.params, 0, cam)
    assert int((pre["tiles"] > 0).sum()) > n // 2
    pl, c = pu.gpu_forward(s.params, 0, cam)
    keys, vals, ranges = pu.sorted_to_numpy(pl)
    assert pl.pairs == len(okeys)
    np.testing.assert_array_equal(keys, pu.tile_of_key(okeys))
    np.testing.assert_array_equal(vals, ovals)
    np.testing.assert_array_equal(ranges, oranges)


def test_capacity_error_writes_nothing(torch_cuda):
    import torch
    from differentiable_tile_gaussian_amd import gs
    cam = scenes.identity_camera(64, 64, 60.0)
    s = scenes.random_scene(9, 300, 0)
    pl, c = pu.gpu_forward(s.params, 0, cam)
    keys = torch.full((pl.pairs - 1,), 7, dtype=torch.int32, device="cuda")
    vals = torch.full((pl.pairs - 1,), 7, dtype=torch.int32, device="cuda")
    ranges = torch.full((2, 16), 7, dtype=torch.int32, device="cuda")
    with pytest.raises(gs.GsError) as e:
        gs.gs_bin_sort(pl.proj, c, pl.pairs, keys, vals, ranges, pl.ws_sort)
    assert e.value.status == gs.GS_ERR_CAPACITY
    torch.cuda.synchronize()
    assert int(keys.min()) == 7 and int(ranges.min()) == 7


# ------------------------------------------------------------- split path
# Small split sizes force every long tile through the chunked forward (exact first
# segment, speculative chunks, combine, re-walk of the stopping chunk) and the
# chunk-parallel backward; results must still match the sequential oracle.
def _deep_case():
    s = scenes.random_scene(501, 2500, 1, spread=2.5, logscale_mean=math.log(0.12), logscale_std=0.4,
                            logit_mean=0.5, logit_std=1.0)
    cam = scenes.identity_camera(72, 56, 60.0)
    return s, cam


# (which scene, (split_first, split_chunk)); the largest split runs on the deep scene only,
# the one whose lists are longer than its 384 pairs
_SPLIT_CASES = [(w, t) for w in ("deep", "small3", "small2") for t in ((16, 8), (64, 32), (12, 4), (256, 128))
                if w == "deep" or t != (256, 128)]


@pytest.mark.parametrize("which,tune", _SPLIT_CASES, ids=[f"{w}-{t[0]}-{t[1]}" for w, t in _SPLIT_CASES])
def test_split_path_parity(torch_cuda, oracle, tune, which):
    torch = torch_cuda
    from differentiable_tile_gaussian_amd import gs
    cfg = gs.GsConfig(split_first=tune[0], split_chunk=tune[1])
    if which == "deep":
        s, cam = _deep_case()
    else:
        s, cam = _scene_and_camera(*_small_cases()[int(which[-1])])
    deg = s.sh_degree
    print(f"split {which} first={tune[0]} chunk={tune[1]}", flush=True)
    dLdI = (np.random.default_rng(11).standard_normal((3, cam.height, cam.width)) * 1e-3).astype(np.float32)
    o = _oracle_all(oracle, s.params, deg, cam, dLdI)
    lens = (o["ranges"][1].astype(np.int64) - o["ranges"][0])
    if lens.max() <= tune[0] + tune[1]:
        pytest.skip("no tile list long enough for this split size")
    pl, c = pu.gpu_forward(s.params, deg, cam, cfg)
    o["risk"] = pu.observed_risk(oracle, o, cam, pu.render_to_numpy(pl), dLdI)
    px = pu.check_render(pu.render_to_numpy(pl), o["fwd"], o["risk"])
    pl.dLdI.copy_(torch.from_numpy(dLdI))
    gs.gs_render_bwd(pl.params, deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI, pl.gscreen,
                     pl.grads, pl.ws_render, cfg=cfg)
    torch.cuda.synchronize()
    pu.check_screen_grads(pl.gscreen[:s.n].T.cpu().numpy(), o["gscreen"], o["risk"]["g"], o["slack"])
    keep = pu.calm(o["risk"]["g"], o["gscreen"])
    g = pl.planar(pl.grads).cpu().numpy()
    pu.check_param_grads(g, o, oracle, s.params, deg, cam, keep)
    stopped = float((o["fwd"]["T"] < 1e-4).mean())
    print(f"  px with a near decision {px['near']}, not calm G {int((~keep).sum())}, saturated px {stopped:.2f}",
          flush=True)


def test_backward_walks_the_forwards_split(torch_cuda):
    """The backward takes the split sizes from the forward's workspace header: a backward
    called with other split sizes than its forward (larger or smaller, so its launch has
    fewer or more chunk blocks than the forward made chunks) gives the same gradients bit
    for bit (fixed-point sums: no reordering); a workspace that no forward of this image
    wrote gives NaN everywhere instead of reading a stale split state."""
    torch = torch_cuda
    from differentiable_tile_gaussian_amd import gs
    s, cam = _deep_case()
    fwd_cfg = gs.GsConfig(grad_sums=gs.GS_GRAD_SUMS_FIXED, split_first=16, split_chunk=8)
    dLdI = torch.from_numpy((np.random.default_rng(12).standard_normal((3, cam.height, cam.width)) * 1e-3)
                            .astype(np.float32)).cuda()
    grads = {}
    for name, bwd in (("same", (16, 8)), ("larger", (2048, 512)), ("smaller", (8, 4))):
        bwd_cfg = gs.GsConfig(grad_sums=gs.GS_GRAD_SUMS_FIXED, split_first=bwd[0], split_chunk=bwd[1])
        pl, c = pu.gpu_forward(s.params, s.sh_degree, cam, fwd_cfg)
        need = gs.gs_workspace_bytes(gs.GS_WS_RENDER, s.n, pl.pairs, cam.width, cam.height, bwd_cfg)
        if pl.ws_render.numel() < need:     # the backward's own sizing may ask for more
            ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
            ws[:pl.ws_render.numel()].copy_(pl.ws_render)
            pl.ws_render = ws
        pl.dLdI.copy_(dLdI)
        gs.gs_render_bwd(pl.params, s.sh_degree, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI,
                         pl.gscreen, pl.grads, pl.ws_render, cfg=bwd_cfg)
        torch.cuda.synchronize()
        grads[name] = pl.planar(pl.grads).cpu().numpy()
    assert np.isfinite(grads["same"]).all() and np.abs(grads["same"]).max() > 0
    for name in ("larger", "smaller"):
        np.testing.assert_array_equal(grads[name].view(np.uint32), grads["same"].view(np.uint32), err_msg=name)
    # a workspace no forward wrote: NaN partials and gradients, in both sum modes
    for mode in (gs.GS_GRAD_SUMS_FLOAT, gs.GS_GRAD_SUMS_FIXED):
        cfg = gs.GsConfig(grad_sums=mode)
        pl, c = pu.gpu_forward(s.params, s.sh_degree, cam, cfg)
        pl.ws_render.zero_()
        gs.gs_render_bwd(pl.params, s.sh_degree, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, dLdI,
                         pl.gscreen, pl.grads, pl.ws_render, cfg=cfg)
        torch.cuda.synchronize()
        assert torch.isnan(pl.gscreen[:s.n]).all()
        vis = torch.from_numpy(pl.proj.tiles[:s.n].cpu().numpy() > 0)
        # mean, scale, rotation and logit come from the (NaN) position, conic and opacity
        # partials; a clamped colour channel's coefficients get an exact 0
        assert torch.isnan(pl.planar(pl.grads).cpu()[0:11, vis]).all()


def test_two_configurations_in_one_process(torch_cuda, oracle):
    """Two pipelines with different settings (SH degree ramp at 1 with Mip compensation;
    the defaults), their calls interleaved: each renders what the oracle renders with its
    own settings.  No setting lives in the library between calls."""
    from differentiable_tile_gaussian_amd import gs
    s, cam = _scene_and_camera(*_small_cases()[3])
    deg = s.sh_degree
    cfg_a = gs.GsConfig(active_sh_degree=1, mip_compensation=True)
    pl_a, c = pu.gpu_forward(s.params, deg, cam, cfg_a)
    pl_b, _ = pu.gpu_forward(s.params, deg, cam)
    pl_a.forward(c)                     # again, after pl_b's calls
    torch_cuda.cuda.synchronize()
    zero = np.zeros((3, cam.height, cam.width), np.float32)
    for pl, active, mip in ((pl_a, 1, True), (pl_b, -1, False)):
        oracle.set_active_sh_degree(active)
        oracle.set_mip_compensation(mip)
        try:
            o = oracle.forward(s.params, deg, cam)
        finally:
            oracle.set_active_sh_degree(-1)
            oracle.set_mip_compensation(False)
        pu.check_preprocess(pu.proj_to_numpy(pl), o[0])
        risk = oracle.flip_risk(o[0], o[2], o[3], cam, zero)
        pu.check_render(pu.render_to_numpy(pl), o[4], risk)
    assert not np.array_equal(pl_a.rgb.cpu().numpy(), pl_b.rgb.cpu().numpy())


# ------------------------------------------------------- fused backward + Adam
@pytest.mark.parametrize("case", [_small_cases()[0], _small_cases()[3], "cfg1"])
def test_fused_backward_adam(torch_cuda, oracle, case):
    """gs_render_bwd_adam equals gs_render_bwd followed by gs_adam_step, and the oracle's
    fp64 Adam applied to the oracle's gradient, on two consecutive steps."""
    torch = torch_cuda
    from differentiable_tile_gaussian_amd import gs
    if case == "cfg1":
        wl = scenes.config1()
        s, cam = wl.scene, wl.cameras[0]
    else:
        s, cam = _scene_and_camera(*case)
    deg = s.sh_degree
    P = scenes.num_planes(deg)
    rng = np.random.default_rng(17)
    m0 = (1e-3 * rng.standard_normal((P, s.n))).astype(np.float32)
    v0 = (1e-6 * rng.random((P, s.n))).astype(np.float32)
    lr = (1.6e-4, 5e-3, 1e-3, 5e-2, 2.5e-3)
    dLdI = (rng.standard_normal((3, cam.height, cam.width)) * 1e-3).astype(np.float32)
    results = {}
    for mode in ("separate", "fused"):
        pl, c = pu.gpu_forward(s.params, deg, cam)
        pl.set_planar(pl.m, torch.from_numpy(m0))
        pl.set_planar(pl.v, torch.from_numpy(v0))
        pl.dLdI.copy_(torch.from_numpy(dLdI))
        if mode == "separate":
            gs.gs_render_bwd(pl.params, deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI,
                             pl.gscreen, pl.grads, pl.ws_render)
            gs.gs_adam_step(pl.params, pl.grads, pl.m, pl.v, s.n, deg, lr, 0.9, 0.999, 1e-8, 3)
        else:
            gs.gs_render_bwd_adam(pl.params, deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI,
                                  pl.gscreen, pl.m, pl.v, lr, 0.9, 0.999, 1e-8, 3, pl.ws_render)
        torch.cuda.synchronize()
        results[mode] = [pl.planar(t).cpu().numpy() for t in (pl.params, pl.m, pl.v)]
    th0 = s.params.astype(np.float64)
    for a, b in zip(results["separate"], results["fused"]):
        np.testing.assert_allclose(b, a, rtol=2e-6, atol=1e-9)
    # against the oracle: gradient from the oracle, Adam in fp64
    o = _oracle_all(oracle, s.params, deg, cam, dLdI)
    pl, _ = pu.gpu_forward(s.params, deg, cam)
    o["risk"] = pu.observed_risk(oracle, o, cam, pu.render_to_numpy(pl), dLdI)
    p_ref, m_ref, v_ref = oracle.adam(th0, o["gparams"].astype(np.float64), m0, v0, deg, np.array(lr), step=3)
    keep = pu.calm(o["risk"]["g"], o["gscreen"])
    # compare the applied updates (theta_new - theta) group by group with the gradient tolerance
    upd_gpu = results["fused"][0].astype(np.float64) - th0
    upd_ref = p_ref - th0
    for name, sl in pu.grad_groups(deg).items():
        pu.check_grad(upd_gpu[sl], upd_ref[sl], keep, rtol=2e-3, name="update " + name)
    pu.check_grad(results["fused"][1].astype(np.float64), m_ref, keep, name="m")


# ------------------------------------------------ larger workloads, whole image
@pytest.mark.timeout(400)        # the oracle alone takes about a minute on the 6M workload
@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_workload_full_step(torch_cuda, oracle, cfg):
    """One training step of each larger workload (camera 0) in the launch configuration the
    benchmark times (default split sizes, fused backward with Adam), against the oracle on
    the whole image: every stage as in _full_step_checks (unfused backward), then the
    fused backward with Adam against the unfused gradient's first Adam step."""
    torch = torch_cuda
    from differentiable_tile_gaussian_amd import gs
    wl = scenes.CONFIGS[cfg]()
    cam = wl.cameras[0]
    deg = wl.scene.sh_degree
    n = wl.scene.n
    print(f"workload {wl.name}: n={n} {cam.width}x{cam.height}", flush=True)
    target = np.random.default_rng(7 + cfg).random((3, cam.height, cam.width), dtype=np.float32)
    ref = oracle.train_step_grads(wl.scene.params, deg, cam, target)
    print(f"  oracle done: {len(ref['keys'])} pairs", flush=True)
    pl, c = pu.gpu_forward(wl.scene.params, deg, cam)
    g = _full_step_checks(torch, gs, oracle, pl, c, ref, target, wl.scene.params, deg, cam)
    # the fused backward with Adam from zero moments: step one moves each parameter by
    # -lr g / (|g| + eps) of its (fused, recomputed) gradient; where the sign of g is well
    # determined this must match the unfused gradient's prediction
    th0 = pl.planar(pl.params).cpu().numpy()
    pl.t = 0
    gs.gs_render_bwd_adam(pl.params, deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc, pl.dLdI,
                          pl.gscreen, pl.m, pl.v, pl.lr, pl.betas[0], pl.betas[1], pl.eps, 1, pl.ws_render)
    torch.cuda.synchronize()
    step = pl.planar(pl.params).cpu().numpy().astype(np.float64) - th0
    for grp, (name, sl) in enumerate(pu.grad_groups(deg).items()):
        lr = pl.lr[min(grp, 4)]
        gg = g[sl].astype(np.float64)
        st = step[sl]
        rms = np.sqrt((gg * gg).mean()) if gg.size else 0.0
        firm = np.abs(gg) >= 1e-2 * rms
        pred = -lr * gg / (np.abs(gg) + pl.eps)
        tol = 2e-3 * lr + 2e-7 * np.abs(th0[sl])
        assert np.all(np.abs(st - pred)[firm] <= tol[firm]), f"fused update {name}"
        assert np.all(np.abs(st) <= 1.01 * lr + 2e-7 * np.abs(th0[sl])), f"fused update bound {name}"


# ------------------------------------ update fused with the next camera's projection
def _proj_arrays(proj, n):
    nv = int(proj.n_visible.cpu().numpy().view(np.uint32)[0])
    return dict(splat=proj.splat[:n].cpu().numpy().view(np.uint32), depth=proj.depth[:n].cpu().numpy().view(np.uint32),
                rect=proj.rect[:n].cpu().numpy(), tiles=proj.tiles[:n].cpu().numpy(), n_visible=np.array([nv]),
                order=proj.order[:nv].cpu().numpy(), rect_order=proj.rect_order[:nv].cpu().numpy(),
                offs=proj.offs[:nv + 1].cpu().numpy())


@pytest.mark.timeout(300)
@pytest.mark.parametrize("case", ["small1", "small3", "small4", "cfg5"])
def test_update_with_next_projection(torch_cuda, case):
    """gs_render_bwd_adam_project (in place, as the benchmark calls it): the next camera's
    records, depths, rectangles, tile counts, depth order, rectangles in that order, pair
    offsets and pair count equal gs_preprocess of the parameters it wrote, bit for bit
    (the same contraction-free fp32 code, fed from registers instead of memory); and the
    update equals gs_render_bwd_adam's up to the order of the gradient atomics."""
    torch = torch_cuda
    from differentiable_tile_gaussian_amd import gs
    if case == "cfg5":
        wl = scenes.CONFIGS[5]()
        s, cam, cam2 = wl.scene, wl.cameras[0], wl.cameras[1]
    else:
        args = _small_cases()[int(case[-1])]
        s, cam = _scene_and_camera(*args)
        cam2 = _scene_and_camera(args[0] + 3, *args[1:])[1]   # the same image size, another orbit angle
    deg, n = s.sh_degree, s.n
    print(f"case {case}: n={n} {cam.width}x{cam.height}", flush=True)
    dLdI = (np.random.default_rng(5).standard_normal((3, cam.height, cam.width)) * 1e-3).astype(np.float32)
    c2 = gs.make_camera(cam2)
    pl, c = pu.gpu_forward(s.params, deg, cam)
    pl.dLdI.copy_(torch.from_numpy(dLdI))
    pairs = gs.gs_render_bwd_adam_project(pl.params, deg, pl.proj, pl.vals, pl.ranges, pl.pairs, c, pl.T, pl.nc,
                                          pl.dLdI, pl.gscreen, pl.m, pl.v, pl.lr, 0.9, 0.999, 1e-8, 1,
                                          pl.ws_render, c2, pl.proj, pl.ws_pre)
    torch.cuda.synchronize()
    fused = _proj_arrays(pl.proj, n)
    proj_b = gs.Proj(n)
    pairs_b = gs.gs_preprocess(pl.params, deg, c2, proj_b, gs.workspace(gs.GS_WS_PREPROCESS, n=n))
    torch.cuda.synchronize()
    ref = _proj_arrays(proj_b, n)
    assert pairs == pairs_b
    for k in ref:
        np.testing.assert_array_equal(fused[k], ref[k], err_msg=k)
    # the update against the call without the projection
    pl2, c_ = pu.gpu_forward(s.params, deg, cam)
    pl2.dLdI.copy_(torch.from_numpy(dLdI))
    gs.gs_render_bwd_adam(pl2.params, deg, pl2.proj, pl2.vals, pl2.ranges, pl2.pairs, c_, pl2.T, pl2.nc, pl2.dLdI,
                          pl2.gscreen, pl2.m, pl2.v, pl2.lr, 0.9, 0.999, 1e-8, 1, pl2.ws_render)
    torch.cuda.synchronize()
    for name, a, b in (("params", pl.params, pl2.params), ("m", pl.m, pl2.m), ("v", pl.v, pl2.v)):
        x, y = pl.planar(a).cpu().numpy(), pl2.planar(b).cpu().numpy()
        scale = np.abs(y).max() + 1e-30
        np.testing.assert_allclose(x, y, rtol=1e-5, atol=1e-5 * scale if name != "params" else 1e-5, err_msg=name)
