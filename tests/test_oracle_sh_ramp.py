"""The SH degree ramp in the oracle ([GSG] "Spherical harmonics": only the first
activeK = (activeDeg + 1)^2 - 1 band weights are summed; inactive ones get no gradient).

Pin: the planes of an SH degree-d scene are the first planes of a degree-3 scene (mean,
log-scale, quaternion, logit, DC, then the bands in order), so a degree-3 scene with the
active degree set to d must project, render and differentiate exactly as the degree-d
scene made of its first planes, with zero gradient on the remaining planes.
"""
import numpy as np
import pytest

from differentiable_tile_gaussian_amd import scenes


@pytest.fixture
def ramp(oracle):
    try:
        yield oracle
    finally:
        oracle.set_active_sh_degree(-1)


@pytest.mark.parametrize("d", [0, 1, 2])
def test_active_degree_equals_the_prefix_scene(ramp, d):
    oracle = ramp
    s = scenes.random_scene(12, 400, 3, spread=1.3)
    s.params[0:3] *= 0.8
    s.params[14:] = np.random.default_rng(3).normal(0, 0.3, s.params[14:].shape).astype(np.float32)
    cam = scenes.look_at_origin((0.5, 0.4, -4.5), 96, 80, 90.0)
    Pd = scenes.num_planes(d)
    prefix = np.ascontiguousarray(s.params[:Pd])
    oracle.set_active_sh_degree(-1)
    pre_d, _, vals_d, ranges_d, fwd_d = oracle.forward(prefix, d, cam)
    dLdI = np.random.default_rng(4).standard_normal((3, 80, 96)).astype(np.float32) * 1e-2
    g_d = oracle.preprocess_bwd(prefix, d, cam, oracle.render_bwd(pre_d, vals_d, ranges_d, cam, fwd_d, dLdI))
    oracle.set_active_sh_degree(d)
    pre_3, _, vals_3, ranges_3, fwd_3 = oracle.forward(s.params, 3, cam)
    for key in ("uv", "conic", "opac", "rgb", "depth", "rect", "tiles"):
        np.testing.assert_array_equal(pre_3[key], pre_d[key], err_msg=key)
    np.testing.assert_array_equal(fwd_3["rgb"], fwd_d["rgb"])
    g_3 = oracle.preprocess_bwd(s.params, 3, cam, oracle.render_bwd(pre_3, vals_3, ranges_3, cam, fwd_3, dLdI))
    np.testing.assert_array_equal(g_3[:Pd], g_d)
    assert not g_3[Pd:].any()
    assert np.abs(g_d[11:]).max() > 0


def test_no_ramp_is_every_band(ramp):
    oracle = ramp
    s = scenes.random_scene(13, 200, 2)
    cam = scenes.look_at_origin((0.0, 0.3, -4.0), 64, 64, 60.0)
    full = oracle.preprocess(s.params, 2, cam)
    for d in (2, 3, -1):
        oracle.set_active_sh_degree(d)
        np.testing.assert_array_equal(oracle.preprocess(s.params, 2, cam)["rgb"], full["rgb"])
