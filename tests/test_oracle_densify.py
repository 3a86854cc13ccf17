"""Density control in the oracle, pinned to hand-built cases and independent references.

[GST] density-control slide: average screen-position gradient over the visible
observations; small Gaussians with a large average are cloned, large ones split into
two children sampled around the parent with smaller scales, very transparent or
oversized ones pruned; opacity reset clamps opacity to at most a cap.  [GSG]
"Densification": split halves shrink by 1.6, a reshaped Gaussian restarts its Adam
moments.  The order of the new population and the thresholds are readings (R34).
"""
import math

import numpy as np
import pytest
from scipy.spatial.transform import Rotation

from differentiable_tile_gaussian_amd import scenes


def _population(n, deg, seed=0):
    s = scenes.random_scene(seed, n, deg)
    return s.params.copy()


def test_accumulate_closed_forms(oracle):
    n = 5
    g = np.zeros((9, n), np.float32)
    g[0], g[1] = [3, 0, 5, -8, 1], [4, 0, 12, 15, 1]
    tiles = np.array([1, 7, 0, 2, 3], np.uint32)
    st = oracle.densify_accumulate(tiles, g, np.zeros((n, 2), np.float32))
    # |(3, 4)| = 5, |(0, 0)| = 0, invisible untouched, |(-8, 15)| = 17, |(1, 1)| = sqrt 2
    np.testing.assert_array_equal(st[:, 0], np.array([5, 0, 0, 17, np.float32(math.sqrt(2))], np.float32))
    np.testing.assert_array_equal(st[:, 1], [1, 1, 0, 1, 1])
    st = oracle.densify_accumulate(tiles, g, st)
    np.testing.assert_array_equal(st[:, 1], [2, 2, 0, 2, 2])
    assert st[0, 0] == 10 and st[3, 0] == 34


THR = dict(grad_threshold=2e-4, prune_opacity=0.005, prune_scale=5.0, split_scale=0.05)


def _hand_case():
    """Seven Gaussians with known fates (comments), SH degree 0 (14 planes)."""
    p = _population(7, 0, seed=4)
    p[10] = 2.0                        # opacity 0.88
    p[3:6] = math.log(0.01)            # small
    stats = np.zeros((7, 2), np.float32)
    stats[:, 1] = 4.0
    stats[:, 0] = 4.0 * 1e-4           # average 1e-4: below the threshold
    p[10, 0] = math.log(0.001 / 0.999)                # 0: opacity 0.001 < 0.005 -> pruned
    p[4, 1] = math.log(10.0)                          # 1: scale 10 > 5 -> pruned
    #                                                   2: low gradient -> kept
    stats[3, 0] = 4.0 * 5e-4                          # 3: high gradient, small -> kept and cloned
    stats[4, 0] = 4.0 * 5e-4; p[5, 4] = math.log(0.2)  # 4: high gradient, scale 0.2 > 0.05 -> split
    stats[5] = (1.0, 0.0)                             # 5: never seen (count 0) -> kept
    stats[6, 0] = 1.0; p[10, 6] = -9.0                # 6: high gradient but opacity 1.2e-4 -> pruned
    return p, stats


def test_hand_built_population(oracle):
    p, stats = _hand_case()
    P, n = p.shape
    rng = np.random.default_rng(3)
    m = rng.standard_normal((P, n)).astype(np.float32)
    v = rng.random((P, n)).astype(np.float32)
    eps = rng.standard_normal((n, 2, 3)).astype(np.float32)
    r = oracle.densify(p, m, v, stats, eps, 0, **THR)
    np.testing.assert_array_equal(r["counts"], [3, 1, 1])        # kept {2, 3, 5}, cloned {3}, split {4}
    out = r["params"]
    assert out.shape == (P, 6)
    # order: kept in order, then clones, then the first and second children
    np.testing.assert_array_equal(out[:, 0], p[:, 2])
    np.testing.assert_array_equal(out[:, 1], p[:, 3])
    np.testing.assert_array_equal(out[:, 2], p[:, 5])
    np.testing.assert_array_equal(out[:, 3], p[:, 3])              # the clone is an exact copy
    np.testing.assert_array_equal(r["m"][:, :3], m[:, [2, 3, 5]])  # kept moments carry over
    np.testing.assert_array_equal(r["v"][:, :3], v[:, [2, 3, 5]])
    assert not r["m"][:, 3:].any() and not r["v"][:, 3:].any()     # new Gaussians start from zero
    assert not r["stats"].any()
    # split children: mean + R(q) (s * eps), scales / 1.6, everything else copied
    q = p[6:10, 4].astype(np.float64)
    rot = Rotation.from_quat([q[1], q[2], q[3], q[0]]).as_matrix()  # scipy takes (x, y, z, w)
    s = np.exp(p[3:6, 4].astype(np.float64))
    for c in range(2):
        child = out[:, 4 + c]
        want = p[0:3, 4].astype(np.float64) + rot @ (s * eps[4, c].astype(np.float64))
        np.testing.assert_allclose(child[0:3], want, rtol=0, atol=1e-6 * (1 + np.abs(want).max()))
        np.testing.assert_allclose(np.exp(child[3:6].astype(np.float64)), s / 1.6, rtol=3e-7)
        np.testing.assert_array_equal(child[6:], p[6:, 4])
    # the two children differ (different normals) and straddle nothing in particular
    assert not np.array_equal(out[0:3, 4], out[0:3, 5])


def test_threshold_is_inclusive_and_count_zero_is_kept(oracle):
    p = _population(3, 0, seed=5)
    p[10] = 3.0
    p[3:6] = math.log(0.01)
    thr = np.float32(2e-4)
    stats = np.array([[thr * 2, 2], [np.nextafter(thr, np.float32(0)) * 2, 2], [5.0, 0]], np.float32)
    z = np.zeros_like(p)
    r = oracle.densify(p, z, z, stats, np.zeros((3, 2, 3), np.float32), 0, **THR)
    # average exactly at the threshold densifies; one ulp below does not; no observations: kept
    np.testing.assert_array_equal(r["counts"], [3, 1, 0])
    np.testing.assert_array_equal(r["params"][:, 3], p[:, 0])


def test_zero_quaternion_splits_along_the_axes(oracle):
    p = _population(1, 0, seed=6)
    p[6:10, 0] = 0.0
    p[10] = 3.0
    p[3:6, 0] = [math.log(0.5), math.log(0.25), math.log(0.125)]
    stats = np.array([[1.0, 1.0]], np.float32)
    eps = np.array([[[1, 2, 3], [-1, 0, 0.5]]], np.float32)
    z = np.zeros_like(p)
    r = oracle.densify(p, z, z, stats, eps, 0, **THR)
    off = r["params"][0:3, :] - p[0:3, :1]
    np.testing.assert_allclose(off[:, 0], [0.5, 0.5, 0.375], rtol=1e-6)
    np.testing.assert_allclose(off[:, 1], [-0.5, 0.0, 0.0625], rtol=1e-6, atol=1e-7)


def test_opacity_reset_clamps_and_restarts_its_moments(oracle):
    p = _population(50, 1, seed=7)
    p[10] = np.linspace(-8, 6, 50, dtype=np.float32)
    rng = np.random.default_rng(8)
    m = rng.standard_normal(p.shape).astype(np.float32)
    v = rng.random(p.shape).astype(np.float32)
    stats = np.zeros((50, 2), np.float32)
    r = oracle.densify(p, m, v, stats, np.zeros((50, 2, 3), np.float32), 1, grad_threshold=1.0,
                       prune_opacity=1e-6, prune_scale=math.inf, split_scale=1.0, reset_opacity=True,
                       opacity_cap=0.01)
    np.testing.assert_array_equal(r["counts"], [50, 0, 0])
    o_in = 1 / (1 + np.exp(-p[10].astype(np.float64)))
    o_out = 1 / (1 + np.exp(-r["params"][10].astype(np.float64)))
    assert np.all(o_out <= 0.01 * (1 + 1e-6))
    low = o_in <= 0.01 * (1 - 1e-6)
    np.testing.assert_array_equal(r["params"][10][low], p[10][low])
    np.testing.assert_allclose(o_out[~low], 0.01, rtol=1e-6)
    assert not r["m"][10].any() and not r["v"][10].any()
    other = [k for k in range(p.shape[0]) if k != 10]
    np.testing.assert_array_equal(r["m"][other], m[other])
    np.testing.assert_array_equal(r["params"][other], p[other])


def test_random_population_invariants(oracle):
    n = 2000
    p = _population(n, 3, seed=9)
    rng = np.random.default_rng(10)
    p[10] = rng.normal(0, 3, n).astype(np.float32)
    stats = np.stack([rng.random(n) * 1e-3, rng.integers(0, 6, n)], 1).astype(np.float32)
    eps = rng.standard_normal((n, 2, 3)).astype(np.float32)
    z = np.zeros_like(p)
    r = oracle.densify(p, z, z, stats, eps, 3, **THR)
    kept, cloned, split = (int(x) for x in r["counts"])
    assert r["params"].shape[1] == kept + cloned + 2 * split
    # recompute the fates from the stated rules in fp64 (up to ties at the rounded thresholds)
    o = 1 / (1 + np.exp(-p[10].astype(np.float64)))
    smax = np.exp(p[3:6].astype(np.float64)).max(axis=0)
    prune = (o < 0.005) | (smax > 5.0)
    avg = np.where(stats[:, 1] > 0, stats[:, 0] / np.maximum(stats[:, 1], 1), 0)
    dens = ~prune & (avg >= 2e-4)
    assert kept == int((~prune & ~(dens & (smax > 0.05))).sum())
    assert cloned == int((dens & (smax <= 0.05)).sum())
    assert split == int((dens & (smax > 0.05)).sum())
    # the kept block is the surviving Gaussians in their original order
    keep_idx = np.nonzero(~prune & ~(dens & (smax > 0.05)))[0]
    np.testing.assert_array_equal(r["params"][:, :kept], p[:, keep_idx])
