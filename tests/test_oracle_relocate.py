"""The oracle's relocation of dead Gaussians ([GSG] "Densification", the MCMC-style pass:
the dead (opacity below about 0.02) are moved next to donors (above about 0.4), the largest
donors first; both shrink by 1.6 and restart their Adam moments).

Pins: a six-Gaussian population worked by hand (which Gaussian moves where, the offset
mean + s eps for an identity rotation, the shrink, which moments are reset and which are
kept, ties between equal donor sizes in index order, the move cap); with a rotated donor,
the offset has the length of s eps; on a random population, the number of moves is the
smaller of the two counts and every moved Gaussian carries its donor's opacity and colour.
"""
import math

import numpy as np

from differentiable_tile_gaussian_amd import scenes

SHRINK = np.float32(math.log(1.6))


def _hand_case():
    P, n = scenes.num_planes(0), 6
    p = np.zeros((P, n), np.float32)
    p[0:3] = np.arange(3 * n, dtype=np.float32).reshape(3, n) * 0.25
    p[3:6] = -2.0
    p[6] = 1.0                                          # identity quaternions
    p[10] = [-5.0, 2.0, -1.0, -4.5, 1.0, 3.0]           # dead, donor, neither, dead, donor, donor
    p[3:6, 1] = (-2.0, -1.0, -3.0)                      # donor sizes: G1 -1, G4 0, G5 -1
    p[3:6, 4] = (0.0, -2.0, -2.0)
    p[3:6, 5] = (-1.0, -1.5, -2.5)
    p[11:14] = np.arange(3 * n, dtype=np.float32).reshape(3, n) / 20.0
    m = np.full((P, n), 0.5, np.float32)
    v = np.full((P, n), 0.25, np.float32)
    rand = np.random.default_rng(0).standard_normal((n, 3)).astype(np.float32)
    return p, m, v, rand


def test_hand_worked_population(oracle):
    p, m, v, rand = _hand_case()
    out = oracle.relocate(p, m, v, rand, 0)
    # ranking: G4 (largest log-scale 0), then G1 and G5 (both -1, index order); dead G0, G3
    assert out["moves"] == 2
    want = p.copy()
    for bi, bd in ((0, 4), (3, 1)):
        s = np.exp(p[3:6, bd].astype(np.float64)).astype(np.float32)
        want[:, bi] = p[:, bd]
        want[0:3, bi] = p[0:3, bd] + s * rand[bi]      # identity rotation: the offset is s eps
        want[3:6, bi] = p[3:6, bd] - SHRINK
        want[3:6, bd] = p[3:6, bd] - SHRINK
    np.testing.assert_array_equal(out["params"], want)
    reset = [0, 1, 3, 4]
    assert not out["m"][:, reset].any() and not out["v"][:, reset].any()
    np.testing.assert_array_equal(out["m"][:, [2, 5]], m[:, [2, 5]])
    np.testing.assert_array_equal(out["v"][:, [2, 5]], v[:, [2, 5]])
    # the cap: one move, to the largest donor
    one = oracle.relocate(p, m, v, rand, 0, max_moves=1)
    assert one["moves"] == 1
    np.testing.assert_array_equal(one["params"][:, 0], want[:, 0])
    np.testing.assert_array_equal(one["params"][:, [1, 2, 3, 5]], p[:, [1, 2, 3, 5]])


def test_rotated_donor_offset_length(oracle):
    p, m, v, rand = _hand_case()
    q = np.array([0.7, -0.3, 0.5, 0.4], np.float32)
    p[6:10, 4] = q * 2.5                               # unnormalised on purpose
    out = oracle.relocate(p, m, v, rand, 0)
    s = np.exp(p[3:6, 4].astype(np.float64))
    off = out["params"][0:3, 0].astype(np.float64) - p[0:3, 4]
    assert math.isclose(np.linalg.norm(off), np.linalg.norm(s * rand[0]), rel_tol=1e-5)
    assert not math.isclose(off[0], s[0] * rand[0, 0], rel_tol=1e-3)   # it is rotated


def test_random_population_invariants(oracle):
    n, deg = 5000, 1
    p = scenes.random_scene(9, n, deg).params.copy()
    rng = np.random.default_rng(9)
    p[10] = rng.normal(-1.0, 2.5, n).astype(np.float32)
    p[3:6] += rng.normal(0, 0.7, (3, n)).astype(np.float32)
    m = rng.standard_normal(p.shape).astype(np.float32)
    v = rng.random(p.shape).astype(np.float32)
    rand = rng.standard_normal((n, 3)).astype(np.float32)
    o = 1.0 / (1.0 + np.exp(-p[10].astype(np.float64)))
    dead, donors = np.nonzero(o < 0.02)[0], np.nonzero(o > 0.4)[0]
    out = oracle.relocate(p, m, v, rand, deg)
    k = min(dead.size, donors.size)
    assert out["moves"] == k > 100
    moved = dead[:k]
    # every moved Gaussian now has a donor's opacity and colour, and the donors used are the
    # k largest by their largest log-scale
    size = p[3:6].max(axis=0)
    used = donors[np.argsort(-size[donors], kind="stable")[:k]]
    np.testing.assert_array_equal(out["params"][10, moved], p[10, used])
    np.testing.assert_array_equal(out["params"][11:, moved], p[11:, used])
    untouched = np.setdiff1d(np.arange(n), np.concatenate([moved, used]))
    np.testing.assert_array_equal(out["params"][:, untouched], p[:, untouched])
    np.testing.assert_array_equal(out["m"][:, untouched], m[:, untouched])
