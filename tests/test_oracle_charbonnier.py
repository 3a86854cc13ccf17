"""The oracle's Charbonnier loss with per-image exposure, pinned to closed forms and to
central finite differences in fp64.

[GSG] the trainer's loss (after "The painting itself"): err = gain C + bias - target,
root = sqrt(err^2 + delta^2), term root - delta, slope gain err / root; "Forgiving the
camera and the light": d/d(log gain) = sum (err / root) C gain, d/d bias = sum err / root.
The mean over the 3HW elements is a reading (the L1 term's normalisation).
"""
import math

import numpy as np


def test_zero_error_is_zero(oracle):
    img = np.random.default_rng(0).random((3, 5, 7))
    loss, g, dlg, db = oracle.loss_charbonnier(img, img)
    assert loss == 0.0 and not g.any() and dlg == 0.0 and db == 0.0
    # an exposure that maps the image exactly onto the target: also zero
    lg, b = math.log(1.3), -0.05
    tgt = 1.3 * img - 0.05
    loss, g, dlg, db = oracle.loss_charbonnier(img, tgt, log_gain=lg, bias=b)
    assert abs(loss) < 1e-15 and np.abs(g).max() < 1e-12 and abs(dlg) < 1e-12 and abs(db) < 1e-12


def test_single_element_closed_form(oracle):
    img = np.zeros((3, 1, 1))
    tgt = np.zeros((3, 1, 1))
    img[0, 0, 0] = 0.4
    loss, g, dlg, db = oracle.loss_charbonnier(img, tgt, delta=0.03)
    r = math.sqrt(0.16 + 0.0009)
    assert math.isclose(loss, (r - 0.03) / 3, rel_tol=1e-14)
    assert math.isclose(g[0, 0, 0], 0.4 / r / 3, rel_tol=1e-14)
    assert g[1, 0, 0] == 0.0 and g[2, 0, 0] == 0.0
    assert math.isclose(db, 0.4 / r / 3, rel_tol=1e-14)
    assert math.isclose(dlg, 0.4 / r * 0.4 / 3, rel_tol=1e-14)


def test_large_errors_behave_like_l1(oracle):
    rng = np.random.default_rng(1)
    img = rng.random((3, 6, 6))
    tgt = img + rng.choice([-5.0, 5.0], img.shape)
    loss, g, _, _ = oracle.loss_charbonnier(img, tgt, delta=0.03)
    n = img.size
    # slope -> sign(err) / n, term -> |err| - delta, to second order in delta / |err|
    np.testing.assert_allclose(g * n, -np.sign(tgt - img), rtol=0, atol=0.03 ** 2 / 25)
    assert math.isclose(loss, np.abs(tgt - img).mean() - 0.03, rel_tol=1e-4)


def test_gradients_match_central_differences(oracle):
    rng = np.random.default_rng(2)
    img = rng.random((3, 4, 5))
    tgt = rng.random((3, 4, 5))
    lg, b, d = 0.2, 0.03, 0.05
    loss, g, dlg, db = oracle.loss_charbonnier(img, tgt, delta=d, log_gain=lg, bias=b)
    h = 1e-6

    def L(im=img, lg_=lg, b_=b):
        return oracle.loss_charbonnier(im, tgt, delta=d, log_gain=lg_, bias=b_)[0]
    for idx in [(0, 0, 0), (1, 2, 3), (2, 3, 4), (0, 1, 1)]:
        p, m = img.copy(), img.copy()
        p[idx] += h
        m[idx] -= h
        assert math.isclose(g[idx], (L(im=p) - L(im=m)) / (2 * h), rel_tol=1e-6)
    assert math.isclose(dlg, (L(lg_=lg + h) - L(lg_=lg - h)) / (2 * h), rel_tol=1e-6)
    assert math.isclose(db, (L(b_=b + h) - L(b_=b - h)) / (2 * h), rel_tol=1e-6)
