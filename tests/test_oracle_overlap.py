"""Depth complexity (the oracle's overlap count): per pixel, the entries of its tile's
list whose alpha reaches 1/255 over the whole list, with no early stop.

A hand-built pin: forty Gaussians of opacity 0.5 centred on one pixel count forty there
although the blend stops after fourteen (0.5^14 < 1e-4, [GSG] "The painting itself"), a
Gaussian of opacity 0.003 (below 1/255 everywhere, [GST] opacity slide) is listed but not
counted, and a pixel of the same tile far from the centre counts none.  Then, per workload,
the tile-list lengths and the overlap over a seeded sample of pixels, and the property the
high depth-complexity workload (3M Gaussians in a slab before a 1280x720 camera) is built
to have: a median overlap of at least 200 entries per pixel."""
import math

import numpy as np
import pytest

from differentiable_tile_gaussian_amd import scenes


def test_overlap_counts_every_entry_at_or_above_the_floor(oracle):
    K = 40
    cam = scenes.identity_camera(32, 32, 32.0)
    zs = (2.0 + 0.1 * np.arange(K + 1)).astype(np.float32)
    p = np.zeros((14, K + 1), np.float32)
    p[0] = p[1] = np.float32((8.5 - 16.0) / 32.0) * zs    # screen centre (8.5, 8.5): pixel (8, 8)
    p[2] = zs
    p[3:6] = math.log(0.05)
    p[6] = 1.0
    p[10, K] = math.log(0.003 / 0.997)                      # the last one: opacity 0.003
    p[11:14] = 0.5
    pre = oracle.preprocess(p, 0, cam)
    assert (pre["tiles"] == 1).all()                        # all listed, in tile 0 only
    _, vals, ranges = oracle.bin_sort(pre, cam)
    c = oracle.overlap_pixels(pre, vals, ranges, cam, [8, 0, 30], [8, 15, 30])
    assert list(c) == [K, 0, 0]
    stop = oracle.render_pixels(pre, vals, ranges, cam, [8], [8])["n_contrib"][0]
    assert stop == 14                                        # the blend itself stops early


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workload_depth_complexity(oracle, cfg):
    """Per workload (camera 0): pairs, median and largest tile-list length, and the overlap
    over 2048 seeded pixels; the high depth-complexity workload (3M Gaussians) must reach a
    median overlap of 200."""
    wl = scenes.CONFIGS[cfg]()
    cam = wl.cameras[0]
    pre = oracle.preprocess(wl.scene.params, wl.scene.sh_degree, cam)
    _, vals, ranges = oracle.bin_sort(pre, cam)
    lens = ranges[1].astype(np.int64) - ranges[0]
    rng = np.random.default_rng(400 + cfg)
    xs, ys = rng.integers(0, cam.width, 2048), rng.integers(0, cam.height, 2048)
    c = oracle.overlap_pixels(pre, vals, ranges, cam, xs, ys)
    q = np.percentile(c, [25, 50, 75])
    print(f"workload {cfg}: {len(vals)} pairs, tile lists median {int(np.median(lens))} max {lens.max()}, "
          f"overlap quartiles {q} max {c.max()}")
    assert lens.sum() == len(vals) and c.max() <= lens.max()
    if cfg == 4:
        assert np.median(c) >= 200
